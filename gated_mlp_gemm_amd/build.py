"""Build the HIP library ``libswiglu.so`` in-tree for gfx950.

    python -m gated_mlp_gemm_amd.build [--jobs N]

Compiles ``csrc/kernels.hip`` (elementwise kernels and the launch dispatch),
``csrc/kernel_instances.hip`` once per group of its instance list (the tile
kernels, one object per group) and ``csrc/api.cpp`` (the C ABI) with hipcc,
in parallel (``--jobs``, else ``MAX_JOBS``, else the CPU count), and links
them into ``gated_mlp_gemm_amd/libswiglu.so``.  The link refuses undefined
symbols, so an instance the dispatch calls but the list leaves out fails the
build.

Every object is compiled with ``-save-temps=obj`` into a folder of its own
under ``_build/obj/``, and the gfx950 assembly of its device code is kept
there beside it (the other intermediates are deleted): the assembly is what
the library's code objects were assembled from.  ``device_assembly()``
returns it, building first unless the last build was of the current sources
and flags.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import glob
import hashlib
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
OBJ = os.path.join(BUILD, "obj")
STAMP = os.path.join(OBJ, "STAMP")
LIBRARY = os.path.join(PKG, "libswiglu.so")
INSTANCES = os.path.join(CSRC, "kernel_instances.hip")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]
DEVICE_ASM = f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def instance_groups() -> int:
    """Number of groups in kernel_instances.hip's instance list (0..n-1)."""
    with open(INSTANCES, encoding="utf-8") as f:
        found = [int(g) for g in re.findall(r"SWIGLU_INSTANCE == (\d+)", f.read())]
    if not found or sorted(found) != list(range(len(found))):
        raise RuntimeError(f"{INSTANCES}: instance groups must be numbered 0..n-1, got {found}")
    return len(found)


def _objects():
    """(name, source, extra flags) of every object of the library, the
    instance groups first (the list puts the longest compiles first)."""
    objs = [(f"inst{g:02d}", INSTANCES, [f"-DSWIGLU_INSTANCE={g}"])
            for g in range(instance_groups())]
    objs.append(("kernels", os.path.join(CSRC, "kernels.hip"), []))
    objs.append(("api", os.path.join(CSRC, "api.cpp"), ["-x", "hip"]))
    return objs


def source_digest() -> str:
    """Hash of the compiler, the flags, the sources under csrc/ and the
    public headers: a build is current when its stamp holds this."""
    h = hashlib.sha256()
    h.update(repr((HIPCC, COMMON, _objects())).encode())
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _compile(name, source, extra):
    d = os.path.join(OBJ, name)
    shutil.rmtree(d, ignore_errors=True)
    os.makedirs(d)
    obj = os.path.join(d, name + ".o")
    out = _run([HIPCC, *COMMON, *extra, "-save-temps=obj", "-c", source, "-o", obj])
    asm = glob.glob(os.path.join(d, DEVICE_ASM))
    if len(asm) != 1:
        raise RuntimeError(f"{name}: expected one device assembly file in {d}, found {asm}")
    for path in os.listdir(d):
        full = os.path.join(d, path)
        if full not in (obj, asm[0]):
            os.remove(full)
    return obj, out


def build(isa: bool = False, verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every object and link the library; returns its path.  (`isa`
    is accepted for compatibility: the device assembly is always kept.)"""
    del isa
    digest = source_digest()
    os.makedirs(OBJ, exist_ok=True)
    if os.path.exists(STAMP):
        os.remove(STAMP)
    jobs = jobs or int(os.environ.get("MAX_JOBS") or os.cpu_count() or 1)
    objs = _objects()
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as pool:
        results = list(pool.map(lambda o: _compile(*o), objs))
    out = "".join(r[1] for r in results)
    tmp = LIBRARY + ".tmp"
    out += _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined",
                 *(r[0] for r in results), "-o", tmp])
    os.replace(tmp, LIBRARY)
    with open(STAMP, "w") as f:
        f.write(digest + "\n")
    if verbose and out.strip():
        print(out)
    return LIBRARY


def device_assembly(path: str) -> str:
    """Write the gfx950 assembly of all of the library's device code to
    `path` (building first unless the last build is current); returns
    `path`."""
    current = False
    if os.path.exists(STAMP):
        with open(STAMP) as f:
            current = f.read().strip() == source_digest()
    if not current:
        build()
    parts = []
    for name, _, _ in _objects():
        asm = glob.glob(os.path.join(OBJ, name, DEVICE_ASM))
        if len(asm) != 1:
            raise RuntimeError(f"no device assembly for {name} under {OBJ}")
        with open(asm[0]) as f:
            parts.append(f.read())
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(parts))
    return path


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--isa", action="store_true", help="(the assembly is always kept)")
    args = ap.parse_args()
    print(build(verbose=True, jobs=args.jobs))
