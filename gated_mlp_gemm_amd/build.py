"""Build the HIP library ``libswiglu.so`` in-tree for gfx950.

    python -m gated_mlp_gemm_amd.build [--isa]

Compiles ``csrc/kernels.hip`` (device code) and ``csrc/api.cpp`` (the C ABI)
with hipcc and links them into ``gated_mlp_gemm_amd/libswiglu.so``.  ``--isa``
also keeps the gfx950 assembly under ``_build/`` for inspection.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libswiglu.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(isa: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    k_obj = os.path.join(BUILD, "kernels.o")
    a_obj = os.path.join(BUILD, "api.o")
    extra = ["-save-temps=obj"] if isa else []
    out = _run([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, "kernels.hip"), "-o", k_obj])
    out += _run([HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", a_obj])
    tmp = LIBRARY + ".tmp"
    out += _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", k_obj, a_obj, "-o", tmp])
    os.replace(tmp, LIBRARY)
    if verbose and out.strip():
        print(out)
    return LIBRARY


def device_assembly(path: str) -> str:
    """Compile csrc/kernels.hip's device code alone, with the library's flags,
    to gfx950 assembly at `path`; returns `path`."""
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    _run([HIPCC, *COMMON, "--cuda-device-only", "-S", os.path.join(CSRC, "kernels.hip"),
          "-o", path])
    return path


if __name__ == "__main__":
    path = build(isa="--isa" in sys.argv, verbose=True)
    print(path)
