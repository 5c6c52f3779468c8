"""Invariants of the compiled gfx950 code (CPU: hipcc cross-compiles).

The 16x16x32 bf16 MFMAs are written as inline assembly (tied accumulator
operands keep the compiler from rotating accumulators through other
registers), so the compiler's hazard recognizer does not see them as MFMAs:
the waits their results need are the kernels' own (wait_mfma_results,
zero_acc's nop).  Those waits only cover the instructions the kernels write.
A copy the register allocator inserts on its own -- an AGPR-to-AGPR move, or
an accumulator read out to a VGPR -- right after an MFMA that still writes
that accumulator reads a stale value, and the result depends on timing.
This test reads the device assembly the library was built from (compiling
it first unless the last build is of the current sources) and checks, in
every kernel that has these MFMAs:

  * no AGPR-to-AGPR copy (v_accvgpr_mov) at all;
  * every read or write of an accumulator by a VALU instruction
    (v_accvgpr_read / v_accvgpr_write) comes at least 19 wait states after the
    last MFMA writing it (the CDNA3/CDNA4 requirement for a VALU access after
    an XDL write is at most 19, for 16-pass MFMAs; 8-pass ones need 11);
  * no MFMA reads an operand a VALU instruction wrote fewer than 2 wait
    states before;

and in every kernel: no VGPR spills.  Wait states are counted backwards
along every control-flow path into the instruction (the previous
instruction unless it is an unconditional branch or the end, and every
branch to a label in front of it): one per instruction, N+1 for s_nop N.
"""
from __future__ import annotations

import os
import re
import tempfile

import pytest

from gated_mlp_gemm_amd import build

ASM_MFMA = "v_mfma_f32_16x16x32_bf16"
XDL_TO_VALU = 19
VALU_TO_XDL = 2

_RANGE = re.compile(r"\b([va])\[(\d+):(\d+)\]")
_SINGLE = re.compile(r"\b([va])(\d+)\b")


def _regs(operand: str) -> set:
    out = set()
    for m in _RANGE.finditer(operand):
        out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
    for m in _SINGLE.finditer(_RANGE.sub(" ", operand)):
        out.add(m.group(1) + m.group(2))
    return out


def _operands(ins: str) -> list:
    parts = ins.split(None, 1)
    return [p.strip() for p in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(ins: str) -> int:
    if ins.startswith("s_nop"):
        return int(ins.split()[1], 0) + 1
    return 1


@pytest.fixture(scope="module")
def assembly():
    with tempfile.TemporaryDirectory() as d:
        path = build.device_assembly(os.path.join(d, "kernels.s"))
        with open(path) as f:
            text = f.read()
    kernels = {}
    functions = set(re.findall(r"\.type\s+(_Z\w+),@function", text))
    for m in re.finditer(r"^(_Z\w+):", text, re.M):
        if m.group(1) not in functions:   # a device variable's label
            continue
        end = text.find(".Lfunc_end", m.end())
        body = text[m.end():end]
        lines = []
        for raw in body.split("\n"):
            line = raw.split(";")[0].strip()
            if not line or (line.startswith(".") and not line.endswith(":")):
                continue
            lines.append(line)
        kernels[m.group(1)] = lines
    spills = {}
    name = None
    for line in text.split("\n"):
        line = line.strip()
        if line.startswith(".name:"):
            name = line.split(":", 1)[1].strip()
        elif line.startswith(".vgpr_spill_count:") and name:
            spills[name] = int(line.split(":", 1)[1])
    return kernels, spills


_NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc_b64")


def _flow(lines):
    """Instructions (labels dropped) and, for each, the instructions that can
    run right before it."""
    ins, label_at, pending = [], {}, []
    for line in lines:
        if line.endswith(":"):
            pending.append(line[:-1])
            continue
        for name in pending:
            label_at[name] = len(ins)
        pending = []
        ins.append(line)
    preds = [[] for _ in ins]
    for i, line in enumerate(ins):
        op = line.split()[0]
        if i + 1 < len(ins) and op not in _NO_FALLTHROUGH:
            preds[i + 1].append(i)
        if op == "s_branch" or op.startswith("s_cbranch"):
            target = line.split()[-1]
            if target in label_at:
                preds[label_at[target]].append(i)
    return ins, preds


def _hit_before(ins, preds, i, hit, limit):
    """(instruction, wait states between) for an instruction satisfying `hit`
    that can run fewer than `limit` wait states before instruction i, or None."""
    stack, seen = [(p, 0) for p in preds[i]], set()
    while stack:
        j, waited = stack.pop()
        if (j, waited) in seen:
            continue
        seen.add((j, waited))
        if hit(ins[j]):
            return ins[j], waited
        waited += _wait_states(ins[j])
        if waited < limit:
            stack.extend((p, waited) for p in preds[j])
    return None


def _asm_mfma_kernels(kernels):
    return {k: v for k, v in kernels.items() if any(i.startswith(ASM_MFMA) for i in v)}


def test_assembly_has_the_kernels(assembly):
    kernels, spills = assembly
    mf = _asm_mfma_kernels(kernels)
    names = " ".join(mf)
    assert "gemm_tiles_kernel" in names and "fused_sequential_persistent_kernel" in names
    assert sum(i.startswith("v_accvgpr_read") for v in mf.values() for i in v) > 0
    assert set(kernels) == set(spills)


def test_no_vgpr_spills(assembly):
    _, spills = assembly
    bad = {k: v for k, v in spills.items() if v}
    assert not bad, bad


def test_no_accumulator_moves(assembly):
    kernels, _ = assembly
    bad = {k: sum(i.startswith("v_accvgpr_mov") for i in v)
           for k, v in _asm_mfma_kernels(kernels).items()}
    bad = {k: n for k, n in bad.items() if n}
    assert not bad, bad


def _late_accumulator_accesses(lines):
    """(access, MFMA, wait states between) for each VALU access of an
    accumulator that can come fewer than XDL_TO_VALU wait states after an
    MFMA writing it."""
    ins, preds = _flow(lines)
    problems = []
    for i, line in enumerate(ins):
        if line.startswith("v_accvgpr_read"):
            regs = _regs(_operands(line)[1])
        elif line.startswith("v_accvgpr_write"):
            regs = _regs(_operands(line)[0])
        else:
            continue
        found = _hit_before(ins, preds, i, lambda x: x.startswith("v_mfma") and
                            bool(_regs(_operands(x)[0]) & regs), XDL_TO_VALU)
        if found:
            problems.append((line, *found))
    return problems


def _early_mfma_operands(lines):
    """(MFMA, VALU write, wait states between) for each MFMA operand that a
    VALU instruction can write fewer than VALU_TO_XDL wait states before."""
    ins, preds = _flow(lines)
    problems = []
    for i, line in enumerate(ins):
        if not line.startswith("v_mfma"):
            continue
        srcs = set()
        for op in _operands(line)[1:]:
            srcs |= _regs(op)

        def writes_src(x):
            if not x.startswith("v_") or x.startswith("v_mfma"):
                return False
            ops = _operands(x)
            return bool(ops) and bool(_regs(ops[0]) & srcs)

        found = _hit_before(ins, preds, i, writes_src, VALU_TO_XDL)
        if found:
            problems.append((line, *found))
    return problems


def test_checkers_on_known_sequences():
    mfma = "v_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[8:11], a[4:7]"
    # read of the result right after the MFMA: flagged; after the kernels' wait: not
    assert _late_accumulator_accesses([mfma, "s_waitcnt lgkmcnt(0)", "v_accvgpr_read_b32 v20, a6"])
    assert not _late_accumulator_accesses([mfma, "s_nop 7", "s_nop 7", "s_nop 7",
                                           "v_accvgpr_read_b32 v20, a6"])
    # a register the MFMA does not write: not flagged
    assert not _late_accumulator_accesses([mfma, "v_accvgpr_read_b32 v20, a8"])
    # overwrite of the result while the MFMA runs: flagged
    assert _late_accumulator_accesses([mfma, "v_accvgpr_write_b32 a7, 0"])
    # an operand written by VALU just before the MFMA: flagged; after s_nop 1: not
    assert _early_mfma_operands(["v_accvgpr_write_b32 a5, 0", mfma])
    assert _early_mfma_operands(["v_mov_b32 v9, 0", mfma])
    assert not _early_mfma_operands(["v_accvgpr_write_b32 a5, 0", "s_nop 1", mfma])
    assert not _early_mfma_operands(["v_mov_b32 v12, 0", mfma])
    # control flow: no path from the MFMA past an unconditional branch ...
    assert not _late_accumulator_accesses([mfma, "s_branch .LBB0_2", ".LBB0_1:",
                                           "v_accvgpr_read_b32 v20, a6", ".LBB0_2:", "s_endpgm"])
    # ... but a branch to the label is one, and so is a loop's back edge
    assert _late_accumulator_accesses([mfma, "s_cbranch_scc1 .LBB0_1", "s_nop 7", "s_nop 7",
                                       "s_nop 7", ".LBB0_1:", "v_accvgpr_read_b32 v20, a6"])
    assert _late_accumulator_accesses([".LBB0_1:", "v_accvgpr_read_b32 v20, a6", "s_nop 7",
                                       "s_nop 7", "s_nop 7", mfma, "s_cbranch_scc1 .LBB0_1"])


def test_accumulator_access_waits_for_mfma(assembly):
    kernels, _ = assembly
    problems = [(k[:60], *p) for k, v in _asm_mfma_kernels(kernels).items()
                for p in _late_accumulator_accesses(v)]
    assert not problems, problems[:5]


def test_mfma_operands_settled(assembly):
    kernels, _ = assembly
    problems = [(k[:60], *p) for k, v in _asm_mfma_kernels(kernels).items()
                for p in _early_mfma_operands(v)]
    assert not problems, problems[:5]
