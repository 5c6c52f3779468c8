"""swiglu_fused_gemm_noalloc (the entry point for callers that cannot
allocate) against swiglu_fused_gemm with a caller workspace, through the C
ABI: the same kernels and schedule, so the outputs must be equal bit for bit,
and both must meet the oracle's bar.  Two calls in a row whose tails are split
along K (so the library's static scratch holds the partials), the second on a
smaller problem, so that partials left by the first call cannot leak into the
second's result; then an AUTO call with the library's own schedule choice."""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import oracle as oracle_pkg
from gated_mlp_gemm_amd import inputs
from gated_mlp_gemm_amd import swiglu as sw

pytestmark = pytest.mark.gpu


def _bits(t):
    return inputs.bits(t.detach().cpu())


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sw.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle_pkg.load()


def _check(dev, orc, M, K, N, seed, variant, forced, expect=None):
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=seed)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad = A.to(dev)
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    n = sw.swiglu_workspace_size(M, N, K, variant)
    ws = torch.full((max(n, 256),), 0xFF, dtype=torch.uint8, device=dev)
    desc = sw.swiglu_describe_launch(M, N, K, variant, n)
    print(f"\n[case] no-alloc {variant} M={M} K={K} N={N}: {desc}", flush=True)
    if forced:
        assert "split_reduce_kernel" in desc, desc
    if expect:
        assert expect in desc, desc
    Y_ws = sw.swiglu_fused_gemm(Ad, Wf, variant=variant, workspace=ws if n else None)
    Y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    sw.swiglu_fused_gemm_noalloc(Ad, Wf, Y_na, variant=variant)
    torch.cuda.synchronize()
    a, b = _bits(Y_na), _bits(Y_ws)
    assert np.array_equal(a, b), f"{int((a != b).sum())} elements differ from the workspace call"
    rep = oracle_pkg.parity_report(a, ref)
    print(f"  {json.dumps(rep)}", flush=True)
    assert rep["mismatches"] == 0, rep


def test_noalloc_matches_workspace_call(dev, orc, monkeypatch):
    monkeypatch.setenv("SWIGLU_I_TILE", "256")
    monkeypatch.setenv("SWIGLU_TAIL", "split")
    # 8 x 9 tiles of 256 x 256 split 3 ways; then 2 x 2 tiles split 16 ways
    _check(dev, orc, 2048, 1536, 1032, 71, "i", forced=True)
    _check(dev, orc, 300, 1000, 136, 72, "i", forced=True)
    monkeypatch.delenv("SWIGLU_I_TILE")
    monkeypatch.delenv("SWIGLU_TAIL")
    _check(dev, orc, 777, 520, 2056, 73, "auto", forced=False)
    _check(dev, orc, 257, 136, 264, 74, "s", forced=False)
    # M <= 128: split along K and reduced in the kernel (library-owned
    # counters beside the static partials), twice in a row, then smaller
    _check(dev, orc, 128, 3584, 4864, 75, "i", forced=False, expect="reduced in the kernel")
    _check(dev, orc, 128, 3584, 4864, 76, "i", forced=False, expect="reduced in the kernel")
    monkeypatch.setenv("SWIGLU_TAIL", "fixup")
    _check(dev, orc, 100, 520, 4600, 77, "auto", forced=False, expect="reduced in the kernel")
