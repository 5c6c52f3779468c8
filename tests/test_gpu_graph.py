"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph): the
launches allocate nothing, clear nothing and synchronise nothing, so a
captured call replays to the eager result bit for bit.  Each replay follows
eager work and a synchronisation, the output is poisoned before it, and the
input is changed in place between replays (the graph reads the live buffers).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_mlp_gemm_amd import inputs
from gated_mlp_gemm_amd import swiglu as sw

pytestmark = pytest.mark.gpu

POISON = -21846   # 0xAAAA as int16: a bf16 pattern no call here produces by chance


@pytest.fixture(autouse=True)
def _default_dispatch(monkeypatch):
    monkeypatch.delenv("SWIGLU_M_SWITCH", raising=False)
    monkeypatch.delenv("SWIGLU_I_TILE", raising=False)
    monkeypatch.delenv("SWIGLU_TAIL", raising=False)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sw.load_library()
    return torch.device("cuda:0")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().copy()


def _setup(case, dev):
    """(call(outputs), outputs, input to perturb, eager work) for one case."""
    kind, M, K, N, use_ws = case
    A, W1, W2, W3 = inputs.make_mlp_inputs(M, K, N, seed=M + K + N)
    Ad = A.to(dev)
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    if kind == "fp8":
        a_exp = sw.swiglu_fp8_scale_exp(float(Ad.float().abs().max()))
        w_exp = sw.swiglu_fp8_scale_exp(float(Wf.float().abs().max()))
        A8 = sw.swiglu_quantize_fp8(Ad, a_exp)
        W8 = sw.swiglu_quantize_fp8(Wf, w_exp)
        ws = sw.make_workspace(M, N, K, "fp8", dev) if use_ws else None
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev)]

        def call(o):
            sw.swiglu_fused_gemm_fp8(A8, W8, a_exp, w_exp, Y=o[0], workspace=ws)
        return call, outs, A8
    if kind == "mlp":
        W3t = W3.t().contiguous().to(dev)
        ws = sw.make_workspace(M, N, K, "down_proj", dev) if use_ws else None
        outs = [torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                torch.empty((M, N), dtype=torch.bfloat16, device=dev)]

        def call(o):
            sw.swiglu_gated_mlp(Ad, Wf, W3t, Out=o[0], H=o[1], workspace=ws)
        return call, outs, Ad
    ws = sw.make_workspace(M, N, K, kind, dev) if use_ws else None
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev)]

    def call(o):
        sw.swiglu_fused_gemm(Ad, Wf, Y=o[0], variant=kind, workspace=ws)
    return call, outs, Ad


CASES = [("i", 128, 896, 4864, False), ("i", 128, 3584, 4864, True), ("i", 2048, 1536, 8960, True),
         ("i", 600, 4096, 392, True), ("s", 300, 512, 1000, False),
         ("fp8", 128, 896, 4864, False), ("fp8", 2048, 1536, 8960, True),
         ("mlp", 256, 512, 768, True)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" + ("-ws" if c[4] else "")
                                             for c in CASES])
def test_graph_replays_match_eager(dev, case):
    print(f"\n[case] graph {case}", flush=True)
    call, outs, inp = _setup(case, dev)
    # eager references, and the capture's lazy initialisation done outside it
    call(outs)
    torch.cuda.synchronize()
    ref = [_bits(o) for o in outs]
    static = [torch.empty_like(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(static)
    torch.cuda.synchronize()
    for r in range(3):
        for o in static:
            o.view(torch.int16).fill_(POISON)
        call(outs)                       # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, o in enumerate(static):
            assert np.array_equal(_bits(o), ref[k]), f"replay {r}, output {k} differs from eager"
    # the graph reads the live input: change it in place, compare with eager
    if inp.dtype == torch.uint8:
        inp.copy_(torch.flip(inp, dims=[0]))
    else:
        inp.mul_(-0.5)
    call(outs)
    torch.cuda.synchronize()
    ref2 = [_bits(o) for o in outs]
    assert any(not np.array_equal(a, b) for a, b in zip(ref, ref2))
    for o in static:
        o.view(torch.int16).fill_(POISON)
    g.replay()
    torch.cuda.synchronize()
    for k, o in enumerate(static):
        assert np.array_equal(_bits(o), ref2[k]), f"replay on new input, output {k}"
