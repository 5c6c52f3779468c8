"""Operands beyond 4 GiB: the 64-bit bases of the weight and activation panels
and of the output tiles (every in-kernel offset is 32 bits, taken from a
per-panel or per-tile base), at the largest K the library accepts.

Inputs are drawn on the device (the make_inputs recipe with a device
generator: several GiB would take the CPU generator minutes); the oracle gets
the drawn values copied to the host, and the parity predicate is the one of
the other parity tests:  |y - ref| <= max(1e-3, 1e-2 |ref|).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as oracle_pkg
from gated_mlp_gemm_amd import inputs
from gated_mlp_gemm_amd import swiglu as sw
from test_gpu_parity import (_intermediate_within_bound, announce, assert_parity, ulp_distance,
                             workspace_for)

pytestmark = pytest.mark.gpu

GIB = 1 << 30
K_MAX = 1 << 21          # largest K swiglu_fused_gemm accepts


@pytest.fixture(autouse=True)
def _default_dispatch(monkeypatch):
    monkeypatch.delenv("SWIGLU_M_SWITCH", raising=False)
    monkeypatch.delenv("SWIGLU_I_TILE", raising=False)
    monkeypatch.delenv("SWIGLU_TAIL", raising=False)


@pytest.fixture(scope="module")
def orc():
    return oracle_pkg.load()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sw.load_library()
    return torch.device("cuda:0")


def _u16(t: torch.Tensor) -> np.ndarray:
    return inputs.bits(t.detach().cpu())


def _run(A, Wf, variant):
    ws = None
    if variant.endswith("+ws"):
        variant = variant[:-3]
        ws = workspace_for(A.shape[0], Wf.shape[0] // 2, A.shape[1], variant, A.device)
    Y = sw.swiglu_fused_gemm(A, Wf, variant=variant, workspace=ws)
    torch.cuda.synchronize()
    return Y


# ---------------------------------------------------------------------------
# K at its maximum: W1 and W2 of 4 GiB each, the packed weight 8 GiB, so the
# weight panels of the later tile columns start beyond 4 GiB
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def max_k(dev):
    M, K, N = 130, K_MAX, 1024
    announce(f"inputs M={M} K={K} N={N} (W_fused {2 * N * K * 2 / GIB:.0f} GiB), device draw")
    A, W1, W2 = inputs.device_inputs(M, K, N, seed=21, device=dev)
    Wf = sw.swiglu_pack_weights(W1, W2)
    torch.cuda.synchronize()
    assert Wf.numel() * 2 > 4 * GIB
    d = dict(M=M, K=K, N=N, A=A, Wf=Wf, hA=_u16(A), hW1=_u16(W1), hW2=_u16(W2), ref={})
    del W1, W2
    yield d
    d.clear()
    torch.cuda.empty_cache()


def _max_k_reference(orc, d, M):
    """Whole rows (every tile column, so every weight panel): the first, the
    middle and the last (ragged tile row at M = 130)."""
    if M not in d["ref"]:
        rows = np.unique(np.array([0, M // 2, M - 1]))
        announce(f"oracle rows {list(rows)}, M={M} K={d['K']}")
        d["ref"][M] = (rows, orc.swiglu_rows(d["hA"][:M], d["hW1"], d["hW2"], rows))
    return d["ref"][M]


@pytest.mark.parametrize("M", [8, 130])
@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_weights_beyond_4gib_at_max_k(dev, orc, max_k, M, variant):
    d = max_k
    rows, ref_rows = _max_k_reference(orc, d, M)
    announce(f"fused {variant} M={M} K={d['K']} N={d['N']}: "
             + sw.swiglu_describe_launch(M, d["N"], d["K"], variant.split("+")[0]))
    Y = _run(d["A"][:M], d["Wf"], variant)
    assert_parity(_u16(Y)[rows], ref_rows, f"{variant} M={M} rows")


# ---------------------------------------------------------------------------
# M near 2^20: A (4 GiB + a ragged tail of 37 rows) and Y (4.5 GiB) both
# extend past 4 GiB, so the late tile rows' A panels and output tiles start
# there
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def big_m(dev, orc):
    M, K, N = (1 << 20) + 37, 2048, 2304
    announce(f"inputs M={M} K={K} N={N} (A {M * K * 2 / GIB:.2f} GiB, "
             f"Y {M * N * 2 / GIB:.2f} GiB), device draw")
    A, W1, W2 = inputs.device_inputs(M, K, N, seed=22, device=dev)
    Wf = sw.swiglu_pack_weights(W1, W2)
    torch.cuda.synchronize()
    assert A.numel() * 2 > 4 * GIB and M * N * 2 > 4 * GIB
    rng = np.random.default_rng(22)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 38, M - 2, M - 1],
                                     rng.integers(M - (1 << 17), M, 4)]))
    pr = rng.integers(0, M, 2000)
    pc = rng.integers(0, N, 2000)
    # the oracle needs only the sampled rows of A
    hA_rows = _u16(A[torch.from_numpy(rows).to(dev)])
    hA_pts = _u16(A[torch.from_numpy(pr).to(dev)])
    hW1, hW2 = _u16(W1), _u16(W2)
    announce(f"oracle rows {list(rows)} and {pr.size} points")
    ref_rows = orc.swiglu_rows(hA_rows, hW1, hW2, np.arange(rows.size))
    ref_pts = orc.swiglu_points(hA_pts, hW1, hW2, np.arange(pr.size), pc)
    d = dict(M=M, K=K, N=N, A=A, Wf=Wf, rows=rows, pr=pr, pc=pc, hA_rows=hA_rows, hW1=hW1,
             hW2=hW2, ref_rows=ref_rows, ref_pts=ref_pts)
    del W1, W2
    yield d
    d.clear()
    torch.cuda.empty_cache()


def _sampled(Y, d):
    dv = Y.device
    yr = _u16(Y[torch.from_numpy(d["rows"]).to(dv)])
    yp = _u16(Y[torch.from_numpy(d["pr"]).to(dv), torch.from_numpy(d["pc"]).to(dv)])
    return yr, yp


@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_activations_and_output_beyond_4gib(dev, big_m, variant):
    d = big_m
    announce(f"fused {variant} M={d['M']} K={d['K']} N={d['N']}: "
             + sw.swiglu_describe_launch(d["M"], d["N"], d["K"], variant.split("+")[0]))
    Y = _run(d["A"], d["Wf"], variant)
    yr, yp = _sampled(Y, d)
    del Y
    assert_parity(yr, d["ref_rows"], f"{variant} rows {list(d['rows'])}")
    assert_parity(yp, d["ref_pts"], f"{variant} points")


def test_ablation_beyond_4gib(dev, orc, big_m):
    """The unfused ablation (Gate, Up and Y each 4.5 GiB) with the workspace
    the benchmark gives it: sampled rows of all three against the oracle."""
    d = big_m
    announce(f"ablation M={d['M']} K={d['K']} N={d['N']}")
    ws = workspace_for(d["M"], d["N"], d["K"], "ablation", dev)
    Y, g, u = sw.swiglu_unfused_ablation(d["A"], d["Wf"], workspace=ws)
    torch.cuda.synchronize()
    idx = torch.from_numpy(d["rows"]).to(dev)
    gb, ub, yb = _u16(g[idx]), _u16(u[idx]), _u16(Y[idx])
    del Y, g, u
    sub = d["hA_rows"]
    g_ref, u_ref, y_ref = orc.swiglu_materialised(sub, d["hW1"], d["hW2"])
    _intermediate_within_bound(orc, sub, d["hW1"], gb, "ablation gate")
    _intermediate_within_bound(orc, sub, d["hW2"], ub, "ablation up")
    same = (gb == g_ref) & (ub == u_ref)
    assert ulp_distance(yb, y_ref)[same].max(initial=0) <= 1
    assert not (oracle_pkg.mismatches(yb, y_ref) & same).any()



def _amax_exp(t: torch.Tensor) -> int:
    return sw.swiglu_fp8_scale_exp(float(t.abs().max()))


# ---------------------------------------------------------------------------
# FP8: A8 (4 GiB + 37 rows of codes, quantized from 8 GiB of bf16) and Y
# (9 GiB) beyond 4 GiB; the oracle quantizes the host values itself
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def big_fp8(dev, orc):
    M, K, N = (1 << 21) + 37, 2048, 2304
    announce(f"inputs M={M} K={K} N={N} (A8 {M * K / GIB:.2f} GiB, Y {M * N * 2 / GIB:.2f} GiB)")
    A, W1, W2 = inputs.device_inputs(M, K, N, seed=23, device=dev)
    a_exp = _amax_exp(A)
    w_exp = max(_amax_exp(W1), _amax_exp(W2))
    Wf = sw.swiglu_pack_weights(W1, W2)
    A8 = sw.swiglu_quantize_fp8(A, a_exp)
    W8 = sw.swiglu_quantize_fp8(Wf, w_exp)
    torch.cuda.synchronize()
    assert A8.numel() > 4 * GIB
    rng = np.random.default_rng(23)
    rows = np.unique(np.concatenate([[0, M // 2, M - 38, M - 1], rng.integers(M - (1 << 18), M, 3)]))
    idx = torch.from_numpy(rows).to(dev)
    hA_rows = _u16(A[idx])
    dA8_rows = A8[idx].cpu().numpy()
    hW1, hW2 = _u16(W1), _u16(W2)
    del A, W1, W2, Wf
    torch.cuda.empty_cache()
    hA8_rows = orc.quantize_fp8(hA_rows, a_exp)
    hWT8 = orc.quantize_fp8(np.ascontiguousarray(orc.pack(hW1, hW2).T), w_exp)
    announce(f"oracle rows {list(rows)}, a_exp={a_exp} w_exp={w_exp}")
    ref = orc.swiglu_fp8(hA8_rows, hWT8, a_exp, w_exp)
    d = dict(M=M, K=K, N=N, A8=A8, W8=W8, a_exp=a_exp, w_exp=w_exp, rows=rows, idx=idx,
             dA8_rows=dA8_rows, hA8_rows=hA8_rows, ref=ref)
    yield d
    d.clear()
    torch.cuda.empty_cache()


def test_fp8_quantizer_beyond_4gib(dev, big_fp8):
    d = big_fp8
    assert np.array_equal(d["dA8_rows"], d["hA8_rows"]), "quantized rows differ from the oracle's"


@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_fp8_beyond_4gib(dev, big_fp8, variant):
    d = big_fp8
    v = variant.split("+")[0]
    ws = workspace_for(d["M"], d["N"], d["K"], "fp8", dev) if variant.endswith("+ws") else None
    announce(f"fp8 {variant} M={d['M']} K={d['K']} N={d['N']}")
    Y = sw.swiglu_fused_gemm_fp8(d["A8"], d["W8"], d["a_exp"], d["w_exp"], variant=v,
                                 workspace=ws)
    torch.cuda.synchronize()
    yb = _u16(Y[d["idx"]])
    del Y
    assert_parity(yb, d["ref"], f"fp8 {variant} rows {list(d['rows'])}")


# ---------------------------------------------------------------------------
# The gated MLP block on the large-M operands: H (4.5 GiB) and Out (4 GiB +
# 37 rows) beyond 4 GiB; the down projection reads H as its activation
# ---------------------------------------------------------------------------
def test_mlp_block_beyond_4gib(dev, orc, big_m):
    d = big_m
    M, K, N = d["M"], d["K"], d["N"]
    g = torch.Generator(device=dev)
    g.manual_seed(24)
    W3 = (torch.randn(N, K, device=dev, generator=g) / N ** 0.5).to(torch.bfloat16)
    W3t = W3.t().contiguous()
    n = sw.swiglu_workspace_size(M, N, K, "down_proj")
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev) if n else None
    announce(f"gated_mlp auto+ws M={M} K={K} N={N}")
    Out, H = sw.swiglu_gated_mlp(d["A"], d["Wf"], W3t, variant="auto", workspace=ws)
    torch.cuda.synchronize()
    idx = torch.from_numpy(d["rows"]).to(dev)
    hb, ob = _u16(H[idx]), _u16(Out[idx])
    del Out, H
    h_ref = orc.swiglu_rows(d["hA_rows"], d["hW1"], d["hW2"], np.arange(d["rows"].size))
    out_ref = orc.down_proj(h_ref, _u16(W3))
    assert_parity(hb, h_ref, f"H rows {list(d['rows'])}")
    assert_parity(ob, out_ref, f"Out rows {list(d['rows'])}")


# ---------------------------------------------------------------------------
# The strided entry point at its largest row pitches: A a column slice of a
# [M, 2^21] matrix (lda = 2^21), Y a column slice of a [M, 2^22] buffer
# (ldy = 2^22).  A whole 256x256 tile with 256 valid rows then spans 2^31
# bytes of Y, which is the largest range an epilogue's buffer resource takes
# (the range limit equals the out-of-range offset): forced through the
# whole-tile epilogue and through the split tail's reduction kernel.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant,tile,tail", [("i", "256", "whole"), ("i+ws", "256", "split"),
                                               ("i", None, None), ("i+ws", None, None),
                                               ("s", None, None)])
def test_strided_at_max_pitches(dev, orc, variant, tile, tail, monkeypatch):
    M, K, N = 300, 200, 136
    lda, ldy = 1 << 21, 1 << 22
    if tile is None:
        monkeypatch.delenv("SWIGLU_I_TILE", raising=False)
        monkeypatch.delenv("SWIGLU_TAIL", raising=False)
    else:
        monkeypatch.setenv("SWIGLU_I_TILE", tile)
        monkeypatch.setenv("SWIGLU_TAIL", tail)
    v = variant.split("+")[0]
    ws = workspace_for(M, N, K, v, dev) if variant.endswith("+ws") else None
    desc = sw.swiglu_describe_launch(M, N, K, v, 0 if ws is None else ws.numel())
    announce(f"strided {variant} M={M} K={K} N={N} lda={lda} ldy={ldy}: {desc}")
    if tail == "whole":
        # tile row 0 is a whole 256x256 tile with 256 valid rows
        assert desc.startswith("gemm_tiles_kernel<256x256x64,") and "(4 tiles;" in desc, desc
    elif tail == "split":
        assert desc.startswith("gemm_tiles_kernel<256x256x64,") and "split_reduce_kernel" in desc \
            and "(0 whole tiles + 4 tiles split" in desc, desc
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=25)
    Abig = torch.full((M, lda), 1e4, dtype=torch.bfloat16, device=dev)
    Abig[:, 8:8 + K] = A.to(dev)
    sentinel = 0x7F7F
    Ybig = torch.full((M, ldy), sentinel, dtype=torch.int16, device=dev)
    Yv = Ybig.view(torch.bfloat16)[:, 16:16 + N]
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    sw.swiglu_fused_gemm_strided(Abig[:, 8:8 + K], Wf, Yv, variant=v, workspace=ws)
    torch.cuda.synchronize()
    stray = int((Ybig[:, :16] != sentinel).sum()) + int((Ybig[:, 16 + N:] != sentinel).sum())
    assert stray == 0, f"{stray} stores outside the Y view"
    yb = _u16(Yv)
    del Abig, Ybig
    assert_parity(yb, orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2)),
                  f"strided {variant} tile={tile} tail={tail} at max pitches")
