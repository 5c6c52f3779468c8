"""Parity of the FP8 (E4M3) path's HIP kernels with the CPU oracle (needs an MI355X).

The product path quantizes on the device (swiglu_quantize_fp8 of A and of the
packed weight) and runs variant I or S on the codes (swiglu_fused_gemm_fp8); the
oracle quantizes the same seeded bf16 inputs on the CPU with its own
quantizer.  The codes must agree bit for bit; Y must meet the bar of the bf16
path, |y_gpu - y_ref| <= max(1e-3, 1e-2 |y_ref|), against the oracle's fused
SwiGLU on the FP8 codes (exact products, fp64 sums, one rounding).
"""
from __future__ import annotations

import json
import math

import numpy as np
import pytest
import torch

import oracle as oracle_pkg
from gated_mlp_gemm_amd import inputs
from gated_mlp_gemm_amd import swiglu as sw

pytestmark = pytest.mark.gpu


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _default_dispatch(monkeypatch):
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


def assert_parity(y_bits, ref_bits, what: str):
    rep = oracle_pkg.parity_report(y_bits, ref_bits)
    print(f"  {what}: {json.dumps(rep)}", flush=True)
    assert rep["mismatches"] == 0, f"{what}: {rep}"


def amax_exp(t: torch.Tensor) -> int:
    return sw.swiglu_fp8_scale_exp(float(t.float().abs().max()))


def prepare(orc, dev, A, W1, W2, a_exp=None, w_exp=None):
    """Device codes (A8, W_fused8) by the product path, host codes by the oracle."""
    a_exp = amax_exp(A) if a_exp is None else a_exp
    w_exp = max(amax_exp(W1), amax_exp(W2)) if w_exp is None else w_exp
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    A8 = sw.swiglu_quantize_fp8(A.to(dev), a_exp)
    W8 = sw.swiglu_quantize_fp8(Wf, w_exp)
    hA8 = orc.quantize_fp8(inputs.bits(A), a_exp)
    hWT8 = orc.quantize_fp8(np.ascontiguousarray(orc.pack(inputs.bits(W1), inputs.bits(W2)).T),
                            w_exp)
    torch.cuda.synchronize()
    return A8, W8, hA8, hWT8, a_exp, w_exp


# ---------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scale_exp", [-6, 0, 4])
def test_quantize_bit_exact(dev, orc, scale_exp):
    announce(f"quantize scale_exp={scale_exp}")
    x = inputs.bits(inputs.random_bf16((4096,), 300 + scale_exp, 2.0 ** (scale_exp + 4)))
    s = 2.0 ** scale_exp
    special = np.array([0.0, -0.0, math.inf, -math.inf, 448 * s, 464 * s, 470 * s, -1e30,
                        1.0625 * s, 1.1875 * s, 2.0 ** -10 * s, 3 * 2.0 ** -10 * s,
                        -(2.0 ** -10) * s, 1e-38, 7.0 * 2.0 ** -9 * s, 2.0 ** -6 * s],
                       dtype=np.float32)
    sb = (special.view(np.uint32) >> 16).astype(np.uint16)
    x[: sb.size] = sb
    x[sb.size] = 0x7FC0                                       # NaN
    q = sw.swiglu_quantize_fp8(inputs.from_bits(x).to(dev), scale_exp)
    torch.cuda.synchronize()
    got = q.cpu().numpy()
    want = orc.quantize_fp8(x, scale_exp)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(x[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


# ---------------------------------------------------------------------------
# the fused FP8 GEMM
# ---------------------------------------------------------------------------
SMALL = [(1, 16, 8), (5, 32, 24), (64, 128, 64), (128, 896, 520), (100, 144, 8960),
         (130, 208, 72), (257, 144, 264), (300, 1008, 136), (513, 64, 1032), (700, 80, 392)]


@pytest.mark.parametrize("M,K,N", SMALL)
@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_fp8_small_shapes(dev, orc, M, K, N, variant):
    announce(f"fused fp8 {variant} M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 29 + K * 5 + N)
    A8, W8, hA8, hWT8, ea, ew = prepare(orc, dev, A, W1, W2)
    assert np.array_equal(A8.cpu().numpy(), hA8)
    assert np.array_equal(W8.cpu().numpy(), hWT8)
    ref = orc.swiglu_fp8(hA8, hWT8, ea, ew)
    v = variant.split("+")[0]
    ws = sw.make_workspace(M, N, K, "fp8", dev) if variant.endswith("+ws") else None
    Y = sw.swiglu_fused_gemm_fp8(A8, W8, ea, ew, variant=v, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(inputs.bits(Y.cpu()), ref, f"fp8 {variant} {M}x{K}x{N}")


@pytest.mark.parametrize("tile", ["256", "128"])
def test_fp8_forced_tile(dev, orc, tile, monkeypatch):
    monkeypatch.setenv("SWIGLU_I_TILE", tile)
    M, K, N = 777, 528, 1032
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=4242)
    A8, W8, hA8, hWT8, ea, ew = prepare(orc, dev, A, W1, W2)
    ref = orc.swiglu_fp8(hA8, hWT8, ea, ew)
    for ws in (None, sw.make_workspace(M, N, K, "fp8", dev)):
        for tail in ("whole", "quarter", "split"):
            monkeypatch.setenv("SWIGLU_TAIL", tail)
            announce(f"fused fp8 tile={tile} tail={tail} ws={ws is not None}")
            Y = sw.swiglu_fused_gemm_fp8(A8, W8, ea, ew, workspace=ws)
            torch.cuda.synchronize()
            assert_parity(inputs.bits(Y.cpu()), ref, f"fp8@{tile} {tail} ws={ws is not None}")


def test_fp8_saturating_and_scaled(dev, orc):
    """A quantized with a too-small exponent (values beyond 448 saturate) and
    weights with a large negative exponent: both sides see the same codes."""
    M, K, N = 256, 256, 264
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=91, a_scale=4.0)
    A8, W8, hA8, hWT8, ea, ew = prepare(orc, dev, A, W1, W2, a_exp=-6)
    assert (np.abs(hA8.astype(np.int32) & 0x7F) == 0x7E).any(), "some A codes saturate"
    ref = orc.swiglu_fp8(hA8, hWT8, ea, ew)
    Y = sw.swiglu_fused_gemm_fp8(A8, W8, ea, ew)
    torch.cuda.synchronize()
    assert_parity(inputs.bits(Y.cpu()), ref, "fp8 saturating")


# Whole-output comparison up to this many GFLOP of oracle work (the three
# smaller workloads: 2.2, 112.7 and 139.1 GFLOP).
WHOLE_OUTPUT_GFLOP = 200.0


@pytest.mark.parametrize("w", inputs.WORKLOADS, ids=[w.name for w in inputs.WORKLOADS])
def test_fp8_workload_rows(dev, orc, w):
    """Each benchmark shape at full size, as the bench runs it (with a
    workspace): the device codes equal the oracle's; Y meets the bar over the
    whole output on the three smaller workloads, and on one whole row in every
    256-row band (plus the first and last rows) on the two large ones."""
    announce(f"generate inputs {w.name}")
    A, W1, W2 = inputs.workload_inputs(w)
    A8, W8, hA8, hWT8, ea, ew = prepare(orc, dev, A, W1, W2)
    assert np.array_equal(A8.cpu().numpy(), hA8)
    assert np.array_equal(W8.cpu().numpy(), hWT8)
    ws = sw.make_workspace(w.M, w.N, w.K, "fp8", dev)
    if w.flops / 1e9 <= WHOLE_OUTPUT_GFLOP:
        rows = None
        announce(f"oracle whole output {w.name}")
    else:
        rng = np.random.default_rng(3000 + w.seed)
        bands = np.arange(0, w.M, 256)
        rows = np.unique(np.concatenate(
            [[0, w.M - 1], bands + rng.integers(0, 256, bands.size) % np.minimum(256, w.M - bands)]))
        announce(f"oracle rows {list(rows)} {w.name}")
    ref = orc.swiglu_fp8(hA8, hWT8, ea, ew, rows=rows)
    for variant in ("auto", "i", "s"):
        announce(f"fused fp8 {variant} {w.name} a_exp={ea} w_exp={ew}")
        Y = sw.swiglu_fused_gemm_fp8(A8, W8, ea, ew, variant=variant,
                                     workspace=ws if variant != "i" else None)
        torch.cuda.synchronize()
        yb = inputs.bits(Y.cpu())
        got = yb if rows is None else yb[rows]
        what = "whole output" if rows is None else "rows"
        assert_parity(got, ref, f"fp8 {variant} {what} {w.name}")
        assert np.isfinite(oracle_pkg.bf16_bits_to_f64(yb)).all()


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 700)), int(rng.integers(1, 70)) * 16, int(rng.integers(1, 140)) * 8)
            for _ in range(count)]


@pytest.mark.parametrize("M,K,N", _random_shapes(2025, 8))
def test_fp8_random_shapes(dev, orc, M, K, N):
    announce(f"fp8 random shape M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=3 * M + K + 11 * N)
    A8, W8, hA8, hWT8, ea, ew = prepare(orc, dev, A, W1, W2)
    assert np.array_equal(A8.cpu().numpy(), hA8) and np.array_equal(W8.cpu().numpy(), hWT8)
    ref = orc.swiglu_fp8(hA8, hWT8, ea, ew)
    for variant, ws in (("i", None), ("i", sw.make_workspace(M, N, K, "fp8", dev)), ("s", None)):
        Y = sw.swiglu_fused_gemm_fp8(A8, W8, ea, ew, variant=variant, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(inputs.bits(Y.cpu()), ref, f"fp8 {variant} {M}x{K}x{N} ws={ws is not None}")
