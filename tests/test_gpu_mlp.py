"""Parity of the gated MLP block's HIP path with the CPU oracle (needs an MI355X).

Covers the linear-layer-layout packer (bit for bit), the down projection
Out = bf16(H . W3) on its own, and the whole block (fused SwiGLU GEMM, then
the down projection), all through the C ABI.  The bar is the one of the
fused SwiGLU GEMM: |y_gpu - y_ref| <= max(1e-3, 1e-2 |y_ref|) for every
compared element, y_ref the oracle's bf16 output.  For the whole block the
oracle's Out is computed from its own H, so the comparison also covers the
GPU's H (whose rare one-ulp differences from the oracle's H move Out by far
less than the bound: Out sums N products with weights ~ N(0, 1/N)).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle as oracle_pkg
from gated_mlp_gemm_amd import inputs
from gated_mlp_gemm_amd import swiglu as sw

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)


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


def bits_of(t: torch.Tensor) -> np.ndarray:
    return inputs.bits(t.detach().cpu())


def assert_parity(y_bits, ref_bits, what: str):
    rep = oracle_pkg.parity_report(y_bits, ref_bits)
    print(f"  {what}: {json.dumps(rep)}", flush=True)
    assert rep["mismatches"] == 0, f"{what}: {rep}"
    return rep


def nan_workspace(M, N, K, dev):
    """The ablation-sized workspace, filled with NaN patterns (needs no init)."""
    n = sw.swiglu_workspace_size(M, N, K, "down_proj")
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=dev) if n else None


# ---------------------------------------------------------------------------
# linear-layer-layout packer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(8, 1), (24, 24), (104, 1000), (72, 137), (896, 4864)])
def test_pack_nk_bit_exact(dev, orc, K, N):
    announce(f"pack_nk K={K} N={N}")
    rng = np.random.default_rng(K * 104729 + N)
    W1t = rng.integers(0, 2 ** 16, size=(N, K), dtype=np.uint16)   # any bits, NaNs included
    W2t = rng.integers(0, 2 ** 16, size=(N, K), dtype=np.uint16)
    Wf = sw.swiglu_pack_weights_nk(inputs.from_bits(W1t).to(dev), inputs.from_bits(W2t).to(dev))
    torch.cuda.synchronize()
    # the packed storage is W_fused column-major: its row c is column c
    assert np.array_equal(bits_of(Wf).T, orc.pack_nk(W1t, W2t))


def test_pack_nk_feeds_the_fused_gemm(dev, orc):
    """Weights given as linear layers ([N][K]) give the same Y as [K][N] ones."""
    M, K, N = 300, 200, 136
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=11)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad = A.to(dev)
    Wf_nk = sw.swiglu_pack_weights_nk(W1.t().contiguous().to(dev), W2.t().contiguous().to(dev))
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(Wf_nk.view(torch.int16), Wf.view(torch.int16))
    Y = sw.swiglu_fused_gemm(Ad, Wf_nk, variant="i")
    torch.cuda.synchronize()
    assert_parity(bits_of(Y), ref, "fused i from pack_nk")


# ---------------------------------------------------------------------------
# down projection alone
# ---------------------------------------------------------------------------
DOWN = [(1, 8, 8), (5, 24, 16), (64, 64, 64), (128, 4864, 896), (130, 72, 200),
        (257, 264, 136), (300, 136, 1000), (513, 1032, 64), (2048, 8960, 1536)]


@pytest.mark.parametrize("M,N,D", DOWN)
@pytest.mark.parametrize("use_ws", [False, True], ids=["nows", "ws"])
def test_down_proj(dev, orc, M, N, D, use_ws):
    announce(f"down_proj M={M} N={N} D={D} ws={use_ws}")
    H = inputs.random_bf16((M, N), seed=M * 13 + N, scale=0.6)
    W3 = inputs.random_bf16((N, D), seed=N * 17 + D, scale=N ** -0.5)
    hH, hW3 = inputs.bits(H), inputs.bits(W3)
    if M * N * D > 5e9:   # full size: sampled rows (each output row needs only its H row)
        rows = np.unique(np.array([0, 1, M // 2, M - 1, 777 % M]))
    else:
        rows = np.arange(M)
    ref = orc.down_proj(np.ascontiguousarray(hH[rows]), hW3)
    ws = nan_workspace(M, N, D, dev) if use_ws else None
    Out = sw.swiglu_down_proj(H.to(dev), W3.t().contiguous().to(dev), workspace=ws)
    torch.cuda.synchronize()
    ob = bits_of(Out)
    assert_parity(ob[rows], ref, f"down_proj {M}x{N}x{D}")
    assert np.isfinite(oracle_pkg.bf16_bits_to_f64(ob)).all()


@pytest.mark.parametrize("tile", ["256", "128"])
def test_down_proj_forced_tile(dev, orc, tile, monkeypatch):
    monkeypatch.setenv("SWIGLU_I_TILE", tile)
    M, N, D = 700, 392, 520
    H = inputs.random_bf16((M, N), seed=5, scale=0.6)
    W3 = inputs.random_bf16((N, D), seed=6, scale=N ** -0.5)
    ref = orc.down_proj(inputs.bits(H), inputs.bits(W3))
    W3t = W3.t().contiguous().to(dev)
    for ws in (None, nan_workspace(M, N, D, dev)):
        announce(f"down_proj tile={tile} ws={ws is not None}")
        Out = sw.swiglu_down_proj(H.to(dev), W3t, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(bits_of(Out), ref, f"down_proj@{tile} ws={ws is not None}")


# ---------------------------------------------------------------------------
# the whole block
# ---------------------------------------------------------------------------
def test_mlp_hand_case_padded(dev, orc):
    """The hand-computed block (golden/mlp_hand_cases.json), zero-padded to
    multiples of 8: zero rows and columns add nothing, so the leading block of
    Out is the hand case's, exactly."""
    with open(os.path.join(HERE, "golden", "mlp_hand_cases.json")) as f:
        case = json.load(f)["cases"][0]
    M, K, N = 2, 8, 8
    A = torch.zeros(M, K)
    A[:, :3] = torch.tensor(case["A"], dtype=torch.float32)
    W1 = torch.zeros(K, N)
    W1[:3, :2] = torch.tensor(case["W1"], dtype=torch.float32)
    W2 = torch.zeros(K, N)
    W2[:3, :2] = torch.tensor(case["W2"], dtype=torch.float32)
    W3 = torch.zeros(N, K)
    W3[:2, :3] = torch.tensor(case["W3"], dtype=torch.float32)
    A, W1, W2, W3 = (t.to(torch.bfloat16) for t in (A, W1, W2, W3))
    h_ref, out_ref = orc.gated_mlp(*(inputs.bits(t) for t in (A, W1, W2, W3)))
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    for variant in ("i", "s"):
        announce(f"mlp hand case variant {variant}")
        Out, H = sw.swiglu_gated_mlp(A.to(dev), Wf, W3.t().contiguous().to(dev), variant=variant)
        torch.cuda.synchronize()
        assert_parity(bits_of(H), h_ref, f"hand H {variant}")
        assert_parity(bits_of(Out), out_ref, f"hand Out {variant}")
        # every value of this case is computed exactly before the single rounding
        assert np.array_equal(bits_of(Out), out_ref)


MLP_SMALL = [(1, 8, 8), (5, 16, 24), (100, 64, 8960), (130, 200, 72), (257, 136, 264),
             (300, 1000, 136), (513, 64, 1032)]


@pytest.mark.parametrize("M,K,N", MLP_SMALL)
@pytest.mark.parametrize("variant", ["i", "i+ws", "s", "auto+ws"])
def test_mlp_small(dev, orc, M, K, N, variant):
    announce(f"gated_mlp {variant} M={M} K={K} N={N}")
    A, W1, W2, W3 = inputs.make_mlp_inputs(M, K, N, seed=M * 7 + K * 3 + N)
    h_ref, out_ref = orc.gated_mlp(*(inputs.bits(t) for t in (A, W1, W2, W3)))
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    v = variant.split("+")[0]
    ws = nan_workspace(M, N, K, dev) if variant.endswith("+ws") else None
    Out, H = sw.swiglu_gated_mlp(A.to(dev), Wf, W3.t().contiguous().to(dev), variant=v,
                                 workspace=ws)
    torch.cuda.synchronize()
    assert_parity(bits_of(H), h_ref, f"H {variant} {M}x{K}x{N}")
    assert_parity(bits_of(Out), out_ref, f"Out {variant} {M}x{K}x{N}")


@pytest.mark.parametrize("w", inputs.WORKLOADS, ids=[w.name for w in inputs.WORKLOADS])
def test_mlp_workload_rows(dev, orc, w):
    """Each benchmark shape at full size, in the launch configuration the bench
    times (AUTO, with a workspace): whole sampled rows of H and Out."""
    announce(f"generate MLP inputs {w.name}")
    A, W1, W2, W3 = inputs.make_mlp_inputs(w.M, w.K, w.N, w.seed)
    Ad = A.to(dev)
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    W3t = W3.t().contiguous().to(dev)
    ws = nan_workspace(w.M, w.N, w.K, dev)
    announce(f"gated_mlp auto+ws {w.name}")
    Out, H = sw.swiglu_gated_mlp(Ad, Wf, W3t, variant="auto", workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2000 + w.seed)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.integers(0, w.M, 3)]))
    announce(f"oracle rows {list(rows)} {w.name}")
    hA, hW1, hW2, hW3 = (inputs.bits(t) for t in (A, W1, W2, W3))
    h_ref = orc.swiglu_rows(hA, hW1, hW2, rows)
    out_ref = orc.down_proj(h_ref, hW3)
    hb, ob = bits_of(H), bits_of(Out)
    assert_parity(hb[rows], h_ref, f"H rows {w.name}")
    assert_parity(ob[rows], out_ref, f"Out rows {w.name}")
    assert np.isfinite(oracle_pkg.bf16_bits_to_f64(ob)).all()
