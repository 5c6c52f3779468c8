"""Parity of the HIP path with the CPU oracle (needs an MI355X).

Every call goes through the C ABI (ctypes binding).  The bar, from the pages'
mismatch criterion (abstract: zero mismatches; gist.science Core
contributions: relative error above 1 % against an FP32 reference counts as a
mismatch), with an absolute floor of 1e-3 for outputs near zero:

    |y_gpu - y_ref| <= max(1e-3, 1e-2 |y_ref|)   for every compared element,

where y_ref is the oracle's bf16-rounded output.  The pack is compared bit
for bit.  Small shapes are checked in full.  The five benchmark workloads
run at their full sizes: the three smaller ones (M=128 K=896 N=4864, M=2048
K=1536 N=8960, M=512 K=3584 N=18944) are compared with the oracle over the
whole output; the two large ones (M=8192 K=5120 N=13824, M=4096 K=8192
N=29568) on one whole row in every 256-row band, every output tile of the
partly idle last round of tiles (the tiles the schedule splits or quarters)
in full, and random single outputs; variants I and S are also compared with
each other over the whole output.
"""
from __future__ import annotations

import json
import math
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
    """Every test starts from the built-in dispatch (tests that force a
    variant threshold or a tile shape set the variable themselves)."""
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


def ordered(b: np.ndarray) -> np.ndarray:
    """bf16 patterns -> integers ordered like the values (+0 and -0 both 0)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(a, b) -> np.ndarray:
    return np.abs(ordered(a) - ordered(b))


def assert_parity(y_bits, ref_bits, what: str):
    rep = oracle_pkg.parity_report(y_bits, ref_bits)
    print(f"  {what}: {json.dumps(rep)}", flush=True)
    assert rep["mismatches"] == 0, f"{what}: {rep}"
    return rep


_WS = {}


def workspace_for(M, N, K, variant, dev):
    """A workspace of the queried size, reused across calls and filled with
    0xFF bytes (NaN as fp32) when allocated: the library needs no
    initialisation, and a stale partial that leaked into a result would show."""
    n = sw.swiglu_workspace_size(M, N, K, variant)
    if n == 0:
        return None
    if _WS.get(dev) is None or _WS[dev].numel() < n:
        _WS[dev] = torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)
    return _WS[dev]


def run_fused(A, Wf, variant):
    """variant 'i' | 's' | 'auto', with '+ws' appended to pass a workspace
    (which lets variant I split the tiles of a partly idle last round)."""
    ws = None
    if variant.endswith("+ws"):
        variant = variant[:-3]
        M, K = A.shape
        ws = workspace_for(M, Wf.shape[0] // 2, K, variant, A.device)
    Y = sw.swiglu_fused_gemm(A, Wf, variant=variant, workspace=ws)
    torch.cuda.synchronize()
    return Y


# ---------------------------------------------------------------------------
# pack
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(8, 8), (24, 24), (104, 1000), (72, 136), (896, 4864)])
def test_pack_bit_exact(dev, orc, K, N):
    announce(f"pack K={K} N={N}")
    rng = np.random.default_rng(K * 7919 + N)
    W1 = rng.integers(0, 2 ** 16, size=(K, N), dtype=np.uint16)   # any bits, NaNs included
    W2 = rng.integers(0, 2 ** 16, size=(K, N), dtype=np.uint16)
    Wf = sw.swiglu_pack_weights(inputs.from_bits(W1).to(dev), inputs.from_bits(W2).to(dev))
    torch.cuda.synchronize()
    # the packed storage is W_fused column-major: its row c is column c
    assert np.array_equal(bits_of(Wf).T, orc.pack(W1, W2))


# ---------------------------------------------------------------------------
# small and ragged shapes, full comparison
# ---------------------------------------------------------------------------
SMALL = [(1, 8, 8), (5, 16, 24), (64, 64, 64), (128, 896, 520), (130, 200, 72),
         (257, 136, 264), (300, 1000, 136), (513, 64, 1032), (700, 72, 392)]


@pytest.mark.parametrize("M,K,N", SMALL)
@pytest.mark.parametrize("variant", ["i", "i+ws", "s", "auto", "auto+ws"])
def test_small_shapes(dev, orc, M, K, N, variant):
    announce(f"fused {variant} M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 31 + K * 7 + N)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wf = sw.swiglu_pack_weights(W1d, W2d)
    Y = run_fused(Ad, Wf, variant)
    assert_parity(bits_of(Y), ref, f"{variant} {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(130, 200, 72), (257, 136, 264), (300, 1000, 136),
                                   (513, 64, 1032), (700, 72, 392)])
@pytest.mark.parametrize("tile", ["256", "128"])
def test_small_shapes_forced_tile(dev, orc, M, K, N, tile, monkeypatch):
    """Both tile shapes of variant I above M = 128, with and without workspace."""
    monkeypatch.setenv("SWIGLU_I_TILE", tile)
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 31 + K * 7 + N)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    for variant in ("i", "i+ws"):
        announce(f"fused {variant} tile={tile} M={M} K={K} N={N}")
        assert_parity(bits_of(run_fused(Ad, Wf, variant)), ref, f"{variant}@{tile} {M}x{K}x{N}")


@pytest.mark.parametrize("K", [128, 192, 320, 136, 264, 1032, 2056])
@pytest.mark.parametrize("tail", ["auto", "whole", "quarter", "split"])
def test_k_step_bodies(dev, orc, K, tail, monkeypatch):
    """Every GEMM and S kernel runs one of two bodies, chosen by K at entry: K a
    multiple of 64 (fixed per-tile load offsets; the steps the ring loads
    ahead past a tile's last step reload that step into unread stages) or
    ragged K (per-lane masking of the chunks past K).  Short K puts most
    steps next to the end (2, 3 and 5 K steps; 17 and 33 ragged ones), on
    ragged M and 2N edges, with every tail schedule and both tile shapes."""
    M, N = 520, 392
    monkeypatch.setenv("SWIGLU_TAIL", tail)
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=K * 13 + 5)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    for tile in ("256", "128"):
        monkeypatch.setenv("SWIGLU_I_TILE", tile)
        for variant in ("i", "i+ws"):
            announce(f"fused {variant} tile={tile} tail={tail} M={M} K={K} N={N}")
            assert_parity(bits_of(run_fused(Ad, Wf, variant)), ref,
                          f"{variant}@{tile}/{tail} {M}x{K}x{N}")
    monkeypatch.delenv("SWIGLU_I_TILE")
    announce(f"fused s tail={tail} M={M} K={K} N={N}")
    assert_parity(bits_of(run_fused(Ad, Wf, "s")), ref, f"s/{tail} {M}x{K}x{N}")


def _pad(a, rows, cols):
    out = np.zeros((rows, cols), dtype=np.float32)
    a = np.asarray(a, dtype=np.float32)
    out[: a.shape[0], : a.shape[1]] = a
    return out


@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_hand_cases_padded(dev, orc, variant):
    """The hand-computed cases, zero-padded to legal shapes (K, N multiples of 8).

    Zero rows of W / zero columns of A add nothing to the dot products, and
    padded output columns have Up = 0, so the leading block is the hand case.
    """
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        announce(f"hand case {case['name']} variant {variant}")
        A = np.asarray(case["A"], dtype=np.float32)
        W1 = np.asarray(case["W1"], dtype=np.float32)
        M, K = A.shape
        N = W1.shape[1]
        Kp, Np = 8 * math.ceil(K / 8), 8 * math.ceil(N / 8)
        At = torch.from_numpy(_pad(case["A"], M, Kp)).to(torch.bfloat16)
        W1t = torch.from_numpy(_pad(case["W1"], Kp, Np)).to(torch.bfloat16)
        W2t = torch.from_numpy(_pad(case["W2"], Kp, Np)).to(torch.bfloat16)
        ref = orc.swiglu(inputs.bits(At), inputs.bits(W1t), inputs.bits(W2t))
        Ad, W1d, W2d = At.to(dev), W1t.to(dev), W2t.to(dev)
        Y = run_fused(Ad, sw.swiglu_pack_weights(W1d, W2d), variant)
        yb = bits_of(Y)
        assert_parity(yb, ref, case["name"])
        # the padded columns are exactly zero (Up = 0)
        assert np.all(oracle_pkg.bf16_bits_to_f64(yb[:, N:]) == 0.0)


def test_saturating_gates(dev, orc):
    """|Gate| up to ~100: SiLU saturates to x on the right and to -0 on the left."""
    M, K, N = 256, 256, 264
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=77, a_scale=25.0)
    ref, ref64 = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2), want_f64=True)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wf = sw.swiglu_pack_weights(W1d, W2d)
    G = orc.matmul(inputs.bits(A), inputs.bits(W1))
    assert (G < -30).any() and (G > 30).any(), "inputs must reach the saturated regions"
    for variant in ("i", "i+ws", "s"):
        announce(f"saturating gates variant {variant}")
        Y = run_fused(Ad, Wf, variant)
        yb = bits_of(Y)
        assert_parity(yb, ref, f"saturating {variant}")
        assert not np.isnan(oracle_pkg.bf16_bits_to_f64(yb)).any()


# ---------------------------------------------------------------------------
# the five workloads at full size (sampled rows + single outputs)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module", params=range(len(inputs.WORKLOADS)),
                ids=[w.name for w in inputs.WORKLOADS])
def workload(request, dev):
    w = inputs.WORKLOADS[request.param]
    announce(f"generate inputs {w.name} M={w.M} K={w.K} N={w.N} seed={w.seed}")
    A, W1, W2 = inputs.workload_inputs(w)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wf = sw.swiglu_pack_weights(W1d, W2d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1000 + w.seed)
    # one row in every 256-row band (the tall tiles' height), and the edges
    bands = np.arange(0, w.M, 256)
    band_rows = bands + rng.integers(0, 256, bands.size) % np.minimum(256, w.M - bands)
    rows = np.unique(np.concatenate([[0, 1, w.M // 2, w.M - 1], band_rows]))
    pr = rng.integers(0, w.M, 20000)
    pc = rng.integers(0, w.N, 20000)
    # edges of the output: last column, first column of the second tile column
    pr = np.concatenate([pr, rng.integers(0, w.M, 64), rng.integers(0, w.M, 64)])
    pc = np.concatenate([pc, np.full(64, w.N - 1), np.full(64, min(128, w.N - 1))])
    hA, hW1, hW2 = inputs.bits(A), inputs.bits(W1), inputs.bits(W2)
    return dict(w=w, A=Ad, W1=W1d, W2=W2d, Wf=Wf, hA=hA, hW1=hW1, hW2=hW2,
                rows=rows, pr=pr, pc=pc, cache={})


# Whole-output comparison up to this many GFLOP of oracle work per workload
# (the oracle runs ~26 GFLOP/s on 16 host cores; the three smaller workloads
# cost 2.2, 112.7 and 139.1 GFLOP).
WHOLE_OUTPUT_GFLOP = 200.0


def _whole(d) -> bool:
    return d["w"].flops / 1e9 <= WHOLE_OUTPUT_GFLOP


def tile_order(t, tiles_m, tiles_n, group_m=8):
    """(tile row, tile column) of tile index t in the GEMM kernels' tile
    order: groups of group_m tile rows, column by column inside a group."""
    width = group_m * tiles_n
    first_m = (t // width) * group_m
    rows_in_group = min(tiles_m - first_m, group_m)
    i = t % width
    return first_m + i % rows_in_group, i // rows_in_group


def tail_windows(M, N, K, ws_bytes):
    """Output windows (row range, Y column range) of the tiles of variant I's
    partly idle last round (split along K or quartered), read from the launch
    the library describes: [] when every tile runs whole."""
    import re
    desc = sw.swiglu_describe_launch(M, N, K, "i", ws_bytes)
    shape = re.search(r"<(\d+)x(\d+)x\d+,", desc)
    tail = re.search(r"\((\d+) (?:whole )?tiles \+ (\d+) tiles", desc)
    if not (shape and tail):
        return desc, []
    bm, bn = int(shape.group(1)), int(shape.group(2))
    dp, L = int(tail.group(1)), int(tail.group(2))
    tiles_m, tiles_n = -(-M // bm), -(-2 * N // bn)
    assert dp + L == tiles_m * tiles_n, desc
    out = []
    # the library's group size: 4 tile rows for at most 8 tile rows and at
    # most 32 K steps of 64, else 8
    group_m = 4 if tiles_m <= 8 and -(-K // 64) <= 32 else 8
    for t in range(dp, dp + L):
        tm, tn = tile_order(t, tiles_m, tiles_n, group_m)
        r0, c0 = tm * bm, tn * bn // 2
        out.append(((r0, min(r0 + bm, M)), (c0, min(c0 + bn // 2, N))))
    return desc, out


def _ref_samples(orc, d):
    c = d["cache"]
    if "ref_rows" in c:
        return
    w = d["w"]
    if _whole(d):
        announce(f"oracle whole output {w.name} ({w.flops / 1e9:.1f} GFLOP)")
        c["ref_full"] = orc.swiglu(d["hA"], d["hW1"], d["hW2"])
        c["ref_rows"] = c["ref_full"][d["rows"]]
        c["ref_pts"] = c["ref_full"][d["pr"], d["pc"]]
        c["ref_tail"] = []
        return
    announce(f"oracle rows {list(d['rows'])}, points and tail tiles {w.name}")
    c["ref_rows"] = orc.swiglu_rows(d["hA"], d["hW1"], d["hW2"], d["rows"])
    c["ref_pts"] = orc.swiglu_points(d["hA"], d["hW1"], d["hW2"], d["pr"], d["pc"])
    ws = sw.swiglu_workspace_size(w.M, w.N, w.K, "i")
    desc, wins = tail_windows(w.M, w.N, w.K, ws)
    announce(f"{len(wins)} tail tiles of {desc}")
    # merge the windows of one tile row that touch into one oracle call
    by_rows = {}
    for (r0, r1), (c0, c1) in wins:
        by_rows.setdefault((r0, r1), []).append((c0, c1))
    c["ref_tail"] = []
    for (r0, r1), cols in sorted(by_rows.items()):
        cols.sort()
        merged = [list(cols[0])]
        for c0, c1 in cols[1:]:
            if c0 == merged[-1][1]:
                merged[-1][1] = c1
            else:
                merged.append([c0, c1])
        for c0, c1 in merged:
            ref = orc.swiglu_block(d["hA"], d["hW1"], d["hW2"], np.arange(r0, r1), c0, c1)
            c["ref_tail"].append(((r0, r1), (c0, c1), ref))


@pytest.mark.parametrize("variant", ["i", "i+ws", "s", "auto+ws"])
def test_workload_full_size(dev, orc, workload, variant):
    d = workload
    w = d["w"]
    _ref_samples(orc, d)
    c = d["cache"]
    announce(f"fused {variant} {w.name}")
    Y = run_fused(d["A"], d["Wf"], variant)
    yb = bits_of(Y)
    if _whole(d):
        assert_parity(yb, c["ref_full"], f"{variant} {w.name} whole output")
    else:
        assert_parity(yb[d["rows"]], c["ref_rows"], f"{variant} {w.name} rows {list(d['rows'])}")
        assert_parity(yb[d["pr"], d["pc"]], c["ref_pts"], f"{variant} {w.name} points")
        assert c["ref_tail"], "the large workloads have a partly idle last round"
        for (r0, r1), (c0, c1), ref in c["ref_tail"]:
            assert_parity(yb[r0:r1, c0:c1], ref, f"{variant} {w.name} tail tiles rows "
                                                 f"{r0}..{r1 - 1} cols {c0}..{c1 - 1}")
    assert np.isfinite(oracle_pkg.bf16_bits_to_f64(yb)).all()
    d["cache"][f"Y_{variant}"] = yb


@pytest.mark.parametrize("variant", ["i+ws", "s"])
def test_workload_whole_output_vs_fp32_gemm(dev, workload, variant):
    """The whole output at full size on the workloads too large for the
    oracle's whole-output run, against an independent reference on the GPU:
    torch's fp32 GEMM (a library kernel sharing no code with this one) for
    Gate and Up, SiLU and the product in fp64, rounded once to bf16, under
    the oracle comparison's rule (max(1e-3, 1 % of |ref|)).  fp32 sums of
    K <= 8192 products of bf16 values are within ~1e-5 (relative to the sum
    of magnitudes) of the exact ones, far inside that rule."""
    d = workload
    w = d["w"]
    if _whole(d):
        pytest.skip("the whole output is compared with the oracle")
    announce(f"fused {variant} {w.name} whole output vs fp32 GEMM")
    Y = run_fused(d["A"], d["Wf"], variant)
    torch.backends.cuda.matmul.allow_tf32 = False
    W1f, W2f = d["W1"].float(), d["W2"].float()
    bad, worst = 0, 0.0
    for r0 in range(0, w.M, 1024):
        a = d["A"][r0:r0 + 1024].float()
        g = (a @ W1f).double()
        u = (a @ W2f).double()
        ref = (g * torch.sigmoid(g) * u).to(torch.bfloat16).float()
        y = Y[r0:r0 + 1024].float()
        err = (y - ref).abs()
        bound = torch.clamp(1e-2 * ref.abs(), min=1e-3)
        bad += int((~(err <= bound)).sum().item())
        big = ref.abs() > 0.1
        if big.any():
            worst = max(worst, float((err[big] / ref[big].abs()).max().item()))
    del W1f, W2f
    print(f"  {variant} {w.name} whole output vs fp32 GEMM: {w.M * w.N} outputs, "
          f"{bad} outside the rule, max rel err {worst:.2e} (|ref| > 0.1)", flush=True)
    assert bad == 0


@pytest.mark.parametrize("pair", [("i", "s"), ("i+ws", "s"), ("i", "i+ws")])
def test_workload_variants_agree(dev, workload, pair):
    """Over the whole output, each path is within 1 % of the truth, hence the
    two are within about 2 % of each other (plus the absolute floor twice)."""
    d = workload
    ya, yb = (d["cache"].get(f"Y_{v}") for v in pair)
    if ya is None or yb is None:
        pytest.skip("variant outputs not computed")
    a, b = oracle_pkg.bf16_bits_to_f64(ya), oracle_pkg.bf16_bits_to_f64(yb)
    bound = np.maximum(2e-3, 2.05e-2 * np.maximum(np.abs(a), np.abs(b)))
    bad = np.abs(a - b) > bound
    assert not bad.any(), f"{int(bad.sum())} elements of {pair} disagree on {d['w'].name}"


def test_workload_pack(dev, orc, workload):
    d = workload
    announce(f"pack check {d['w'].name}")
    K, N = d["w"].K, d["w"].N
    cols = np.unique(np.array([0, 1, N // 3, N - 2, N - 1]))
    packed_rows = np.stack([2 * cols, 2 * cols + 1], axis=1).reshape(-1)
    got = bits_of(d["Wf"][torch.as_tensor(packed_rows, device=dev)]).T
    assert np.array_equal(got, orc.pack(d["hW1"][:, cols], d["hW2"][:, cols]))


# ---------------------------------------------------------------------------
# ablation (unfused) pipeline
# ---------------------------------------------------------------------------
def _intermediate_within_bound(orc, a_bits, w_bits, got_bits, what):
    """bf16(fp32 sum) vs the exact sum: |got - G| <= 2^-8 |G| + K 2^-23 sum|a w|.

    The first term is the final rounding to bf16 (half a spacing, relative);
    the second is twice the classical bound for K-term fp32 accumulation.  Near
    zero (cancellation) the second term dominates, which is why a fixed ulp
    count is not a valid criterion for the intermediates.
    """
    G = orc.matmul(a_bits, w_bits)
    a64, w64 = oracle_pkg.bf16_bits_to_f64(a_bits), oracle_pkg.bf16_bits_to_f64(w_bits)
    K = a_bits.shape[1]
    bound = 2.0 ** -8 * np.abs(G) + K * 2.0 ** -23 * (np.abs(a64) @ np.abs(w64)) + 1e-37
    err = np.abs(oracle_pkg.bf16_bits_to_f64(got_bits) - G)
    assert np.all(err <= bound), f"{what}: max err/bound {float((err / bound).max()):.3f}"


def test_ablation_workload_full_size(dev, orc, workload):
    """The unfused ablation at each workload's full size, with the workspace
    the benchmark gives it: sampled rows of Gate, Up and Y against the oracle."""
    d = workload
    w = d["w"]
    announce(f"ablation {w.name} full size, workspace")
    ws = workspace_for(w.M, w.N, w.K, "ablation", dev)
    Y, g, u = sw.swiglu_unfused_ablation(d["A"], d["Wf"], workspace=ws)
    torch.cuda.synchronize()
    rows = d["rows"]
    _verify_ablation(orc, Y, g, u, d["hA"][rows], d["hW1"], d["hW2"], rows,
                     f"ablation {w.name}")
    assert np.isfinite(oracle_pkg.bf16_bits_to_f64(bits_of(Y))).all()


def _check_ablation(orc, A, W1, W2, rows, dev, what, use_ws=False):
    Ad = A.to(dev)
    M, K = A.shape
    ws = workspace_for(M, W1.shape[1], K, "ablation", dev) if use_ws else None
    Y, g, u = sw.swiglu_unfused_ablation(Ad, sw.swiglu_pack_weights(W1.to(dev), W2.to(dev)),
                                         workspace=ws)
    torch.cuda.synchronize()
    _verify_ablation(orc, Y, g, u, inputs.bits(A)[rows], inputs.bits(W1), inputs.bits(W2),
                     rows, what)
    return Y


def _verify_ablation(orc, Y, g, u, sub, hW1, hW2, rows, what):
    """Rows `rows` of the ablation's Gate, Up and Y (device) against the oracle,
    given those rows of A (`sub`) and the weights as bf16 bits."""
    g_ref, u_ref, y_ref = orc.swiglu_materialised(sub, hW1, hW2)
    gb, ub, yb = bits_of(g)[rows], bits_of(u)[rows], bits_of(Y)[rows]
    # the intermediates: fp32 accumulation + one rounding, against the exact sums
    _intermediate_within_bound(orc, sub, hW1, gb, what + " gate")
    _intermediate_within_bound(orc, sub, hW2, ub, what + " up")
    # the activation stage: within 1 ulp wherever the intermediates equal the oracle's
    same = (gb == g_ref) & (ub == u_ref)
    assert ulp_distance(yb, y_ref)[same].max(initial=0) <= 1, f"{what}: silu-mul off by >1 ulp"
    bad = oracle_pkg.mismatches(yb, y_ref)
    assert not (bad & same).any(), f"{what}: mismatch not explained by intermediate rounding"
    print(f"  {what}: intermediates differing from the oracle's rounding "
          f"{int((~same).sum())} of {same.size}, y mismatches {int(bad.sum())}", flush=True)


@pytest.mark.parametrize("M,K,N", [(5, 16, 24), (130, 200, 72), (257, 136, 264),
                                   (128, 896, 4864), (600, 4096, 392)])
@pytest.mark.parametrize("use_ws", [False, True], ids=["dp", "ws"])
@pytest.mark.parametrize("tile", [None, "256", "128"])
def test_ablation_small(dev, orc, M, K, N, use_ws, tile, monkeypatch):
    if tile is None:
        monkeypatch.delenv("SWIGLU_I_TILE", raising=False)
    else:
        if M <= 128:
            pytest.skip("one tile shape at M <= 128")
        monkeypatch.setenv("SWIGLU_I_TILE", tile)
    announce(f"ablation M={M} K={K} N={N} workspace={use_ws} tile={tile}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + K + N)
    _check_ablation(orc, A, W1, W2, np.arange(M), dev, f"ablation {M}x{K}x{N}", use_ws)


@pytest.mark.parametrize("use_ws", [False, True], ids=["dp", "ws"])
def test_ablation_workload_rows(dev, orc, use_ws):
    w = inputs.WORKLOADS[1]
    announce(f"ablation {w.name} workspace={use_ws}")
    A, W1, W2 = inputs.workload_inputs(w)
    rows = np.array([0, 1, 777, w.M - 1])
    _check_ablation(orc, A, W1, W2, rows, dev, f"ablation {w.name}", use_ws)


def test_silu_mul_stage(dev, orc):
    announce("silu_mul stage")
    n = (1 << 20) + 8
    g = inputs.random_bf16((n,), 5, scale=6.0)
    u = inputs.random_bf16((n,), 6, scale=1.0)
    Y = sw.swiglu_silu_mul(g.to(dev), u.to(dev))
    torch.cuda.synchronize()
    ref = orc.silu_mul(inputs.bits(g), inputs.bits(u))
    yb = bits_of(Y)
    assert ulp_distance(yb, ref).max() <= 1
    assert_parity(yb, ref, "silu_mul")


# ---------------------------------------------------------------------------
# determinism, dispatcher, streams, empty problems
# ---------------------------------------------------------------------------
def test_determinism(dev):
    w = inputs.WORKLOADS[1]
    announce(f"determinism {w.name}")
    A, W1, W2 = (t.to(dev) for t in inputs.workload_inputs(w))
    Wf = sw.swiglu_pack_weights(W1, W2)
    for variant in ("i", "i+ws", "s"):
        y1 = run_fused(A, Wf, variant).clone()
        y2 = run_fused(A, Wf, variant)
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), variant
    ws = workspace_for(w.M, w.N, w.K, "ablation", dev)
    for workspace in (None, ws):
        Y1, g1, u1 = sw.swiglu_unfused_ablation(A, Wf, workspace=workspace)
        Y1 = Y1.clone()
        Y2, g2, u2 = sw.swiglu_unfused_ablation(A, Wf, workspace=workspace)
        torch.cuda.synchronize()
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


# (M, K, N) for the two tile shapes above M = 128 (forced through
# SWIGLU_I_TILE) and their schedules on 256 CUs: split tails of 2 to 21
# pieces, whole tiles for a full round plus split tail tiles, tiles whole
# with K tails, and the 128x64 tiles of M <= 128 split 32 ways over a long K
# (the exact schedule of each case is what swiglu_describe_launch reports).
SPLIT_TAIL = [(300, 1000, 136), (2048, 1536, 1032), (600, 4096, 392), (777, 520, 2056),
              (3000, 2048, 3000), (70, 128, 520), (128, 8192, 256)]


@pytest.mark.parametrize("M,K,N", SPLIT_TAIL)
@pytest.mark.parametrize("tile", ["256", "128"])
def test_split_tail_shapes(dev, orc, M, K, N, tile, monkeypatch):
    if M <= 128 and tile == "128":
        pytest.skip("one tile shape at M <= 128")
    monkeypatch.setenv("SWIGLU_I_TILE", tile)
    monkeypatch.setenv("SWIGLU_TAIL", "split")
    announce(f"split tail M={M} K={K} N={N} tile={tile}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 3 + K * 5 + N)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wf = sw.swiglu_pack_weights(W1d, W2d)
    Y = run_fused(Ad, Wf, "i+ws")
    yb = bits_of(Y)
    hA, hW1, hW2 = inputs.bits(A), inputs.bits(W1), inputs.bits(W2)
    if M * N * K <= 2 ** 31:
        assert_parity(yb, orc.swiglu(hA, hW1, hW2), f"split tail {M}x{K}x{N}")
    else:
        rng = np.random.default_rng(M + N + K)
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
        assert_parity(yb[rows], orc.swiglu_rows(hA, hW1, hW2, rows),
                      f"split tail rows {M}x{K}x{N}")
        pr, pc = rng.integers(0, M, 4000), rng.integers(0, N, 4000)
        assert_parity(yb[pr, pc], orc.swiglu_points(hA, hW1, hW2, pr, pc),
                      f"split tail points {M}x{K}x{N}")
    # the one-kernel schedule agrees within the accuracy bound
    yd = bits_of(run_fused(Ad, Wf, "i"))
    a, b = oracle_pkg.bf16_bits_to_f64(yb), oracle_pkg.bf16_bits_to_f64(yd)
    assert np.all(np.abs(a - b) <= np.maximum(2e-3, 2.05e-2 * np.maximum(np.abs(a), np.abs(b))))


# (M, K, N) whose 256x256 tiles leave a partly idle last round on 256 CUs, run
# with that round's tiles as quarter-size (128x128) tiles: quarters past the
# output's bottom or right edge (M = 300, 777, 3000; 2N = 272, 784, 4112,
# 6000), no whole tile at all (300 x 136), a full round plus quarters
# (3000 x 3000: 12 x 24 tiles), K tails (1000, 520, 136), and one K step.
QUARTER_TAIL = [(300, 1000, 136), (2048, 1536, 1032), (600, 4096, 392), (777, 520, 2056),
                (3000, 2048, 3000), (257, 64, 1032), (513, 136, 640)]


@pytest.mark.parametrize("M,K,N", QUARTER_TAIL)
def test_quarter_tail_shapes(dev, orc, M, K, N, monkeypatch):
    monkeypatch.setenv("SWIGLU_I_TILE", "256")
    monkeypatch.setenv("SWIGLU_TAIL", "quarter")
    desc = sw.swiglu_describe_launch(M, N, K, "i", 0)
    announce(f"quarter tail M={M} K={K} N={N}: {desc}")
    assert "run as" in desc and "128x128 tiles" in desc, desc
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 7 + K * 3 + N)
    Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
    Wf = sw.swiglu_pack_weights(W1d, W2d)
    # poison the output: every element must be written
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    sw.swiglu_fused_gemm(Ad, Wf, Y=Y, variant="i")
    torch.cuda.synchronize()
    yb = bits_of(Y)
    hA, hW1, hW2 = inputs.bits(A), inputs.bits(W1), inputs.bits(W2)
    if M * N * K <= 2 ** 31:
        assert_parity(yb, orc.swiglu(hA, hW1, hW2), f"quarter tail {M}x{K}x{N}")
    else:
        rng = np.random.default_rng(M + N + K)
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 6)]))
        assert_parity(yb[rows], orc.swiglu_rows(hA, hW1, hW2, rows),
                      f"quarter tail rows {M}x{K}x{N}")
        pr, pc = rng.integers(0, M, 4000), rng.integers(0, N, 4000)
        assert_parity(yb[pr, pc], orc.swiglu_points(hA, hW1, hW2, pr, pc),
                      f"quarter tail points {M}x{K}x{N}")
    # a quarter tile sums each output over the same K steps in the same order
    # as the whole tile: bit-identical to the all-whole schedule
    monkeypatch.setenv("SWIGLU_TAIL", "whole")
    assert "run as" not in sw.swiglu_describe_launch(M, N, K, "i", 0)
    yw = bits_of(run_fused(Ad, Wf, "i"))
    assert np.array_equal(yb, yw)


@pytest.mark.parametrize("M,K,N", [(300, 1000, 136), (777, 520, 1032)])
def test_ablation_quarter_tail(dev, orc, M, K, N, monkeypatch):
    monkeypatch.setenv("SWIGLU_I_TILE", "256")
    monkeypatch.setenv("SWIGLU_TAIL", "quarter")
    desc = sw.swiglu_describe_launch(M, N, K, "ablation", 0)
    announce(f"ablation quarter tail M={M} K={K} N={N}: {desc}")
    assert "run as" in desc, desc
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + 2 * K + N)
    _check_ablation(orc, A, W1, W2, np.arange(M), dev, f"ablation quarter {M}x{K}x{N}")


def test_workspace_reuse_sizes(dev, orc):
    """One workspace across calls of different shapes, large then small then
    large: counters left by a call never leak into the next."""
    ws = None
    for (M, K, N) in [(1030, 512, 1000), (260, 264, 136), (1030, 512, 1000), (70, 128, 520)]:
        announce(f"workspace reuse M={M} K={K} N={N}")
        A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + 2 * K + 3 * N)
        need = sw.swiglu_workspace_size(M, N, K, "i")
        if ws is None:
            ws = torch.empty(sw.swiglu_workspace_size(1030, 1000, 512, "i"), dtype=torch.uint8,
                             device=dev)
        assert ws.numel() >= need
        Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
        Y = sw.swiglu_fused_gemm(Ad, Wf, variant="i", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(bits_of(Y), orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2)),
                      f"reuse {M}x{K}x{N}")


def test_workspace_too_small_falls_back(dev, orc):
    announce("workspace too small")
    M, K, N = 300, 256, 264
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=5)
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    small = torch.zeros(1024, dtype=torch.uint8, device=dev)
    Y = sw.swiglu_fused_gemm(Ad, Wf, variant="i", workspace=small)
    Yd = run_fused(Ad, Wf, "i")
    assert torch.equal(Y.view(torch.int16), Yd.view(torch.int16))   # the same DP schedule
    assert int(small.abs().sum().item()) == 0                          # untouched


@pytest.mark.parametrize("M,switch,expect", [(2047, None, "i"), (2049, None, "i"),
                                             (2048, "2048", "i"), (2049, "2048", "s")])
def test_auto_dispatch_matches_named_variant(dev, M, switch, expect, monkeypatch):
    if switch is None:
        monkeypatch.delenv("SWIGLU_M_SWITCH", raising=False)
    else:
        monkeypatch.setenv("SWIGLU_M_SWITCH", switch)
    announce(f"dispatch M={M}")
    A, W1, W2 = (t.to(dev) for t in inputs.make_inputs(M, 64, 64, seed=M))
    Wf = sw.swiglu_pack_weights(W1, W2)
    ya = run_fused(A, Wf, "auto")
    yv = run_fused(A, Wf, expect)
    assert torch.equal(ya.view(torch.int16), yv.view(torch.int16))


def test_non_default_stream(dev, orc):
    announce("non-default stream")
    M, K, N = 300, 256, 200
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=11)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ad, W1d, W2d = A.to(dev), W1.to(dev), W2.to(dev)
        Wf = sw.swiglu_pack_weights(W1d, W2d)
        Yi = sw.swiglu_fused_gemm(Ad, Wf, variant="i")
        Ys = sw.swiglu_fused_gemm(Ad, Wf, variant="s")
        ws = torch.empty(sw.swiglu_workspace_size(M, N, K, "i"), dtype=torch.uint8, device=dev)
        Yk = sw.swiglu_fused_gemm(Ad, Wf, variant="i", workspace=ws)
    s.synchronize()
    assert_parity(bits_of(Yi), ref, "stream i")
    assert_parity(bits_of(Ys), ref, "stream s")
    assert_parity(bits_of(Yk), ref, "stream i+ws")


def test_describe_launch(dev, monkeypatch):
    """The launch description names the kernels the dispatch picks."""
    ws = sw.swiglu_workspace_size(2048, 8960, 1536, "i")
    d = sw.swiglu_describe_launch(2048, 8960, 1536, "auto", ws)
    assert d.startswith("gemm_tiles_kernel<") and "PairMulEpilogue" in d
    monkeypatch.setenv("SWIGLU_I_TILE", "256")
    d = sw.swiglu_describe_launch(2048, 8960, 1536, "i", ws)
    assert "256x256x64" in d and "512 tiles + 48 tiles run as 192 128x128 tiles; 256 workgroups" in d, d
    assert "split" not in sw.swiglu_describe_launch(2048, 8960, 1536, "i", 0)
    monkeypatch.setenv("SWIGLU_TAIL", "split")
    d = sw.swiglu_describe_launch(2048, 8960, 1536, "i", ws)
    assert "256x256x64" in d and "split 5 ways" in d and d.endswith("split_reduce_kernel")
    assert "split" not in sw.swiglu_describe_launch(2048, 8960, 1536, "i", 0)
    monkeypatch.setenv("SWIGLU_TAIL", "whole")
    assert sw.swiglu_describe_launch(2048, 8960, 1536, "i", ws).endswith("(560 tiles; 256 workgroups)")
    monkeypatch.delenv("SWIGLU_TAIL")
    monkeypatch.setenv("SWIGLU_I_TILE", "128")
    assert "128x128x64" in sw.swiglu_describe_launch(2048, 8960, 1536, "i", 0)
    d = sw.swiglu_describe_launch(2048, 8960, 1536, "s")
    assert d == ("fused_sequential_persistent_kernel<256x128x64> (512 tiles + 48 tiles run as "
                 "192 128x64 tiles; 256 workgroups)"), d
    monkeypatch.setenv("SWIGLU_TAIL", "whole")
    d = sw.swiglu_describe_launch(2048, 8960, 1536, "s")
    assert d == "fused_sequential_persistent_kernel<256x128x64> (560 tiles; 256 workgroups)", d
    monkeypatch.delenv("SWIGLU_TAIL")
    assert sw.swiglu_describe_launch(128, 8960, 1536, "s").startswith("fused_sequential_kernel<")
    assert sw.swiglu_describe_launch(2048, 8960, 1536, "ablation").startswith("2 x gemm_tiles")
    assert "128x128x64" in sw.swiglu_describe_launch(128, 4864, 896, "i")    # forced at M <= 128
    monkeypatch.setenv("SWIGLU_I_TILE", "256")
    assert "128x64x64" in sw.swiglu_describe_launch(128, 8960, 1536, "i")    # forced at M <= 128
    monkeypatch.delenv("SWIGLU_I_TILE")
    # M <= 128: 128x128 tiles where they put no more weight rows on a CU (M > 64)
    assert "128x64x64" in sw.swiglu_describe_launch(128, 4864, 896, "i")     # 152 vs 76 tiles
    assert "128x128x64" in sw.swiglu_describe_launch(128, 8960, 1536, "i")   # 280 vs 140 tiles
    assert "128x64x64" in sw.swiglu_describe_launch(64, 8960, 1536, "i")
    assert "128x64x64" in sw.swiglu_describe_launch(128, 18944, 3584, "i")   # 592 vs 296 tiles
    assert "128x128x128" in sw.swiglu_describe_launch(128, 8960, 1536, "fp8")


def test_empty_and_invalid_on_device(dev):
    A = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    Y = sw.swiglu_fused_gemm(A, sw.swiglu_pack_weights(W, W))
    assert Y.shape == (0, 64)
    with pytest.raises(sw.SwigluError):      # K = 20 is not a multiple of 8
        sw.swiglu_fused_gemm(torch.empty((8, 20), dtype=torch.bfloat16, device=dev),
                             torch.empty((128, 20), dtype=torch.bfloat16, device=dev))


# ---------------------------------------------------------------------------
# row-strided views of A and Y (swiglu_fused_gemm_strided)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 16, 8), (130, 200, 72), (300, 1000, 136),
                                   (513, 64, 1032), (2048, 1536, 8960)])
@pytest.mark.parametrize("variant", ["i", "i+ws", "s"])
def test_strided_views(dev, orc, M, K, N, variant):
    """A is columns [8, 8+K) of an [M, K+24] matrix whose other columns hold
    1e4 (reading them would wreck the result); Y is columns [16, 16+N) of an
    [M, N+40] buffer of sentinels, which must be untouched outside the view."""
    announce(f"strided {variant} M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 13 + K * 3 + N)
    Abig = torch.full((M, K + 24), 1e4, dtype=torch.bfloat16, device=dev)
    Abig[:, 8:8 + K] = A.to(dev)
    Av = Abig[:, 8:8 + K]
    sentinel = 0x7F7F                                    # a large finite bf16 pattern
    Ybig = torch.full((M, N + 40), 0, dtype=torch.int16, device=dev)
    Ybig.fill_(sentinel)
    Ybig = Ybig.view(torch.bfloat16)
    Yv = Ybig[:, 16:16 + N]
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    v = variant.split("+")[0]
    ws = workspace_for(M, N, K, v, dev) if variant.endswith("+ws") else None
    sw.swiglu_fused_gemm_strided(Av, Wf, Yv, variant=v, workspace=ws)
    torch.cuda.synchronize()
    big = bits_of(Ybig)
    outside = np.concatenate([big[:, :16].ravel(), big[:, 16 + N:].ravel()])
    assert np.all(outside == sentinel), "stores outside the Y view"
    yb = np.ascontiguousarray(big[:, 16:16 + N])
    hA, hW1, hW2 = inputs.bits(A), inputs.bits(W1), inputs.bits(W2)
    if M * N * K > 1e9:
        rows = np.array([0, 1, M // 2, M - 1])
        assert_parity(yb[rows], orc.swiglu_rows(hA, hW1, hW2, rows), f"strided {variant} rows")
    else:
        assert_parity(yb, orc.swiglu(hA, hW1, hW2), f"strided {variant} {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(100, 136, 8960), (128, 64, 13824)])
@pytest.mark.parametrize("variant", ["i", "i+ws", "auto"])
def test_small_m_quad_tiles(dev, orc, M, K, N, variant):
    """M <= 128 shapes for which variant I takes 128x128 tiles (two per CU)."""
    assert "128x128x64" in sw.swiglu_describe_launch(M, N, K, "i")
    announce(f"small-M 128x128 {variant} M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M * 7 + N)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    assert_parity(bits_of(run_fused(A.to(dev), Wf, variant)), ref, f"{variant} {M}x{K}x{N}")


# ---------------------------------------------------------------------------
# seeded random ragged shapes (deterministic; whole outputs against the oracle)
# ---------------------------------------------------------------------------
def _random_shapes(seed, count, k_mult):
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(count):
        M = int(rng.integers(1, 700))
        K = int(rng.integers(1, 1100 // k_mult + 1)) * k_mult
        N = int(rng.integers(1, 140)) * 8
        shapes.append((M, K, N))
    return shapes


@pytest.mark.parametrize("M,K,N", _random_shapes(2024, 12, 8))
def test_random_shapes(dev, orc, M, K, N):
    announce(f"random shape M={M} K={K} N={N}")
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + 7 * K + 13 * N)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad = A.to(dev)
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    for variant in ("i", "i+ws", "s"):
        assert_parity(bits_of(run_fused(Ad, Wf, variant)), ref, f"{variant} {M}x{K}x{N}")


# Variant S above 128 rows: whole 256x128 tiles, and the last round's tiles as
# 128x64 quarters.  Forced each way on ragged shapes: a partial last tile row
# and column, a quarter wholly past the M edge (M=300: rows 384..511) and one
# past the N edge (N=904: columns 960..1023), a K tail (K=200), and more tiles
# than compute units so the persistent loop takes several tiles (M=4100).
@pytest.mark.parametrize("tail", ["whole", "quarter"])
@pytest.mark.parametrize("M,K,N", [(300, 200, 1000), (300, 520, 904), (4100, 136, 2056)])
def test_sequential_tail_modes(dev, orc, monkeypatch, tail, M, K, N):
    announce(f"S tail={tail} M={M} K={K} N={N}")
    monkeypatch.setenv("SWIGLU_TAIL", tail)
    d = sw.swiglu_describe_launch(M, N, K, "s")
    tiles = math.ceil(M / 256) * math.ceil(N / 128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rem = tiles % cus
    if tail == "quarter" and rem:
        assert f"{tiles - rem} tiles + {rem} tiles run as {4 * rem} 128x64 tiles" in d, d
    else:
        assert f"({tiles} tiles;" in d, d
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + N + K)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    Y = sw.swiglu_fused_gemm(Ad, Wf, variant="s")
    torch.cuda.synchronize()
    assert_parity(bits_of(Y), ref, f"S tail={tail}")
    # the same arithmetic per element whichever way the tile runs
    Yi = sw.swiglu_fused_gemm(Ad, Wf, variant="i")
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yi.view(torch.int16))


# Variant S runs its quarter tail before its whole tiles when a tile is at
# most 64 K steps long, after them on longer tiles.  The cases above take the
# first order; these the second: M=2048, N=4224 is 264 tiles of 256x128, so
# 256 run whole and 8 as 32 quarters (the last tile column, every tile row),
# with 66 K steps (K a multiple of 64, and ragged).  Rows sampled against the
# oracle cross whole and quarter tiles; the whole output against variant I.
@pytest.mark.parametrize("K", [4224, 4168])
def test_sequential_quarters_after_long_tiles(dev, orc, monkeypatch, K):
    M, N = 2048, 4224
    monkeypatch.setenv("SWIGLU_TAIL", "quarter")
    announce(f"S long tiles, quarter tail last M={M} K={K} N={N}")
    d = sw.swiglu_describe_launch(M, N, K, "s")
    tiles = math.ceil(M / 256) * math.ceil(N / 128)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rem = tiles % cus
    if rem and tiles > cus:
        assert f"{tiles - rem} tiles + {rem} tiles run as {4 * rem} 128x64 tiles" in d, d
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=K + 17)
    rows = np.array([0, 1, 127, 128, 255, 256, 700, 1023, 1024, 1535, 1792, 2047])
    ref = orc.swiglu_rows(inputs.bits(A), inputs.bits(W1), inputs.bits(W2), rows)
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    Y = sw.swiglu_fused_gemm(Ad, Wf, variant="s")
    torch.cuda.synchronize()
    assert_parity(bits_of(Y)[rows], ref, f"S long tiles K={K} rows")
    Yi = sw.swiglu_fused_gemm(Ad, Wf, variant="i")
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yi.view(torch.int16))


# Variant I at M <= 128 with a workspace: every 128x128 tile split into
# s = min(CUs / tiles, K steps) pieces along K and reduced in the kernel by its
# last piece (device-scope partials in the workspace, library-owned arrival
# counters), by default when 3 <= s <= 4 with at least 16 K steps a piece,
# forced by SWIGLU_TAIL=fixup (s capped at 4).  Ragged M, a K tail, a single
# row, uneven pieces (14 steps in 3), a shape the default takes (3584 = 56
# steps in 3 pieces), and a long K with more tiles' pieces than the cap.  Each
# case runs twice on the same workspace (filled with NaN patterns): both calls
# equal bit for bit, which also shows the counters were left at zero.
@pytest.mark.parametrize("M,K,N", [(128, 896, 4864), (100, 520, 4600), (1, 896, 4864),
                                   (64, 200, 8192), (128, 3584, 4864), (128, 4864, 896)])
def test_reduce_in_kernel(dev, orc, monkeypatch, M, K, N):
    A, W1, W2 = inputs.make_inputs(M, K, N, seed=M + 3 * K + 7 * N)
    ref = orc.swiglu(inputs.bits(A), inputs.bits(W1), inputs.bits(W2))
    Ad, Wf = A.to(dev), sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    tiles = math.ceil(2 * N / 128)
    s = min(cus // tiles, math.ceil(K / 64))
    ws = workspace_for(M, N, K, "i", dev)
    for tail in ("auto", "fixup"):
        if tail == "auto":
            monkeypatch.delenv("SWIGLU_TAIL", raising=False)
        else:
            monkeypatch.setenv("SWIGLU_TAIL", tail)
        announce(f"I tail={tail} M={M} K={K} N={N}")
        d = sw.swiglu_describe_launch(M, N, K, "i", ws.numel())
        nk = math.ceil(K / 64)
        in_kernel = s >= 2 if tail == "fixup" else (3 <= s <= 4 and nk >= 16 * s)
        assert ("reduced in the kernel" in d) == in_kernel, d
        if in_kernel:
            assert f"({tiles} tiles split {min(s, 4)} ways along K" in d, d
        y1 = sw.swiglu_fused_gemm(Ad, Wf, variant="i", workspace=ws)
        y2 = sw.swiglu_fused_gemm(Ad, Wf, variant="i", workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        assert_parity(bits_of(y1), ref, f"I tail={tail} {M}x{K}x{N}")
    monkeypatch.delenv("SWIGLU_TAIL", raising=False)
    assert "reduced in the kernel" not in sw.swiglu_describe_launch(M, N, K, "i", 0)
