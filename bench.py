"""Benchmark of the fused SwiGLU GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload IDX]
                    [--variant auto|i|s] [--no-cpu-baseline] [--no-per-workload]
    python bench.py --sweep [--sweep-m 128,256,...]

A step is one pass of the hot path over one batch of synthetic input: the
fused call Y = SiLU(A.W1) (.) (A.W2) with the M-based dispatch (the weight
pack is offline and untimed).  The headline workload is the largest one,
M=4096, K=8192, N=29568 (seed 4; a 72B-class gated MLP, 969 MB of packed
weights).  Inputs are resident in HBM before timing starts; when a step's
working set is below 512 MB the timed steps rotate over R copies of (A,
weights, Y), so the 256 MB Infinity Cache cannot hold it across steps.

Protocol: W warm-up steps, continued until at least --warmup-seconds of GPU
work has run, then exactly K timed steps (HIP events on the launch stream):
the headline.  Then AUTO again, variant I, variant S and the unfused ablation
(two GEMMs + SiLU-mul from the same mainloop) run K-step loops in
alternating repeats, whose medians give the speedup over the ablation.

Prints ONE JSON line: TFLOP/s (4 M N K per step), the fraction of the bf16
dense MFMA peak, the speedup over the unfused ablation, a roofline record for
the fused call, `per_workload` sub-records for the other four workloads
(AUTO / I / S / ablation medians and minima per call, TFLOP/s, fraction of
peak, speedup), the CPU oracle's throughput on a bounded sample of the
headline workload, and for context the same call on FP8 E4M3 operands
(`fp8`: operands quantized beforehand, and with the activation quantized
inside each step).

--sweep instead times variant I, variant S and the ablation over a range of M
for each of the five K x N shapes of the workloads (inputs drawn on the
device from the same distributions; the same rotation rule) and prints one
JSON line per (shape, M): the data behind the M threshold of the dispatcher.

--mlp times the gated MLP block (the fused SwiGLU GEMM, then the down
projection back to the model width) against the unfused pipeline followed by
the same down projection, on the five workloads: one JSON line each.

--fp8 times the fused GEMM (variant I) on FP8 E4M3 operands against the same
call on bf16, on the five workloads: one JSON line each.

--schedule-calibration times variant I at the same shapes over a finer range
of M, once with the library's own choice and once forced (SWIGLU_I_TILE,
SWIGLU_TAIL) through each tile shape and tail schedule, one JSON line per
(shape, M, schedule): the data the schedule cost model is fitted to
(``python -m gated_mlp_gemm_amd.schedule_fit FILE``).

--launch-cost times the fused call (bf16 and FP8) on warm inputs through the
Python binding, straight through the C ABI, and replayed from a HIP graph:
the host cost per call and where it stops mattering (one JSON line per
workload; by default the M=128 one).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
METRIC = "fused SwiGLU-GEMM TFLOP/s + % bf16 MFMA peak; speedup vs unfused ablation"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # The clock settles under sustained MFMA load (durations of back-to-back
    # calls rise by ~10 % before levelling off), so every warm-up also runs
    # for at least --warmup-seconds of GPU work, whatever --warmup says.
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--warmup-seconds", type=float, default=0.3,
                   help="minimum GPU time of the headline's warm-up (partners: a quarter)")
    p.add_argument("--repeats", type=int, default=5,
                   help="alternating repeats of the partner loops (medians and minima)")
    # the headline workload: M=4096 K=8192 N=29568, the largest configuration
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--no-per-workload", action="store_true",
                   help="skip the sub-records of the other four workloads")
    p.add_argument("--variant", default="auto", choices=["auto", "i", "s"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--no-fp8", action="store_true",
                   help="skip the FP8 context timing of the default line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one device copy of known size (for HBM counter scaling)")
    p.add_argument("--sweep", action="store_true",
                   help="time I, S and the ablation over M for the five K x N shapes")
    p.add_argument("--sweep-m", default="128,256,512,1024,2048,3072,4096,8192,16384")
    p.add_argument("--mlp", action="store_true",
                   help="time the gated MLP block (SwiGLU + down projection), fused vs "
                        "unfused, on the five workloads")
    p.add_argument("--mlp-workloads", default="0,1,2,3,4")
    p.add_argument("--fp8", action="store_true",
                   help="time the fused GEMM on FP8 (E4M3) operands against bf16, five workloads")
    p.add_argument("--fp8-workloads", default="0,1,2,3,4")
    p.add_argument("--launch-cost", action="store_true",
                   help="host cost per call: binding vs C-ABI vs HIP-graph replay (warm inputs)")
    p.add_argument("--launch-workloads", default="0")
    p.add_argument("--schedule-calibration", action="store_true",
                   help="time variant I under every forced tile shape / tail schedule")
    p.add_argument("--calibration-m",
                   default="256,512,640,768,1024,1280,1536,2048,2560,3072,4096,5120,6144,8192,16384")
    return p.parse_args()


def _time_call(fn, copies, stream, budget_s=0.03, max_reps=100):
    """Per-call microseconds of fn over rotated input copies (3 warm-up calls,
    then enough timed calls for about budget_s), with HIP events on `stream`."""
    import torch

    R = len(copies)
    for r in range(3):
        fn(*copies[r % R])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn(*copies[0])
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-6)
    reps = int(min(max_reps, max(5, budget_s / est)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        fn(*copies[r % R])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _sweep_shapes(dev, ms_list, body):
    """For each K x N shape of the workloads (smallest first): draw the weights
    and a tall A on the device, then call body(K, N, M, copies, Wf) per M with
    R rotated copies of (A[:M], W_fused), R x step bytes >= 512 MiB."""
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    shapes = sorted({(w.K, w.N) for w in inputs.WORKLOADS}, key=lambda kn: kn[0] * kn[1])
    for K, N in shapes:
        g = torch.Generator(device=dev)
        g.manual_seed(K * 131 + N)
        W1 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        W2 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        Wf = sw.swiglu_pack_weights(W1, W2)
        del W1, W2
        A_all = torch.randn(max(ms_list), K, device=dev, generator=g).to(torch.bfloat16)
        for M in ms_list:
            step_bytes = 2 * (M * K + 2 * K * N + M * N)
            R = max(1, -(-512 * 2 ** 20 // step_bytes))
            A = A_all[:M]
            copies = [(A, Wf)] + [(A.clone(), Wf.clone()) for _ in range(R - 1)]
            body(K, N, M, copies, Wf)
            del copies
        del Wf, A_all
        torch.cuda.empty_cache()


def schedule_calibration(args):
    """Variant I per (shape, M) under the library's choice and every forced
    (tile, tail) schedule; one JSON line each."""
    import torch

    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sw.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    ms_list = [int(x) for x in args.calibration_m.split(",")]
    schedules = [("auto", "auto"), ("256", "whole"), ("256", "split"), ("256", "quarter"),
                 ("128", "whole"), ("128", "split")]
    saved = {k: os.environ.get(k) for k in ("SWIGLU_I_TILE", "SWIGLU_TAIL")}

    def body(K, N, M, copies, Wf):
        ws = sw.make_workspace(M, N, K, "i", dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for tile, tail in schedules:
            for k, v in (("SWIGLU_I_TILE", tile), ("SWIGLU_TAIL", tail)):
                if v == "auto":
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
            desc = sw.swiglu_describe_launch(M, N, K, "i", ws.numel() if ws is not None else 0)
            us = _time_call(lambda a, w: sw.swiglu_fused_gemm(a, w, Y=Y, variant="i",
                                                              workspace=ws),
                            copies, stream, budget_s=0.04, max_reps=200)
            print(json.dumps({"K": K, "N": N, "M": M, "tile": tile, "tail": tail,
                              "us": round(us, 2), "launch": desc}), flush=True)

    try:
        _sweep_shapes(dev, ms_list, body)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def mlp_blocks(args):
    """The gated MLP block per workload (one JSON line each): the fused SwiGLU
    GEMM followed by the down projection Out = H . W3 (W3 in R^{N x K}), against
    the unfused pipeline (two GEMMs materialising Gate and Up, the SiLU-mul
    kernel) followed by the same down projection; plus each stage alone.  The
    share of the unfused block spent in the activation kernel, and the share
    the fusion removes, are the MI355X counterparts of the paper's Figure 1
    (SwiGLU and its materialisation as a fraction of MLP time)."""
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sw.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for idx in (int(x) for x in args.mlp_workloads.split(",")):
        w = inputs.WORKLOADS[idx]
        M, K, N = w.M, w.K, w.N
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed)
        # the workload's distributions, drawn on the device (same recipe as
        # the parity tests' generator, different stream of numbers)
        A = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        W1 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        W2 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        Wf = sw.swiglu_pack_weights(W1, W2)
        del W1, W2
        W3t = (torch.randn(K, N, device=dev, generator=g) / N ** 0.5).to(torch.bfloat16)
        in_bytes = 2 * (M * K + 2 * K * N + K * N)
        R = max(1, -(-512 * 2 ** 20 // in_bytes))
        copies = []
        for r in range(R):
            a, wf, w3 = (A, Wf, W3t) if r == 0 else (A.clone(), Wf.clone(), W3t.clone())
            bufs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
            out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            copies.append((a, wf, w3, bufs[0], bufs[1], bufs[2], out))
        ws = sw.make_workspace(M, N, K, "ablation", dev)
        torch.cuda.synchronize()

        def unfused(a, wf, w3, h, gt, up, out):
            sw.swiglu_unfused_ablation(a, wf, gate_ws=gt, up_ws=up, Y=h, workspace=ws)
            sw.swiglu_down_proj(h, w3, Out=out, workspace=ws)

        calls = {
            "fused_swiglu": lambda a, wf, w3, h, gt, up, out:
                sw.swiglu_fused_gemm(a, wf, Y=h, variant="auto", workspace=ws),
            "ablation_swiglu": lambda a, wf, w3, h, gt, up, out:
                sw.swiglu_unfused_ablation(a, wf, gate_ws=gt, up_ws=up, Y=h, workspace=ws),
            "silu_mul": lambda a, wf, w3, h, gt, up, out: sw.swiglu_silu_mul(gt, up, Y=h),
            "down_proj": lambda a, wf, w3, h, gt, up, out:
                sw.swiglu_down_proj(h, w3, Out=out, workspace=ws),
            "mlp_fused": lambda a, wf, w3, h, gt, up, out:
                sw.swiglu_gated_mlp(a, wf, w3, H=h, Out=out, variant="auto", workspace=ws),
            "mlp_unfused": unfused,
        }
        us = {}
        for name, fn in calls.items():
            us[name] = round(_time_call(fn, copies, stream, budget_s=0.25, max_reps=2000), 2)
        mlp_flops = 6 * M * N * K
        rec = {
            "workload": f"gated MLP block M={M} K={K} N={N} (seed {w.seed})",
            "M": M, "K": K, "N": N, "rotation_copies": R, "us": us,
            "down_proj_launch": sw.swiglu_describe_launch(M, N, K, "down_proj",
                                                          0 if ws is None else ws.numel()),
            "down_proj_tflops": round(2 * M * N * K / (us["down_proj"] * 1e-6) / 1e12, 1),
            "mlp_tflops_fused": round(mlp_flops / (us["mlp_fused"] * 1e-6) / 1e12, 1),
            "mlp_tflops_unfused": round(mlp_flops / (us["mlp_unfused"] * 1e-6) / 1e12, 1),
            "mlp_speedup_fused_vs_unfused": round(us["mlp_unfused"] / us["mlp_fused"], 3),
            "activation_share_of_unfused_mlp": round(us["silu_mul"] / us["mlp_unfused"], 4),
            "fusion_saving_share_of_unfused_mlp":
                round((us["mlp_unfused"] - us["mlp_fused"]) / us["mlp_unfused"], 4),
        }
        print(json.dumps(rec), flush=True)
        del copies, A, Wf, W3t, ws
        torch.cuda.empty_cache()


def launch_cost(args, calls=3000, per_graph=20, replays=100):
    """Per-call cost of the fused call, bf16 and FP8, on warm inputs (one copy):
    through the Python binding and straight through the C ABI (host time of
    `calls` back-to-back calls, and wall time to their completion), and
    replayed from a HIP graph of `per_graph` captured calls.  One JSON line
    per workload."""
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    lib = sw.load_library()
    dev = torch.device("cuda:0")

    def loop(fn):
        for _ in range(100):
            fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(calls):
            fn()
        host = time.perf_counter() - t
        torch.cuda.synchronize()
        wall = time.perf_counter() - t
        return round(host / calls * 1e6, 2), round(wall / calls * 1e6, 2)

    def graph(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        return round((time.perf_counter() - t) / (replays * per_graph) * 1e6, 2)

    for idx in (int(x) for x in args.launch_workloads.split(",")):
        w = inputs.WORKLOADS[idx]
        M, K, N = w.M, w.K, w.N
        A, W1, W2 = inputs.workload_inputs(w)
        Ad = A.to(dev)
        Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
        a_exp = sw.swiglu_fp8_scale_exp(float(Ad.float().abs().max()))
        w_exp = sw.swiglu_fp8_scale_exp(float(Wf.float().abs().max()))
        A8, W8 = sw.swiglu_quantize_fp8(Ad, a_exp), sw.swiglu_quantize_fp8(Wf, w_exp)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        s = torch.cuda.current_stream(dev).cuda_stream
        pa, pw, p8a, p8w, py = Ad.data_ptr(), Wf.data_ptr(), A8.data_ptr(), W8.data_ptr(), Y.data_ptr()
        paths = {
            "bf16": (lambda: sw.swiglu_fused_gemm(Ad, Wf, Y=Y),
                     lambda: lib.swiglu_fused_gemm(pa, pw, py, M, N, K, 0, None, 0, s)),
            "fp8": (lambda: sw.swiglu_fused_gemm_fp8(A8, W8, a_exp, w_exp, Y=Y),
                    lambda: lib.swiglu_fused_gemm_fp8(p8a, p8w, py, M, N, K, a_exp, w_exp, 0,
                                                      None, 0, s)),
        }
        rec = {"workload": f"fused SwiGLU GEMM M={M} K={K} N={N} (seed {w.seed}), warm inputs",
               "M": M, "K": K, "N": N, "calls": calls, "graph_calls": per_graph * replays,
               "us_per_call": {}}
        for name, (bound, direct) in paths.items():
            bh, bw = loop(bound)
            ch, cw = loop(direct)
            rec["us_per_call"][name] = {"binding_host": bh, "binding_wall": bw, "c_abi_host": ch,
                                        "c_abi_wall": cw, "graph_replay": graph(bound)}
        print(json.dumps(rec), flush=True)


def fp8_compare(args):
    """The fused GEMM (AUTO, i.e. variant I) on FP8 E4M3 operands against the
    same call on bf16, and variant S on FP8, per workload (one JSON line each).  The operands are quantized once,
    untimed (power-of-two tensor scales from the absolute maxima), like the
    weight pack; the timed call is the fused GEMM alone."""
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sw.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for idx in (int(x) for x in args.fp8_workloads.split(",")):
        w = inputs.WORKLOADS[idx]
        M, K, N = w.M, w.K, w.N
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed)
        A = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
        W1 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        W2 = (torch.randn(K, N, device=dev, generator=g) / K ** 0.5).to(torch.bfloat16)
        Wf = sw.swiglu_pack_weights(W1, W2)
        del W1, W2
        a_exp = sw.swiglu_fp8_scale_exp(float(A.float().abs().max()))
        w_exp = sw.swiglu_fp8_scale_exp(float(Wf.float().abs().max()))
        A8 = sw.swiglu_quantize_fp8(A, a_exp)
        W8 = sw.swiglu_quantize_fp8(Wf, w_exp)
        step16 = 2 * (M * K + 2 * K * N + M * N)
        R = max(1, -(-512 * 2 ** 20 // step16))
        # inputs and outputs rotate together, as in the default line
        Ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        bf = [(A, Wf, Ys[0])] + [(A.clone(), Wf.clone(), Ys[r]) for r in range(1, R)]
        f8 = [(A8, W8, Ys[0])] + [(A8.clone(), W8.clone(), Ys[r]) for r in range(1, R)]
        ws = sw.make_workspace(M, N, K, "i", dev)
        torch.cuda.synchronize()
        us16 = _time_call(lambda a, wf, y: sw.swiglu_fused_gemm(a, wf, Y=y, variant="auto",
                                                                workspace=ws),
                          bf, stream, budget_s=0.25, max_reps=2000)
        us8 = _time_call(lambda a, wf, y: sw.swiglu_fused_gemm_fp8(a, wf, a_exp, w_exp, Y=y,
                                                                   workspace=ws),
                         f8, stream, budget_s=0.25, max_reps=2000)
        us8s = _time_call(lambda a, wf, y: sw.swiglu_fused_gemm_fp8(a, wf, a_exp, w_exp, Y=y,
                                                                    variant="s"),
                          f8, stream, budget_s=0.25, max_reps=2000)
        flops = 4 * M * N * K
        t8 = flops / (us8 * 1e-6) / 1e12
        rec = {
            "workload": f"fused SwiGLU GEMM M={M} K={K} N={N} (seed {w.seed})",
            "M": M, "K": K, "N": N, "rotation_copies": R, "a_exp": a_exp, "w_exp": w_exp,
            "us": {"bf16": round(us16, 2), "fp8": round(us8, 2), "fp8_s": round(us8s, 2)},
            "tflops": {"bf16": round(flops / (us16 * 1e-6) / 1e12, 1), "fp8": round(t8, 1),
                       "fp8_s": round(flops / (us8s * 1e-6) / 1e12, 1)},
            "fp8_pct_of_fp8_peak": round(100 * t8 / PEAK_FP8_TFLOPS, 2),
            "fp8_speedup_vs_bf16": round(us16 / us8, 3),
            "fp8_launch": sw.swiglu_describe_launch(M, N, K, "fp8",
                                                    0 if ws is None else ws.numel()),
        }
        print(json.dumps(rec), flush=True)
        del bf, f8, Ys, A, Wf, A8, W8, ws
        torch.cuda.empty_cache()
    if args.copy_calibration:
        # one plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()


def sweep(args):
    """Variant I vs S vs the ablation over M, per K x N shape (one JSON line each)."""
    import torch

    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sw.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    ms_list = [int(x) for x in args.sweep_m.split(",")]
    ws = {}

    def body(K, N, M, copies, Wf):
        if (K, N) not in ws:
            ws.clear()
            ws[(K, N)] = {v: sw.make_workspace(max(ms_list), N, K, v, dev)
                          for v in ("i", "ablation")}
        w = ws[(K, N)]
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        G = torch.empty_like(Y)
        U = torch.empty_like(Y)
        calls = {
            "i": lambda a, wf: sw.swiglu_fused_gemm(a, wf, Y=Y, variant="i", workspace=w["i"]),
            "s": lambda a, wf: sw.swiglu_fused_gemm(a, wf, Y=Y, variant="s"),
            "ablation": lambda a, wf: sw.swiglu_unfused_ablation(a, wf, G, U, Y,
                                                                 workspace=w["ablation"]),
        }
        rec = {"K": K, "N": N, "M": M, "rotation_copies": len(copies), "us": {}, "tflops": {}}
        for name, fn in calls.items():
            us = _time_call(fn, copies, stream)
            rec["us"][name] = round(us, 2)
            rec["tflops"][name] = round(4 * M * N * K / (us * 1e-6) / 1e12, 1)
        rec["fastest_fused"] = min(("i", "s"), key=lambda v: rec["us"][v])
        rec["speedup_i_vs_ablation"] = round(rec["us"]["ablation"] / rec["us"]["i"], 3)
        rec["speedup_s_vs_ablation"] = round(rec["us"]["ablation"] / rec["us"]["s"], 3)
        print(json.dumps(rec), flush=True)

    _sweep_shapes(dev, ms_list, body)


def kernel_source_hash() -> str:
    from gated_mlp_gemm_amd.counters import kernel_source_hash as h
    return h()


def traffic_record(variant: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    table_path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(table_path):
        return None
    with open(table_path) as f:
        table = json.load(f)
    rec = table.get(f"{variant}|{workload}")
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _warm_up(step_fn, steps, min_s):
    """`steps` untimed steps, continued until at least `min_s` seconds of GPU
    work have run (the clock settles under sustained MFMA load: short runs
    read fast).  Returns the number of steps run."""
    import torch

    s = 0
    t0 = time.perf_counter()
    while s < steps or time.perf_counter() - t0 < min_s:
        step_fn(s)
        s += 1
        if s % 8 == 0:
            torch.cuda.synchronize()   # so that wall time follows GPU time
    torch.cuda.synchronize()
    return s


def _timed(step_fn, steps, stream, start=0):
    """Milliseconds per step over `steps` back-to-back steps, HIP events on
    `stream` (the stream the library launches on)."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(start, start + steps):
        step_fn(s)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _alternating(paths, steps, stream, repeats):
    """Per-step ms of each path over `repeats` rounds in which every path runs
    one loop of `steps` steps in turn (so clock drift hits all paths alike):
    {name: {"median": ms, "min": ms, "all": [ms, ...]}}."""
    import statistics

    runs = {name: [] for name in paths}
    for r in range(repeats):
        for name, fn in paths.items():
            runs[name].append(_timed(fn, steps, stream, start=r * steps))
    return {name: {"median": statistics.median(v), "min": min(v), "all": v}
            for name, v in runs.items()}


def _workload_record(args, idx, dev, stream):
    """One workload (inputs drawn on the device with the workload's recipe and
    seed): AUTO, variant I, variant S and the unfused ablation in alternating
    repeats; per-call median and min, TFLOP/s and the fraction of the bf16
    peak from the median, speedup over the ablation (median over median)."""
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    w = inputs.WORKLOADS[idx]
    M, K, N = w.M, w.K, w.N
    flops = 4 * M * N * K
    A, W1, W2 = inputs.device_inputs(M, K, N, w.seed, dev)
    Wf = sw.swiglu_pack_weights(W1, W2)
    del W1, W2
    step_bytes = 2 * (M * K + 2 * K * N + M * N)
    R = max(1, -(-512 * 2 ** 20 // step_bytes))
    copies = [(A, Wf)] + [(A.clone(), Wf.clone()) for _ in range(R - 1)]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    gu = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    scratch = {v: sw.make_workspace(M, N, K, v, dev) for v in ("auto", "i", "ablation")}
    torch.cuda.synchronize()

    def fused(variant, wsname):
        def step(s):
            a, wf = copies[s % R]
            sw.swiglu_fused_gemm(a, wf, Y=outs[s % R], variant=variant,
                                 workspace=scratch.get(wsname))
        return step

    def ablation(s):
        a, wf = copies[s % R]
        sw.swiglu_unfused_ablation(a, wf, gate_ws=gu[0], up_ws=gu[1], Y=outs[s % R],
                                   workspace=scratch["ablation"])

    paths = {"auto": fused("auto", "auto"), "i": fused("i", "i"), "s": fused("s", None),
             "ablation": ablation}
    # loops of at least --steps steps and about 5 ms each
    t0 = time.perf_counter()
    for s in range(4):
        paths["auto"](s)
    torch.cuda.synchronize()
    est_ms = (time.perf_counter() - t0) * 1e3 / 4
    steps = max(args.steps, int(5.0 / max(est_ms, 1e-3)))
    for fn in paths.values():
        _warm_up(fn, args.warmup, args.warmup_seconds / 4)
    t = _alternating(paths, steps, stream, args.repeats)
    med = t["auto"]["median"]
    tflops = flops / (med * 1e-3) / 1e12
    ws = scratch["auto"]
    rec = {
        "workload": f"fused SwiGLU GEMM M={M} K={K} N={N} (seed {w.seed}, A~N(0,1), "
                    f"W~N(0,1/K), bf16, drawn on the device)",
        "M": M, "K": K, "N": N, "rotation_copies": R, "steps_per_loop": steps,
        "repeats": args.repeats,
        "us_per_call": {k: {"median": round(v["median"] * 1e3, 2), "min": round(v["min"] * 1e3, 2)}
                        for k, v in t.items()},
        "tflops": round(tflops, 2),
        "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "tflops_per_variant": {k: round(flops / (v["median"] * 1e-3) / 1e12, 2)
                               for k, v in t.items()},
        "speedup_vs_ablation": round(t["ablation"]["median"] / med, 4),
        "speedup_s_vs_ablation": round(t["ablation"]["median"] / t["s"]["median"], 4),
        "kernel": sw.swiglu_describe_launch(M, N, K, "auto", 0 if ws is None else ws.numel()),
    }
    if M <= 1024:
        # HBM-bound end of the range: algorithmic bytes over the call time
        rec["hbm_gbs_algorithmic"] = round(step_bytes / (med * 1e-3) / 1e9, 1)
        rec["frac_hbm_peak"] = round(step_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    del copies, outs, gu, scratch, A, Wf
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the fused SwiGLU GEMM is a single-device "
              "kernel here (a column split of N needs no communication, so each GPU would "
              "run this same call on its share of the columns); --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return
    if args.mlp:
        mlp_blocks(args)
        return
    if args.fp8:
        fp8_compare(args)
        return
    if args.schedule_calibration:
        schedule_calibration(args)
        return
    if args.launch_cost:
        launch_cost(args)
        return

    import numpy as np
    import torch

    from gated_mlp_gemm_amd import inputs
    from gated_mlp_gemm_amd import swiglu as sw

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    sw.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = inputs.WORKLOADS[args.workload]
    M, K, N = w.M, w.K, w.N
    flops = 4 * M * N * K

    print(f"[bench] headline workload M={M} K={K} N={N} (seed {w.seed}): drawing inputs",
          file=sys.stderr, flush=True)
    A, W1, W2 = inputs.workload_inputs(w)
    Ad = A.to(dev)
    Wf = sw.swiglu_pack_weights(W1.to(dev), W2.to(dev))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    chosen = {"auto": sw.swiglu_select_variant(M, N, K), "i": sw.SWIGLU_VARIANT_I,
              "s": sw.SWIGLU_VARIANT_S}[args.variant]
    vname = "i" if chosen == sw.SWIGLU_VARIANT_I else "s"

    # rotation copies: fused working set (A + packed weights + Y) times R >= 512 MB
    ws_bytes = 2 * (M * K + 2 * K * N + M * N)
    R = max(1, -(-512 * 2 ** 20 // ws_bytes))
    copies = [(Ad, Wf)]
    for _ in range(R - 1):
        copies.append((Ad.clone(), Wf.clone()))
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    gate_up = (torch.empty((M, N), dtype=torch.bfloat16, device=dev),
               torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    # scratch for the split-tail schedule (one per path, reused by every step)
    scratch = {v: sw.make_workspace(M, N, K, v, dev) for v in ("auto", "i", "s", "ablation")}
    torch.cuda.synchronize()

    def fused_step(variant):
        def step(s):
            a, wf = copies[s % R]
            sw.swiglu_fused_gemm(a, wf, Y=outs[s % R], variant=variant,
                                 workspace=scratch[variant])
        return step

    def ablation_step(s):
        a, wf = copies[s % R]
        sw.swiglu_unfused_ablation(a, wf, gate_ws=gate_up[0], up_ws=gate_up[1], Y=outs[s % R],
                                   workspace=scratch["ablation"])

    # the headline: W warm-up steps (and at least --warmup-seconds of work),
    # then exactly K timed steps of the dispatched fused call
    head = fused_step(args.variant)
    warm_steps = _warm_up(head, args.warmup, args.warmup_seconds)
    wall0 = time.perf_counter()
    ms = _timed(head, args.steps, stream, start=warm_steps)
    wall = time.perf_counter() - wall0
    tflops = flops / (ms * 1e-3) / 1e12
    print(f"[bench] fused {args.variant}->{vname}: {ms * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s "
          f"(R={R}, {warm_steps} warm-up steps, timed wall {wall:.3f}s)", file=sys.stderr,
          flush=True)

    # the partners, in alternating repeats of K-step loops (AUTO again, each
    # fused variant, the unfused ablation): medians and minima per call
    partners = {"auto": head, "i": fused_step("i"), "s": fused_step("s"),
                "ablation": ablation_step}
    for name, fn in partners.items():
        if name != "auto":
            _warm_up(fn, args.warmup, args.warmup_seconds / 4)
    per = _alternating(partners, args.steps, stream, args.repeats)
    for k, v in per.items():
        print(f"[bench] {k}: median {v['median'] * 1e3:.1f} us, min {v['min'] * 1e3:.1f} us "
              f"({flops / (v['median'] * 1e-3) / 1e12:.1f} TFLOP/s)", file=sys.stderr, flush=True)

    # context, not the headline: the same call on FP8 E4M3 operands (power-of-two
    # tensor scales from the absolute maxima), with the operands quantized
    # beforehand, and with the activation quantized inside each timed step
    fp8 = None
    if not args.no_fp8:
        a_exp = sw.swiglu_fp8_scale_exp(float(A.float().abs().max()))
        w_exp = sw.swiglu_fp8_scale_exp(float(Wf.float().abs().max()))
        copies8 = [(sw.swiglu_quantize_fp8(a, a_exp), sw.swiglu_quantize_fp8(wf, w_exp))
                   for a, wf in copies]
        torch.cuda.synchronize()

        def fp8_step(quantize_a):
            def step(s):
                a8, w8 = copies8[s % R]
                if quantize_a:
                    sw.swiglu_quantize_fp8(copies[s % R][0], a_exp, Q=a8)
                sw.swiglu_fused_gemm_fp8(a8, w8, a_exp, w_exp, Y=outs[s % R],
                                         workspace=scratch["i"])
            return step

        _warm_up(fp8_step(False), args.warmup, args.warmup_seconds / 4)
        t8 = _alternating({"fp8": fp8_step(False), "fp8_quantize_a": fp8_step(True)},
                          args.steps, stream, args.repeats)
        ms8, msq = t8["fp8"]["median"], t8["fp8_quantize_a"]["median"]
        tf8 = flops / (ms8 * 1e-3) / 1e12
        fp8 = {
            "ms": round(ms8, 5), "tflops": round(tf8, 2),
            "pct_fp8_peak": round(100 * tf8 / PEAK_FP8_TFLOPS, 2),
            "speedup_vs_bf16": round(per["auto"]["median"] / ms8, 4),
            "ms_with_activation_quantize": round(msq, 5),
            "a_exp": a_exp, "w_exp": w_exp,
            "kernel": sw.swiglu_describe_launch(M, N, K, "fp8", scratch["i"].numel()
                                                if scratch["i"] is not None else 0),
        }
        print(f"[bench] fp8: {ms8 * 1e3:.1f} us, {tf8:.1f} TFLOP/s "
              f"({msq * 1e3:.1f} us with A quantized per step)", file=sys.stderr, flush=True)
        del copies8

    if args.copy_calibration:
        # one plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # what the fused call launches (tile shape and schedule chosen by the
    # library; with a split tail, two kernels: the time covers the whole call)
    ws_used = scratch[args.variant]
    kernel = sw.swiglu_describe_launch(M, N, K, args.variant,
                                       0 if ws_used is None else ws_used.numel())
    workload = f"M={M},K={K},N={N}"
    roofline = {
        "bound": "mfma",
        "achieved": round(tflops, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        # FETCH_SIZE + WRITE_SIZE per call from rocprofv3 counter passes on the
        # current kernel sources (else null): bytes between the L2 caches and
        # the memory fabric, an upper bound on HBM bytes (the Infinity Cache
        # serves some of the fetches)
        "traffic": traffic_record(vname, workload),
        "traffic_kind": "L2-fabric bytes (FETCH_SIZE + WRITE_SIZE), copy-calibrated",
        "kernel": kernel,
        "timed": "the whole call (every launch of it), HIP events on the launch stream",
        "algorithmic_flops_per_launch": flops,
        "algorithmic_hbm_bytes_per_launch": ws_bytes,
    }
    del copies, outs, gate_up, scratch, Ad, Wf
    torch.cuda.empty_cache()

    # the other workloads, each with its own partners (sub-records)
    per_workload = []
    if not args.no_per_workload:
        for idx in range(len(inputs.WORKLOADS)):
            if idx == args.workload:
                continue
            rec = _workload_record(args, idx, dev, stream)
            print(f"[bench] {rec['workload']}: {rec['us_per_call']['auto']['median']} us, "
                  f"{rec['tflops']} TFLOP/s, {rec['speedup_vs_ablation']}x vs ablation",
                  file=sys.stderr, flush=True)
            per_workload.append(rec)

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle as it stands, on a bounded sample of the same workload:
        # whole output rows (all N columns, full K), as many rows -- and, if one
        # pass over all M rows is shorter than the target, as many passes --
        # as fit in about --cpu-seconds of CPU work
        import oracle
        orc = oracle.load()
        hA, hW1, hW2 = inputs.bits(A), inputs.bits(W1), inputs.bits(W2)
        probe = min(M, 8)
        t = time.perf_counter()
        orc.swiglu_rows(hA, hW1, hW2, np.arange(probe))
        per_row = (time.perf_counter() - t) / probe
        rows = int(min(M, max(probe, args.cpu_seconds / max(per_row, 1e-9))))
        # whole passes until two thirds of the target have elapsed (at most 20)
        passes = 0
        t = time.perf_counter()
        while True:
            orc.swiglu_rows(hA, hW1, hW2, np.arange(rows))
            passes += 1
            dt = time.perf_counter() - t
            if rows < M or passes >= 20 or dt >= args.cpu_seconds * 2.0 / 3.0:
                break
        cpu = {
            "value": round(4 * passes * rows * N * K / dt / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"{passes} pass(es) over rows 0..{rows - 1} of M={M} (all N={N} "
                      f"columns, K={K}), fp64 oracle; {dt:.1f} s",
        }

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"fused SwiGLU GEMM M={M} K={K} N={N} (seed {w.seed}, A~N(0,1), "
                        f"W~N(0,1/K), bf16)",
            "M": M, "K": K, "N": N,
            "variant": f"{args.variant}->{vname}",
            "rotation_copies": R,
            "warmup_steps_run": warm_steps,
            "workspace_bytes": int(ws_used.numel()) if ws_used is not None else 0,
        },
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_ablation": round(per["ablation"]["median"] / per["auto"]["median"], 4),
        "per_variant": {k: {"ms_median": round(v["median"], 5), "ms_min": round(v["min"], 5),
                            "tflops_median": round(flops / (v["median"] * 1e-3) / 1e12, 2)}
                        for k, v in per.items()},
        "partner_protocol": f"{args.repeats} alternating repeats of {args.steps}-step loops",
        "roofline": roofline,
        "fp8": fp8,
        "per_workload": per_workload,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
