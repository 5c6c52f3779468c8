"""Fit the schedule cost model of the variant-I / ablation GEMM launcher.

    python -m gated_mlp_gemm_amd.schedule_fit CALIBRATION.jsonl [--cus 256]

Input: the JSON lines of ``python bench.py --schedule-calibration`` -- per
(K, N, M) the time of variant I under each forced (tile, tail) schedule and
under the library's own choice ("auto").

The model (the one ``make_schedule`` / ``quad_tiles_faster`` in
``csrc/kernels.hip`` evaluate) prices a schedule in microseconds:

* every round of workgroups costs ``round_us`` plus nk K steps of its tile:
  ``step_256`` for 256x256x64 tiles (one workgroup per CU, G = CUs slots),
  ``step_128`` for 128x128x64 tiles (two per CU, G = 2 CUs), ``step_quarter``
  for the 128x128 quarter tiles a 256x256 kernel runs in a tail round;
* T tiles take T // G full rounds; the L = T mod G tiles of a partly idle
  last round run whole (one more round), as 4L quarter tiles (ceil(4L / G)
  rounds, 256x256 only), or split along K into s = min(G // L, nk) >= 2
  pieces: one round of ceil(nk / s) steps plus ``reduce_us`` and the fp32
  partials (L s BM BN 4 bytes, written and read back) at ``partial_bytes_per_us``.

The six constants are fitted by least squares on log time over all forced
rows (Nelder-Mead).  Printed: the constants, the fit's RMS error, and the
regret of the model's pick against the measured-fastest schedule per point;
with "auto" rows present, also the measured regret of the library's pick.
"""
from __future__ import annotations

import argparse
import collections
import json
import math

PARAMS = ("round_us", "step_256", "step_quarter", "step_128", "reduce_us",
          "partial_bytes_per_us")
START = (4.0, 1.7, 0.6, 1.0, 3.0, 6.0e6)


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def schedule_times(p, M: int, N: int, K: int, tile: str, cus: int = 256) -> dict:
    """Predicted microseconds of each tail schedule of the given tile shape."""
    round_us, step_256, step_quarter, step_128, reduce_us, bw = p
    bm, G, step = (256, cus, step_256) if tile == "256" else (128, 2 * cus, step_128)
    T = cdiv(M, bm) * cdiv(2 * N, bm)
    nk = cdiv(K, 64)
    rnd = round_us + nk * step
    R, L = divmod(T, G)
    if L == 0:
        return {"whole": R * rnd}
    out = {"whole": (R + 1) * rnd}
    if tile == "256":
        out["quarter"] = R * rnd + cdiv(4 * L, G) * (round_us + nk * step_quarter)
    s = min(G // L, nk)
    if s >= 2:
        out["split"] = (R * rnd + round_us + cdiv(nk, s) * step + reduce_us +
                        L * s * bm * bm * 4 * 2 / bw)
    return out


def predict(p, M, N, K, tile, tail, cus=256) -> float:
    t = schedule_times(p, M, N, K, tile, cus)
    return t.get(tail, t["whole"])


def fit(rows, cus=256):
    from scipy.optimize import minimize

    forced = [r for r in rows if r["tile"] != "auto"]

    def loss(p):
        if min(p) <= 0:
            return 1e9
        return sum(math.log(predict(p, r["M"], r["N"], r["K"], r["tile"], r["tail"], cus) /
                            r["us"]) ** 2 for r in forced)

    res = minimize(loss, START, method="Nelder-Mead",
                   options={"maxiter": 20000, "xatol": 1e-6, "fatol": 1e-9})
    return list(res.x), math.sqrt(res.fun / len(forced))


def regrets(p, rows, cus=256):
    """Per point: (model pick, its measured us, measured-fastest, its us)."""
    by = collections.defaultdict(dict)
    for r in rows:
        by[(r["K"], r["N"], r["M"])][(r["tile"], r["tail"])] = r["us"]
    out = []
    for (K, N, M), d in sorted(by.items()):
        forced = {c: v for c, v in d.items() if c[0] != "auto"}
        pred = {}
        for tile in ("256", "128"):
            for tail, v in schedule_times(p, M, N, K, tile, cus).items():
                pred[(tile, tail)] = v
        pick = min(pred, key=pred.get)
        got = forced.get(pick, forced.get((pick[0], "whole")))
        best = min(forced, key=forced.get)
        out.append(((K, N, M), pick, got, best, forced[best], d.get(("auto", "auto"))))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("calibration")
    ap.add_argument("--cus", type=int, default=256)
    args = ap.parse_args()
    rows = [json.loads(line) for line in open(args.calibration) if line.strip()]
    p, rms = fit(rows, args.cus)
    print("fitted constants:")
    for name, v in zip(PARAMS, p):
        print(f"  {name:22s} {v:.4g}")
    print(f"RMS error of log time: {rms:.4f} ({len([r for r in rows if r['tile'] != 'auto'])} "
          "forced timings)")
    reg = regrets(p, rows, args.cus)
    model = [got / best_us - 1 for _, _, got, _, best_us, _ in reg]
    print(f"model pick vs measured-fastest: mean regret {100 * sum(model) / len(model):.2f} %, "
          f"max {100 * max(model):.1f} %")
    auto = [a / best_us - 1 for _, _, _, _, best_us, a in reg if a is not None]
    if auto:
        print(f"library pick (auto rows) vs measured-fastest: mean regret "
              f"{100 * sum(auto) / len(auto):.2f} %, max {100 * max(auto):.1f} % "
              f"({len(auto)} points)")


if __name__ == "__main__":
    main()
