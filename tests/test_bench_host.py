"""CPU tests of bench.py's host-side bookkeeping (no GPU, no kernel launch)."""
from __future__ import annotations

import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_record_looks_up_variant_and_workload():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        table = json.load(f)
    current = bench.kernel_source_hash()
    for key, rec in table.items():
        variant, workload = key.split("|")
        got = bench.traffic_record(variant, workload)
        if rec["kernel_source_hash"] == current:
            # counters taken on these sources: the record carries their bytes
            assert got == rec["hbm_bytes_per_launch"], key
        else:
            # counters of other sources are never reported
            assert got is None, key
    assert bench.traffic_record("i", "M=1,K=8,N=8") is None
    assert bench.traffic_record("no-such-variant", "M=2048,K=1536,N=8960") is None


def _write_csv(directory, counter, rows):
    import csv
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "bench_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, value) in enumerate(rows):
            w.writerow([i + 1, name, counter, value])


def test_counter_table_from_synthetic_passes(tmp_path):
    from gated_mlp_gemm_amd import counters

    gemm_i = "gemm_tiles_kernel<TileShape<256, 256, 64, 2, 2, 2>, PairMulEpilogueT<false>, 2>"
    gemm_s = "gemm_tiles_kernel<TileShape<256, 256, 64, 2, 2, 2>, StoreEpilogue, 2>"
    copy = "__amd_rocclr_copyBuffer"
    # the copy reads half of what it moves on the fetch counter (scale 2)
    fetch = [(copy, 10.0), (gemm_i, 100.0), (gemm_i, 104.0), (gemm_i, 102.0),
             (gemm_s, 50.0), (gemm_s, 50.0), ("silu_mul_kernel", 30.0), (copy, 131072.0)]
    write = [(copy, 10.0), (gemm_i, 40.0), (gemm_i, 40.0), (gemm_i, 40.0),
             (gemm_s, 40.0), (gemm_s, 40.0), ("silu_mul_kernel", 20.0), (copy, 262144.0)]
    _write_csv(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_csv(str(tmp_path / "w"), "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    counters.main([str(tmp_path / "f"), str(tmp_path / "w"), "--workload", "M=8,K=8,N=8",
                   "--out", str(out)])
    table = json.loads(out.read_text())
    i = table["i|M=8,K=8,N=8"]
    assert i["fetch_scale"] == 2.0 and i["write_scale"] == 1.0
    assert i["fetch_kib_raw"] == [102.0]                       # median of the dispatches
    assert i["hbm_bytes_per_launch"] == (102 * 2 + 40) * 1024
    ab = table["ablation|M=8,K=8,N=8"]
    assert ab["launches_per_call"] == [2, 1]
    assert ab["hbm_bytes_per_launch"] == (2 * (50 * 2 + 40) + (30 * 2 + 20)) * 1024
    assert "s|M=8,K=8,N=8" not in table                        # no sequential kernel ran
    assert i["kernel_source_hash"] == counters.kernel_source_hash()


def test_source_hash_ignores_comments_only():
    from gated_mlp_gemm_amd import counters

    a = 'int f(int x) { return x + 1; }  // one\n/* block\n comment */\nconst char *s = "//x";\n'
    b = '// header\nint f(int x)\n{\n    return x + 1;   /* inline */\n}\nconst char *s = "//x";\n'
    c = 'int f(int x) { return x + 2; }\nconst char *s = "//x";\n'
    d = 'int f(int x) { return x + 1; }\nconst char *s = "//y";\n'
    assert counters._code_only(a) == counters._code_only(b)
    assert counters._code_only(a) != counters._code_only(c)
    assert counters._code_only(a) != counters._code_only(d)     # strings are code
    assert counters._code_only('char q[] = "a\\\\"b"; int z;') == 'char q[] = "a\\\\"b"; int z;'
