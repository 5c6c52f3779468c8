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
