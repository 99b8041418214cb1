"""The committed HBM traffic records against the benchmark's byte model.

Each record holds the bytes per decode launch measured with rocprofv3's
FETCH_SIZE and WRITE_SIZE counters (scaled by a plain device copy) for the
OPT-6.7B-shaped layer. The algorithmic bytes it was compared with must be
what bench.py's byte model gives for that layer today, and the measured
traffic must lie within 10% of it (no wasted re-reads, nothing skipped).
"""
import glob
import json
import os

import pytest

import bench
from workload import ELEM_BYTES, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.json")))
BITS = {"u8": 8, "u4": 4, "u2": 2}


def algorithmic_bytes(name: str) -> float:
    base = os.path.basename(name)[len("decode_"):-len("_hbm_traffic.json")]
    mode, _, wname = base.partition("_") if base.split("_")[0] in BITS else ("bf16", "", base)
    wl = WORKLOADS[wname]
    d, e, k, n, T = wl.head_dim, ELEM_BYTES[wl.dtype], wl.k, wl.prompt_len, wl.steps
    used = [min(k, n + t) for t in range(T)]
    if mode in BITS:
        per = [bench.decode_bytes_per_head_quant(u, d, e, BITS[mode]) for u in used]
    else:
        per = [bench.decode_bytes_per_head(u, d, e) for u in used]
    return wl.n_heads_total * sum(per) / T


def test_records_exist():
    assert len(RECORDS) >= 4


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_record_matches_byte_model(path):
    with open(path) as f:
        rec = json.load(f)
    alg = algorithmic_bytes(path)
    assert rec["algorithmic_bytes_per_launch"] == pytest.approx(alg, rel=1e-9)
    ratio = rec["bytes_per_launch"] / alg
    assert 0.9 <= ratio <= 1.1, f"measured traffic {ratio:.3f}x the byte model"
    assert rec["bytes_per_launch"] == pytest.approx(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])
