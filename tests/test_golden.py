"""Values the pages print, checked against this repo's byte accounting (CPU only)."""
import json
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def test_lut_overhead_bits_per_param():
    """16 bf16 table entries per row of K = 4096 cost 0.0625 bit per weight."""
    with open(os.path.join(HERE, "golden", "lut_overhead.json")) as f:
        gold = json.load(f)
    K = gold["K"]
    N = 1000
    g = K     # one group: isolate the table term from alpha/beta
    # algorithmic bytes with M = 0 activations: idx + alpha/beta + table
    total_bits = 8 * bench.algorithmic_bytes(0, N, K, g)
    per_param = total_bits / (N * K)
    idx_bits = 4.0
    ab_bits = 2 * 16 / g
    assert abs(per_param - idx_bits - ab_bits - gold["bits_per_param"]) < 1e-12
    assert gold["lut_entries"] * gold["entry_bits"] / K == gold["bits_per_param"]
