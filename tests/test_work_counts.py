"""The work-count conventions against numbers printed on the pages (CPU only)."""

import json
import os

import numpy as np

import oracle
from paged_attention_prefill_amd import workload

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_flop_convention_reproduces_the_pages_tflops():
    g = GOLDEN["turing_d256_chunk"]
    L = g["q_len"] + g["prefix"]
    cu = [0, g["q_len"]]
    flops = workload.prefill_flops(cu, [L], g["num_q_heads"], g["head_dim"])
    for ms, tflops in g["timings_ms_and_tflops"]:
        got = flops / (ms * 1e-3) / 1e12
        assert abs(got / tflops - 1) < g["tolerance_rel"], (ms, got, tflops)


def test_closed_form_pair_count_equals_oracle_loop():
    rng = np.random.default_rng(0)
    for _ in range(20):
        B = int(rng.integers(1, 6))
        q = rng.integers(0, 40, B)
        L = rng.integers(0, 60, B)
        cu = np.concatenate([[0], np.cumsum(q)])
        assert workload.attended_pairs(cu, L) == oracle.attended_pairs(cu, L)
    # the long-chunk workload: 2048 after 150,000
    assert workload.attended_pairs([0, 2048], [152048]) == 309298176


def test_decode_bytes_counts_kv_once_per_kv_head():
    b = workload.decode_bytes([0, 1], [100000], 24, 4, 256, 64, "f16", "f16", 1)
    kv = 100000 * 4 * 256 * 2 * 2
    assert kv < b < kv * 1.01


def test_windowed_counts_equal_a_brute_force_count():
    """Under a left window W the token at key position p sees keys max(0, p - W)
    .. p: the pair count is the sum of those ranges (counted one key at a time
    here), and the decode rows' bytes cover the keys some token of the row sees."""
    rng = np.random.default_rng(1)
    for _ in range(30):
        B = int(rng.integers(1, 5))
        q = rng.integers(0, 30, B)
        L = rng.integers(0, 80, B)
        W = int(rng.integers(0, 50))
        cu = np.concatenate([[0], np.cumsum(q)])
        brute = 0
        for b in range(B):
            for i in range(int(q[b])):
                p = int(L[b]) - int(q[b]) + i
                brute += sum(1 for j in range(max(0, p - W), p + 1) if j >= 0)
        assert workload.attended_pairs(cu, L, W) == brute
        assert workload.attended_pairs(cu, L, int(L.max()) + 1) == workload.attended_pairs(cu, L)
    # a q=1 row at 100,000 keys with W = 8191 reads 8192 keys per kv head
    b = workload.decode_bytes([0, 1], [100000], 24, 4, 256, 64, "f16", "f16", 1, window_left=8191)
    kv = 8192 * 4 * 256 * 2 * 2
    assert kv < b < kv * 1.02
