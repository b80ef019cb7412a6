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
