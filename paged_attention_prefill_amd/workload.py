"""Algorithmic work of one call: the units the throughput figures are priced in.

Prefill FLOPs count only attended (query, key) pairs, causal-exact: 2*D for the
QK^T dot product and 2*D for the PV update per pair and query head (the
convention that reproduces the pages' "about 23 TFLOPS" at 165.8 ms and "61
TFLOPS" at 61.5 ms for a 2048-token chunk after 150k tokens, 12 query heads,
D 256: 1CatAI/1Cat-vLLM PR #1279, commit 1).

Decode bytes count K and V of every row once per kv head (GQA heads re-read
from cache are not counted again), plus q, the output, the block-table entries
read and the FP32 partial states written and read back by the merge.
"""

import numpy as np

KV_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e5m2": 1, "e4m3": 1}
Q_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def attended_pairs(cu_seqlens_q, seq_lens, window_left=-1):
    """Per query head: sum over tokens of the visible keys, max(0, L - Q + i + 1)
    (closed form per sequence), each capped at window_left + 1 under a window."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    if window_left is not None and window_left >= 0:
        total = 0
        for b in range(len(L)):
            Q = int(cu[b + 1] - cu[b])
            n = int(L[b]) - Q + 1 + np.arange(Q, dtype=np.int64)
            total += int(np.minimum(np.maximum(n, 0), window_left + 1).sum())
        return total
    total = 0
    for b in range(len(L)):
        Q = int(cu[b + 1] - cu[b])
        lo = int(L[b]) - Q + 1          # visible count of token 0
        hi = int(L[b])                  # visible count of token Q-1
        first = max(lo, 1)
        if hi >= first:
            total += (first + hi) * (hi - first + 1) // 2
    return total


def prefill_flops(cu_seqlens_q, seq_lens, num_q_heads, head_dim, window_left=-1):
    return 4 * int(head_dim) * int(num_q_heads) * attended_pairs(cu_seqlens_q, seq_lens, window_left)


def decode_bytes(cu_seqlens_q, seq_lens, num_q_heads, num_kv_heads, head_dim, page_size,
                 q_kind, kv_kind, num_splits, window_left=-1):
    L = np.asarray(seq_lens, dtype=np.int64)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    total_q = int(cu[-1])
    if window_left is not None and window_left >= 0:  # keys some token of the row can see
        Q = np.diff(cu)
        keys = np.minimum(L, window_left + Q)
    else:
        keys = L
    kv = int(keys.sum()) * int(num_kv_heads) * int(head_dim) * 2 * KV_BYTES[kv_kind]
    qo = 2 * total_q * int(num_q_heads) * int(head_dim) * Q_BYTES[q_kind]
    bt = int(sum(-(-int(x) // int(page_size)) for x in keys)) * 4
    partial = 2 * total_q * int(num_q_heads) * int(num_splits) * (int(head_dim) + 2) * 4
    return kv + qo + bt + partial


def kv_write_bytes(cu_seqlens_q, seq_lens, num_kv_heads, head_dim, page_size, src_kind, kv_kind):
    """KV write: the new K and V rows read once and written once into the cache,
    plus cu_seqlens_q, seq_lens and the block-table entries the new tokens map to."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    total_q = int(cu[-1])
    rows = total_q * int(num_kv_heads) * int(head_dim) * 2
    pages = 0
    for b in range(len(L)):
        q = int(cu[b + 1] - cu[b])
        lo = max(0, int(L[b]) - q)
        if int(L[b]) > lo:
            pages += (int(L[b]) - 1) // int(page_size) - lo // int(page_size) + 1
    return rows * (Q_BYTES[src_kind] + KV_BYTES[kv_kind]) + (2 * len(L) + 1) * 4 + pages * 4
