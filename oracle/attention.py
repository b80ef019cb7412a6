"""numpy float64 oracle of paged softmax attention (test infrastructure only).

The method computes exact softmax attention; the kernels on the pages only
change where the keys come from (pages reached through a block table) and in
what order partial sums are formed.  So this oracle is the definition written
out in float64:

  for sequence b with L = seq_lens[b] keys and Q = cu_seqlens_q[b+1] -
  cu_seqlens_q[b] query tokens, query token i (0 <= i < Q) of query head h
  attends to keys j < n_i = L - Q + i + 1 of kv head h // (Hq / Hkv)
  (bottom-right causal alignment: InferMatrixLab/vllm-rlt PR #128, "Purpose",
  Prefill; the chunk sits at the end of the context as in 1CatAI/1Cat-vLLM
  PR #1279, commit 1 and its kernel microbenchmarks).  Key j of sequence b
  lives at page block_tables[b, j // P], slot j % P.
  s_j = scale * <q, K_j>;  m = max_j s_j;  w_j = exp(s_j - m);
  o = sum_j w_j V_j / sum_j w_j;  lse = m + log(sum_j w_j)  (natural log).
  A row with n_i <= 0 has no visible key: o = 0 and lse = -inf (the zero
  output for empty rows of PR #128, "Test Plan").

Split-KV (PR #128, "Purpose", Decode): the context of a row is cut into
S equal parts aligned to a tile of T keys, a function of the row's own length
only; every part yields an FP32 partial state (o_s normalised, lse_s) and a
second pass merges them by log-sum-exp.  The exact tile is not stated; the
reading used here is T = 32 and per = ceil(ceil(L/T)/S) tiles per part, part s
covering keys [s*per*T, min((s+1)*per*T, L)).

Rows are processed in blocks so that no score matrix of a long context exists
whole in memory.  Everything is float64; inputs are upcast exactly.
"""

import numpy as np

from .fp8 import e4m3_to_float64, e5m2_to_float64

# Decode split tile (keys); see the module docstring for the reading.
SPLIT_TILE = 32


def dequantize_pool(pool, kind, scale=1.0):
    """Exact float64 values of a KV page pool.

    ``kind`` is 'float' for any IEEE float storage (fp32, fp16, or bf16 already
    widened by the caller), 'e5m2' or 'e4m3' for a uint8 array of fp8 bytes, whose
    values are decode(byte) * scale; ``scale`` is one number or one per kv head (per-tensor scale; 1CatAI/1Cat-vLLM PR #616,
    fp8_e5m2 KV paragraph of "Test Result").
    """
    if kind == "float":
        return np.asarray(pool, dtype=np.float64)
    sc = np.asarray(scale, dtype=np.float64)
    if sc.ndim == 1:  # one factor per kv head (axis 2 of [pages, page_size, Hkv, D])
        sc = sc[None, None, :, None]
    if kind == "e5m2":
        return e5m2_to_float64(np.asarray(pool)) * sc
    if kind == "e4m3":
        return e4m3_to_float64(np.asarray(pool)) * sc
    raise ValueError(f"unknown pool kind {kind!r}")


def gather_dense_kv(pool, block_table_row, seq_len, kv_head):
    """Dense [seq_len, D] keys (or values) of one sequence and one kv head.

    ``pool`` is [num_pages, page_size, Hkv, D]; key j is read from page
    block_table_row[j // page_size], slot j % page_size.  Only the first
    ceil(seq_len / page_size) table entries are read.
    """
    page_size = pool.shape[1]
    j = np.arange(int(seq_len))
    pages = np.asarray(block_table_row, dtype=np.int64)[j // page_size]
    return np.asarray(pool[pages, j % page_size, kv_head, :], dtype=np.float64)


def visible_key_count(seq_len, q_len, i):
    """n_i = L - Q + i + 1: keys visible to query token i under bottom-right alignment."""
    return seq_len - q_len + i + 1


def window_start(seq_len, q_len, i, window_left):
    """First key visible to query token i under a left window: the token sits
    at key L - Q + i and sees keys j >= L - Q + i - window_left (window_left < 0:
    no window, start 0)."""
    i = np.asarray(i, dtype=np.int64)
    if window_left is None or window_left < 0:
        return np.zeros_like(i)
    return np.maximum(0, seq_len - q_len + i - int(window_left))


def add_sink(o, lse, sink):
    """The softmax with one more logit `sink` in its denominator and no value:
    o * sum_j e^s_j / (sum_j e^s_j + e^sink), lse = log(sum_j e^s_j + e^sink)."""
    new = np.logaddexp(lse, sink)
    with np.errstate(invalid="ignore"):
        f = np.where(np.isfinite(lse), np.exp(lse - new), 0.0)
    return o * f[..., None], new


def modified_logits(s, softcap=0.0, slopes=None, dist=None):
    """Score modifiers on natural-unit logits s = scale * q.k (both readings of
    variants the pages only name: 1CatAI/1Cat-vLLM PR #1279, commit 1, the
    Turing selection rule).  softcap > 0: s -> softcap * tanh(s / softcap),
    which bounds every logit to (-softcap, softcap).  slopes: ALiBi, then
    s -> s - slope * dist, dist = p - j for the query token at key position p
    and key j (slopes broadcast against s's rows).  Softcap comes first."""
    if softcap:
        s = softcap * np.tanh(s / softcap)
    if slopes is not None:
        s = s - np.asarray(slopes, dtype=np.float64).reshape(-1, 1) * dist
    return s


def attention_rows(qrows, K, V, counts, scale, key_lo=0, key_hi=None, block=128, starts=None,
                   softcap=0.0, alibi=None):
    """Softmax attention of query rows over a key range.

    Row r attends to keys j with max(key_lo, starts[r]) <= j < min(counts[r],
    key_hi, len(K)).  Returns (o [n, D], lse [n]); a row with no key in range
    gets o = 0 and lse = -inf.  softcap / alibi (a slope per row, or one for
    all rows): see modified_logits; row r's query token sits at key position
    counts[r] - 1.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    counts = np.asarray(counts, dtype=np.int64)
    starts = np.zeros_like(counts) if starts is None else np.asarray(starts, dtype=np.int64)
    n, D = qrows.shape
    if alibi is not None:
        alibi = np.broadcast_to(np.asarray(alibi, dtype=np.float64), (n,))
    L = K.shape[0]
    hi = L if key_hi is None else min(int(key_hi), L)
    o = np.zeros((n, D), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    for r0 in range(0, n, block):
        qb = qrows[r0:r0 + block]
        end = np.minimum(counts[r0:r0 + block], hi)
        emax = int(end.max()) if end.size else 0
        if emax <= key_lo:
            continue
        Kb = K[key_lo:emax]
        Vb = V[key_lo:emax]
        s = scale * (qb @ Kb.T)
        j = np.arange(key_lo, emax)
        if softcap or alibi is not None:
            dist = (counts[r0:r0 + block] - 1)[:, None] - j[None, :]
            s = modified_logits(s, softcap, None if alibi is None else alibi[r0:r0 + block], dist)
        vis = (j[None, :] < end[:, None]) & (j[None, :] >= starts[r0:r0 + block][:, None])
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        has = np.isfinite(m)
        w = np.where(vis, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
        den = w.sum(axis=1)
        ob = (w @ Vb) / np.where(has, den, 1.0)[:, None]
        o[r0:r0 + block] = np.where(has[:, None], ob, 0.0)
        with np.errstate(divide="ignore"):
            lse[r0:r0 + block] = np.where(has, m + np.log(np.where(has, den, 1.0)), -np.inf)
    return o, lse


def _token_to_seq(cu):
    total = int(cu[-1])
    return np.searchsorted(cu, np.arange(total), side="right") - 1


def paged_attention(q, k_pool, v_pool, cu_seqlens_q, seq_lens, block_tables, scale, rows=None,
                    window_left=-1, sinks=None, softcap=0.0, alibi_slopes=None):
    """Varlen paged attention in float64.

    q            [total_q, Hq, D]
    k_pool/v_pool [num_pages, page_size, Hkv, D] (float64 values; see dequantize_pool)
    cu_seqlens_q [B + 1], seq_lens [B], block_tables [B, max_pages]
    rows         optional [n, 2] array of (token, q head) pairs to compute.
    window_left  >= 0: token i also needs j >= L - Q + i - window_left (see window_start).
    sinks        optional [Hq] logits, one more term in each head's softmax denominator.
    softcap      > 0: logits capped by softcap * tanh(logit / softcap) (see modified_logits).
    alibi_slopes optional [Hq]: head h's logit of key j for the token at key position p
                 loses alibi_slopes[h] * (p - j).

    Returns (out [total_q, Hq, D], lse [total_q, Hq]) or, with ``rows``,
    (out [n, D], lse [n]) in the order given.
    """
    q = np.asarray(q, dtype=np.float64)
    total_q, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    if cu[-1] != total_q:
        raise ValueError("cu_seqlens_q[-1] must equal total_q")

    if rows is None:
        out = np.zeros((total_q, Hq, D))
        lse = np.full((total_q, Hq), -np.inf)
        want = None
    else:
        want = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        out = np.zeros((len(want), D))
        lse = np.full(len(want), -np.inf)
        seq_of = _token_to_seq(cu)[want[:, 0]]

    for b in range(len(L)):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        Qb, Lb = t1 - t0, int(L[b])
        if Qb == 0:
            continue
        for h in range(Hkv):
            heads = range(h * g, (h + 1) * g)
            if want is not None:
                sel = np.nonzero((seq_of == b) & (want[:, 1] // g == h))[0]
                if sel.size == 0:
                    continue
            K = gather_dense_kv(k_pool, bt[b], Lb, h)
            V = gather_dense_kv(v_pool, bt[b], Lb, h)
            if want is None:
                i = np.arange(Qb)
                counts = visible_key_count(Lb, Qb, i)
                starts = window_start(Lb, Qb, i, window_left)
                for qh in heads:
                    sl = None if alibi_slopes is None else float(alibi_slopes[qh])
                    o, s = attention_rows(q[t0:t1, qh, :], K, V, counts, scale, starts=starts,
                                          softcap=softcap, alibi=sl)
                    if sinks is not None:
                        o, s = add_sink(o, s, float(sinks[qh]))
                    out[t0:t1, qh, :] = o
                    lse[t0:t1, qh] = s
            else:
                toks = want[sel, 0]
                qrows = q[toks, want[sel, 1], :]
                counts = visible_key_count(Lb, Qb, toks - t0)
                starts = window_start(Lb, Qb, toks - t0, window_left)
                sl = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64)[want[sel, 1]]
                o, s = attention_rows(qrows, K, V, counts, scale, starts=starts, softcap=softcap, alibi=sl)
                if sinks is not None:
                    o, s = add_sink(o, s, np.asarray(sinks, dtype=np.float64)[want[sel, 1]])
                out[sel] = o
                lse[sel] = s
    return out, lse


def window_base(seq_len, q_len, window_left, tile=SPLIT_TILE):
    """First key any token of a sequence can see under a left window (its first
    token's window start), rounded down to the tile grid; 0 without a window."""
    if window_left is None or window_left < 0:
        return 0
    return (max(0, int(seq_len) - int(q_len) - int(window_left)) // tile) * tile


def split_ranges(seq_len, num_splits, tile=SPLIT_TILE, part_keys=0, base=0):
    """Key ranges of the S parts of a row of length seq_len.

    part_keys == 0: S tile-aligned parts cut from the row's own length
    (InferMatrixLab/vllm-rlt PR #128, "Purpose", Decode).  part_keys > 0:
    absolute parts [s * part_keys, (s + 1) * part_keys) clipped to the row,
    the last part running on to seq_len -- boundaries that do not move with the
    row's length, which is what lets a verify row be compared with serial
    decoding token for token (same page, "Purpose", Prefill)."""
    L = int(seq_len)
    if part_keys:
        C = int(part_keys)
        return [(min(s * C, L), L if s == num_splits - 1 else min((s + 1) * C, L)) for s in range(num_splits)]
    # parts of the keys the sequence can see, [base, L) (base: window_base)
    tiles = -(-(L - base) // tile)
    per = -(-tiles // num_splits)
    return [(min(base + s * per * tile, L), min(base + (s + 1) * per * tile, L)) for s in range(num_splits)]


def split_partials(qrows, K, V, counts, scale, num_splits, tile=SPLIT_TILE, part_keys=0, starts=None, base=0,
                   softcap=0.0, alibi=None):
    """Per-part partial states of rows over one sequence: (o_s [S, n, D], lse_s [S, n])."""
    ranges = split_ranges(K.shape[0], num_splits, tile, part_keys, base)
    os_, ls_ = [], []
    for lo, hi in ranges:
        o, s = attention_rows(qrows, K, V, counts, scale, key_lo=lo, key_hi=hi, starts=starts,
                              softcap=softcap, alibi=alibi)
        os_.append(o)
        ls_.append(s)
    return np.stack(os_), np.stack(ls_)


def merge_partials(o_s, lse_s):
    """Log-sum-exp merge over axis 0 of partial states (o_s normalised per part).

    M = max_s lse_s; w_s = exp(lse_s - M); o = sum_s w_s o_s / sum_s w_s;
    lse = M + log sum_s w_s.  All parts empty: o = 0, lse = -inf.
    """
    o_s = np.asarray(o_s, dtype=np.float64)
    lse_s = np.asarray(lse_s, dtype=np.float64)
    M = lse_s.max(axis=0)
    has = np.isfinite(M)
    w = np.exp(lse_s - np.where(has, M, 0.0))
    den = w.sum(axis=0)
    o = (w[..., None] * o_s).sum(axis=0) / np.where(has, den, 1.0)[..., None]
    o = np.where(has[..., None], o, 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, M + np.log(np.where(has, den, 1.0)), -np.inf)
    return o, lse


def attended_pairs(cu_seqlens_q, seq_lens):
    """Sum over query tokens of their visible key count (per query head)."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    L = np.asarray(seq_lens, dtype=np.int64)
    total = 0
    for b in range(len(L)):
        Qb = int(cu[b + 1] - cu[b])
        for i in range(Qb):
            total += max(0, int(L[b]) - Qb + i + 1)
    return total

