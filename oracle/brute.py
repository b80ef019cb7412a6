"""Pure-Python brute force of paged attention for tiny cases (test infrastructure only).

An independent second writing of the same definition as ``attention.py``
(softmax attention with bottom-right causal alignment through a block table;
InferMatrixLab/vllm-rlt PR #128, "Purpose", Prefill), using Python floats,
``math.exp``/``math.log`` and ``math.fsum`` and no numpy arithmetic, so that the
vectorised oracle can be pinned against it to ~1e-12 on inputs small enough
for a triple loop (a few thousand attended pairs).
"""

import math


def _f(x):
    return float(x)


def brute_paged_attention(q, k_pool, v_pool, cu_seqlens_q, seq_lens, block_tables, scale, window_left=-1,
                          sinks=None, softcap=0.0, alibi_slopes=None):
    """q [total_q][Hq][D]; pools [num_pages][page_size][Hkv][D] (float values).
    window_left >= 0: the token at key position p sees keys p - window_left .. p;
    sinks[h]: a logit with no value added to head h's softmax denominator;
    softcap > 0: each logit z becomes softcap * tanh(z / softcap), then
    alibi_slopes[h]: the logit of key j drops by alibi_slopes[h] * (p - j).

    Returns (out, lse) as nested Python lists: out[t][h][d], lse[t][h].
    """
    total_q = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    page_size = len(k_pool[0])
    Hkv = len(k_pool[0][0])
    g = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(total_q)]
    lse = [[-math.inf] * Hq for _ in range(total_q)]
    for b in range(len(seq_lens)):
        t0 = int(cu_seqlens_q[b])
        t1 = int(cu_seqlens_q[b + 1])
        Q = t1 - t0
        L = int(seq_lens[b])
        for i in range(Q):
            n_vis = L - Q + i + 1
            first = 0 if window_left is None or window_left < 0 else max(0, n_vis - 1 - window_left)
            for h in range(Hq):
                kvh = h // g
                sink = None if sinks is None else _f(sinks[h])
                if n_vis <= first:
                    if sink is not None:
                        lse[t0 + i][h] = sink  # only the sink: zeros and lse = sink
                    continue  # no visible key: zeros and -inf
                qv = [_f(x) for x in q[t0 + i][h]]
                scores = []
                vals = []
                for j in range(first, n_vis):
                    page = int(block_tables[b][j // page_size])
                    slot = j % page_size
                    kj = k_pool[page][slot][kvh]
                    z = scale * math.fsum(qv[d] * _f(kj[d]) for d in range(D))
                    if softcap:
                        z = softcap * math.tanh(z / softcap)
                    if alibi_slopes is not None:
                        z -= _f(alibi_slopes[h]) * (n_vis - 1 - j)
                    scores.append(z)
                    vals.append([_f(x) for x in v_pool[page][slot][kvh]])
                m = max(scores) if sink is None else max(max(scores), sink)
                w = [math.exp(s - m) for s in scores]
                den = math.fsum(w + ([math.exp(sink - m)] if sink is not None else []))
                out[t0 + i][h] = [math.fsum(w[j] * vals[j][d] for j in range(len(w))) / den
                                  for d in range(D)]
                lse[t0 + i][h] = m + math.log(den)
    return out, lse
