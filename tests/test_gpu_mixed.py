"""A mixed step (pa_mixed_step) on the GPU, through the C ABI (needs an MI355X):
a batch in any order, its rows routed by query length on the device (small-q
rows to the split-KV decode, the others to the prefill), against the separate
calls on the two sub-batches, bit for bit (the same work items and kernel
code), and against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops
from parity_bars import compare, say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def pools64(case):
    kind = case.kv_kind if case.kv_kind in ("e5m2", "e4m3") else "float"
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), kind, case.k_scale)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), kind, case.v_scale)
    return k, v


# rows in no particular order: chunks, q = 1, an empty row, a verify row of 5,
# a chunk with more query tokens than keys (its first rows see no key), rows of
# 16 and 17 tokens on both sides of the default threshold
Q_LENS = [150, 1, 0, 5, 40, 300, 16, 17]
SEQ_LENS = [900, 700, 64, 1300, 30, 2000, 500, 1000]

MIXED_CASES = [
    # (q dtype, KV dtype, D, Hq, Hkv, page, prefill parts, decode parts, part_keys, decode_max_q, options)
    ("f16", "f16", 256, 12, 2, 64, 3, 8, 0, 0, {}),
    ("bf16", "bf16", 256, 6, 1, 48, 1, 12, 128, 0, {"window_left": 300}),
    ("f16", "e5m2", 256, 8, 2, 64, 2, 8, 0, 5, {"sinks": True}),
    ("bf16", "e4m3", 256, 8, 2, 816, 2, 16, 0, 0, {"softcap": 3.0, "alibi": True}),
    ("f16", "f16", 208, 8, 8, 32, 4, 8, 0, 0, {"softcap": 2.0, "window_left": 100, "sinks": True}),
    ("bf16", "bf16", 128, 8, 2, 32, 3, 8, 0, 16, {}),
    ("f16", "e5m2", 128, 8, 2, 32, 1, 8, 0, 1, {}),
    ("f32", "f32", 64, 4, 1, 16, 2, 4, 0, 0, {"sinks": True}),
]


def _options(Hq, opts, seed):
    rng = np.random.default_rng(seed)
    host = {"window_left": opts.get("window_left", -1), "softcap": opts.get("softcap", 0.0), "sinks": None,
            "alibi_slopes": None}
    if opts.get("sinks"):
        host["sinks"] = rng.normal(size=Hq).astype(np.float32)
    if opts.get("alibi"):
        host["alibi_slopes"] = gen.geometric_alibi_slopes(Hq)
    dev = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in host.items()}
    return host, dev


def token_index(case, seqs):
    cu = case.cu_seqlens_q
    parts = [np.arange(cu[b], cu[b + 1]) for b in seqs]
    return torch.from_numpy(np.concatenate(parts).astype(np.int64)) if parts else torch.zeros(0, dtype=torch.int64)


@pytest.mark.parametrize("qk,kvk,D,Hq,Hkv,P,sp,sd,part_keys,dmq,opts", MIXED_CASES)
def test_mixed_step_routes_rows_and_equals_separate_calls(qk, kvk, D, Hq, Hkv, P, sp, sd, part_keys, dmq, opts):
    c = gen.make_case(f"mixed_{qk}_{kvk}_D{D}", q_lens=Q_LENS, seq_lens=SEQ_LENS, num_q_heads=Hq,
                      num_kv_heads=Hkv, head_dim=D, page_size=P, q_kind=qk, kv_kind=kvk, seed=3 * D + Hq)
    host, dev = _options(Hq, opts, D + P)
    d = gen.to_device(c)
    thr = dmq or ops.MIXED_DECODE_MAX_Q
    small = [b for b, q in enumerate(Q_LENS) if 1 <= q <= thr]
    chunks = [b for b, q in enumerate(Q_LENS) if q > thr]
    say(f"  mixed step {qk}/{kvk} D {D}: decode_max_q {thr} -> small-q rows {small}, chunks {chunks}; "
        f"prefill parts {sp}, decode parts {sd}, part_keys {part_keys}, {opts}")
    out, lse = ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], Q_LENS, d["seq_lens"], d["bt"], c.scale,
                              decode_max_q=dmq, decode_splits=sd, decode_part_keys=part_keys, prefill_splits=sp,
                              k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True, **dev)
    torch.cuda.synchronize()

    # the separate calls on the two sub-batches
    dec, pre = gen.select_seqs(c, small), gen.select_seqs(c, chunks)
    dd, dp = gen.to_device(dec), gen.to_device(pre)
    o_d, l_d = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"],
                                   max(1, dec.max_seqlen_q), c.scale, num_splits=sd, part_keys=part_keys,
                                   k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True, **dev)
    o_p, l_p = ops.paged_prefill(dp["q"], dp["k"], dp["v"], dp["cu"], dp["seq_lens"], dp["bt"], pre.max_seqlen_q,
                                 c.scale, num_kv_splits=sp, k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True,
                                 **dev)
    torch.cuda.synchronize()
    ti_d, ti_p = token_index(c, small).cuda(), token_index(c, chunks).cuda()
    assert torch.equal(bits(out[ti_d]), bits(o_d)), "small-q rows differ from pa_split_kv_decode_ex"
    assert torch.equal(bits(lse[ti_d]), bits(l_d))
    assert torch.equal(bits(out[ti_p]), bits(o_p)), "chunks differ from pa_paged_prefill_ex"
    assert torch.equal(bits(lse[ti_p]), bits(l_p))

    # and the oracle over the whole batch
    k, v = pools64(c)
    ref, rl = oracle.paged_attention(gen.to_numpy64(c.q), k, v, c.cu_seqlens_q, c.seq_lens, c.block_tables, c.scale,
                                     window_left=host["window_left"], sinks=host["sinks"], softcap=host["softcap"],
                                     alibi_slopes=host["alibi_slopes"])
    kind = kvk if kvk in ("e5m2", "e4m3") else qk
    compare("mixed step vs oracle", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)


def test_mixed_step_with_only_one_kind_of_row():
    """Only small-q rows, or only chunks: the other class's grid finds no row."""
    c = gen.make_case("mixed_one", q_lens=[1, 4, 200], seq_lens=[500, 900, 1200], num_q_heads=8, num_kv_heads=2,
                      head_dim=256, page_size=64, q_kind="f16", seed=91)
    d = gen.to_device(c)
    full = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], 200, c.scale)
    dec = gen.select_seqs(c, [0, 1])
    dd = gen.to_device(dec)
    o1 = ops.mixed_step(dd["q"], dd["k"], dd["v"], dd["cu"], dec.q_lens, dd["seq_lens"], dd["bt"], c.scale,
                        decode_splits=8)
    o2 = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 4, c.scale, num_splits=8)
    pre = gen.select_seqs(c, [2])
    dp = gen.to_device(pre)
    o3 = ops.mixed_step(dp["q"], dp["k"], dp["v"], dp["cu"], pre.q_lens, dp["seq_lens"], dp["bt"], c.scale,
                        prefill_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2))
    assert torch.equal(bits(o3), bits(full[5:]))


def test_mixed_step_batch_order_does_not_change_a_row():
    """The same rows in two orders: every row's output and lse have the same bits."""
    c = gen.make_case("mixed_order", q_lens=[3, 120, 1, 64, 9], seq_lens=[800, 1500, 77, 64, 2222], num_q_heads=12,
                      num_kv_heads=2, head_dim=256, page_size=64, q_kind="bf16", seed=17)
    perm = [3, 1, 4, 0, 2]
    r = gen.select_seqs(c, perm)
    outs = []
    for case in (c, r):
        d = gen.to_device(case)
        o, l = ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], case.q_lens, d["seq_lens"], d["bt"], case.scale,
                              decode_splits=8, prefill_splits=2, return_lse=True)
        torch.cuda.synchronize()
        outs.append((o, l))
    (o0, l0), (o1, l1) = outs
    idx = token_index(c, perm).cuda()
    assert torch.equal(bits(o0[idx]), bits(o1)) and torch.equal(bits(l0[idx]), bits(l1))


@pytest.mark.parametrize("D,kvk", [(256, "f16"), (64, "bf16")])
def test_mixed_step_many_rows(D, kvk):
    """1,500 rows (more than the routing's work group of 1,024 threads, so its
    scans run over several waves and two chunks of rows): every row's output
    and lse equal the separate decode and prefill calls on the two classes."""
    rng = np.random.default_rng(D)
    q_lens = rng.choice([0, 1, 1, 2, 5, 16, 17, 40], size=1500)
    seq_lens = q_lens + rng.integers(0, 200, size=1500)
    c = gen.make_case(f"mixed_many_{D}", q_lens=q_lens.tolist(), seq_lens=seq_lens.tolist(), num_q_heads=8,
                      num_kv_heads=2, head_dim=D, page_size=32, q_kind=kvk, seed=D + 1)
    d = gen.to_device(c)
    small = [b for b, q in enumerate(q_lens) if 1 <= q <= ops.MIXED_DECODE_MAX_Q]
    chunks = [b for b, q in enumerate(q_lens) if q > ops.MIXED_DECODE_MAX_Q]
    say(f"  mixed step, {len(q_lens)} rows, D {D} {kvk}: {len(small)} small-q rows, {len(chunks)} chunks")
    out, lse = ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], q_lens, d["seq_lens"], d["bt"], c.scale,
                              decode_splits=4, prefill_splits=1, return_lse=True)
    torch.cuda.synchronize()
    dec, pre = gen.select_seqs(c, small), gen.select_seqs(c, chunks)
    dd, dp = gen.to_device(dec), gen.to_device(pre)
    o_d, l_d = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"],
                                   max(1, dec.max_seqlen_q), c.scale, num_splits=4, return_lse=True)
    o_p, l_p = ops.paged_prefill(dp["q"], dp["k"], dp["v"], dp["cu"], dp["seq_lens"], dp["bt"], pre.max_seqlen_q,
                                 c.scale, num_kv_splits=1, return_lse=True)
    torch.cuda.synchronize()
    ti_d, ti_p = token_index(c, small).cuda(), token_index(c, chunks).cuda()
    assert torch.equal(bits(out[ti_d]), bits(o_d)) and torch.equal(bits(lse[ti_d]), bits(l_d))
    assert torch.equal(bits(out[ti_p]), bits(o_p)) and torch.equal(bits(lse[ti_p]), bits(l_p))
