"""One launch for a mixed step (pa_mixed_step) on the GPU, through the C ABI
(needs an MI355X): the small-q rows and the chunks of one batch against the
separate calls on the two sub-batches, bit for bit (the same work items and
kernel code), and against the fp64 oracle."""

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


# small-q rows first (q 1 and a verify row of 5, one row with q = 0), then chunks
# (one with more query tokens than keys, so that its first rows see no key)
Q_LENS = [1, 5, 0, 150, 40, 300]
SEQ_LENS = [700, 1300, 64, 900, 30, 2000]
ND = 3

MIXED_CASES = [
    # (q dtype, KV dtype, D, Hq, Hkv, page, prefill parts, decode parts, part_keys, options)
    ("f16", "f16", 256, 12, 2, 64, 3, 8, 0, {}),
    ("bf16", "bf16", 256, 6, 1, 48, 1, 12, 128, {"window_left": 300}),
    ("f16", "e5m2", 256, 8, 2, 64, 0, 8, 0, {"sinks": True}),
    ("f16", "e4m3", 256, 8, 2, 816, 2, 16, 0, {"softcap": 3.0, "alibi": True}),
    ("f16", "f16", 208, 8, 8, 32, 4, 8, 0, {"softcap": 2.0, "window_left": 100, "sinks": True}),
    ("bf16", "bf16", 128, 8, 2, 32, 3, 8, 0, {}),
    ("f32", "f32", 64, 4, 1, 16, 2, 4, 0, {"sinks": True}),
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


@pytest.mark.parametrize("qk,kvk,D,Hq,Hkv,P,sp,sd,part_keys,opts", MIXED_CASES)
def test_mixed_step_equals_separate_calls_and_oracle(qk, kvk, D, Hq, Hkv, P, sp, sd, part_keys, opts):
    c = gen.make_case(f"mixed_{qk}_{kvk}_D{D}", q_lens=Q_LENS, seq_lens=SEQ_LENS, num_q_heads=Hq,
                      num_kv_heads=Hkv, head_dim=D, page_size=P, q_kind=qk, kv_kind=kvk, seed=3 * D + Hq)
    host, dev = _options(Hq, opts, D + P)
    d = gen.to_device(c)
    dec_tok = int(c.cu_seqlens_q[ND])
    max_q = int(max(Q_LENS[:ND]))
    chunk_max = int(max(Q_LENS[ND:]))
    say(f"  mixed step {qk}/{kvk} D {D}: prefill parts {sp}, decode parts {sd}, part_keys {part_keys}, {opts}")
    out, lse = ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], ND, dec_tok, max_q, chunk_max,
                              c.scale, decode_splits=sd, decode_part_keys=part_keys, prefill_splits=sp,
                              k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True, **dev)
    torch.cuda.synchronize()

    # the separate calls on the two sub-batches
    dec, pre = gen.select_seqs(c, range(ND)), gen.select_seqs(c, range(ND, c.num_seqs))
    dd, dp = gen.to_device(dec), gen.to_device(pre)
    o_d, l_d = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], max_q, c.scale,
                                   num_splits=sd, part_keys=part_keys, k_scale=c.k_scale, v_scale=c.v_scale,
                                   return_lse=True, **dev)
    o_p, l_p = ops.paged_prefill(dp["q"], dp["k"], dp["v"], dp["cu"], dp["seq_lens"], dp["bt"], chunk_max, c.scale,
                                 num_kv_splits=sp, k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True, **dev)
    torch.cuda.synchronize()
    assert torch.equal(bits(out[:dec_tok]), bits(o_d)), "small-q rows differ from pa_split_kv_decode_ex"
    assert torch.equal(bits(lse[:dec_tok]), bits(l_d))
    assert torch.equal(bits(out[dec_tok:]), bits(o_p)), "chunks differ from pa_paged_prefill_ex"
    assert torch.equal(bits(lse[dec_tok:]), bits(l_p))

    # and the oracle over the whole batch
    k, v = pools64(c)
    ref, rl = oracle.paged_attention(gen.to_numpy64(c.q), k, v, c.cu_seqlens_q, c.seq_lens, c.block_tables, c.scale,
                                     window_left=host["window_left"], sinks=host["sinks"], softcap=host["softcap"],
                                     alibi_slopes=host["alibi_slopes"])
    kind = kvk if kvk in ("e5m2", "e4m3") else qk
    compare("mixed step vs oracle", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)


def test_mixed_step_with_only_one_kind_of_row():
    """No chunks, or no small-q rows: the call runs the one part there is."""
    c = gen.make_case("mixed_one", q_lens=[1, 4, 200], seq_lens=[500, 900, 1200], num_q_heads=8, num_kv_heads=2,
                      head_dim=256, page_size=64, q_kind="f16", seed=91)
    d = gen.to_device(c)
    full = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], 200, c.scale)
    dec = gen.select_seqs(c, [0, 1])
    dd = gen.to_device(dec)
    o1 = ops.mixed_step(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 2, 5, 4, 1, c.scale,
                        decode_splits=8)
    o2 = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 4, c.scale, num_splits=8)
    pre = gen.select_seqs(c, [2])
    dp = gen.to_device(pre)
    o3 = ops.mixed_step(dp["q"], dp["k"], dp["v"], dp["cu"], dp["seq_lens"], dp["bt"], 0, 0, 1, 200, c.scale,
                        prefill_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2))
    assert torch.equal(bits(o3), bits(full[5:]))
