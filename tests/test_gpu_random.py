"""Seeded random configurations against the fp64 oracle (needs an MI355X).

Each case draws a dtype pair, a head dim (any multiple of 16 up to 256), a GQA
ratio, a page size, ragged query and key lengths (some rows with more query
tokens than keys, some empty), a part count and a combination of the options
(window, sinks, softcap, ALiBi), then checks the prefill of the whole batch
and the split-KV decode of its small-q rows (proportional or absolute parts)
against the oracle with the bars of parity_bars.py (max-abs, rms ratio and lse).  Sizes stay
small enough for the oracle to finish each case in about a second.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops
from parity_bars import compare, say

pytestmark = pytest.mark.gpu

KINDS = [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"), ("f16", "e5m2"), ("f16", "e4m3")]
PAGES = [16, 32, 48, 64, 128, 816]


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    qk, kvk = KINDS[seed % len(KINDS)]
    D = 16 * int(rng.integers(1, 17))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8]))
    P = int(rng.choice(PAGES))
    B = int(rng.integers(1, 5))
    q_lens, seq_lens = [], []
    for b in range(B):
        small = rng.random() < 0.5
        q = int(rng.integers(0, 17)) if small else int(rng.integers(17, 200))
        prefix = int(rng.integers(0, 1500))
        L = q + prefix if rng.random() < 0.85 else int(rng.integers(0, max(1, q)))  # q > L: empty first rows
        q_lens.append(q)
        seq_lens.append(L)
    opts = {}
    if rng.random() < 0.4:
        opts["window_left"] = int(rng.integers(0, 300))
    if rng.random() < 0.3:
        opts["sinks"] = rng.normal(size=Hkv * g).astype(np.float32)
    if rng.random() < 0.3:
        opts["softcap"] = float(rng.uniform(1.0, 20.0))
    if rng.random() < 0.3:
        opts["alibi_slopes"] = gen.geometric_alibi_slopes(Hkv * g)
    splits = int(rng.choice([0, 1, 2, 3, 5]))
    parts = int(rng.integers(1, 20))
    part_keys = int(rng.choice([0, 0, 32, 96, 512]))
    return dict(qk=qk, kvk=kvk, D=D, Hkv=Hkv, Hq=Hkv * g, P=P, q_lens=q_lens, seq_lens=seq_lens, opts=opts,
                splits=splits, parts=parts, part_keys=part_keys)


@pytest.mark.parametrize("seed", range(96))
def test_random_configuration(seed):
    c = draw(seed)
    say(f"  case {seed}: {c['qk']}/{c['kvk']} D {c['D']} Hq {c['Hq']} Hkv {c['Hkv']} P {c['P']} q {c['q_lens']} "
        f"L {c['seq_lens']} splits {c['splits']} parts {c['parts']} part_keys {c['part_keys']} "
        f"options {sorted(c['opts'])}")
    case = gen.make_case(f"random_{seed}", q_lens=c["q_lens"], seq_lens=c["seq_lens"], num_q_heads=c["Hq"],
                         num_kv_heads=c["Hkv"], head_dim=c["D"], page_size=c["P"], q_kind=c["qk"], kv_kind=c["kvk"],
                         seed=seed, k_scale=0.8 if c["kvk"] in ("e5m2", "e4m3") else 1.0,
                         v_scale=1.25 if c["kvk"] in ("e5m2", "e4m3") else 1.0)
    kind = c["kvk"] if c["kvk"] in ("e5m2", "e4m3") else c["qk"]
    opts = c["opts"]
    host = dict(window_left=opts.get("window_left", -1), sinks=opts.get("sinks"), softcap=opts.get("softcap", 0.0),
                alibi_slopes=opts.get("alibi_slopes"))
    dev = {k: (torch.from_numpy(v).cuda() if isinstance(v, np.ndarray) else v) for k, v in host.items()}
    dk = "float" if kind not in ("e5m2", "e4m3") else kind
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), dk, case.k_scale)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), dk, case.v_scale)
    ref, rl = oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                     case.block_tables, case.scale, **host)
    if case.total_q == 0:
        return
    d = gen.to_device(case)
    out, lse = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], max(1, case.max_seqlen_q),
                                 case.scale, k_scale=case.k_scale, v_scale=case.v_scale, num_kv_splits=c["splits"],
                                 return_lse=True, **dev)
    torch.cuda.synchronize()
    compare("prefill", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)

    small = [b for b, q in enumerate(c["q_lens"]) if q <= 16]
    if not small:
        return
    dec = gen.select_seqs(case, small)
    if dec.total_q == 0:
        return
    dd = gen.to_device(dec)
    out, lse = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"],
                                   max(1, dec.max_seqlen_q), case.scale, num_splits=c["parts"],
                                   part_keys=c["part_keys"], k_scale=case.k_scale, v_scale=case.v_scale,
                                   return_lse=True, **dev)
    torch.cuda.synchronize()
    cu = case.cu_seqlens_q
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in small]).astype(np.int64)
    compare("decode", kind, out.float().cpu().numpy(), ref[idx], lse.cpu().numpy(), rl[idx])
