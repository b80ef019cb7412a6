"""The C ABI's plain entry points and 64-bit cache offsets on the GPU (needs an MI355X).

* pa_paged_prefill, pa_split_kv_decode and pa_split_kv_decode_fixed are called
  directly through ctypes (the binding's torch helpers go through the _ex forms)
  and checked against the fp64 oracle (InferMatrixLab/vllm-rlt PR #128,
  "Purpose": the prefill call, the split-KV decode call and its merge).
* Pools larger than 4 GiB: the Turing kernel of 1CatAI/1Cat-vLLM PR #1279
  (commit 1, the selection rule) is only taken when every cache offset stays
  below 2^31.  Here page offsets are 64-bit, so the same case is run on a
  compact pool and on one of more than 4 GiB per K and V with the sequences'
  pages at the highest page ids; every kernel family must give the same bits.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops
from parity_bars import compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def kind_of(case):
    return case.kv_kind if case.kv_kind in ("e5m2", "e4m3") else case.q_kind


def oracle_ref(case):
    kind = case.kv_kind if case.kv_kind in ("e5m2", "e4m3") else "float"
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), kind, case.k_scale)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), kind, case.v_scale)
    return oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                  case.block_tables, case.scale)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ plain entry points


def plain_call(fn, case, d, count, part_keys=None, decode=False):
    """One of the three plain calls on device tensors; returns (out, lse)."""
    L = ops.lib()
    kv = ops.kv_cache(d["k"], d["v"], case.k_scale, case.v_scale)
    q = d["q"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    total_q, Hq, D = q.shape
    if decode:
        nb = ops.decode_workspace_bytes(total_q, Hq, D, count)
    else:
        nb = ops.prefill_workspace_bytes(total_q, Hq, D, count)
    ws = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=q.device)
    args = [_p(q), ops._dtype(q), _p(out), _p(lse), _p(d["cu"]), _p(d["seq_lens"]), _p(d["bt"]), case.num_seqs,
            d["bt"].shape[1], total_q, max(1, case.max_seqlen_q), Hq, ctypes.byref(kv), ctypes.c_float(case.scale)]
    if part_keys is not None:
        args += [part_keys, count]
    else:
        args += [count]
    st = fn(*args, _p(ws), ws.numel() * 4, _stream())
    assert st == 0, (st, L.pa_last_error())
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("qk,kvk,D", [("bf16", "bf16", 128), ("f16", "f16", 256), ("f32", "f32", 64),
                                      ("f16", "e5m2", 256)])
def test_plain_entry_points_match_oracle(qk, kvk, D):
    c = gen.make_case(f"plain_{qk}_{kvk}_{D}", q_lens=[90, 1, 5, 16], seq_lens=[1200, 777, 2050, 16],
                      num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=32, q_kind=qk, kv_kind=kvk, seed=D + 11)
    ref, rl = oracle_ref(c)
    kind = kind_of(c)
    d = gen.to_device(c)
    L = ops.lib()
    for splits in (1, 3):
        say(f"  pa_paged_prefill {qk}/{kvk} D={D} splits={splits}")
        out, lse = plain_call(L.pa_paged_prefill, c, d, splits)
        compare(f"pa_paged_prefill S={splits}", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)
    dec = gen.select_seqs(c, [1, 2, 3])
    dd = gen.to_device(dec)
    tok = slice(int(c.cu_seqlens_q[1]), int(c.cu_seqlens_q[4]))
    say(f"  pa_split_kv_decode {qk}/{kvk} D={D}")
    out, lse = plain_call(L.pa_split_kv_decode, dec, dd, 16, decode=True)
    compare("pa_split_kv_decode", kind, out.float().cpu().numpy(), ref[tok], lse.cpu().numpy(), rl[tok])
    say(f"  pa_split_kv_decode_fixed {qk}/{kvk} D={D}")
    out, lse = plain_call(L.pa_split_kv_decode_fixed, dec, dd, 5, part_keys=256, decode=True)
    compare("pa_split_kv_decode_fixed", kind, out.float().cpu().numpy(), ref[tok], lse.cpu().numpy(), rl[tok])


# ------------------------------------------------------------------ pools beyond 4 GiB

POOL_BYTES = (9 << 30) // 2  # 4.5 GiB per K and per V


def relocated(case, d):
    """The case's pages moved to the highest ids of pools of more than 4 GiB each
    (nothing else in the big pools is written: those pages are never read)."""
    n = case.num_pages
    page_bytes = d["k"][0].numel() * d["k"].element_size()
    total = max(n + 1, -(-POOL_BYTES // page_bytes) + n)
    rng = np.random.default_rng(n)
    big_id = (total - 1 - rng.permutation(n)).astype(np.int64)
    ids = torch.from_numpy(big_id).cuda()
    big = {}
    for name in ("k", "v"):
        src = d[name]
        t = torch.empty((total,) + tuple(src.shape[1:]), dtype=src.dtype, device="cuda")
        if src.element_size() == 1:  # fp8 bytes: copied as bytes
            t.view(torch.uint8).index_copy_(0, ids, src.view(torch.uint8))
        else:
            t.index_copy_(0, ids, src)
        big[name] = t
    bt = torch.from_numpy(big_id[case.block_tables].astype(np.int32)).cuda()
    say(f"  pools of {total} pages ({total * page_bytes / 2**30:.2f} GiB each), "
        f"highest byte offset used {int(big_id.max() + 1) * page_bytes / 2**30:.2f} GiB")
    return dict(d, k=big["k"], v=big["v"], bt=bt), ids


BIG_CASES = [  # (q dtype, KV dtype, head dim, kernels exercised)
    ("f16", "f16", 128, "DMA prefill (D <= 128), decode D 128, KV write"),
    ("bf16", "bf16", 256, "prefill D 256 (4 waves x 64 rows), decode D 256"),
    ("f16", "e5m2", 256, "fp8 prefill and decode D 256, fp8 KV write"),
    ("f16", "e4m3", 128, "register-staged fp8 prefill and decode (D <= 128)"),
    ("f32", "f32", 64, "fp32 VALU prefill and decode"),
]


@pytest.mark.parametrize("qk,kvk,D,what", BIG_CASES)
def test_pools_beyond_4gib_give_the_same_bits(qk, kvk, D, what):
    c = gen.make_case(f"big_{qk}_{kvk}_{D}", q_lens=[300, 1, 5, 16], seq_lens=[2100, 3000, 1777, 600],
                      num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=16, q_kind=qk, kv_kind=kvk, seed=3 * D + 1)
    say(f"  {qk}/{kvk} D={D}: {what}")
    d = gen.to_device(c)
    big, ids = relocated(c, d)
    ref, rl = oracle_ref(c)
    kind = kind_of(c)
    kw = dict(k_scale=c.k_scale, v_scale=c.v_scale, return_lse=True)

    def prefill(t, splits):
        o, l = ops.paged_prefill(t["q"], t["k"], t["v"], t["cu"], t["seq_lens"], t["bt"], c.max_seqlen_q, c.scale,
                                 num_kv_splits=splits, **kw)
        torch.cuda.synchronize()
        return o, l
    for splits in (1, 3):
        o_s, l_s = prefill(d, splits)
        o_b, l_b = prefill(big, splits)
        assert torch.equal(bits(o_s), bits(o_b)) and torch.equal(bits(l_s), bits(l_b)), f"prefill S={splits}"
        compare(f"prefill S={splits} (compact pool)", kind, o_s.float().cpu().numpy(), ref, l_s.cpu().numpy(), rl)

    dec = gen.select_seqs(c, [1, 2, 3])
    tok = slice(int(c.cu_seqlens_q[1]), int(c.cu_seqlens_q[4]))
    for t, tag in ((d, "compact"), (big, "big")):
        sub = dict(t, q=t["q"][tok], cu=torch.from_numpy(dec.cu_seqlens_q.astype(np.int32)).cuda(),
                   seq_lens=t["seq_lens"][1:], bt=t["bt"][1:].contiguous())
        o1, l1 = ops.split_kv_decode(sub["q"], sub["k"], sub["v"], sub["cu"], sub["seq_lens"], sub["bt"], 16,
                                     c.scale, num_splits=8, **kw)
        o2, l2 = ops.split_kv_decode(sub["q"], sub["k"], sub["v"], sub["cu"], sub["seq_lens"], sub["bt"], 16,
                                     c.scale, num_splits=6, part_keys=512, **kw)
        torch.cuda.synchronize()
        if tag == "compact":
            first = (o1, l1, o2, l2)
            compare("decode (compact pool)", kind, o1.float().cpu().numpy(), ref[tok], l1.cpu().numpy(), rl[tok])
            compare("fixed-part decode (compact pool)", kind, o2.float().cpu().numpy(), ref[tok], l2.cpu().numpy(),
                    rl[tok])
        else:
            for a, b in zip(first, (o1, l1, o2, l2)):
                assert torch.equal(bits(a), bits(b)), "decode differs on the big pool"

    if qk == "f32" or kvk == "e4m3":
        return
    # KV write of the chunk's 300 new rows at the top of the big pool: the same bytes as on the compact pool
    g = torch.Generator(device="cuda").manual_seed(D)
    src = torch.float16 if qk == "f16" else torch.bfloat16
    kn = torch.randn((c.total_q, c.num_kv_heads, D), generator=g, device="cuda").to(src)
    vn = torch.randn((c.total_q, c.num_kv_heads, D), generator=g, device="cuda").to(src)
    for t in (d, big):
        ops.write_kv(kn, vn, t["k"], t["v"], t["cu"], t["seq_lens"], t["bt"], c.max_seqlen_q,
                     k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    for name in ("k", "v"):
        a = d[name].view(torch.uint8) if d[name].element_size() == 1 else bits(d[name])
        b = big[name][ids]
        b = b.view(torch.uint8) if b.element_size() == 1 else bits(b)
        assert torch.equal(a, b), f"KV write of {name} differs on the big pool"
