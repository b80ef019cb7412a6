"""Parity of the HIP path with the fp64 oracle, through the C ABI (needs an MI355X).

Bars (max-abs error against the oracle): fp32 1e-5; fp16/bf16 2e-2; fp8 KV
(E5M2 or E4M3) 5e-2 against the oracle fed the same dequantized values.  Besides the
max-abs bar every comparison also reports max|err| / max|ref| and
rms(err) / rms(ref), with a self-imposed bar of 1e-2 on the rms ratio for
16-bit inputs (at long contexts the outputs are small and the absolute bar
alone would be loose).  Bitwise checks: a decode row alone vs in a batch; page
permutation, page size and KV layout leave outputs unchanged.
"""

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops
from parity_bars import RMS_BAR, TOL, compare, say  # noqa: F401

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.lib()  # raises if the library is missing
    yield
    torch.cuda.synchronize()


def oracle_pools(case):
    kind = case.kv_kind if case.kv_kind in ("e5m2", "e4m3") else "float"
    ks = case.k_scale if case.k_head_scales is None else case.k_scale * np.asarray(case.k_head_scales, np.float64)
    vs = case.v_scale if case.v_head_scales is None else case.v_scale * np.asarray(case.v_head_scales, np.float64)
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), kind, ks)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), kind, vs)
    return k, v


def run_oracle(case, rows=None, pools=None):
    k, v = pools if pools is not None else oracle_pools(case)
    return oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                  case.block_tables, case.scale, rows=rows)


def gpu_prefill(case, d=None, splits=1):
    d = d or gen.to_device(case)
    say(f"  prefill {case.name}: total_q={case.total_q} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} P={case.page_size} splits={splits}")
    out, lse = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], case.max_seqlen_q,
                                 case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                                 num_kv_splits=splits, return_lse=True, k_head_scales=d.get("k_head_scales"),
                                 v_head_scales=d.get("v_head_scales"))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def gpu_decode(case, d=None, splits=None, max_q=None):
    d = d or gen.to_device(case)
    splits = splits or case.num_splits
    max_q = max_q or max(1, case.max_seqlen_q)
    say(f"  decode {case.name}: rows={case.num_seqs} total_q={case.total_q} Hq={case.num_q_heads} "
        f"Hkv={case.num_kv_heads} D={case.head_dim} P={case.page_size} S={splits} max_q={max_q}")
    out, lse = ops.split_kv_decode(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], max_q, case.scale,
                                   num_splits=splits, k_scale=case.k_scale, v_scale=case.v_scale,
                                   return_lse=True, k_head_scales=d.get("k_head_scales"),
                                   v_head_scales=d.get("v_head_scales"))
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------------ tiny fp32

def test_tiny_fp32_prefill_all_rows():
    c = gen.tiny_fp32()
    ref, rl = run_oracle(c)
    for splits in (1, 2, 16):
        out, lse = gpu_prefill(c, splits=splits)
        compare(f"tiny prefill S={splits}", "f32", out, ref, lse, rl)


def test_tiny_fp32_decode_row_and_verify_row():
    c = gen.tiny_fp32()
    ref, rl = run_oracle(c)
    out, lse = gpu_decode(c, splits=16, max_q=16)   # the 16-token chunk as a verify row + the q=1 row
    compare("tiny decode (both rows)", "f32", out.cpu().numpy(), ref, lse.cpu().numpy(), rl)
    b = gen.select_seqs(c, [1])
    out1, lse1 = gpu_decode(b, splits=16, max_q=1)
    compare("tiny decode row", "f32", out1.cpu().numpy(), ref[16:], lse1.cpu().numpy(), rl[16:])


# ------------------------------------------------------------------ decode batch

@pytest.fixture(scope="module")
def decode_bf16():
    c = gen.decode_batch(kind="bf16")
    return c, gen.to_device(c), run_oracle(c)


def test_decode_batch_bf16_matches_oracle(decode_bf16):
    c, d, (ref, rl) = decode_bf16
    out, lse = gpu_decode(c, d, splits=16)
    compare("decode bf16 S=16", "bf16", out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)
    # the empty row (length 0) is exactly zero with lse -inf
    z = int(np.nonzero(c.seq_lens == 0)[0][0])
    assert not out[z].float().abs().sum().item() and torch.isinf(lse[z]).all()


def test_decode_row_alone_equals_row_in_batch_bitwise(decode_bf16):
    c, d, _ = decode_bf16
    out_b, lse_b = gpu_decode(c, d, splits=16, max_q=1)
    for b in [0, 1, 4, 5, 9, 13, 31]:
        one = gen.select_seqs(c, [b])
        out1, lse1 = gpu_decode(one, splits=16, max_q=1)
        assert torch.equal(out1.view(torch.int16), out_b[b:b + 1].view(torch.int16)), f"row {b}"
        assert torch.equal(lse1, lse_b[b:b + 1]), f"row {b} lse"
    # and in another batch composition
    sub = gen.select_seqs(c, [13, 5, 31])
    out3, _ = gpu_decode(sub, splits=16, max_q=1)
    for i, b in enumerate([13, 5, 31]):
        assert torch.equal(out3[i].view(torch.int16), out_b[b].view(torch.int16))


@pytest.mark.parametrize("splits", [1, 3, 8, 64])
def test_decode_other_split_counts(decode_bf16, splits):
    c, d, (ref, rl) = decode_bf16
    out, lse = gpu_decode(c, d, splits=splits)
    compare(f"decode bf16 S={splits}", "bf16", out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)


def test_decode_batch_fp32_matches_oracle():
    c = gen.decode_batch(kind="f32")
    ref, rl = run_oracle(c)
    out, lse = gpu_decode(c, splits=16)
    compare("decode f32 S=16", "f32", out.cpu().numpy(), ref, lse.cpu().numpy(), rl)


# ------------------------------------------------------------------ varlen prefill

@pytest.fixture(scope="module")
def varlen_bf16():
    c = gen.varlen_prefill(kind="bf16")
    return c, gen.to_device(c), run_oracle(c)


@pytest.mark.parametrize("splits", [1, 2, 4, 0])
def test_varlen_prefill_bf16(varlen_bf16, splits):
    c, d, (ref, rl) = varlen_bf16
    out, lse = gpu_prefill(c, d, splits=splits)
    compare(f"varlen bf16 S={splits}", "bf16", out, ref, lse, rl)


def test_varlen_prefill_fp16_and_fp32():
    for kind in ("f16", "f32"):
        c = gen.varlen_prefill(kind=kind)
        if kind == "f32":  # the exact-product path at a size the fp32 kernel finishes quickly
            c = gen.select_seqs(c, [0, 1, 2])
        ref, rl = run_oracle(c)
        out, lse = gpu_prefill(c)
        compare(f"varlen {kind}", kind, out, ref, lse, rl)


def test_prefill_splits_agree_with_unsplit(varlen_bf16):
    c, d, _ = varlen_bf16
    o1, _ = gpu_prefill(c, d, splits=1)
    o4, _ = gpu_prefill(c, d, splits=4)
    assert np.abs(o1 - o4).max() < 1e-2


# ------------------------------------------------------------------ invariants (bitwise)

def _repage(case, P2, seed):
    """Same dense K/V in another page size / permutation / layout (built on the CPU)."""
    rng = np.random.default_rng(seed)
    B = case.num_seqs
    need = [-(-int(L) // P2) for L in case.seq_lens]
    n_pages = sum(need) + 1
    perm = rng.permutation(n_pages)
    shape = (n_pages, P2) + tuple(case.k_pool.shape[2:])
    k2 = torch.full(shape, float("nan"), dtype=case.k_pool.dtype)
    v2 = torch.full(shape, float("nan"), dtype=case.v_pool.dtype)
    bt2 = np.full((B, max(need)), perm[-1], dtype=np.int32)
    off = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        j = np.arange(L)
        src_p = case.block_tables[b, j // case.page_size]
        src_s = j % case.page_size
        dst_p = perm[off + j // P2]
        k2[torch.from_numpy(dst_p), torch.from_numpy(j % P2)] = case.k_pool[torch.from_numpy(src_p), torch.from_numpy(src_s)]
        v2[torch.from_numpy(dst_p), torch.from_numpy(j % P2)] = case.v_pool[torch.from_numpy(src_p), torch.from_numpy(src_s)]
        bt2[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    from dataclasses import replace
    return replace(case, k_pool=k2, v_pool=v2, block_tables=bt2, page_size=P2)


def test_page_size_permutation_and_layout_leave_output_bitwise_unchanged():
    c = gen.make_case("inv", q_lens=[37, 1, 100], seq_lens=[300, 77, 700], num_q_heads=8, num_kv_heads=2,
                      head_dim=128, page_size=32, q_kind="f16", seed=31)
    base, base_lse = gpu_prefill(c, splits=1)
    dec, _ = gpu_decode(gen.select_seqs(c, [1]), splits=4, max_q=1)
    for P2 in (16, 48, 816):
        c2 = _repage(c, P2, seed=P2)
        o2, l2 = gpu_prefill(c2, splits=1)
        assert np.array_equal(o2, base) and np.array_equal(l2, base_lse), f"page {P2}"
        d2, _ = gpu_decode(gen.select_seqs(c2, [1]), splits=4, max_q=1)
        assert torch.equal(d2, dec)
    # the same logical cache stored [pages, Hkv, page_size, D]
    from dataclasses import replace
    h = replace(c, layout="HND", k_pool=c.k_pool.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3),
                v_pool=c.v_pool.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3))
    assert h.k_pool.stride(2) == c.page_size * c.head_dim
    oh, lh = gpu_prefill(h, splits=1)
    assert np.array_equal(oh, base) and np.array_equal(lh, base_lse)


# ------------------------------------------------------------------ shapes and edge cases

@pytest.mark.parametrize("D", [16, 48, 64, 80, 96, 112, 128, 144, 160, 192, 224, 240, 256])
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_head_dims(D, kind):
    c = gen.make_case(f"hd{D}", q_lens=[70, 3, 129], seq_lens=[70, 200, 1000], num_q_heads=6, num_kv_heads=2,
                      head_dim=D, page_size=16, q_kind=kind, seed=D)
    ref, rl = run_oracle(c)
    out, lse = gpu_prefill(c)
    compare(f"prefill {kind} D={D}", kind, out, ref, lse, rl)
    out, lse = gpu_decode(gen.select_seqs(c, [1]), splits=5, max_q=3)
    compare(f"decode {kind} D={D}", kind, out.float().cpu().numpy(), ref[70:73], lse.cpu().numpy(), rl[70:73])


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (12, 2), (24, 4), (16, 2)])
def test_gqa_ratios(Hq, Hkv):
    c = gen.make_case(f"gqa{Hq}-{Hkv}", q_lens=[50, 16], seq_lens=[333, 16], num_q_heads=Hq,
                      num_kv_heads=Hkv, head_dim=64, page_size=32, q_kind="f16", seed=Hq * 10 + Hkv)
    ref, rl = run_oracle(c)
    out, lse = gpu_prefill(c, splits=2)
    compare(f"prefill gqa {Hq}/{Hkv}", "f16", out, ref, lse, rl)
    one = gen.select_seqs(c, [1])
    out, lse = gpu_decode(one, splits=3, max_q=16)
    compare(f"decode gqa {Hq}/{Hkv}", "f16", out.float().cpu().numpy(), ref[50:], lse.cpu().numpy(), rl[50:])


def test_edge_cases_empty_and_ragged():
    # q_len > seq_len (leading rows see nothing), seq_len 0 with q > 0, q_len 0,
    # single key, lengths just off tile and page boundaries
    c = gen.make_case("edge", q_lens=[5, 3, 0, 1, 33, 1], seq_lens=[2, 0, 10, 1, 31, 33], num_q_heads=4,
                      num_kv_heads=2, head_dim=64, page_size=16, q_kind="bf16", seed=41)
    ref, rl = run_oracle(c)
    for s in (1, 3):
        out, lse = gpu_prefill(c, splits=s)
        compare(f"edge prefill S={s}", "bf16", out, ref, lse, rl)
        assert not out[:3].any() and np.isneginf(lse[:3]).all()
        assert not out[5:8].any()
    dec = gen.select_seqs(c, [1, 2, 3, 5])
    out, lse = gpu_decode(dec, splits=16, max_q=3)
    ref_d, rl_d = run_oracle(dec)
    compare("edge decode", "bf16", out.float().cpu().numpy(), ref_d, lse.cpu().numpy(), rl_d)


def test_peaked_scores():
    # planted high-score keys (scale x 8): outputs are O(1), so the absolute bar is tight
    c = gen.make_case("peaked", q_lens=[200], seq_lens=[3000], num_q_heads=8, num_kv_heads=2, head_dim=128,
                      page_size=64, q_kind="f16", seed=51)
    c.scale *= 8.0
    ref, rl = run_oracle(c)
    assert np.abs(ref).max() > 0.5
    out, lse = gpu_prefill(c, splits=1)
    compare("peaked prefill", "f16", out, ref, lse, rl)
    dec = gen.select_seqs(c, [0])
    dec.q = c.q[-4:].clone()
    dec.cu_seqlens_q = np.array([0, 4], dtype=np.int32)
    out, lse = gpu_decode(dec, splits=16, max_q=4)
    compare("peaked decode", "f16", out.float().cpu().numpy(), ref[-4:], lse.cpu().numpy(), rl[-4:])


# ------------------------------------------------- absolute parts: verify row == serial decode

def gpu_decode_fixed(case, d=None, part_keys=512, parts=8, max_q=None):
    d = d or gen.to_device(case)
    max_q = max_q or max(1, case.max_seqlen_q)
    say(f"  fixed-part decode {case.name}: rows={case.num_seqs} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} P={case.page_size} part_keys={part_keys} parts={parts} max_q={max_q}")
    out, lse = ops.split_kv_decode(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], max_q, case.scale,
                                   num_splits=parts, part_keys=part_keys, k_scale=case.k_scale,
                                   v_scale=case.v_scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("part_keys,parts", [(512, 20), (256, 4), (2048, 64)])
def test_fixed_part_decode_matches_oracle(decode_bf16, part_keys, parts):
    """Absolute parts, including a last part that runs on past parts * part_keys."""
    c, d, (ref, rl) = decode_bf16
    out, lse = gpu_decode_fixed(c, d, part_keys, parts, max_q=1)
    compare(f"fixed-part decode C={part_keys} S={parts}", "bf16", out.float().cpu().numpy(), ref,
            lse.cpu().numpy(), rl)


# (q dtype, KV dtype, D, Hq, Hkv, page, L, q of the verify row)
VERIFY_CASES = [
    ("f16", "f16", 256, 24, 4, 816, 5000, 5),
    ("f16", "e5m2", 256, 24, 4, 816, 5000, 5),
    ("bf16", "bf16", 128, 16, 16, 16, 3001, 5),
    ("f16", "f16", 64, 8, 2, 32, 1234, 16),
    ("f32", "f32", 64, 4, 1, 16, 700, 4),
    ("f16", "e5m2", 128, 8, 2, 48, 2000, 3),
]


@pytest.mark.parametrize("qk,kvk,D,Hq,Hkv,P,L,q", VERIFY_CASES)
def test_verify_row_equals_serial_decode_bitwise(qk, kvk, D, Hq, Hkv, P, L, q):
    """Token i of a verify row (q tokens at length L, in a batch with other rows)
    gives the same bits as a q=1 row at length L - q + 1 + i, with absolute parts
    and a different part count in the two calls."""
    case = gen.make_case(f"verify_{qk}_{kvk}_D{D}", q_lens=[q, 1, 7], seq_lens=[L, 900, 1500], num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=D, page_size=P, q_kind=qk, kv_kind=kvk, seed=41 + D + q)
    ser = gen.expand_row(case, 0)
    C = 256
    parts = -(-L // C)
    out_v, lse_v = gpu_decode_fixed(case, part_keys=C, parts=parts + 3, max_q=7 if q < 7 else q)
    out_s, lse_s = gpu_decode_fixed(ser, part_keys=C, parts=parts, max_q=1)
    assert torch.equal(bits(out_v[:q]), bits(out_s)), "verify row differs from the serial decode rows"
    assert torch.equal(lse_v[:q].view(torch.int32), lse_s.view(torch.int32)), "lse differs"
    ref, rl = run_oracle(case)
    compare(f"verify {qk}/{kvk} D{D}", kvk, out_v.float().cpu().numpy(), ref, lse_v.cpu().numpy(), rl)


def test_merge_states_matches_oracle_merge():
    rng = np.random.default_rng(61)
    N, H, S, D = 7, 3, 5, 128
    o = rng.standard_normal((N, H, S, D))
    l = rng.standard_normal((N, H, S)) * 3
    l[0, 0, :] = -np.inf          # all parts empty
    l[1, 1, 2] = -np.inf          # one empty part
    o[1, 1, 2] = np.nan           # its output must be ignored
    rec = np.concatenate([o, l[..., None], np.zeros((N, H, S, 1))], -1).astype(np.float32)
    ro, rlse = oracle.merge_partials(np.moveaxis(rec[..., :D].astype(np.float64), 2, 0),
                                     np.moveaxis(rec[..., D].astype(np.float64), 2, 0))
    ro[1, 1] = oracle.merge_partials(np.delete(rec[1, 1, :, :D], 2, 0).astype(np.float64),
                                     np.delete(rec[1, 1, :, D], 2, 0).astype(np.float64))[0]
    out, lse = ops.merge_states(torch.from_numpy(rec).cuda(), torch.float32, return_lse=True)
    torch.cuda.synchronize()
    compare("merge f32", "f32", out.cpu().numpy(), ro)
    assert np.isneginf(lse[0, 0].item()) and not out[0, 0].any()


def test_first_pass_only_then_merge_equals_the_merged_call():
    """out = NULL leaves the FP32 records in the workspace; merge_states over them gives the merged call's
    output and lse bit for bit (prefill with a key split, and decode)."""
    c = gen.make_case("p1", q_lens=[40, 3], seq_lens=[500, 1300], num_q_heads=8, num_kv_heads=2, head_dim=128,
                      page_size=48, q_kind="bf16", seed=63)
    d = gen.to_device(c)
    out, lse = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q, c.scale,
                                 num_kv_splits=3, return_lse=True)
    parts = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q, c.scale,
                              num_kv_splits=3, merge=False)
    assert parts.shape == (c.total_q, 8, 3, 130)
    o2, l2 = ops.merge_states(parts, torch.bfloat16, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), out.view(torch.int16)) and torch.equal(l2, lse)
    one = gen.select_seqs(c, [1])
    dd = gen.to_device(one)
    out, lse = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 3, one.scale,
                                   num_splits=7, return_lse=True)
    parts = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 3, one.scale,
                                num_splits=7, merge=False)
    o2, l2 = ops.merge_states(parts, torch.bfloat16, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), out.view(torch.int16)) and torch.equal(l2, lse)


# ------------------------------------------------------------------ fp8 KV

def test_fp8_prefill_and_decode_small():
    c = gen.make_case("fp8", q_lens=[100, 5], seq_lens=[900, 2000], num_q_heads=12, num_kv_heads=2,
                      head_dim=256, page_size=816, q_kind="f16", kv_kind="e5m2", seed=71,
                      k_scale=0.5, v_scale=2.0)
    ref, rl = run_oracle(c)
    out, lse = gpu_prefill(c, splits=2)
    compare("fp8 prefill", "e5m2", out, ref, lse, rl)
    one = gen.select_seqs(c, [1])
    out, lse = gpu_decode(one, splits=16, max_q=5)
    compare("fp8 decode", "e5m2", out.float().cpu().numpy(), ref[100:], lse.cpu().numpy(), rl[100:])


@pytest.mark.parametrize("D,P", [(64, 16), (128, 48), (160, 16), (256, 16), (256, 48), (256, 64)])
def test_fp8_head_dims_and_page_sizes(D, P):
    # fp8 KV: every head-dim bucket, page sizes that make tiles straddle pages
    # (16, 48) or not (64); chunk and verify rows, k/v scales != 1
    c = gen.make_case(f"fp8hd{D}p{P}", q_lens=[70, 5, 129], seq_lens=[70, 300, 1000], num_q_heads=6,
                      num_kv_heads=2, head_dim=D, page_size=P, q_kind="f16", kv_kind="e5m2", seed=D + P,
                      k_scale=0.75, v_scale=1.5)
    ref, rl = run_oracle(c)
    for splits in (1, 3):
        out, lse = gpu_prefill(c, splits=splits)
        compare(f"fp8 prefill D={D} P={P} S={splits}", "e5m2", out, ref, lse, rl)
    out, lse = gpu_decode(gen.select_seqs(c, [1]), splits=4, max_q=5)
    compare(f"fp8 decode D={D} P={P}", "e5m2", out.float().cpu().numpy(), ref[70:75], lse.cpu().numpy(), rl[70:75])


@pytest.mark.parametrize("fmt,D,P", [("e5m2", 256, 64), ("e4m3", 256, 816), ("e5m2", 128, 32), ("e4m3", 64, 16),
                                     ("e5m2", 160, 48)])
def test_bf16_queries_with_fp8_kv(fmt, D, P):
    """bf16 q and out over fp8 KV (widened to bf16 in the kernels): prefill with
    1 and 3 parts, the decode of the small-q rows, and a verify row bit for bit
    equal to its token-wise expansion, against the oracle fed the decoded values."""
    c = gen.make_case(f"bf16_{fmt}_D{D}_P{P}", q_lens=[70, 5, 1], seq_lens=[700, 1300, 333], num_q_heads=12,
                      num_kv_heads=2, head_dim=D, page_size=P, q_kind="bf16", kv_kind=fmt, seed=D + P + 5,
                      k_scale=0.75, v_scale=1.5)
    ref, rl = run_oracle(c)
    for splits in (1, 3):
        out, lse = gpu_prefill(c, splits=splits)
        compare(f"bf16/{fmt} prefill D={D} P={P} S={splits}", fmt, out, ref, lse, rl)
    dec = gen.select_seqs(c, [1, 2])
    out, lse = gpu_decode(dec, splits=8, max_q=5)
    compare(f"bf16/{fmt} decode D={D} P={P}", fmt, out.float().cpu().numpy(), ref[70:], lse.cpu().numpy(), rl[70:])
    ver = gen.select_seqs(c, [1])
    ser = gen.expand_row(ver, 0)
    out_v, lse_v = gpu_decode_fixed(ver, part_keys=256, parts=7, max_q=5)
    out_s, lse_s = gpu_decode_fixed(ser, part_keys=256, parts=6, max_q=1)  # both cover the 1300 keys
    assert torch.equal(bits(out_v), bits(out_s)) and torch.equal(bits(lse_v), bits(lse_s))


FP8_FINITE = {"e5m2": [b for b in range(256) if (b & 0x7F) < 0x7C], "e4m3": [b for b in range(256) if (b & 0x7F) != 0x7F]}


@pytest.mark.parametrize("qk", ["f16", "bf16"])
@pytest.mark.parametrize("fmt,D", [("e5m2", 256), ("e4m3", 256), ("e5m2", 128), ("e4m3", 64)])
def test_fp8_values_widen_exactly(qk, fmt, D):
    """A row that sees one key outputs that key's value exactly (its weight is 1,
    the sum 1, v_scale 1), so the first token of a chunk without prefix, and a
    q=1 row of length 1, give the decoded fp8 values of that key exactly:
    every finite code of the format goes through the kernels' widening to fp16
    or bf16, in the prefill and in the decode kernels."""
    c = gen.make_case(f"widen_{qk}_{fmt}_{D}", q_lens=[40, 1], seq_lens=[40, 1], num_q_heads=4, num_kv_heads=2,
                      head_dim=D, page_size=16, q_kind=qk, kv_kind=fmt, seed=D + 1)
    codes = np.array(FP8_FINITE[fmt], dtype=np.uint8)
    for b in range(2):  # key 0 of each sequence holds the codes, shifted per head
        page = int(c.block_tables[b, 0])
        for h in range(2):
            row = np.roll(np.resize(codes, D), 37 * h + 101 * b)
            c.v_pool[page, 0, h] = torch.from_numpy(row)
    dk = oracle.dequantize_pool(gen.to_numpy64(c.v_pool, fmt), fmt, 1.0)
    want = {b: torch.from_numpy(np.stack([dk[int(c.block_tables[b, 0]), 0, h // 2] for h in range(4)])).to(
        {"f16": torch.float16, "bf16": torch.bfloat16}[qk]) for b in range(2)}
    out, _ = gpu_prefill(gen.select_seqs(c, [0]), splits=1)
    # values compared exactly (not bits: the accumulation turns the code for -0 into +0)
    got = torch.from_numpy(out[0]).to(want[0].dtype)
    bad = torch.nonzero(got.float() != want[0].float())
    for h, j in bad[:8].tolist():
        say(f"  prefill head {h} d {j}: got {float(got[h, j])!r} want {float(want[0][h, j])!r}")
    assert len(bad) == 0, f"prefill widening: {len(bad)} values differ"
    od, _ = gpu_decode(gen.select_seqs(c, [1]), splits=4, max_q=1)
    got = od[0].cpu()
    bad = torch.nonzero(got.float() != want[1].float())
    for h, j in bad[:8].tolist():
        say(f"  decode head {h} d {j}: got {float(got[h, j])!r} want {float(want[1][h, j])!r}")
    assert len(bad) == 0, f"decode widening: {len(bad)} values differ"


# ------------------------------------------------------------------ full-size workloads (every row)


@pytest.fixture(scope="module")
def long_chunk_ref():
    """The 2048-token chunk after 150,000 cached tokens and the q=1 row over the
    same cache, with the oracle's output for every (token, head) row of both."""
    c = gen.long_chunk()
    pre, dec = gen.select_seqs(c, [0]), gen.select_seqs(c, [1])
    k, v = oracle_pools(pre)
    say(f"  oracle: all {pre.total_q} x {pre.num_q_heads} rows of the long chunk ...")
    ref, rl = run_oracle(pre, pools=(k, v))
    rd, rld = run_oracle(dec, pools=(k, v))
    return pre, dec, ref, rl, rd, rld


@pytest.mark.parametrize("splits", [1, 0])
def test_long_chunk_prefill_every_row(long_chunk_ref, splits):
    """Every output and lse of the long chunk, unsplit and at the automatic part
    count (4 on 256 compute units), against the oracle."""
    pre, dec, ref, rl, rd, rld = long_chunk_ref
    out, lse = gpu_prefill(pre, splits=splits)
    compare(f"long chunk S={splits} (all {ref.shape[0] * ref.shape[1]} rows)", "f16", out, ref, lse, rl)
    if splits == 1:  # the q=1 decode row over the same cache
        od, ld = gpu_decode(dec, splits=64, max_q=1)
        compare("long chunk decode row", "f16", od.float().cpu().numpy(), rd, ld.cpu().numpy(), rld)


@pytest.mark.parametrize("splits", [1, 2])
def test_prefill_page_ids_past_the_lds_table(splits):
    """A work group whose keys span more pages than its LDS page-id table holds
    (8192): 140,000 keys at page 16 are 8750 pages, read from the block table at
    every tile when unsplit; with 2 parts each group's 4375 pages come from the
    table.  Every row against the oracle."""
    case = gen.make_case("page ids past the table", q_lens=[32], seq_lens=[140_000], num_q_heads=4,
                         num_kv_heads=1, head_dim=256, page_size=16, q_kind="f16", seed=41)
    ref, rl = run_oracle(case)
    out, lse = gpu_prefill(case, splits=splits)
    compare(f"8750 pages, S={splits}", "f16", out, ref, lse, rl)


@pytest.mark.parametrize("kv_kind", ["f16", "e5m2"])
def test_mixed_step_every_row(kv_kind):
    """The mixed step: the verify row (q=5 at 240,000 keys, 64 parts) and every
    row of the 784-token chunk after 104,000 (automatic parts) against the oracle,
    then the same step as one pa_mixed_step call, bit for bit."""
    c = gen.mixed_step(kv_kind=kv_kind)
    k, v = oracle_pools(c)
    ver = gen.select_seqs(c, [0])
    od, ld = gpu_decode(ver, splits=64, max_q=5)
    rd, rld = run_oracle(ver, pools=(k, v))
    compare(f"mixed verify row {kv_kind}", kv_kind, od.float().cpu().numpy(), rd, ld.cpu().numpy(), rld)
    chunk = gen.select_seqs(c, [1])
    out, lse = gpu_prefill(chunk, splits=0)
    say(f"  oracle: all {chunk.total_q} x {chunk.num_q_heads} rows of the chunk ...")
    ref, rl = run_oracle(chunk, pools=(k, v))
    del k, v
    compare(f"mixed chunk {kv_kind} (all {ref.shape[0] * ref.shape[1]} rows)", kv_kind, out, ref, lse, rl)
    # the whole step as one pa_mixed_step call (the launch bench.py times as
    # mixed_step_fused): the same bits as the two calls above
    d = gen.to_device(c)
    sp = ops.auto_splits(chunk.total_q, 1, chunk.max_seqlen_q, chunk.num_q_heads, chunk.num_kv_heads,
                         chunk.head_dim, ops.PA_F16, ops.PA_FP8_E5M2 if kv_kind == "e5m2" else ops.PA_F16)
    say(f"  mixed step in one launch {kv_kind}: verify row (64 parts) + chunk ({sp} parts, its automatic count)")
    fo, fl = ops.mixed_step(d["q"], d["k"], d["v"], d["cu"], c.q_lens, d["seq_lens"], d["bt"], c.scale,
                            decode_splits=64, prefill_splits=sp, k_scale=c.k_scale, v_scale=c.v_scale,
                            return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(bits(fo[:5]), bits(od)) and torch.equal(bits(fl[:5]), bits(ld))
    assert np.array_equal(fo[5:].float().cpu().numpy().astype(np.float64), out)
    assert np.array_equal(fl[5:].cpu().numpy().astype(np.float64), lse)


# ------------------------------------------------------------------ fp8 E4M3 KV

@pytest.mark.parametrize("D,P", [(64, 16), (128, 48), (256, 16), (256, 64), (160, 32)])
def test_e4m3_prefill_and_decode(D, P):
    """E4M3 KV (fp16 q) against the oracle fed the same decoded values: prefill
    with 1 and 3 parts, and the decode of the two last rows."""
    c = gen.make_case(f"e4m3_D{D}_P{P}", q_lens=[70, 1, 5], seq_lens=[400, 333, 1200], num_q_heads=8,
                      num_kv_heads=2, head_dim=D, page_size=P, q_kind="f16", kv_kind="e4m3", seed=D + 3 * P,
                      k_scale=0.75, v_scale=1.5)
    ref, rl = run_oracle(c)
    for splits in (1, 3):
        out, lse = gpu_prefill(c, splits=splits)
        compare(f"e4m3 prefill D={D} P={P} S={splits}", "e4m3", out, ref, lse, rl)
    dec = gen.select_seqs(c, [1, 2])
    out, lse = gpu_decode(dec, splits=8, max_q=5)
    compare(f"e4m3 decode D={D} P={P}", "e4m3", out.float().cpu().numpy(), ref[70:], lse.cpu().numpy(), rl[70:])


def test_e4m3_verify_row_equals_serial_decode_bitwise():
    case = gen.make_case("verify_e4m3", q_lens=[5, 1], seq_lens=[3000, 900], num_q_heads=24, num_kv_heads=4,
                         head_dim=256, page_size=816, q_kind="f16", kv_kind="e4m3", seed=77)
    ser = gen.expand_row(case, 0)
    out_v, lse_v = gpu_decode_fixed(case, part_keys=512, parts=9, max_q=5)
    out_s, lse_s = gpu_decode_fixed(ser, part_keys=512, parts=6, max_q=1)
    assert torch.equal(bits(out_v[:5]), bits(out_s)) and torch.equal(lse_v[:5].view(torch.int32),
                                                                       lse_s.view(torch.int32))


# ------------------------------------------------------------------ graphs and prefill batch invariance

def test_calls_replay_under_a_hip_graph():
    """The grid depends on host scalars only, so a prefill (split, with merge),
    a decode, an absolute-part decode and a KV write can be captured in one HIP
    graph.  The graph is replayed several times with eager work and
    synchronisations in between; every replay must equal the eager results bit
    for bit (the pages keep the static grid for CUDA graphs: InferMatrixLab/
    vllm-rlt PR #128, "Purpose", Decode)."""
    c = gen.make_case("graph", q_lens=[300, 1, 5], seq_lens=[1000, 700, 2000], num_q_heads=16, num_kv_heads=4,
                      head_dim=128, page_size=32, q_kind="bf16", seed=91)
    d = gen.to_device(c)
    pre = gen.select_seqs(c, [0])
    dec = gen.select_seqs(c, [1, 2])
    dp, dd = gen.to_device(pre), gen.to_device(dec)
    dp["k"], dp["v"], dd["k"], dd["v"] = d["k"], d["v"], d["k"], d["v"]
    kn = torch.randn((5, 4, 128), device="cuda").to(torch.bfloat16)
    vn = torch.randn((5, 4, 128), device="cuda").to(torch.bfloat16)
    ws_p = torch.empty(ops.prefill_workspace_bytes(pre.total_q, 16, 128, 3) // 4, dtype=torch.float32, device="cuda")
    ws_d = torch.empty(ops.decode_workspace_bytes(dec.total_q, 16, 128, 8) // 4, dtype=torch.float32, device="cuda")
    ws_f = torch.empty_like(ws_d)
    outs = [torch.empty_like(dp["q"]), torch.empty_like(dd["q"]), torch.empty_like(dd["q"])]
    lses = [torch.empty(dp["q"].shape[:2], dtype=torch.float32, device="cuda") for _ in range(1)]
    kv_copy = [d["k"].clone(), d["v"].clone()]
    bt_w = torch.from_numpy(np.ascontiguousarray(c.block_tables[2:3])).cuda()
    cu_w = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    sl_w = torch.tensor([int(c.seq_lens[2])], dtype=torch.int32, device="cuda")

    def step(stream):
        ops.paged_prefill(dp["q"], dp["k"], dp["v"], dp["cu"], dp["seq_lens"], dp["bt"], pre.max_seqlen_q, c.scale,
                          num_kv_splits=3, out=outs[0], lse=lses[0], workspace=ws_p, stream=stream)
        ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 5, c.scale, num_splits=8,
                            out=outs[1], workspace=ws_d, stream=stream)
        ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 5, c.scale, num_splits=8,
                            part_keys=256, out=outs[2], workspace=ws_f, stream=stream)
        ops.write_kv(kn, vn, kv_copy[0], kv_copy[1], cu_w, sl_w, bt_w, 5, stream=stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs] + [lses[0].clone(), kv_copy[0].clone(), kv_copy[1].clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        lses[0].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(outs) + [lses[0], kv_copy[0], kv_copy[1]]
        for i, (a, b) in enumerate(zip(got, eager)):
            assert torch.equal(bits(a), bits(b)), f"replay {rep}, output {i}"
        _ = torch.ones(1 << 20, device="cuda").sum().item()  # eager work between replays
    ref, rl = run_oracle(c)
    compare("graph prefill", "bf16", outs[0].float().cpu().numpy(), ref[:300])
    compare("graph decode", "bf16", outs[1].float().cpu().numpy(), ref[300:])


def test_prefill_with_fixed_splits_is_batch_invariant_bitwise(varlen_bf16):
    """A sequence's prefill output does not depend on the other sequences of the
    call when num_kv_splits is fixed (the grid order only changes which work
    group runs when)."""
    c, d, _ = varlen_bf16
    for splits in (1, 3):
        out_b, lse_b = gpu_prefill(c, d, splits=splits)
        cu = c.cu_seqlens_q
        for b in (3, 1):
            one, lo = gpu_prefill(gen.select_seqs(c, [b]), splits=splits)
            assert np.array_equal(one.view(np.uint64), out_b[cu[b]:cu[b + 1]].view(np.uint64)), (splits, b)
            assert np.array_equal(lo.view(np.uint64), lse_b[cu[b]:cu[b + 1]].view(np.uint64)), (splits, b)
        sub = gen.select_seqs(c, [2, 0])
        two, _ = gpu_prefill(sub, splits=splits)
        assert np.array_equal(two[:cu[3] - cu[2]].view(np.uint64), out_b[cu[2]:cu[3]].view(np.uint64))


@pytest.mark.parametrize("fmt,D,P", [("e5m2", 256, 64), ("e4m3", 256, 816), ("e4m3", 128, 32), ("e5m2", 64, 16)])
def test_fp8_per_head_scales(fmt, D, P):
    """fp8 KV with a factor per kv head on top of the per-tensor one, prefill
    (1 and 2 parts) and decode, against the oracle fed decode(byte) * k_scale *
    k_head_scales[h]."""
    c = gen.make_case(f"headscale_{fmt}_D{D}", q_lens=[90, 1, 4], seq_lens=[700, 500, 1500], num_q_heads=12,
                      num_kv_heads=4, head_dim=D, page_size=P, q_kind="f16", kv_kind=fmt, seed=7 * D + P,
                      k_scale=0.5, v_scale=2.0)
    c.k_head_scales = np.array([1.0, 0.25, 3.0, 0.7], dtype=np.float32)
    c.v_head_scales = np.array([0.5, 1.5, 1.0, 4.0], dtype=np.float32)
    ref, rl = run_oracle(c)
    d = gen.to_device(c)
    for splits in (1, 2):
        out, lse = gpu_prefill(c, d, splits=splits)
        compare(f"{fmt} per-head prefill D={D} S={splits}", fmt, out, ref, lse, rl)
    dec = gen.select_seqs(c, [1, 2])
    out, lse = gpu_decode(dec, splits=8, max_q=4)
    compare(f"{fmt} per-head decode D={D}", fmt, out.float().cpu().numpy(), ref[90:], lse.cpu().numpy(), rl[90:])


# ------------------------------------------------------------------ sliding window and sinks

WINDOW_CASES = [
    # (q dtype, KV dtype, D, Hq, Hkv, page, window_left, with sinks)
    ("bf16", "bf16", 128, 8, 2, 32, 37, True),
    ("f16", "f16", 256, 12, 2, 64, 300, True),
    ("f16", "f16", 64, 4, 4, 16, 0, False),
    ("f16", "f16", 256, 6, 1, 48, 1000, False),
    ("f32", "f32", 64, 4, 1, 16, 50, True),
    ("f16", "e5m2", 256, 8, 2, 64, 129, True),
    ("f16", "e4m3", 128, 8, 2, 16, 64, True),
]


@pytest.mark.parametrize("qk,kvk,D,Hq,Hkv,P,window,with_sinks", WINDOW_CASES)
def test_window_and_sinks(qk, kvk, D, Hq, Hkv, P, window, with_sinks):
    """Left sliding window and attention sinks against the oracle: prefill with
    1 and 3 parts (sinks in the epilogue, then in the merge) and decode with
    proportional and absolute parts."""
    c = gen.make_case(f"win_{qk}_{kvk}_D{D}_W{window}", q_lens=[150, 1, 5, 40], seq_lens=[900, 700, 1300, 30],
                      num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, q_kind=qk, kv_kind=kvk,
                      seed=5 * D + window)
    rng = np.random.default_rng(window + D)
    sinks = rng.normal(size=Hq).astype(np.float32) * 2 if with_sinks else None
    k, v = oracle_pools(c)
    ref, rl = oracle.paged_attention(gen.to_numpy64(c.q), k, v, c.cu_seqlens_q, c.seq_lens, c.block_tables,
                                     c.scale, window_left=window, sinks=sinks)
    d = gen.to_device(c)
    sk = None if sinks is None else torch.from_numpy(sinks).cuda()
    kind = kvk if kvk in ("e5m2", "e4m3") else qk
    for splits in (1, 3):
        say(f"  window {window} sinks {with_sinks}: prefill S={splits}")
        out, lse = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q,
                                     c.scale, num_kv_splits=splits, return_lse=True, sinks=sk, window_left=window)
        torch.cuda.synchronize()
        compare(f"window prefill S={splits}", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)
    dec = gen.select_seqs(c, [1, 2])
    dd = gen.to_device(dec)
    for part_keys, parts in ((0, 8), (128, 12)):
        say(f"  window {window} sinks {with_sinks}: decode part_keys={part_keys}")
        out, lse = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 5, c.scale,
                                       num_splits=parts, part_keys=part_keys, return_lse=True, sinks=sk,
                                       window_left=window)
        torch.cuda.synchronize()
        compare(f"window decode C={part_keys}", kind, out.float().cpu().numpy(), ref[150:156], lse.cpu().numpy(),
                rl[150:156])


def test_window_verify_row_equals_serial_decode_bitwise():
    """With a window, absolute parts still give a verify row the bits of its
    token-wise expansion (each wave's tiles stay anchored at the part start)."""
    case = gen.make_case("verify_window", q_lens=[5, 1], seq_lens=[3000, 900], num_q_heads=24, num_kv_heads=4,
                         head_dim=256, page_size=816, q_kind="f16", seed=83)
    ser = gen.expand_row(case, 0)
    sk = torch.linspace(-1, 1, 24, device="cuda")
    d, ds = gen.to_device(case), gen.to_device(ser)
    outs = []
    for c, dd, parts, mq in ((case, d, 10, 5), (ser, ds, 6, 1)):
        out = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], mq, c.scale,
                                  num_splits=parts, part_keys=512, sinks=sk, window_left=777)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0][:5]), bits(outs[1]))


# ------------------------------------------------------------------ softcap and ALiBi

MOD_CASES = [
    # (q dtype, KV dtype, D, Hq, Hkv, page, softcap, with ALiBi, window_left, with sinks)
    ("f32", "f32", 64, 4, 2, 16, 5.0, True, -1, False),
    ("bf16", "bf16", 128, 8, 2, 32, 0.0, True, 37, True),
    ("f16", "f16", 64, 4, 4, 16, 2.0, False, -1, False),
    ("f16", "f16", 256, 12, 2, 64, 3.0, True, -1, True),
    ("bf16", "bf16", 256, 6, 1, 48, 0.0, True, 300, False),
    ("f16", "e5m2", 128, 8, 2, 16, 4.0, True, 64, False),
    ("f16", "e4m3", 256, 8, 2, 64, 1.5, True, -1, True),
    ("f16", "e5m2", 256, 8, 2, 64, 10.0, False, 129, False),
    # softcap alone at D <= 128 (the reciprocal form of the cap), with a window and sinks
    ("bf16", "bf16", 128, 8, 2, 32, 1.0, False, -1, False),
    ("f16", "f16", 128, 8, 4, 16, 0.5, False, 100, True),
]


alibi_slopes = gen.geometric_alibi_slopes


@pytest.mark.parametrize("qk,kvk,D,Hq,Hkv,P,softcap,with_alibi,window,with_sinks", MOD_CASES)
def test_softcap_and_alibi(qk, kvk, D, Hq, Hkv, P, softcap, with_alibi, window, with_sinks):
    """Softcap and ALiBi (with windows and sinks in some cases) against the
    oracle on every kernel: prefill with 1 and 3 parts, decode with
    proportional and absolute parts."""
    c = gen.make_case(f"mod_{qk}_{kvk}_D{D}", q_lens=[150, 1, 5, 40], seq_lens=[900, 700, 1300, 30],
                      num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P, q_kind=qk, kv_kind=kvk,
                      seed=7 * D + Hq)
    rng = np.random.default_rng(D + Hq)
    sinks = rng.normal(size=Hq).astype(np.float32) if with_sinks else None
    slopes = alibi_slopes(Hq) if with_alibi else None
    k, v = oracle_pools(c)
    ref, rl = oracle.paged_attention(gen.to_numpy64(c.q), k, v, c.cu_seqlens_q, c.seq_lens, c.block_tables,
                                     c.scale, window_left=window, sinks=sinks, softcap=softcap, alibi_slopes=slopes)
    d = gen.to_device(c)
    sk = None if sinks is None else torch.from_numpy(sinks).cuda()
    al = None if slopes is None else torch.from_numpy(slopes).cuda()
    kind = kvk if kvk in ("e5m2", "e4m3") else qk
    mods = dict(sinks=sk, window_left=window, softcap=softcap, alibi_slopes=al)
    for splits in (1, 3):
        say(f"  softcap {softcap} alibi {with_alibi} window {window}: prefill S={splits}")
        out, lse = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], c.max_seqlen_q,
                                     c.scale, num_kv_splits=splits, return_lse=True, **mods)
        torch.cuda.synchronize()
        compare(f"modified prefill S={splits}", kind, out.float().cpu().numpy(), ref, lse.cpu().numpy(), rl)
    dec = gen.select_seqs(c, [1, 2])
    dd = gen.to_device(dec)
    for part_keys, parts in ((0, 8), (128, 12)):
        say(f"  softcap {softcap} alibi {with_alibi} window {window}: decode part_keys={part_keys}")
        out, lse = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], 5, c.scale,
                                       num_splits=parts, part_keys=part_keys, return_lse=True, **mods)
        torch.cuda.synchronize()
        compare(f"modified decode C={part_keys}", kind, out.float().cpu().numpy(), ref[150:156], lse.cpu().numpy(),
                rl[150:156])


def test_modified_verify_row_equals_serial_decode_bitwise():
    """Softcap and ALiBi are per-score functions of the row's own key position:
    with absolute parts a verify row still has the bits of its token-wise
    expansion."""
    case = gen.make_case("verify_mod", q_lens=[5, 1], seq_lens=[3000, 900], num_q_heads=24, num_kv_heads=4,
                         head_dim=256, page_size=816, q_kind="f16", seed=84)
    ser = gen.expand_row(case, 0)
    al = torch.from_numpy(alibi_slopes(24)).cuda()
    d, ds = gen.to_device(case), gen.to_device(ser)
    outs = []
    for c, dd, parts, mq in ((case, d, 10, 5), (ser, ds, 6, 1)):
        out = ops.split_kv_decode(dd["q"], dd["k"], dd["v"], dd["cu"], dd["seq_lens"], dd["bt"], mq, c.scale,
                                  num_splits=parts, part_keys=512, softcap=20.0, alibi_slopes=al)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0][:5]), bits(outs[1]))
