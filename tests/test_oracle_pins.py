"""Pins of the fp64 oracle to things other than itself (CPU only).

* brute force: a pure-Python triple loop (oracle/brute.py) on tiny inputs;
* closed forms: zero query / zero scale -> uniform weights, constant V,
  a single visible key, two visible keys (logistic weights), empty rows;
* a library routine: torch float64 scaled_dot_product_attention with a causal
  mask equals a whole-sequence prefill on an identity block table, and a chunk
  equals the last rows of the whole-sequence attention (bottom-right alignment);
* invariants: page permutation, page size, GQA == MHA with repeated kv heads,
  verify row (q = K+1) == K+1 decode rows, split + merge == unsplit;
* the E5M2 decoder against torch's float8_e5m2 for all 256 bytes;
* planted mistakes in the oracle are caught by at least one of the pins above.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from paged_attention_prefill_amd import inputs as gen


def assert_same(a, b):
    """Equal up to the rounding of a different BLAS blocking (row counts differ)."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert (np.isfinite(a) == np.isfinite(b)).all()
    fin = np.isfinite(a)
    np.testing.assert_allclose(a[fin], b[fin], rtol=0, atol=1e-14)
    assert (a[~fin] == b[~fin]).all()


def run_oracle(case, rows=None):
    kvk = "e5m2" if case.kv_kind == "e5m2" else "float"
    k = oracle.dequantize_pool(gen.to_numpy64(case.k_pool, case.kv_kind), kvk, case.k_scale)
    v = oracle.dequantize_pool(gen.to_numpy64(case.v_pool, case.kv_kind), kvk, case.v_scale)
    return oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q,
                                  case.seq_lens, case.block_tables, case.scale, rows=rows)


def brute(case):
    q = gen.to_numpy64(case.q).tolist()
    k = gen.to_numpy64(case.k_pool).tolist()
    v = gen.to_numpy64(case.v_pool).tolist()
    o, l = oracle.brute_paged_attention(q, k, v, case.cu_seqlens_q.tolist(), case.seq_lens.tolist(),
                                        case.block_tables.tolist(), case.scale)
    return np.array(o), np.array(l)


def small_gqa_case(seed=11, **kw):
    args = dict(q_lens=[5, 1, 3, 4], seq_lens=[9, 7, 2, 20], num_q_heads=6, num_kv_heads=2,
                head_dim=16, page_size=4, q_kind="f32", seed=seed)
    args.update(kw)
    return gen.make_case("small_gqa", **args)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("maker", [lambda: gen.tiny_fp32(), lambda: small_gqa_case()])
def test_numpy_oracle_matches_brute_force(maker):
    case = maker()
    o, l = run_oracle(case)
    bo, bl = brute(case)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert (fin == np.isfinite(l)).all()
    np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-12)


def test_sampled_rows_equal_full_output():
    case = small_gqa_case(seed=12)
    o, l = run_oracle(case)
    rows = np.array([[0, 5], [4, 0], [5, 3], [12, 1], [8, 2]])
    so, sl = run_oracle(case, rows=rows)
    # same arithmetic, possibly another BLAS blocking: equal up to rounding
    np.testing.assert_allclose(so, o[rows[:, 0], rows[:, 1]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sl, l[rows[:, 0], rows[:, 1]], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed forms

def _dense_v(case, b, kvh):
    v = gen.to_numpy64(case.v_pool)
    return oracle.gather_dense_kv(v, case.block_tables[b], int(case.seq_lens[b]), kvh)


def test_zero_query_gives_uniform_mean():
    case = small_gqa_case(seed=13)
    case.q.zero_()
    o, l = run_oracle(case)
    g = case.num_q_heads // case.num_kv_heads
    for b in range(case.num_seqs):
        t0, t1 = case.cu_seqlens_q[b], case.cu_seqlens_q[b + 1]
        Q, L = t1 - t0, int(case.seq_lens[b])
        for i in range(Q):
            n = L - Q + i + 1
            for h in range(case.num_q_heads):
                if n <= 0:
                    assert not o[t0 + i, h].any() and l[t0 + i, h] == -np.inf
                    continue
                V = _dense_v(case, b, h // g)
                np.testing.assert_allclose(o[t0 + i, h], V[:n].mean(0), atol=1e-14)
                assert abs(l[t0 + i, h] - math.log(n)) < 1e-14


def test_zero_scale_gives_uniform_mean():
    a = small_gqa_case(seed=14)
    a.scale = 0.0
    o, l = run_oracle(a)
    b2 = small_gqa_case(seed=14)
    b2.q.zero_()
    o2, l2 = run_oracle(b2)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(l[np.isfinite(l)], l2[np.isfinite(l2)], atol=1e-14)


def test_constant_values_pass_through():
    case = small_gqa_case(seed=15)
    c = torch.linspace(-3, 3, case.head_dim)
    case.v_pool[:] = c  # every slot of every page, poison included
    o, _ = run_oracle(case)
    vis = np.abs(o).sum(-1) > 0
    np.testing.assert_allclose(o[vis], np.broadcast_to(c.double().numpy(), o[vis].shape), atol=1e-13)


def test_single_and_two_visible_keys():
    # prefix 0: token 0 sees key 0 only, token 1 sees keys 0 and 1
    case = gen.make_case("first_tokens", q_lens=[3], seq_lens=[3], num_q_heads=2, num_kv_heads=1,
                         head_dim=8, page_size=16, q_kind="f32", seed=16)
    o, l = run_oracle(case)
    q = gen.to_numpy64(case.q)
    K = oracle.gather_dense_kv(gen.to_numpy64(case.k_pool), case.block_tables[0], 3, 0)
    V = _dense_v(case, 0, 0)
    for h in range(2):
        s0 = case.scale * q[0, h] @ K[0]
        np.testing.assert_allclose(o[0, h], V[0], atol=0)
        assert abs(l[0, h] - s0) < 1e-14
        s = case.scale * np.array([q[1, h] @ K[0], q[1, h] @ K[1]])
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        np.testing.assert_allclose(o[1, h], w0 * V[0] + (1 - w0) * V[1], atol=1e-14)
        assert abs(l[1, h] - (max(s) + math.log(math.exp(s[0] - max(s)) + math.exp(s[1] - max(s))))) < 1e-14


def test_rows_without_visible_keys_are_zero():
    # q_len 6 > seq_len 3: tokens 0..2 see no key (n_i = 3 - 6 + i + 1 <= 0)
    case = gen.make_case("empty_rows", q_lens=[6, 2], seq_lens=[3, 0], num_q_heads=2,
                         num_kv_heads=2, head_dim=8, page_size=16, q_kind="f32", seed=17)
    o, l = run_oracle(case)
    assert not o[:3].any() and np.all(l[:3] == -np.inf)
    assert not o[6:].any() and np.all(l[6:] == -np.inf)
    assert np.isfinite(l[3:6]).all()


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_matches_torch_causal_sdpa(Hq, Hkv):
    L, D = 37, 24
    case = gen.make_case("sdpa", q_lens=[L], seq_lens=[L], num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, page_size=L, q_kind="f32", seed=18, shuffle=False)
    o, l = run_oracle(case)
    g = Hq // Hkv
    qt = case.q.double().permute(1, 0, 2)                       # [Hq, L, D]
    kt = case.k_pool[0].double().permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    vt = case.v_pool[0].double().permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=case.scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-13)
    # logsumexp from the same library: logsumexp of the masked scores
    sc = (qt @ kt.transpose(1, 2)) * case.scale
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    ref_lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
    np.testing.assert_allclose(l, ref_lse.T.numpy(), atol=1e-13)


def test_chunk_equals_last_rows_of_full_causal_attention():
    L, Q = 50, 13
    full = gen.make_case("full", q_lens=[L], seq_lens=[L], num_q_heads=3, num_kv_heads=1,
                         head_dim=16, page_size=16, q_kind="f32", seed=19)
    chunk = gen.select_seqs(full, [0])
    chunk.q = full.q[L - Q:].clone()
    chunk.cu_seqlens_q = np.array([0, Q], dtype=np.int32)
    o_full, l_full = run_oracle(full)
    o_chunk, l_chunk = run_oracle(chunk)
    assert_same(o_chunk, o_full[L - Q:])
    assert_same(l_chunk, l_full[L - Q:])


# ---------------------------------------------------------------- invariants

def _repage(case, new_page_size, seed):
    """Same dense K/V, laid out again with another page size and a fresh permutation."""
    P2 = new_page_size
    rng = np.random.default_rng(seed)
    k = case.k_pool
    v = case.v_pool
    B = case.num_seqs
    need = [-(-int(L) // P2) for L in case.seq_lens]
    n_pages = sum(need) + 1
    perm = rng.permutation(n_pages)
    shape = (n_pages, P2) + tuple(k.shape[2:])
    k2 = torch.full(shape, float("nan"), dtype=k.dtype)
    v2 = torch.full(shape, float("nan"), dtype=v.dtype)
    bt2 = np.full((B, max(need)), perm[-1], dtype=np.int32)
    off = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        for j in range(L):
            src_p, src_s = case.block_tables[b, j // case.page_size], j % case.page_size
            dst_p = perm[off + j // P2]
            k2[dst_p, j % P2] = k[src_p, src_s]
            v2[dst_p, j % P2] = v[src_p, src_s]
        bt2[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    from dataclasses import replace
    return replace(case, k_pool=k2, v_pool=v2, block_tables=bt2, page_size=P2)


@pytest.mark.parametrize("P2", [4, 16, 48])
def test_page_size_and_permutation_leave_output_unchanged(P2):
    case = small_gqa_case(seed=20, page_size=16)
    o, l = run_oracle(case)
    o2, l2 = run_oracle(_repage(case, P2, seed=P2))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_gqa_equals_mha_with_repeated_kv_heads():
    case = small_gqa_case(seed=21)
    g = case.num_q_heads // case.num_kv_heads
    from dataclasses import replace
    mha = replace(case, k_pool=case.k_pool.repeat_interleave(g, 2),
                  v_pool=case.v_pool.repeat_interleave(g, 2), num_kv_heads=case.num_q_heads)
    o, l = run_oracle(case)
    o2, l2 = run_oracle(mha)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_verify_row_equals_token_wise_decode_rows():
    K1 = 5  # MTP verify row q = K + 1 with K = 4
    L = 70
    ver = gen.make_case("verify", q_lens=[K1], seq_lens=[L], num_q_heads=4, num_kv_heads=2,
                        head_dim=16, page_size=16, q_kind="f32", seed=22)
    o, l = run_oracle(ver)
    from dataclasses import replace
    dec = replace(ver, cu_seqlens_q=np.arange(K1 + 1, dtype=np.int32),
                  seq_lens=np.array([L - K1 + 1 + i for i in range(K1)], dtype=np.int32),
                  block_tables=np.repeat(ver.block_tables, K1, axis=0))
    o2, l2 = run_oracle(dec)
    assert_same(o, o2)
    assert_same(l, l2)


@pytest.mark.parametrize("S", [1, 2, 3, 16, 40])
def test_split_merge_equals_unsplit(S):
    case = gen.make_case("split", q_lens=[4], seq_lens=[300], num_q_heads=2, num_kv_heads=1,
                         head_dim=16, page_size=16, q_kind="f32", seed=23)
    q = gen.to_numpy64(case.q)[:, 0, :]
    K = oracle.gather_dense_kv(gen.to_numpy64(case.k_pool), case.block_tables[0], 300, 0)
    V = oracle.gather_dense_kv(gen.to_numpy64(case.v_pool), case.block_tables[0], 300, 0)
    counts = oracle.visible_key_count(300, 4, np.arange(4))
    o, l = oracle.attention_rows(q, K, V, counts, case.scale)
    os_, ls_ = oracle.split_partials(q, K, V, counts, case.scale, S)
    om, lm = oracle.merge_partials(os_, ls_)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)
    # an empty partial merges as the identity
    oe = np.concatenate([os_, np.zeros((1,) + os_.shape[1:])])
    le = np.concatenate([ls_, np.full((1,) + ls_.shape[1:], -np.inf)])
    om2, lm2 = oracle.merge_partials(oe, le)
    np.testing.assert_array_equal(om2, om)
    np.testing.assert_array_equal(lm2, lm)


def test_split_ranges_partition_properties():
    for L in [0, 1, 31, 32, 33, 511, 512, 513, 4097, 10000]:
        for S in [1, 2, 16]:
            r = oracle.split_ranges(L, S)
            assert len(r) == S
            assert r[0][0] == 0 and r[-1][1] == L
            for (a, b), (c, d) in zip(r, r[1:]):
                assert b == c and a <= b
            for a, b in r:
                assert a % 32 == 0 or a == L
            sizes = [b - a for a, b in r]
            # equal parts of whole tiles, the last one possibly shorter or empty
            full = [s for s in sizes if s > 0][:-1]
            assert len(set(full)) <= 1
    assert oracle.split_ranges(0, 4) == [(0, 0)] * 4
    assert oracle.split_ranges(100, 16)[:4] == [(0, 32), (32, 64), (64, 96), (96, 100)]


def test_absolute_split_ranges_partition_properties():
    """Absolute parts: [s C, (s + 1) C) clipped to the row, the last part running on
    to L; the boundaries of a shorter row are those of a longer row cut at its end."""
    for C in [32, 96, 512]:
        for S in [1, 3, 8]:
            longest = oracle.split_ranges(10 ** 6, S, part_keys=C)
            for L in [0, 1, 31, 32, 33, 95, 96, 97, 511, 512, 513, 1500, 4097]:
                r = oracle.split_ranges(L, S, part_keys=C)
                assert len(r) == S and r[0][0] == 0 and r[-1][1] == L
                for (a, b), (c, d) in zip(r, r[1:]):
                    assert b == c and a <= b
                for s, (a, b) in enumerate(r[:-1]):
                    assert (a, b) == (min(s * C, L), min((s + 1) * C, L))
                    assert (a, b) == (min(longest[s][0], L), min(longest[s][1], L))
                assert r[-1][0] == min((S - 1) * C, L)
    assert oracle.split_ranges(100, 4, part_keys=32) == [(0, 32), (32, 64), (64, 96), (96, 100)]
    assert oracle.split_ranges(300, 2, part_keys=64) == [(0, 64), (64, 300)]
    assert oracle.split_ranges(50, 3, part_keys=64) == [(0, 50), (50, 50), (50, 50)]


@pytest.mark.parametrize("C,S", [(32, 10), (64, 2), (96, 4), (512, 1)])
def test_absolute_split_merge_equals_unsplit(C, S):
    case = gen.make_case("split_abs", q_lens=[5], seq_lens=[300], num_q_heads=2, num_kv_heads=1,
                         head_dim=16, page_size=16, q_kind="f32", seed=29)
    q = gen.to_numpy64(case.q)[:, 0, :]
    K = oracle.gather_dense_kv(gen.to_numpy64(case.k_pool), case.block_tables[0], 300, 0)
    V = oracle.gather_dense_kv(gen.to_numpy64(case.v_pool), case.block_tables[0], 300, 0)
    counts = oracle.visible_key_count(300, 5, np.arange(5))
    o, l = oracle.attention_rows(q, K, V, counts, case.scale)
    os_, ls_ = oracle.split_partials(q, K, V, counts, case.scale, S, part_keys=C)
    om, lm = oracle.merge_partials(os_, ls_)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)


def test_token_wise_expansion_of_a_verify_row():
    """A verify row of q tokens at length L equals q decode rows at lengths
    L - q + 1 .. L over the same pages (the token-wise expansion), in the oracle."""
    case = gen.make_case("verify", q_lens=[5, 3], seq_lens=[200, 90], num_q_heads=4, num_kv_heads=2,
                         head_dim=32, page_size=16, q_kind="f32", seed=31)
    k = gen.to_numpy64(case.k_pool)
    v = gen.to_numpy64(case.v_pool)
    o, l = oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                  case.block_tables, case.scale)
    for b in range(2):
        ex = gen.expand_row(case, b)
        assert list(ex.seq_lens) == [int(case.seq_lens[b]) - int(case.q_lens[b]) + 1 + i
                                     for i in range(int(case.q_lens[b]))]
        oe, le = oracle.paged_attention(gen.to_numpy64(ex.q), k, v, ex.cu_seqlens_q, ex.seq_lens,
                                        ex.block_tables, ex.scale)
        t0, t1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        np.testing.assert_allclose(oe, o[t0:t1], atol=1e-13)
        np.testing.assert_allclose(le, l[t0:t1], atol=1e-13)


# ---------------------------------------------------------------- fp8

def test_e5m2_decoder_matches_torch_on_all_bytes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e5m2_to_float64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert (np.isnan(mine) == np.isnan(ref)).all()
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])
    # a few values fixed by the bit layout alone
    assert oracle.e5m2_to_float64(np.array([0x3C]))[0] == 1.0
    assert oracle.e5m2_to_float64(np.array([0x01]))[0] == 2.0 ** -16
    assert oracle.e5m2_to_float64(np.array([0x7B]))[0] == 57344.0
    assert oracle.e5m2_to_float64(np.array([0xC0]))[0] == -2.0
    assert np.isinf(oracle.e5m2_to_float64(np.array([0x7C]))[0])


def test_e5m2_pool_dequantizes_with_scale():
    case = gen.make_case("fp8", q_lens=[3], seq_lens=[20], num_q_heads=2, num_kv_heads=1,
                         head_dim=16, page_size=16, q_kind="f16", kv_kind="e5m2", seed=24,
                         k_scale=0.5, v_scale=2.0)
    raw = case.k_pool.numpy()
    k = oracle.dequantize_pool(raw, "e5m2", 0.5)
    ref = torch.from_numpy(raw.copy()).view(torch.float8_e5m2).to(torch.float64).numpy() * 0.5
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(k[fin], ref[fin])


# ---------------------------------------------------------------- planted mistakes

def _pin_suite_passes():
    """Runs the pins that planted mistakes must trip; True if all hold."""
    try:
        test_numpy_oracle_matches_brute_force(lambda: small_gqa_case())
        test_matches_torch_causal_sdpa(6, 2)
        test_chunk_equals_last_rows_of_full_causal_attention()
        test_zero_query_gives_uniform_mean()
        test_rows_without_visible_keys_are_zero()
        for S in (2, 3):
            test_split_merge_equals_unsplit(S)
    except AssertionError:
        return False
    return True


MUTATIONS = {
    "top_left_causal": ("visible_key_count", lambda L, Q, i: i + 1),
    "off_by_one_visible": ("visible_key_count", lambda L, Q, i: L - Q + i),
    "wrong_kv_head": ("gather_dense_kv",
                      lambda pool, bt, L, h, _f=oa.gather_dense_kv: _f(pool, bt, L, (h + 1) % pool.shape[2])),
    "page_slot_swapped": ("gather_dense_kv",
                          lambda pool, bt, L, h: np.asarray(pool[np.asarray(bt)[np.arange(L) % pool.shape[1] % len(bt)],
                                                                 np.arange(L) // pool.shape[1] % pool.shape[1], h, :], np.float64)),
    "scale_dropped": ("attention_rows",
                      lambda q, K, V, c, scale, key_lo=0, key_hi=None, block=128, starts=None, _f=oa.attention_rows,
                      **kw: _f(q, K, V, c, 1.0, key_lo, key_hi, block, starts, **kw)),
    "lse_base2": ("attention_rows",
                  lambda q, K, V, c, scale, key_lo=0, key_hi=None, block=128, starts=None, _f=oa.attention_rows,
                  **kw: (lambda r: (r[0], r[1] / math.log(2)))(_f(q, K, V, c, scale, key_lo, key_hi, block, starts,
                                                                   **kw))),
    "merge_unweighted": ("merge_partials",
                         lambda o, l: (np.asarray(o).mean(0), np.asarray(l).max(0))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    assert _pin_suite_passes()
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    assert not _pin_suite_passes(), f"mutation {name} survived every pin"


# ---------------------------------------------------------------- window and sinks

def _dense(case):
    k = gen.to_numpy64(case.k_pool)
    v = gen.to_numpy64(case.v_pool)
    return k, v


@pytest.mark.parametrize("window,sinks", [(0, None), (3, None), (7, [0.5, -1.0, 2.0, 0.0, 1.0, -3.0]),
                                          (-1, [0.5, -1.0, 2.0, 0.0, 1.0, -3.0]), (100, None)])
def test_window_and_sinks_match_brute_force(window, sinks):
    case = small_gqa_case(seed=13)
    k, v = _dense(case)
    o, l = oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                  case.block_tables, case.scale, window_left=window, sinks=sinks)
    bo, bl = oracle.brute_paged_attention(gen.to_numpy64(case.q).tolist(), k.tolist(), v.tolist(),
                                          case.cu_seqlens_q.tolist(), case.seq_lens.tolist(),
                                          case.block_tables.tolist(), case.scale, window_left=window, sinks=sinks)
    bo, bl = np.array(bo), np.array(bl)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert (fin == np.isfinite(l)).all()
    np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-12)


def test_window_special_cases():
    case = small_gqa_case(seed=14)
    k, v = _dense(case)
    q = gen.to_numpy64(case.q)
    args = (case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale)
    full, fl = oracle.paged_attention(q, k, v, *args)
    wide, wl = oracle.paged_attention(q, k, v, *args, window_left=int(case.seq_lens.max()))
    np.testing.assert_array_equal(wide, full)
    np.testing.assert_array_equal(wl, fl)
    # window 0: each token sees only its own key: o = v at that key, lse = its score
    o0, l0 = oracle.paged_attention(q, k, v, *args, window_left=0)
    g = case.num_q_heads // case.num_kv_heads
    for b in range(case.num_seqs):
        L, Q = int(case.seq_lens[b]), int(case.q_lens[b])
        for i in range(Q):
            t, p = int(case.cu_seqlens_q[b]) + i, L - Q + i
            for h in range(case.num_q_heads):
                if p < 0:
                    assert not o0[t, h].any() and l0[t, h] == -np.inf
                    continue
                page, slot = int(case.block_tables[b][p // case.page_size]), p % case.page_size
                np.testing.assert_allclose(o0[t, h], v[page, slot, h // g], atol=1e-15)
                np.testing.assert_allclose(l0[t, h], case.scale * q[t, h] @ k[page, slot, h // g], atol=1e-13)


def test_sink_closed_forms():
    case = small_gqa_case(seed=15)
    k, v = _dense(case)
    q = gen.to_numpy64(case.q)
    args = (case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale)
    base, bl = oracle.paged_attention(q, k, v, *args)
    none, nl = oracle.paged_attention(q, k, v, *args, sinks=[-np.inf] * case.num_q_heads)
    np.testing.assert_array_equal(none, base)
    np.testing.assert_array_equal(nl, bl)
    # zero queries: n visible keys of weight 1 and a sink of weight e^s: o = sum v / (n + e^s)
    z, zl = oracle.paged_attention(np.zeros_like(q), k, v, *args, sinks=[0.7] * case.num_q_heads)
    g = case.num_q_heads // case.num_kv_heads
    for b in range(case.num_seqs):
        L, Q = int(case.seq_lens[b]), int(case.q_lens[b])
        for i in range(Q):
            t, n = int(case.cu_seqlens_q[b]) + i, L - Q + i + 1
            for h in range(case.num_q_heads):
                V = oracle.gather_dense_kv(v, case.block_tables[b], L, h // g)[:max(n, 0)]
                want = V.sum(axis=0) / (max(n, 0) + np.exp(0.7))
                np.testing.assert_allclose(z[t, h], want, atol=1e-14)
                np.testing.assert_allclose(zl[t, h], np.log(max(n, 0) + np.exp(0.7)), atol=1e-13)


@pytest.mark.parametrize("S,window", [(3, 5), (4, 0), (2, 12), (5, 200)])
def test_window_split_merge_equals_unsplit(S, window):
    case = gen.make_case("wsplit", q_lens=[6], seq_lens=[300], num_q_heads=2, num_kv_heads=1, head_dim=16,
                         page_size=16, q_kind="f32", seed=33)
    q = gen.to_numpy64(case.q)[:, 0, :]
    K = oracle.gather_dense_kv(gen.to_numpy64(case.k_pool), case.block_tables[0], 300, 0)
    V = oracle.gather_dense_kv(gen.to_numpy64(case.v_pool), case.block_tables[0], 300, 0)
    i = np.arange(6)
    counts = oracle.visible_key_count(300, 6, i)
    starts = oracle.window_start(300, 6, i, window)
    o, l = oracle.attention_rows(q, K, V, counts, case.scale, starts=starts)
    for base in (0, oracle.window_base(300, 6, window)):
        # parts of [0, L) or of the window range [base, L): both cover every visible key
        assert base <= starts.min() and base % 32 == 0
        os_, ls_ = oracle.split_partials(q, K, V, counts, case.scale, S, starts=starts, base=base)
        assert oracle.split_ranges(300, S, base=base)[0][0] == base
        om, lm = oracle.merge_partials(os_, ls_)
        np.testing.assert_allclose(om, o, atol=1e-13)
        np.testing.assert_allclose(lm, l, atol=1e-13)


# ---------------------------------------------------------------- softcap and ALiBi

SLOPES6 = [0.5, 0.25, 0.125, 0.0625, 1.0, 0.03125]


def _brute_vs_oracle(case, **kw):
    k, v = _dense(case)
    o, l = oracle.paged_attention(gen.to_numpy64(case.q), k, v, case.cu_seqlens_q, case.seq_lens,
                                  case.block_tables, case.scale, **kw)
    bo, bl = oracle.brute_paged_attention(gen.to_numpy64(case.q).tolist(), k.tolist(), v.tolist(),
                                          case.cu_seqlens_q.tolist(), case.seq_lens.tolist(),
                                          case.block_tables.tolist(), case.scale, **kw)
    bo, bl = np.array(bo), np.array(bl)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert (fin == np.isfinite(l)).all()
    np.testing.assert_allclose(l[fin], bl[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kw", [dict(softcap=0.8), dict(softcap=5.0), dict(alibi_slopes=SLOPES6),
                                dict(softcap=1.5, alibi_slopes=SLOPES6),
                                dict(softcap=2.0, alibi_slopes=SLOPES6, window_left=3, sinks=[0.5] * 6)])
def test_softcap_and_alibi_match_brute_force(kw):
    _brute_vs_oracle(small_gqa_case(seed=16, scale=1.5), **kw)


def test_softcap_limits():
    """A cap far above every logit changes nothing (tanh(x) = x - x^3/3 + ...);
    logits far above (below) the cap all become +cap (-cap): equal weights,
    o = the mean of the visible values and lse = +-cap + log(n)."""
    case = small_gqa_case(seed=17)
    k, v = _dense(case)
    q = gen.to_numpy64(case.q)
    args = (case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale)
    base, bl = oracle.paged_attention(q, k, v, *args)
    far, fl = oracle.paged_attention(q, k, v, *args, softcap=1e9)
    np.testing.assert_allclose(far, base, atol=1e-12)
    fin = np.isfinite(bl)
    np.testing.assert_allclose(fl[fin], bl[fin], atol=1e-12)
    # every key along +u with a positive length, q = +-big * u
    u = np.ones(case.head_dim) / np.sqrt(case.head_dim)
    rng = np.random.default_rng(3)
    ks = u[None, None, None, :] * rng.uniform(1.0, 2.0, size=k.shape[:3] + (1,))
    g = case.num_q_heads // case.num_kv_heads
    for sign in (1.0, -1.0):
        qs = np.broadcast_to(sign * 1e4 * u, q.shape).copy()
        o, l = oracle.paged_attention(qs, ks, v, *args, softcap=0.75)
        for b in range(case.num_seqs):
            L, Q = int(case.seq_lens[b]), int(case.q_lens[b])
            for i in range(Q):
                t, n = int(case.cu_seqlens_q[b]) + i, L - Q + i + 1
                for h in range(case.num_q_heads):
                    if n <= 0:
                        assert l[t, h] == -np.inf
                        continue
                    V = oracle.gather_dense_kv(v, case.block_tables[b], L, h // g)[:n]
                    np.testing.assert_allclose(o[t, h], V.mean(axis=0), atol=1e-13)
                    np.testing.assert_allclose(l[t, h], sign * 0.75 + np.log(n), atol=1e-13)


def _key_index_values(case):
    """A V pool whose dimension 0 holds the key index j of each (sequence) slot."""
    v = np.zeros((case.k_pool.shape[0], case.page_size, case.num_kv_heads, case.head_dim))
    for b in range(case.num_seqs):
        for j in range(int(case.seq_lens[b])):
            v[int(case.block_tables[b][j // case.page_size]), j % case.page_size, :, 0] = j
    return v


def test_alibi_closed_form_for_zero_queries():
    """q = 0: the logits are -slope * d for distances d = 0 .. n-1, so with r =
    e^-slope the weights are geometric: lse = log((1 - r^n) / (1 - r)) and the
    mean key index is p - r (1 - n r^(n-1) + (n-1) r^n) / ((1 - r)(1 - r^n))."""
    case = small_gqa_case(seed=18, seq_lens=[30, 7, 2, 64], q_lens=[5, 1, 3, 4])
    k, _ = _dense(case)
    v = _key_index_values(case)
    q = np.zeros(gen.to_numpy64(case.q).shape)
    o, l = oracle.paged_attention(q, k, v, case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale,
                                  alibi_slopes=SLOPES6)
    for b in range(case.num_seqs):
        L, Q = int(case.seq_lens[b]), int(case.q_lens[b])
        for i in range(Q):
            t, n = int(case.cu_seqlens_q[b]) + i, L - Q + i + 1
            p = n - 1
            for h in range(case.num_q_heads):
                if n <= 0:  # no visible key
                    assert l[t, h] == -np.inf and not o[t, h].any()
                    continue
                r = math.exp(-SLOPES6[h])
                geo = (1 - r ** n) / (1 - r)
                mean_d = r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / ((1 - r) ** 2 * geo)
                np.testing.assert_allclose(l[t, h], math.log(geo), rtol=0, atol=1e-13)
                np.testing.assert_allclose(o[t, h, 0], p - mean_d, rtol=0, atol=1e-11)
                assert not o[t, h, 1:].any()


def test_alibi_equals_plain_attention_with_one_more_dimension():
    """slope * j is a dot product: with q' = [q, slope / scale] and k'_j = [k_j, j]
    the plain logits are scale q.k + slope j, which differ from the ALiBi ones by
    slope * p per row: the same o, and lse shifted by slope * p."""
    case = small_gqa_case(seed=19, seq_lens=[40, 9, 3, 33])
    k, v = _dense(case)
    q = gen.to_numpy64(case.q)
    o, l = oracle.paged_attention(q, k, v, case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale,
                                  alibi_slopes=SLOPES6)
    kj = _key_index_values(case)[..., :1]
    k2 = np.concatenate([k, kj], axis=-1)
    v2 = np.concatenate([v, np.zeros_like(kj)], axis=-1)
    q2 = np.concatenate([q, np.broadcast_to(np.array(SLOPES6)[None, :, None] / case.scale, q.shape[:2] + (1,))], -1)
    o2, l2 = oracle.paged_attention(q2, k2, v2, case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale)
    np.testing.assert_allclose(o, o2[..., :-1], atol=1e-12)
    pos = np.concatenate([int(case.seq_lens[b]) - int(case.q_lens[b]) + np.arange(int(case.q_lens[b]))
                          for b in range(case.num_seqs)])
    want = l2 - np.array(SLOPES6)[None, :] * pos[:, None]
    fin = np.isfinite(l)
    assert (fin == np.isfinite(want)).all()
    np.testing.assert_allclose(l[fin], want[fin], atol=1e-11)


def test_alibi_matches_torch_sdpa_with_a_bias_matrix():
    """One sequence, MHA, dense: torch's fp64 scaled_dot_product_attention with an
    additive mask holding -slope (p - j) on visible keys and -inf elsewhere."""
    import torch
    Q, L, H, D = 6, 23, 3, 16
    case = gen.make_case("alibi_sdpa", q_lens=[Q], seq_lens=[L], num_q_heads=H, num_kv_heads=H, head_dim=D,
                         page_size=8, q_kind="f32", seed=20)
    k, v = _dense(case)
    q = gen.to_numpy64(case.q)
    slopes = [0.3, 0.05, 1.2]
    o, l = oracle.paged_attention(q, k, v, case.cu_seqlens_q, case.seq_lens, case.block_tables, case.scale,
                                  alibi_slopes=slopes)
    K = np.stack([oracle.gather_dense_kv(k, case.block_tables[0], L, h) for h in range(H)])
    V = np.stack([oracle.gather_dense_kv(v, case.block_tables[0], L, h) for h in range(H)])
    p = L - Q + np.arange(Q)
    j = np.arange(L)
    dist = p[:, None] - j[None, :]
    bias = np.where(dist[None] >= 0, -np.array(slopes)[:, None, None] * dist[None], -np.inf)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2).copy()), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=torch.from_numpy(bias), scale=case.scale).numpy()
    np.testing.assert_allclose(o, ref.transpose(1, 0, 2), atol=1e-12)


@pytest.mark.parametrize("S,window,softcap,slope", [(3, -1, 1.0, 0.2), (4, 7, 0.0, 0.05), (2, -1, 3.0, 0.0),
                                                    (5, 40, 0.5, 0.7)])
def test_softcap_alibi_split_merge_equals_unsplit(S, window, softcap, slope):
    case = gen.make_case("msplit", q_lens=[6], seq_lens=[300], num_q_heads=1, num_kv_heads=1, head_dim=16,
                         page_size=16, q_kind="f32", seed=34)
    q = gen.to_numpy64(case.q)[:, 0, :] * 4
    K = oracle.gather_dense_kv(gen.to_numpy64(case.k_pool), case.block_tables[0], 300, 0)
    V = oracle.gather_dense_kv(gen.to_numpy64(case.v_pool), case.block_tables[0], 300, 0)
    i = np.arange(6)
    counts = oracle.visible_key_count(300, 6, i)
    starts = oracle.window_start(300, 6, i, window)
    al = slope if slope else None
    o, l = oracle.attention_rows(q, K, V, counts, case.scale, starts=starts, softcap=softcap, alibi=al)
    base = oracle.window_base(300, 6, window)
    os_, ls_ = oracle.split_partials(q, K, V, counts, case.scale, S, starts=starts, base=base, softcap=softcap,
                                     alibi=al)
    om, lm = oracle.merge_partials(os_, ls_)
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, l, atol=1e-13)


def _mods_pins_pass():
    try:
        test_softcap_and_alibi_match_brute_force(dict(softcap=1.5, alibi_slopes=SLOPES6))
        test_softcap_limits()
        test_alibi_closed_form_for_zero_queries()
        test_alibi_equals_plain_attention_with_one_more_dimension()
    except AssertionError:
        return False
    return True


MOD_MUTATIONS = {
    "softcap_outer_factor_dropped": lambda s, softcap=0.0, slopes=None, dist=None, _f=oa.modified_logits:
        _f(np.tanh(s / softcap) if softcap else s, 0.0, slopes, dist),
    "alibi_sign": lambda s, softcap=0.0, slopes=None, dist=None, _f=oa.modified_logits:
        _f(s, softcap, None if slopes is None else -np.asarray(slopes), dist),
    "alibi_before_softcap": lambda s, softcap=0.0, slopes=None, dist=None, _f=oa.modified_logits:
        _f(_f(s, 0.0, slopes, dist), softcap, None, dist),
    "alibi_distance_off_by_one": lambda s, softcap=0.0, slopes=None, dist=None, _f=oa.modified_logits:
        _f(s, softcap, slopes, None if dist is None else dist + 1),
}


@pytest.mark.parametrize("name", sorted(MOD_MUTATIONS))
def test_planted_score_modifier_mistake_is_caught(name, monkeypatch):
    assert _mods_pins_pass()
    monkeypatch.setattr(oa, "modified_logits", MOD_MUTATIONS[name])
    assert not _mods_pins_pass(), f"mutation {name} survived every pin"
