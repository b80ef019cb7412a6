"""The seeded generators lay out valid paged caches with poison where nothing may be read (CPU)."""

import numpy as np
import torch

from paged_attention_prefill_amd import inputs as gen


def _check_layout(case):
    P = case.page_size
    seen = set()
    for b in range(case.num_seqs):
        L = int(case.seq_lens[b])
        n = -(-L // P)
        pages = case.block_tables[b, :n].tolist()
        assert len(set(pages)) == n
        assert not (set(pages) & seen) or case.name.startswith("long_chunk")
        seen |= set(pages)
        for j in range(L):
            k = case.k_pool[pages[j // P], j % P].float()
            assert torch.isfinite(k).all() if case.kv_kind not in ("e5m2", "e4m3") else (
                (case.k_pool[pages[j // P], j % P] & 0x7F) != gen.FP8_NAN_BYTE).all()
        if n and L % P:
            tail = case.k_pool[pages[-1], L % P:]
            if case.kv_kind in ("e5m2", "e4m3"):
                assert (tail == gen.FP8_NAN_BYTE).all()
            else:
                assert torch.isnan(tail.float()).all()
        # entries past the sequence's pages point at a poisoned spare page
        for p in case.block_tables[b, n:]:
            assert int(p) not in seen
    assert case.block_tables.min() >= 0 and case.block_tables.max() < case.num_pages


def test_tiny_case_layout():
    c = gen.tiny_fp32()
    assert c.num_pages == 16 and c.total_q == 17 and list(c.seq_lens) == [64, 64]
    _check_layout(c)
    # 8 pages in use, 8 poisoned
    assert c.meta["spare_pages"] == 8


def test_generators_are_deterministic():
    a = gen.make_case("x", [3, 4], [10, 40], 4, 2, 32, 16, q_kind="bf16", seed=7)
    b = gen.make_case("x", [3, 4], [10, 40], 4, 2, 32, 16, q_kind="bf16", seed=7)
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k_pool.nan_to_num(), b.k_pool.nan_to_num())
    assert (a.block_tables == b.block_tables).all()


def test_fp8_and_hnd_layouts():
    c = gen.make_case("f8", [2, 5], [33, 100], 6, 2, 64, 16, q_kind="f16", kv_kind="e5m2", seed=3)
    assert c.k_pool.dtype == torch.uint8
    _check_layout(c)
    e = gen.make_case("e4", [2, 5], [33, 100], 6, 2, 64, 16, q_kind="f16", kv_kind="e4m3", seed=3)
    assert e.k_pool.dtype == torch.uint8
    _check_layout(e)
    # E4M3 bytes of N(0, 1) draws: decoded values are the draws rounded to E4M3
    vals = e.k_pool[e.block_tables[1, 0]].view(torch.float8_e4m3fn).float()
    assert torch.isfinite(vals).all() and vals.abs().max() < 8
    h = gen.make_case("hnd", [2, 5], [33, 100], 6, 2, 64, 16, q_kind="f16", seed=3, layout="HND")
    assert h.k_pool.shape == (h.num_pages, 16, 2, 64)
    assert h.k_pool.stride(1) == 64 and h.k_pool.stride(2) == 16 * 64
    _check_layout(h)


def test_decode_batch_lengths():
    lens = gen.decode_batch_lengths(np.random.default_rng(2))
    assert len(lens) == 32
    assert list(lens[:10]) == gen.DECODE_FIXED_LENS
    assert lens.max() <= 10000 and lens[10:].min() >= 1
    small = gen.decode_batch(extra_rows=2, max_len=64)
    assert small.num_seqs == 12 and small.total_q == 12


def test_select_seqs():
    c = gen.make_case("x", [3, 4, 2], [10, 40, 9], 4, 2, 32, 16, q_kind="f32", seed=8)
    s = gen.select_seqs(c, [2, 0])
    assert list(s.cu_seqlens_q) == [0, 2, 5]
    assert torch.equal(s.q[:2], c.q[7:9]) and torch.equal(s.q[2:], c.q[0:3])
    assert (s.block_tables[0] == c.block_tables[2]).all()
