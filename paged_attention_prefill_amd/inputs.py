"""Seeded synthetic inputs for paged attention (shared by tests and the benchmark).

This module only draws random numbers and lays them out as a paged KV cache:
it holds none of the attention arithmetic, so both the fp64 oracle and the HIP
path can be fed from it without sharing any of the method's code.

Recipe (every case):
  * ``rng = numpy.random.default_rng(seed)``; draws in this order: extra row
    lengths (decode batch only), the page permutation, q, k pages, v pages.
  * q, k, v ~ N(0, 1) drawn in float32, then rounded to the storage dtype
    (round-to-nearest-even through torch's casts); fp8 KV is N(0, 1) rounded
    to E5M2 (or E4M3) with per-tensor scale 1.0, stored as bytes.
  * Each sequence gets ceil(seq_len / page_size) pages.  The pool holds those
    plus spare pages (10 % by default, at least ``min_spare``); the page ids
    are a random permutation of the pool, so pages are out of order.
  * Poison: spare pages and the slots past seq_len in a sequence's last page
    hold NaN (byte 0x7F for fp8, a NaN in both formats).  Block-table entries past a sequence's
    pages point at a poisoned spare page, so any read outside the visible
    range turns the result into NaN instead of touching memory out of bounds.
  * KV layout: logical [num_pages, page_size, Hkv, D] with D contiguous; the
    'HND' layout stores [num_pages, Hkv, page_size, D] and exposes the same
    logical view through strides.
"""

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

FP8_NAN_BYTE = 0x7F  # a NaN of both E5M2 and E4M3
E5M2_NAN_BYTE = FP8_NAN_BYTE

_TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
}


@dataclass
class PagedCase:
    name: str
    q: torch.Tensor                 # [total_q, Hq, D], dtype q_dtype (CPU)
    k_pool: torch.Tensor            # logical [num_pages, page_size, Hkv, D] view (CPU)
    v_pool: torch.Tensor
    cu_seqlens_q: np.ndarray        # int32 [B + 1]
    seq_lens: np.ndarray            # int32 [B]
    block_tables: np.ndarray        # int32 [B, max_pages]
    page_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    q_kind: str                     # 'f32' | 'f16' | 'bf16'
    kv_kind: str                    # 'f32' | 'f16' | 'bf16' | 'e5m2' | 'e4m3'
    k_scale: float = 1.0
    v_scale: float = 1.0
    num_splits: int = 16
    layout: str = "NHD"
    k_head_scales: Optional[np.ndarray] = None  # fp8 only: float32 [Hkv] per-head factors
    v_head_scales: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.seq_lens)

    @property
    def total_q(self):
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self):
        return np.diff(self.cu_seqlens_q.astype(np.int64))

    @property
    def max_seqlen_q(self):
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def num_pages(self):
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self):
        return int(self.block_tables.shape[1])


_FP8_TORCH = {"e5m2": torch.float8_e5m2, "e4m3": torch.float8_e4m3fn}


def _fill_normal(dst, rng, chunk=1 << 24, fp8="e5m2"):
    """Fill a contiguous CPU tensor with N(0,1) float32 draws rounded to its dtype
    (uint8 storage: the bytes of the fp8 format `fp8`)."""
    flat = dst.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        src = torch.from_numpy(rng.standard_normal(e - s, dtype=np.float32))
        if dst.dtype == torch.uint8:  # fp8 storage
            flat[s:e] = src.to(_FP8_TORCH[fp8]).view(torch.uint8)
        else:
            flat[s:e] = src.to(dst.dtype)


def make_case(name, q_lens, seq_lens, num_q_heads, num_kv_heads, head_dim, page_size,
              q_kind="bf16", kv_kind=None, seed=0, scale=None, spare_frac=0.10,
              min_spare=1, shuffle=True, poison=True, layout="NHD", num_splits=16,
              k_scale=1.0, v_scale=1.0, pool_pages=None, rng=None, extra_pages_per_seq=0):
    """Build one varlen paged case.  ``q_lens[b] <= seq_lens[b]`` is not required
    (rows without a visible key are legal and must come out as zeros)."""
    kv_kind = kv_kind or q_kind
    rng = rng if rng is not None else np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    P = int(page_size)
    need = [-(-int(L) // P) for L in seq_lens]
    used = int(sum(need))
    spare = max(int(min_spare), int(np.ceil(used * spare_frac)))
    num_pages = used + spare if pool_pages is None else int(pool_pages)
    if num_pages < used + 1:
        raise ValueError("pool too small (needs at least one spare page for poison)")
    perm = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    owned = perm[:used]
    spare_ids = perm[used:]
    poison_page = int(spare_ids[0])
    max_pages = max(1, max(need) + int(extra_pages_per_seq)) if B else 1
    bt = np.full((B, max_pages), poison_page, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = owned[off:off + need[b]]
        off += need[b]

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    total_q = int(cu[-1])

    D, Hq, Hkv = int(head_dim), int(num_q_heads), int(num_kv_heads)
    q = torch.empty((total_q, Hq, D), dtype=_TORCH_DTYPES[q_kind])
    _fill_normal(q, rng)

    store_dtype = torch.uint8 if kv_kind in _FP8_TORCH else _TORCH_DTYPES[kv_kind]
    phys_shape = (num_pages, P, Hkv, D) if layout == "NHD" else (num_pages, Hkv, P, D)
    pools = []
    for _ in range(2):
        t = torch.empty(phys_shape, dtype=store_dtype)
        _fill_normal(t, rng, fp8=kv_kind if kv_kind in _FP8_TORCH else "e5m2")
        view = t if layout == "NHD" else t.permute(0, 2, 1, 3)
        if poison:
            bad = FP8_NAN_BYTE if kv_kind in _FP8_TORCH else float("nan")
            view[torch.from_numpy(spare_ids.astype(np.int64))] = bad
            for b in range(B):
                tail = int(seq_lens[b]) % P
                if need[b] and tail:
                    view[int(bt[b, need[b] - 1]), tail:] = bad
        pools.append(view)

    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    return PagedCase(name=name, q=q, k_pool=pools[0], v_pool=pools[1], cu_seqlens_q=cu,
                     seq_lens=seq_lens.astype(np.int32), block_tables=bt, page_size=P,
                     num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, scale=float(scale),
                     q_kind=q_kind, kv_kind=kv_kind, k_scale=float(k_scale),
                     v_scale=float(v_scale), num_splits=int(num_splits), layout=layout,
                     meta={"seed": seed, "spare_pages": int(len(spare_ids))})


def select_seqs(case, idx, name=None):
    """Sub-batch of sequences ``idx`` over the same page pool (q rows copied)."""
    idx = list(idx)
    cu = case.cu_seqlens_q.astype(np.int64)
    parts = [case.q[int(cu[b]):int(cu[b + 1])] for b in idx]
    q = torch.cat(parts, 0) if parts else case.q[:0]
    ql = np.array([cu[b + 1] - cu[b] for b in idx], dtype=np.int64)
    new_cu = np.zeros(len(idx) + 1, dtype=np.int32)
    new_cu[1:] = np.cumsum(ql)
    return replace(case, name=name or f"{case.name}[{idx}]", q=q, cu_seqlens_q=new_cu,
                   seq_lens=case.seq_lens[idx].copy(), block_tables=case.block_tables[idx].copy())


def expand_row(case, b, name=None):
    """Row b (q tokens at length L) as q separate q=1 rows at lengths
    L - q + 1 .. L over the same pages: the token-wise expansion of a verify row."""
    cu = case.cu_seqlens_q.astype(np.int64)
    t0, q_len = int(cu[b]), int(cu[b + 1] - cu[b])
    L = int(case.seq_lens[b])
    lens = np.array([L - q_len + 1 + i for i in range(q_len)], dtype=np.int32)
    return replace(case, name=name or f"{case.name}[{b}] token-wise", q=case.q[t0:t0 + q_len].clone(),
                   cu_seqlens_q=np.arange(q_len + 1, dtype=np.int32), seq_lens=lens,
                   block_tables=np.repeat(case.block_tables[b:b + 1], q_len, axis=0))


# ---------------------------------------------------------------------------
# The five workloads, shaped like the pages' measurements
# ---------------------------------------------------------------------------

def tiny_fp32(seed=1):
    """fp32, Hq 4 / Hkv 1, D 64, page 16: a 48-token prefix + 16-token chunk (seq_len 64)
    and a q=1 decode row at seq_len 64 on its own 4 pages; 16-page pool, 8 poisoned."""
    return make_case("tiny_fp32", q_lens=[16, 1], seq_lens=[64, 64], num_q_heads=4,
                     num_kv_heads=1, head_dim=64, page_size=16, q_kind="f32", seed=seed,
                     pool_pages=16, num_splits=16)


DECODE_FIXED_LENS = [0, 1, 31, 32, 33, 511, 512, 513, 4097, 10000]


def decode_batch_lengths(rng, extra_rows=22, max_len=10000):
    """Row lengths of the decode batch: the fixed list, then uniform[1, max_len] draws."""
    extra = rng.integers(1, max_len + 1, extra_rows)
    return np.concatenate([np.array(DECODE_FIXED_LENS), extra]).astype(np.int64)


def decode_batch(seed=2, kind="bf16", extra_rows=22, max_len=10000):
    """32 decode rows (q=1): lengths 0/1/31/32/33/511/512/513/4097/10000 plus
    uniform[1, 10000]; MHA 16 heads, D 128, page 16, 16 splits."""
    rng = np.random.default_rng(seed)
    lens = decode_batch_lengths(rng, extra_rows, max_len)
    return make_case(f"decode_batch_{kind}", q_lens=[1] * len(lens), seq_lens=lens,
                     num_q_heads=16, num_kv_heads=16, head_dim=128, page_size=16,
                     q_kind=kind, seed=seed, num_splits=16, rng=rng)


def varlen_prefill(seed=3, kind="bf16"):
    """4 sequences, q lens 64/300/1024/2048 after prefixes 0/777/4096/8192;
    Hq 32 / Hkv 8, D 128, page 32."""
    q_lens = [64, 300, 1024, 2048]
    prefix = [0, 777, 4096, 8192]
    return make_case(f"varlen_prefill_{kind}", q_lens=q_lens,
                     seq_lens=[a + b for a, b in zip(q_lens, prefix)], num_q_heads=32,
                     num_kv_heads=8, head_dim=128, page_size=32, q_kind=kind, seed=seed)


def long_chunk(seed=4, kind="f16", q_len=2048, prefix=150000, num_q_heads=24, num_kv_heads=4):
    """One 2048-token causal chunk after 150,000 cached tokens; Hq 24 / Hkv 4, D 256,
    page 64, scale 1/16.  Adds a q=1 decode row over the same cache (seq 1)."""
    L = q_len + prefix
    case = make_case(f"long_chunk_{kind}", q_lens=[q_len, 1], seq_lens=[L, L],
                     num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=256,
                     page_size=64, q_kind=kind, seed=seed, spare_frac=0.01)
    # the decode row reads the very same pages as the chunk
    case.block_tables[1] = case.block_tables[0]
    return case


def geometric_alibi_slopes(num_heads):
    """The usual ALiBi slopes 2^(-8 (h + 1) / H), float32 [H] (an input of the
    ALiBi option; nothing of the method's arithmetic)."""
    return (2.0 ** (-8.0 * (np.arange(num_heads) + 1) / num_heads)).astype(np.float32)


def mixed_step(seed=5, kv_kind="f16"):
    """D 256, Hq 24 / Hkv 4, page 816: a verify row (q=5, seq_len 240,000) and a
    784-token chunk after 104,000 cached tokens; fp16 or fp8_e5m2 KV, fp16 q."""
    return make_case(f"mixed_step_{kv_kind}", q_lens=[5, 784], seq_lens=[240000, 104784],
                     num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=816,
                     q_kind="f16", kv_kind=kv_kind, seed=seed, spare_frac=0.02,
                     num_splits=16)


def to_numpy64(t: torch.Tensor, kv_kind: Optional[str] = None):
    """Exact widening of a CPU tensor for the oracle (fp8 stays as raw bytes)."""
    if kv_kind in _FP8_TORCH:
        return t.numpy()
    return t.to(torch.float64).numpy()


def to_device(case, device="cuda"):
    """Copies of a case's tensors on the GPU (the pools keep their logical strides)."""
    def dev(t):
        return t.to(device)
    k = case.k_pool
    v = case.v_pool
    if case.layout != "NHD":
        # move the physical storage, then rebuild the same logical view
        k = k.permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().to(device).permute(0, 2, 1, 3)
    else:
        k, v = dev(k.contiguous()), dev(v.contiguous())
    if case.kv_kind == "e4m3":  # the binding reads the fp8 format from the dtype (uint8 = E5M2)
        k, v = k.view(torch.float8_e4m3fn), v.view(torch.float8_e4m3fn)
    extra = {}
    for name in ("k_head_scales", "v_head_scales"):
        val = getattr(case, name)
        if val is not None:
            extra[name] = torch.from_numpy(np.asarray(val, dtype=np.float32)).to(device)
    return dict(q=dev(case.q.contiguous()), k=k, v=v, **extra,
                cu=torch.from_numpy(case.cu_seqlens_q.astype(np.int32)).to(device),
                seq_lens=torch.from_numpy(case.seq_lens.astype(np.int32)).to(device),
                bt=torch.from_numpy(np.ascontiguousarray(case.block_tables, dtype=np.int32)).to(device))
