"""Oracle of the KV write: new tokens' K and V into their cache pages (test
infrastructure only).

What is computed (the pages give the step, not its arithmetic):
* the chunk's K/V are in the cache before its attention runs (1CatAI/1Cat-vLLM
  PR #1279, commit 3: the second half of a split batch reads the first half's
  KV writes); token t of a sequence with q new tokens and length L (counting
  them) lands at position L - q + t, page block_table[pos // P], slot pos % P;
* an fp8_e5m2 cache with a per-tensor scale (1CatAI/1Cat-vLLM PR #616,
  original description, "Test Result", fp8_e5m2 KV paragraph), and an e4m3
  path named by the same page's "Test Plan".  The pages do not say how a value
  becomes a byte.  Reading: byte = the fp8 value nearest to x / scale, the
  quotient taken in float32 (as the kernel takes it), ties to the even code,
  magnitudes past the largest finite value (57344 for E5M2, 448 for E4M3)
  saturated to it, NaN kept NaN (0x7F with the sign bit).

The encoder is written as that definition: it searches the table of all
finite E5M2 values (decoded by ``oracle.fp8`` from the bit layout) for the
nearest one; no bit tricks.  Pinned against torch's float8_e5m2 conversion
inside the finite range and against hand-checked values.  The float32
quotient is pinned by exact rational arithmetic on inputs where a float64
quotient would give another byte.
"""

import numpy as np

from .fp8 import e4m3_to_float64, e5m2_to_float64

E5M2_MAX = 57344.0
E4M3_MAX = 448.0
# every finite non-negative code of each format, in ascending order of value
_TABLES = {"e5m2": (np.arange(0, 0x7C), e5m2_to_float64(np.arange(0, 0x7C)), E5M2_MAX),
           "e4m3": (np.arange(0, 0x7F), e4m3_to_float64(np.arange(0, 0x7F)), E4M3_MAX)}


def fp8_encode(y, fmt):
    """fp8 bytes (uint8) of the float values y: the nearest finite value of the
    format, ties to the even code, saturating at the largest finite magnitude,
    NaN -> 0x7F | sign (a NaN code of both formats)."""
    codes, values, vmax = _TABLES[fmt]
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    sign = np.signbit(y).astype(np.int64) << 7
    a_sat = np.minimum(np.where(np.isnan(a), 0.0, a), vmax)
    hi = np.searchsorted(values, a_sat, side="left")     # first table value >= a
    hi = np.minimum(hi, len(values) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a_sat - values[lo]
    d_hi = values[hi] - a_sat
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    code = np.where(pick_hi, codes[hi], codes[lo])
    code = np.where(a_sat == values[hi], codes[hi], code)
    code = np.where(np.isnan(y), 0x7F, code)
    return (code | sign).astype(np.uint8)


def e5m2_encode(y):
    """E5M2 bytes: nearest finite value, ties to even, saturating at +-57344."""
    return fp8_encode(y, "e5m2")


def e4m3_encode(y):
    """E4M3 bytes: nearest finite value, ties to even, saturating at +-448."""
    return fp8_encode(y, "e4m3")


def quantize_fp8(x, scale, fmt="e5m2"):
    """fp8 bytes of x / scale, the quotient formed in float32."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return fp8_encode(q.astype(np.float64), fmt)


def quantize_e5m2(x, scale):
    """E5M2 bytes of x / scale, the quotient formed in float32."""
    return quantize_fp8(x, scale, "e5m2")


def write_kv(k_pool, v_pool, k_new, v_new, cu_seqlens_q, seq_lens, block_tables, fp8=False,
             k_scale=1.0, v_scale=1.0, k_head_scales=None, v_head_scales=None):
    """Copies of the pools [num_pages, P, Hkv, D] with the new tokens written.

    k_new, v_new [total_q, Hkv, D] (float values); fp8 pools are uint8 byte
    arrays, fp8 = True or "e5m2" for E5M2 bytes, "e4m3" for E4M3 bytes.
    """
    fmt = "e5m2" if fp8 is True else fp8

    def head_scales(scale, per_head):
        # the per-tensor factor times the head's own, the product rounded to float32
        ph = np.ones(H, dtype=np.float32) if per_head is None else np.asarray(per_head, dtype=np.float32)
        return np.float32(scale) * ph
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    H = k_out.shape[2]
    P = k_out.shape[1]
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for b in range(len(seq_lens)):
        q_len = int(cu[b + 1] - cu[b])
        L = int(seq_lens[b])
        for t in range(q_len):
            pos = L - q_len + t
            if pos < 0:
                continue
            page = int(block_tables[b][pos // P])
            row = int(cu[b]) + t
            if fp8:
                ks, vs = head_scales(k_scale, k_head_scales), head_scales(v_scale, v_head_scales)
                for h in range(H):
                    k_out[page, pos % P, h] = quantize_fp8(k_new[row, h], ks[h], fmt)
                    v_out[page, pos % P, h] = quantize_fp8(v_new[row, h], vs[h], fmt)
            else:
                k_out[page, pos % P] = k_new[row]
                v_out[page, pos % P] = v_new[row]
    return k_out, v_out
