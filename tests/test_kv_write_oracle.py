"""Pins of the KV-write oracle (CPU): the E5M2 encoder against torch's
float8_e5m2 conversion and hand-checked values, and the slot arithmetic of the
write against the oracle's own gather."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen


def test_e5m2_encoder_matches_torch_on_every_finite_fp16_value():
    """Every fp16 bit pattern below the saturation point: ties, subnormals,
    both signs (torch's conversion rounds to nearest even, without saturation)."""
    h = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.float16)
    x = h.to(torch.float32)
    keep = torch.isfinite(x) & (x.abs() < 61440)
    x = x[keep]
    want = x.to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = oracle.e5m2_encode(x.numpy().astype(np.float64))
    assert (got == want).all(), int((got != want).sum())


def test_e5m2_encoder_matches_torch_on_random_float32():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 12, 200000))).astype(np.float32)
    x = x[np.abs(x) < 61440]
    want = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert (oracle.e5m2_encode(x.astype(np.float64)) == want).all()


def test_e5m2_encoder_special_values():
    cases = [(1.0, 0x3C), (1.125, 0x3C), (1.375, 0x3E), (1.25, 0x3D), (57344.0, 0x7B), (61439.0, 0x7B),
             (61440.0, 0x7B), (1e30, 0x7B), (np.inf, 0x7B), (-np.inf, 0xFB), (-70000.0, 0xFB), (2.0 ** -16, 0x01),
             (2.0 ** -17, 0x00), (3 * 2.0 ** -18, 0x01), (2.0 ** -14, 0x04), (0.875 * 2.0 ** -14, 0x04),
             (-0.0, 0x80), (0.0, 0x00), (-1e-9, 0x80)]
    for v, c in cases:
        assert int(oracle.e5m2_encode(np.array([v]))[0]) == c, (v, hex(c))
    nan = oracle.e5m2_encode(np.array([np.nan, -np.nan]))
    assert list(nan) == [0x7F, 0xFF]


def test_e5m2_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) < 0x7C])
    vals = oracle.e5m2_to_float64(codes)
    back = oracle.e5m2_encode(vals)
    assert (back == codes).all()


def _round_fraction(q, mant_bits, min_exp):
    """The binary float nearest to the rational q (ties to the even significand):
    mant_bits fraction bits, smallest normal exponent min_exp, exact arithmetic."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, min_exp) - mant_bits)
    n, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _nearest_code(v, fmt):
    """fp8 code of the exact rational v: nearest finite value of the format,
    ties to the even code (the values come from the bit-layout decoder, which is
    pinned against torch on all 256 bytes)."""
    top = 0x7C if fmt == "e5m2" else 0x7F
    dec = oracle.e5m2_to_float64 if fmt == "e5m2" else oracle.e4m3_to_float64
    vals = [Fraction(float(x)) for x in dec(np.arange(top))]
    a = abs(v)
    best = min(range(top), key=lambda c: (abs(vals[c] - a), c % 2))
    return best | (0x80 if v < 0 else 0)


# (fmt, source value, scale): the fp32 quotient and the fp64 quotient of these
# land on different sides of a rounding boundary of the fp8 grid
DIVERGENT = [("e5m2", 0.000194549560546875, 1.7), ("e5m2", 1.1444091796875e-05, 0.1),
             ("e5m2", 7.62939453125e-06, 1 / 3), ("e5m2", 2.6702880859375e-05, 0.7),
             ("e5m2", -2.6702880859375e-05, 0.7), ("e4m3", 0.02490234375, 1.7), ("e4m3", 0.00146484375, 0.1),
             ("e4m3", 0.0009765625, 1 / 3), ("e4m3", 0.01708984375, 0.7), ("e4m3", -0.00341796875, 0.7)]


def _exact_codes(fmt, x, scale):
    """(code of the quotient rounded to float32, code of it rounded to float64),
    from the exact rational quotient."""
    q = Fraction(float(np.float32(x))) / Fraction(float(np.float32(scale)))
    return _nearest_code(_round_fraction(q, 23, -126), fmt), _nearest_code(_round_fraction(q, 52, -1022), fmt)


@pytest.mark.parametrize("fmt,x,scale", DIVERGENT)
def test_quantize_divides_in_float32(fmt, x, scale):
    """The reading: byte = fp8 code of the IEEE float32 quotient x / scale.  The
    expected byte is derived here from the exact rational quotient, rounded to
    float32 by exact arithmetic; the inputs are chosen so that an fp64 quotient
    gives another byte, so the test tells the two readings apart."""
    want32, want64 = _exact_codes(fmt, x, scale)
    assert want32 != want64
    got = int(oracle.quantize_fp8(np.array([x], dtype=np.float32), scale, fmt)[0])
    assert got == want32, (fmt, x, scale, hex(got), hex(want32))


def test_quantize_pin_trips_on_fp64_division(monkeypatch):
    """A planted mistake: the quotient formed in float64 instead of float32."""
    from oracle import kv_write

    def fp64_quotient(x, scale, fmt="e5m2"):
        q = np.asarray(x, dtype=np.float32).astype(np.float64) / np.float64(np.float32(scale))
        return kv_write.fp8_encode(q, fmt)
    monkeypatch.setattr(oracle, "quantize_fp8", fp64_quotient)
    tripped = 0
    for fmt, x, scale in DIVERGENT:
        try:
            test_quantize_divides_in_float32(fmt, x, scale)
        except AssertionError:
            tripped += 1
    assert tripped == len(DIVERGENT)


def test_write_places_each_token_at_its_slot():
    """After the write, the sequence's last q_len keys (gathered by the oracle
    through the block table) are exactly the new rows, and nothing else moved."""
    case = gen.make_case("kvw", q_lens=[5, 0, 17], seq_lens=[40, 9, 17], num_q_heads=4, num_kv_heads=2,
                         head_dim=32, page_size=16, q_kind="f32", seed=51, poison=False)
    rng = np.random.default_rng(52)
    T = case.total_q
    kn = rng.standard_normal((T, 2, 32))
    vn = rng.standard_normal((T, 2, 32))
    kp = gen.to_numpy64(case.k_pool)
    vp = gen.to_numpy64(case.v_pool)
    ko, vo = oracle.write_kv(kp, vp, kn, vn, case.cu_seqlens_q, case.seq_lens, case.block_tables)
    changed = np.zeros(kp.shape[:2], dtype=bool)
    for b in range(case.num_seqs):
        L, q = int(case.seq_lens[b]), int(case.q_lens[b])
        t0 = int(case.cu_seqlens_q[b])
        for h in range(2):
            K = oracle.gather_dense_kv(ko, case.block_tables[b], L, h)
            V = oracle.gather_dense_kv(vo, case.block_tables[b], L, h)
            np.testing.assert_array_equal(K[L - q:], kn[t0:t0 + q, h])
            np.testing.assert_array_equal(V[L - q:], vn[t0:t0 + q, h])
            K0 = oracle.gather_dense_kv(kp, case.block_tables[b], L, h)
            np.testing.assert_array_equal(K[:L - q], K0[:L - q])
        for pos in range(L - q, L):
            changed[int(case.block_tables[b][pos // 16]), pos % 16] = True
    np.testing.assert_array_equal(ko[~changed], kp[~changed])
    np.testing.assert_array_equal(vo[~changed], vp[~changed])


# ---------------------------------------------------------------- E4M3

def test_e4m3_decoder_matches_torch_on_all_bytes():
    codes = np.arange(256)
    want = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_to_float64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.nanmax(got) == 448.0 and int(np.isnan(got).sum()) == 2


def test_e4m3_encoder_matches_torch_on_every_fp16_value_in_range():
    """Every fp16 bit pattern up to 464 (torch's conversion, which rounds to
    nearest even and turns larger magnitudes into NaN)."""
    h = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.float16)
    x = h.to(torch.float32)
    x = x[torch.isfinite(x) & (x.abs() <= 464)]
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x.numpy().astype(np.float64))
    assert (got == want).all(), int((got != want).sum())


def test_e4m3_encoder_specials_and_round_trip():
    cases = [(448.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE),
             (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -11, 0x01),
             (2.0 ** -6, 0x08), (-0.0, 0x80)]
    for v, c in cases:
        assert int(oracle.e4m3_encode(np.array([v]))[0]) == c, (v, hex(c))
    assert list(oracle.e4m3_encode(np.array([np.nan, -np.nan]))) == [0x7F, 0xFF]
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert (oracle.e4m3_encode(oracle.e4m3_to_float64(codes)) == codes).all()



def test_per_head_scales_in_dequantisation_and_write():
    """A per-head factor multiplies head h only (axis 2 of the pool), and the
    write divides by the float32 product of the two factors."""
    rng = np.random.default_rng(3)
    pool = rng.integers(0, 0x7B, size=(3, 16, 4, 8), dtype=np.uint8)
    hs = np.array([0.5, 2.0, 1.0, 3.0], dtype=np.float32)
    got = oracle.dequantize_pool(pool, "e5m2", 0.25 * hs.astype(np.float64))
    for h in range(4):
        np.testing.assert_array_equal(got[:, :, h], oracle.e5m2_to_float64(pool[:, :, h]) * 0.25 * float(hs[h]))
    case = gen.make_case("hs", q_lens=[3], seq_lens=[20], num_q_heads=4, num_kv_heads=4, head_dim=16,
                         page_size=16, q_kind="f16", kv_kind="e4m3", seed=5, poison=False)
    kn = rng.standard_normal((3, 4, 16))
    ko, _ = oracle.write_kv(case.k_pool.numpy(), case.v_pool.numpy(), kn, kn, case.cu_seqlens_q, case.seq_lens,
                            case.block_tables, fp8="e4m3", k_scale=0.3, k_head_scales=hs)
    for h in range(4):
        want = oracle.quantize_fp8(kn[:, h], np.float32(0.3) * hs[h], "e4m3")
        K = oracle.gather_dense_kv(ko, case.block_tables[0], 20, h)
        np.testing.assert_array_equal(K[17:20], want)
