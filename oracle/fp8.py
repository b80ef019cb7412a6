"""fp8 byte decoding for the oracle (test infrastructure only): E5M2 and E4M3.

The pages name the KV format "fp8_e5m2" (1CatAI/1Cat-vLLM PR #616, original
description, "Test Plan" and the fp8_e5m2 KV paragraph of "Test Result") and
give no bit layout.  The reading taken here is the common E5M2 layout that
torch.float8_e5m2 also uses: 1 sign bit, 5 exponent bits with bias 15, 2
mantissa bits, subnormals at exponent 0, and exponent 31 reserved for
infinities (mantissa 0) and NaNs (mantissa != 0).

Written from that definition with integer arithmetic; no table and no library
conversion.  Pinned against torch's own float8_e5m2 conversion for all 256
bytes in the oracle tests.
"""

import numpy as np


def e5m2_to_float64(codes):
    """Decode an array of E5M2 bytes (any integer dtype, values 0..255) to float64."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E5M2 codes must be bytes")
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 2) & 0x1F
    man = c & 0x3
    # normal numbers: (1 + m/4) * 2^(e-15); subnormals: (m/4) * 2^(1-15)
    normal = (1.0 + man / 4.0) * np.exp2(exp.astype(np.float64) - 15.0)
    subnormal = (man / 4.0) * np.exp2(-14.0)
    val = np.where(exp == 0, subnormal, normal)
    val = np.where(exp == 31, np.where(man == 0, np.inf, np.nan), val)
    return sign * val


def e4m3_to_float64(codes):
    """Decode an array of E4M3 bytes to float64.

    The pages' tests name an e4m3 KV path (1CatAI/1Cat-vLLM PR #616, original
    description, "Test Plan": an e4m3 scalar fp32 test) without a layout; the
    reading is the OCP E4M3 ("fn") layout that torch.float8_e4m3fn uses: 1 sign,
    4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
    infinities, and only exponent 15 with mantissa 7 as NaN (so 448 is the
    largest magnitude).  Pinned against torch on all 256 bytes."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes must be bytes")
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * np.exp2(-6.0)
    val = np.where(exp == 0, subnormal, normal)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val
