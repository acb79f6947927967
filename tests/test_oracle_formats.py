"""Pins for the oracle's format decoders and the generator's encoders.

The fp8 values are those of the OCP 8-bit floating-point specification
(E4M3 "FN": bias 7, no infinities, S.1111.111 = NaN, max normal 448, min
normal 2^-6, min subnormal 2^-9).  The generator's integer encoder and the
oracle's definition-based decoder were written separately; they must agree.
"""
import math

import numpy as np

from oracle.formats import decode_bf16, decode_e4m3fn, e4m3fn_value
from synth import gen


def test_e4m3fn_spec_values():
    assert e4m3fn_value(0x00) == 0.0
    assert e4m3fn_value(0x80) == 0.0 and math.copysign(1, e4m3fn_value(0x80)) < 0
    assert e4m3fn_value(0x38) == 1.0
    assert e4m3fn_value(0x7E) == 448.0
    assert e4m3fn_value(0xFE) == -448.0
    assert e4m3fn_value(0x08) == 2.0 ** -6
    assert e4m3fn_value(0x07) == 7 * 2.0 ** -9
    assert e4m3fn_value(0x01) == 2.0 ** -9
    assert math.isnan(e4m3fn_value(0x7F)) and math.isnan(e4m3fn_value(0xFF))
    # 0x78 (exponent field 15, mantissa 0) is a finite 256 in the FN variant.
    assert e4m3fn_value(0x78) == 256.0
    # Monotone over the positive codes.
    vals = [e4m3fn_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_generator_integer_codes_decode_exactly():
    ints = np.arange(-7, 8)
    codes = gen.encode_e4m3_int(ints)
    assert np.array_equal(decode_e4m3fn(codes), ints.astype(np.float64))
    # Zero is encoded as +0.
    assert codes[7] == 0


def test_bf16_decode_and_rounding():
    assert decode_bf16(np.array([0x3F80]))[0] == 1.0
    assert decode_bf16(np.array([0xC000]))[0] == -2.0
    assert decode_bf16(np.array([0x7F80]))[0] == np.inf
    # Round to nearest even at the exact halfway points.
    one_plus_half_ulp = np.float32(1.0 + 2.0 ** -8)
    three_half_ulps = np.float32(1.0 + 3 * 2.0 ** -8)
    assert gen.f32_to_bf16_bits(np.array([one_plus_half_ulp]))[0] == 0x3F80
    assert gen.f32_to_bf16_bits(np.array([three_half_ulps]))[0] == 0x3F82
    # Just above halfway rounds up.
    above = np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20)
    assert gen.f32_to_bf16_bits(np.array([above]))[0] == 0x3F81
    # Values already on the bf16 grid round-trip.
    x = np.array([0.5, -0.25, 3.0, 1e-3], np.float32)
    bits = gen.f32_to_bf16_bits(x)
    assert np.array_equal(gen.f32_to_bf16_bits(decode_bf16(bits).astype(np.float32)), bits)


def test_generator_query_drift_statistics():
    from synth import get_workload
    wl = get_workload("tiny-4k").with_(steps=64, idx_heads=64)
    q = gen.index_query_ints(wl, 0, 0, 0).astype(np.float64)
    assert q.min() >= -7 and q.max() <= 7
    # Clipping at +-7 trims the Gaussian innovations' tails, so the spread
    # settles a little below the uniform-integer std and then stays there;
    # the lag-1 correlation stays near rho.
    early, late = q[1:16].std(), q[32:].std()
    assert 3.2 < late < math.sqrt(56 / 3) and abs(early - late) < 0.3
    a, b = q[:-1].ravel(), q[1:].ravel()
    corr = np.corrcoef(a, b)[0, 1]
    assert abs(corr - wl.rho) < 0.05
