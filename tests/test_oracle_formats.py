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


def test_656_byte_entry_decodes_by_hand():
    # One entry built by hand: c_KV block 0 holds 1.0 (0x38) and -448 (0xFE)
    # at scale 2^-3; block 1 the smallest subnormal 2^-9 (0x01) at scale 1;
    # block 2 the value 3.5 (0x46: 1.75 * 2) at scale 16; block 3 zeros at
    # scale 2^-9; k_R: bf16 1.5 (0x3FC0) and -0.25 (0xBE80).
    from oracle.formats import decode_entries
    e = np.zeros((1, 656), np.uint8)
    e[0, 0], e[0, 1] = 0x38, 0xFE
    e[0, 128] = 0x01
    e[0, 256] = 0x46
    e[0, 512:528] = np.array([2.0 ** -3, 1.0, 16.0, 2.0 ** -9], np.float32).view(np.uint8)
    kr = np.zeros(64, np.uint16)
    kr[0], kr[63] = 0x3FC0, 0xBE80
    e[0, 528:] = kr.view(np.uint8)
    v = decode_entries(e)[0]
    assert v[0] == 0.125 and v[1] == -56.0
    assert v[128] == 2.0 ** -9 and v[256] == 56.0
    assert v[512] == 1.5 and v[575] == -0.25
    assert np.count_nonzero(v) == 6


def test_656_byte_entries_round_trip_the_generator():
    # The generator's entries: per block a power-of-two scale, every c_KV
    # value within half an fp8 step of the bf16 latent (relative 2^-4 for
    # normal codes, 2^-10 * scale absolute for subnormal ones), k_R exact,
    # and every decoded value exactly a bf16 value.
    from oracle.formats import decode_entries
    from synth.gen import encode_entries
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((200, 576)) * 0.5).astype(np.float32)
    x[7, :128] = 0.0                                   # an all-zero block
    rows = gen.f32_to_bf16_bits(x)
    ent = encode_entries(rows)
    got = decode_entries(ent)
    ref = decode_bf16(rows)
    scale = np.ascontiguousarray(ent[:, 512:528]).view(np.float32).astype(np.float64)
    m, ex = np.frexp(scale)
    assert np.all(m == 0.5)                            # powers of two
    s = np.repeat(scale, 128, axis=1)
    err = np.abs(got[:, :512] - ref[:, :512])
    assert np.all(err <= np.maximum(np.abs(ref[:, :512]) * 2.0 ** -4, s * 2.0 ** -10))
    assert np.array_equal(got[:, 512:], ref[:, 512:])
    assert np.array_equal(decode_bf16(gen.f32_to_bf16_bits(got.astype(np.float32))), got)
    assert np.all(got[7, :128] == 0.0)


def test_oracle_entry_encoder_by_hand():
    # Block 0: 1.0 and 448 (scale 1), the midpoint 1.0625 of codes 0x38 and
    # 0x39 (tie -> even 0x38), 1.1875 between 0x39 and 0x3A (tie -> 0x3A),
    # -0 -> +0; block 1: max 450 needs scale 2 (450 / 2 = 225 -> 224, 0x76);
    # block 2 all zero: scale 1; block 3: max 0.5 -> scale 2^-9 (0.5 / 2^-9
    # = 256 -> 0x78).
    from oracle.formats import decode_entries, encode_entries
    x = np.zeros(576, np.float32)
    x[0], x[1], x[2], x[3], x[4] = 1.0, 448.0, 1.0625, 1.1875, -0.0
    x[128] = 450.0
    x[384] = 0.5
    x[512], x[575] = 1.5, -3.0
    e = encode_entries(gen.f32_to_bf16_bits(x)[None])[0]
    assert e[:5].tolist() == [0x38, 0x7E, 0x38, 0x3A, 0x00]
    assert e[128] == 0x76
    assert e[384] == 0x78
    sc = e[512:528].view(np.float32).tolist()
    assert sc == [1.0, 2.0, 1.0, 2.0 ** -9]
    d = decode_entries(e[None])[0]
    assert d[1] == 448.0 and d[128] == 448.0 and d[384] == 0.5
    assert d[512] == 1.5 and d[575] == -3.0


def test_oracle_entry_encoder_agrees_with_the_generator():
    # Two separate implementations of the same quantization (the generator's
    # vectorised one and the oracle's brute-force one) agree bit for bit.
    from oracle.formats import encode_entries
    rng = np.random.default_rng(11)
    x = rng.standard_normal((24, 576)).astype(np.float32) * rng.choice([1e-3, 0.5, 30.0], (24, 1)).astype(np.float32)
    x[3, 128:256] = 0.0
    rows = gen.f32_to_bf16_bits(x)
    assert np.array_equal(encode_entries(rows), gen.encode_entries(rows))
