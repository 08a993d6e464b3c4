"""Pins for the oracle's codecs against library routines and worked examples."""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def _e2m1_as_e4m3_code(c):
    # Re-encode an E2M1 code as the e4m3 code of the same value (both are
    # sign/exponent/mantissa formats; E2M1 bias 1, e4m3 bias 7), so that
    # torch's e4m3 decoder can check the E2M1 decoder.
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if e == 0 and m == 0:
        return s << 7
    if e == 0:                                    # 0.5 = 2^-1
        return (s << 7) | (6 << 3)
    return (s << 7) | ((e + 6) << 3) | (m << 2)


def test_e2m1_all_codes_match_torch_via_e4m3():
    codes = np.arange(16)
    e4 = np.array([_e2m1_as_e4m3_code(int(c)) for c in codes], dtype=np.uint8)
    ref = torch.from_numpy(e4).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e2m1_value(codes)
    assert np.array_equal(got, ref)
    assert sorted(set(np.abs(got))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_int4_matches_int8_arithmetic_shift():
    codes = np.arange(16, dtype=np.uint8)
    ref = ((codes << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int64)
    assert np.array_equal(oracle.int4_value(codes), ref)
    assert oracle.int4_value(np.array([7, 8, 15])).tolist() == [7, -8, -1]


def test_nibble_order_worked_example():
    # Reading: element 2b is the low nibble of byte b.
    got = oracle.unpack_nibbles(np.array([[0x21, 0xF8]], dtype=np.uint8))
    assert got.tolist() == [[1, 2, 8, 15]]
    assert oracle.int4_value(got).tolist() == [[1, 2, -8, -1]]


def test_ue4m3_rejects_sign_and_nan():
    assert oracle.ue4m3_value(np.array([0x30, 0x47])).tolist() == [0.5, 3.75]
    with pytest.raises(ValueError):
        oracle.ue4m3_value(np.array([0xB0]))
    with pytest.raises(ValueError):
        oracle.ue4m3_value(np.array([0x7F]))


def test_e2m1_times_ue4m3_exact_in_bf16_and_f16():
    # Every weight x block-scale product is a bf16 and an fp16 value, so a
    # kernel may dequantize into either type without rounding.
    v = oracle.e2m1_value(np.arange(16))[:, None] * oracle.ue4m3_value(np.arange(127))[None, :]
    t = torch.from_numpy(v)
    assert torch.equal(t.to(torch.bfloat16).to(torch.float64), t)
    assert torch.equal(t.to(torch.float16).to(torch.float64), t)


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, 5000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_value(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def _ties_and_randoms(rng):
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(3.0) ** rng.integers(-30, 30, 20000)
    # exact halfway points between neighbouring bf16 values, and near the
    # largest finite values
    b = rng.integers(0, 2 ** 15, 4000).astype(np.uint32) << 16
    half = (b | 0x8000).view(np.float32)
    big = np.array([3.3895e38, 3.39e38, -3.3895e38, 65504.0, 65520.0, 1e-40, -1e-42],
                   np.float32)
    return np.concatenate([x, half, big])


def test_round_to_bf16_matches_torch_from_f32():
    x = _ties_and_randoms(np.random.default_rng(1))
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_to_bf16_rounds_once_from_f64():
    # values off the fp32 grid, where rounding to fp32 first (to a tie) and
    # then to bf16 would land on the other neighbour; expected values from
    # the definition of nearest-even on the bf16 grid (8 significant bits)
    cases = [
        (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7),   # above the midpoint: up
        (1 + 2.0 ** -8 - 2.0 ** -30, 1.0),              # below it: down
        (1 + 2.0 ** -8, 1.0),                           # the tie: even (1.0)
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),             # tie between odd and even: even
        (-(3 + 2.0 ** -7 + 2.0 ** -40), -(3 + 2.0 ** -6)),
        (2.0 ** -134 * (1 + 2.0 ** -40), 2.0 ** -133),  # subnormal grid, just above half
        (2.0 ** -134, 0.0),                             # subnormal tie: even (zero)
        # the largest bf16, (2 - 2^-7) 2^127, has spacing 2^120 above it
        ((2 - 2.0 ** -7) * 2.0 ** 127 + 2.0 ** 119 - 2.0 ** 90, (2 - 2.0 ** -7) * 2.0 ** 127),
        ((2 - 2.0 ** -7) * 2.0 ** 127 + 2.0 ** 119, np.inf),   # tie at the top: even is 2^128
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    assert np.array_equal(oracle.round_to_bf16(x), want)


def test_round_to_f16_matches_torch_from_f32():
    x = _ties_and_randoms(np.random.default_rng(2))
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    got = oracle.round_to_f16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_f16_value_known_patterns():
    bits = np.array([0x0000, 0x3C00, 0xC000, 0x7BFF, 0x0001, 0x0400, 0x3555, 0x7C00], np.uint16)
    v = oracle.f16_value(bits)
    assert list(v[:7]) == [0.0, 1.0, -2.0, 65504.0, 2.0 ** -24, 2.0 ** -14, 0.25 * (1 + 341 / 1024)]
    assert np.isposinf(v[7])
    assert np.array_equal(oracle.f16_bits(v[:7]), bits[:7])


def test_bf16_to_f16_exact_in_range_and_matches_torch_everywhere():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f16_bits(bits)
    # every bf16 value of magnitude in [2^-14, 65504] converts exactly
    v = oracle.bf16_value(bits)
    m = np.isfinite(v) & (np.abs(v) >= 2.0 ** -14) & (np.abs(v) <= 65504)
    assert np.array_equal(oracle.f16_value(got[m]), v[m])
    # overflow and the largest finite boundary
    assert oracle.bf16_to_f16_bits(np.array([0x4780], np.uint16))[0] == 0x7C00     # 65536 -> inf
    assert oracle.bf16_to_f16_bits(np.array([0x477F], np.uint16))[0] == 0x7BF8     # 65280, exact
    # all 65536 patterns against torch's own bf16 -> f16 conversion (NaNs: both NaN)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float16)
    ref = t.view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.f16_value(got[nan])))
