"""Pins for the oracle's per-row INT4 quantizer: a hand-worked row, the
rounding and range invariants of the rule, exactness of the fp32 steps
against Python's own float arithmetic, and the packing against the INT4
unpacker."""
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def test_hand_worked_row():
    # amax = 3.5 -> s = 0.5, 7/amax = 2: codes are rne(2x)
    x = np.array([[3.5, -3.5, 1.25, -0.25, 0.75, 0.0, 2.25, -1.0]], np.float32)
    q, s = oracle.quantize_int4_rows(x)
    assert s[0] == np.float32(0.5)
    codes = oracle.int4_value(oracle.unpack_nibbles(q))[0]
    # 2x = 7, -7, 2.5, -0.5, 1.5, 0, 4.5, -2 -> half to even: 2, -0, 2, 4
    assert list(codes) == [7, -7, 2, 0, 2, 0, 4, -2]
    # packing: element 0 in the low nibble of byte 0
    assert q[0, 0] == (7 | ((-7 & 15) << 4))


def test_python_float_arithmetic_agrees():
    # the same steps done with Python floats rounded to fp32 one by one
    rng = np.random.default_rng(3)
    x = synth.uniform_f32(rng, (5, 64), -3.0, 3.0)
    q, s = oracle.quantize_int4_rows(x)
    codes = oracle.int4_value(oracle.unpack_nibbles(q))
    for r in range(5):
        amax = max(abs(float(v)) for v in x[r])
        assert s[r] == np.float32(f32(amax / 7.0))
        rec = f32(7.0 / amax)
        for k in range(64):
            t = f32(float(x[r, k]) * rec)
            # Python's round() is half to even
            assert codes[r, k] == max(-8, min(7, round(t)))


def test_invariants():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    q, s = oracle.quantize_int4_rows(x)
    codes = oracle.int4_value(oracle.unpack_nibbles(q)).astype(np.float64)
    # every row reaches +-7 at its amax element and never -8
    assert np.all(np.max(np.abs(codes), axis=1) == 7)
    assert codes.min() >= -7
    # dequantized error within half a step, up to the fp32 rounding of the rule
    err = np.abs(codes * s[:, None].astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # scaling a row by a power of two scales s exactly and keeps the codes
    q2, s2 = oracle.quantize_int4_rows(x * np.float32(8))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8))


def test_zero_and_tiny_rows():
    x = np.zeros((3, 32), np.float32)
    x[1, 5] = 2.0 ** -130
    x[2, :] = -1.0
    q, s = oracle.quantize_int4_rows(x)
    assert np.all(q[:2] == 0) and s[0] == 1 and s[1] == 1
    assert np.all(oracle.int4_value(oracle.unpack_nibbles(q[2:])) == -7)
    assert s[2] == np.float32(1 / 7)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_input_dtype_is_read_exactly(dtype):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128)).astype(dtype)
    qa, sa = oracle.quantize_int4_rows(x)
    qb, sb = oracle.quantize_int4_rows(x.astype(np.float64))
    assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


# Rows on which the two readings of the rule differ: codes from the
# reciprocal, rne(fl32(x * fl32(7 / amax))) (the reading taken), against the
# quotient, rne(fl32(x / fl32(amax / 7))).  Each row is [amax, x] as fp32
# bits; the last two fields are the code of x under each reading.
SEPARATING = [
    (0x4012A5E6, 0x3F92A5E6, 3, 4),    # x = amax / 2: exactly 3.5 in the reals
    (0x3F809561, 0x3F6ECC47, 7, 6),
    (0x401B1BE7, 0xBF04F358, -2, -1),
    (0x3F18B166, 0x3EEFF232, 5, 6),
    (0x3FD3B845, 0xBDF1F72B, 0, -1),
    (0x3F9B25E0, 0x3DB14FDC, 0, 1),
]


def _fp32_from_bits(b):
    return struct.unpack("<f", struct.pack("<I", b))[0]


def _nearest_fp32(q):
    """Correctly rounded fp32 value (ties to even) of a nonzero rational q in
    the normal range, from the definition: q / 2^(e-23) rounded to an
    integer, e = floor(log2 |q|)."""
    from fractions import Fraction
    s, q = (-1, -q) if q < 0 else (1, q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    quantum = Fraction(2) ** (e - 23)
    n = q / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * quantum


def _rne_int(q):
    from fractions import Fraction
    fl = q.numerator // q.denominator
    rem = q - fl
    return fl + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1) else fl


@pytest.mark.parametrize("amax_bits,x_bits,code_recip,code_quot", SEPARATING)
def test_reading_separates_reciprocal_from_quotient(amax_bits, x_bits, code_recip, code_quot):
    from fractions import Fraction
    amax, x = Fraction(_fp32_from_bits(amax_bits)), Fraction(_fp32_from_bits(x_bits))
    # both readings in exact rational arithmetic with explicit fp32 roundings
    recip = _nearest_fp32(Fraction(7) / amax)
    t_recip = _nearest_fp32(x * recip) if x else Fraction(0)
    s = _nearest_fp32(amax / 7)
    t_quot = _nearest_fp32(x / s) if x else Fraction(0)
    assert _rne_int(t_recip) == code_recip and _rne_int(t_quot) == code_quot
    assert code_recip != code_quot
    # the oracle follows the reciprocal reading, and its scale is fl32(amax/7)
    row = np.array([[_fp32_from_bits(amax_bits), _fp32_from_bits(x_bits)]], np.float32)
    q, sc = oracle.quantize_int4_rows(row)
    codes = oracle.int4_value(oracle.unpack_nibbles(q))[0]
    assert codes[0] == 7 and codes[1] == code_recip
    assert Fraction(float(sc[0])) == s
