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
