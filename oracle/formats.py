"""Codecs of the low-precision formats (oracle; test infrastructure only).

Each decoder is the closed form of the format, applied to integer codes.
"""
from __future__ import annotations

import numpy as np


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes.

    Element 2b sits in the low nibble of byte b and element 2b+1 in the high
    nibble.  The pages do not state the nibble order for INT4 (CUTLASS
    discussion #2855 only says K/2 bytes per row) nor for E2M1
    (tilelang_kernels.py stores (E, N, K//2)); megamoe_rm.cu's chunk_mma
    feeds the first byte of a row to k+0..1, which this reading follows."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


# Each decoder below is a pure function of its code.  The closed form is
# evaluated once over the format's whole code alphabet and each code then
# looks its value up: the same values as evaluating it per element, without
# a large array's worth of temporaries (a code outside the alphabet raises
# IndexError).


def _int4_closed_form(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    return c - 16 * (c >= 8)


def _e2m1_closed_form(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int32)))
    return np.where(s == 1, -mag, mag)


def _e4m3fn_closed_form(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((e == 15) & (b & 7 == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_INT4 = _int4_closed_form(np.arange(16))
_E2M1 = _e2m1_closed_form(np.arange(16))
_E4M3FN = _e4m3fn_closed_form(np.arange(256))


def _codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes)
    if c.dtype.kind not in "iu":
        raise TypeError("codes must be integers")
    if c.size and c.min() < 0:
        raise IndexError("negative code")
    return c


def int4_value(codes: np.ndarray) -> np.ndarray:
    """Two's-complement 4-bit integer: code c in [0,15] -> c - 16*[c >= 8],
    range [-8, 7] (W4A4 INT4 of CUTLASS discussion #2855).  int64."""
    return _INT4[_codes(codes)]


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.
    exponent 0 is subnormal: m/2; otherwise 2^(e-1) * (1 + m/2).
    (The NVFP4 element format of tilelang_kernels.py and megamoe_rm.cu.)"""
    return _E2M1[_codes(codes)]


def e4m3fn_value(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 e4m3fn: sign bit 7, exponent bits 6:3 (bias 7), mantissa 2:0.
    exponent 0 is subnormal: 2^-6 * m/8; exponent 15 with mantissa 7 is NaN
    (no infinities); otherwise 2^(e-7) * (1 + m/8).  Largest finite 448.
    (cutlass::float_e4m3_t of CUTLASS issue #2087; float8_e4m3fn of
    tilelang_kernels.py.)"""
    return _E4M3FN[_codes(codes)]


def ue4m3_value(codes: np.ndarray) -> np.ndarray:
    """Unsigned e4m3 block scale (NVFP4 per-16 scale): e4m3fn with the sign bit
    clear.  A sign-set or NaN byte is not a valid scale; the oracle rejects it."""
    b = np.asarray(codes).astype(np.int64)
    if np.any(b & 0x80) or np.any(b == 0x7F):
        raise ValueError("UE4M3 scale byte with sign bit set or NaN encoding")
    return e4m3fn_value(b)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_value(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary16 bits, rounded once to nearest even (overflow
    to +-inf, gradual underflow), as numpy's double->half conversion does."""
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def bf16_to_f16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> binary16 bits of the nearest binary16 value (ties to
    even).  Exact for every bf16 value of magnitude in [2^-14, 65504]: bf16
    carries 8 significant bits and binary16 11.  Used when bf16 activations
    are handed to the fp16 form of the NVFP4 GEMM (megamoe_rm.cu converts its
    bf16 input to fp16 in route_prep the same way)."""
    return f16_bits(bf16_value(bits))


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest IEEE binary16 (ties to even); returned as
    float64.  numpy's double->half conversion rounds once, to nearest even."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 (8 significant bits, exponent range
    of float32; ties to even; overflow to +-inf); returned as float64.  Rounds
    once, directly from float64."""
    x = np.asarray(x, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)
        e = np.maximum(e, -125)                      # below 2^-126: fixed quantum 2^-133
        q = np.ldexp(1.0, (e - 8).astype(np.int32))  # spacing of bf16 values near x
        r = np.rint(x / q) * q                       # np.rint rounds half to even
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
        return np.where(np.isfinite(x), r, x)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits (rounded as round_to_bf16)."""
    r = round_to_bf16(x).astype(np.float32)         # exact: r is a bf16 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to an output dtype name: 'f16', 'bf16', 'f32' (values as float64)."""
    if dtype == "f16":
        return round_to_f16(x)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)
