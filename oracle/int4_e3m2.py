"""INT4 values stored as FP6 E3M2 codes (oracle; test infrastructure only).

The INT4 grouped GEMM's operands are int4 values in [-8, 7] (CUTLASS
discussion #2855, "How to implement dequantization of row and column
broadcast in Epilogue of GroupGemm": W4A4, int32 accumulation).  Besides
the packed two-per-byte layout, the library reads the same values stored as
6-bit FP6 E3M2 codes, each code exactly the value (every integer of
magnitude up to 8 is an E3M2 number), laid out as the operands of a 32 x 64
block-scaled MFMA step.

E3M2 (the 6-bit float of the OCP microscaling formats): sign bit 5,
exponent bits 4:2 with bias 3, mantissa bits 1:0; exponent 0 is subnormal,
(m / 4) * 2^-2; otherwise 2^(e - 3) * (1 + m / 4).  No infinities or NaNs.

Row layout ("e3m2 rows"): a row of K values (K % 64 == 0) is K/64 blocks of
48 bytes.  Block b holds values k = 64 b + 32 h + i (half h in {0, 1}, i in
[0, 32)).  The 32 codes c_i of half h form the 192-bit number
S_h = sum_i c_i * 2^(6 i), cut into six 32-bit words D_h[0..5]
(D_h[j] = bits 32 j .. 32 j + 31 of S_h).  The block's twelve little-endian
words are, in order,
    D_0[0..3], D_1[0..3], D_0[4..5], D_1[4..5].
"""
from __future__ import annotations

import numpy as np

from .formats import unpack_nibbles, int4_value


def e3m2_value(codes) -> np.ndarray:
    """FP6 E3M2 code (0..63) -> float64, the closed form above."""
    c = np.asarray(codes).astype(np.int64)
    if c.size and (c.min() < 0 or c.max() > 63):
        raise ValueError("E3M2 codes are 6-bit")
    s = (c >> 5) & 1
    e = (c >> 2) & 7
    m = (c & 3).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 4.0, -2), np.ldexp(1.0 + m / 4.0, (e - 3).astype(np.int32)))
    return np.where(s == 1, -mag, mag)


# The code whose value is v, for v in [-8, 8]: found by decoding all 64 codes
# (+0 for zero).  Every such integer has exactly one code (two for 0).
_ALL = e3m2_value(np.arange(64))
_CODE_OF = {}
for _c in range(63, -1, -1):                 # descending: +0 (code 0) wins over -0
    _v = float(_ALL[_c])
    if _v == int(_v) and -8 <= _v <= 8:
        _CODE_OF[int(_v)] = _c
assert sorted(_CODE_OF) == list(range(-8, 9))


def e3m2_code_of_int(v) -> np.ndarray:
    """Exact E3M2 code of each integer of v (each in [-8, 8])."""
    v = np.asarray(v, np.int64)
    table = np.array([_CODE_OF[i] for i in range(-8, 9)], np.int64)
    if v.size and (v.min() < -8 or v.max() > 8):
        raise ValueError("value outside [-8, 8]")
    return table[v + 8]


def _block_words(codes_block: np.ndarray) -> list:
    """Twelve 32-bit words of one block from its 64 codes (Python integers)."""
    words = {}
    for h in range(2):
        S = 0
        for i in range(32):
            S |= int(codes_block[32 * h + i]) << (6 * i)
        words[h] = [(S >> (32 * j)) & 0xFFFFFFFF for j in range(6)]
    return words[0][:4] + words[1][:4] + words[0][4:] + words[1][4:]


def int4_to_e3m2_rows(packed) -> np.ndarray:
    """Packed int4 rows [..., K/2] (two's complement, element 2b in the low
    nibble of byte b) -> e3m2 rows [..., 3K/4] bytes in the layout above."""
    packed = np.asarray(packed, np.uint8)
    vals = int4_value(unpack_nibbles(packed))             # [..., K]
    K = vals.shape[-1]
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    codes = e3m2_code_of_int(vals).reshape(-1, K)
    out = np.zeros((codes.shape[0], K // 64 * 12), np.uint32)
    for r in range(codes.shape[0]):
        for b in range(K // 64):
            out[r, 12 * b:12 * b + 12] = _block_words(codes[r, 64 * b:64 * b + 64])
    return out.astype("<u4").view(np.uint8).reshape(packed.shape[:-1] + (3 * K // 4,))


def e3m2_rows_values(rows) -> np.ndarray:
    """e3m2 rows [..., 3K/4] bytes -> their values [..., K] as float64
    (each code decoded by e3m2_value, placed by the layout above)."""
    rows = np.asarray(rows, np.uint8)
    nb = rows.shape[-1] // 48
    w = rows.reshape(-1, nb, 48).copy().view("<u4").astype(np.uint64)      # [R][nb][12]
    out = np.zeros((w.shape[0], nb, 64), np.float64)
    for h in range(2):
        D = [w[:, :, 4 * h + j] for j in range(4)] + [w[:, :, 8 + 2 * h + j] for j in range(2)]
        for i in range(32):
            bit = 6 * i
            j, o = bit // 32, bit % 32
            c = D[j] >> np.uint64(o)
            if o > 26:
                c = c | (D[j + 1] << np.uint64(32 - o))
            out[:, :, 32 * h + i] = e3m2_value((c & np.uint64(63)).astype(np.int64))
    return out.reshape(rows.shape[:-1] + (64 * nb,))
