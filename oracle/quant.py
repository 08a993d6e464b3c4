"""Per-row symmetric INT4 activation quantizer (oracle; test infrastructure only).

CUTLASS discussion #2855 states that the W4A4 activations start as fp16 and
are quantized per token to int4, their scale applied with the weight scale
in the epilogue.  The page gives no rounding rule; the reading taken here is
the symmetric one: for a row x,

    amax = max |x|,  s = amax / 7,  q = clamp(rne(x * (7 / amax)), -8, 7)

with s and 7/amax each one correctly rounded fp32 division and the product
x * (7/amax) one fp32 multiplication, because the fp32 result decides the
integer code and the kernel computes it exactly so.  Rows whose amax is
below 2^-120 (including all-zero rows) quantize to zeros with scale 1.
Codes are packed two per byte, element 2b in the low nibble of byte b.
"""
from __future__ import annotations

import numpy as np

TINY = np.float32(2.0 ** -120)


def quantize_int4_rows(x: np.ndarray):
    """x [rows][K] (any float dtype, values taken as fp32) ->
    (packed uint8 [rows][K/2], scale float32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    amax = np.max(np.abs(x), axis=1) if K else np.zeros(rows, np.float32)
    amax = amax.astype(np.float32)
    tiny = amax < TINY
    safe = np.where(tiny, np.float32(1), amax).astype(np.float32)
    scale = np.where(tiny, np.float32(1), safe / np.float32(7)).astype(np.float32)
    recip = np.where(tiny, np.float32(0), np.float32(7) / safe).astype(np.float32)
    t = (x * recip[:, None]).astype(np.float32)          # one fp32 product
    q = np.clip(np.rint(t), -8, 7).astype(np.int64)      # round half to even
    codes = (q & 15).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale
