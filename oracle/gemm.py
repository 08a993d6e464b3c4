"""Grouped GEMMs with dequantization (oracle; test infrastructure only).

Common grouped structure (CUTLASS discussion #2855's per-expert problem list;
tilelang_kernels.py's per-expert F.linear): sorted position s in
[0, offsets[E]) belongs to the expert e with offsets[e] <= s < offsets[e+1];
its output row is y[s, :] = (row of A) . W[e]^T with W stored [N][K]
(K contiguous).  The row of A is
  * 'token':  A[sorted_pair_ids[s] // topk]  (each token's row feeds its k
    experts; megamoe_rm.cu gathers x by token = pair / topk), or
  * 'sorted': A[s]  (A already in sorted order, as in CUTLASS discussion
    #2855 where the input arrives permuted, and for the second GEMM).
With sorted_pair_ids None the rows are the identity ('sorted').

All arithmetic is exact or float64: the integer contraction is an fp64 BLAS
product of integer values (every partial sum is an integer below 2^53, so
exact), the floating contractions are float64 products of exactly decoded
values.  `rows` restricts the computation to a subset of sorted positions
(for sampled checks of large problems); the result then has len(rows) rows.
`cols` likewise restricts it to a subset of output columns: the weight rows
those columns need are selected before the contraction (with act 'silu_mul',
output column j takes weight rows j and I + j), and the result has
len(cols) columns.  Neither changes any arithmetic.
"""
from __future__ import annotations

import numpy as np

from .formats import (unpack_nibbles, int4_value, e4m3fn_value, e2m1_value, ue4m3_value,
                      bf16_value, f16_value)


def gemm_rows(offsets, sorted_pair_ids, topk: int, a_row: str, rows=None):
    """(s, e, r): sorted positions, their experts and their A rows."""
    offsets = np.asarray(offsets, np.int64)
    n = int(offsets[-1])
    s = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    if s.size and (s.min() < 0 or s.max() >= n):
        raise ValueError("row outside [0, offsets[E])")
    e = np.searchsorted(offsets, s, side="right") - 1
    if sorted_pair_ids is None or a_row == "sorted":
        r = s
    elif a_row == "token":
        p = np.asarray(sorted_pair_ids, np.int64)[s]
        assert np.all(p >= 0)
        r = p // topk
    else:
        raise ValueError(a_row)
    return s, e, r


def weight_rows(N: int, act: str, cols):
    """Weight rows (output channels of the GEMM) that the output columns
    `cols` depend on, in the order the contraction returns them: all N when
    cols is None; cols itself for act 'none'; for 'silu_mul' the gate rows
    cols followed by the up rows I + cols, so that silu_mul's halves line up."""
    if cols is None:
        return np.arange(N)
    c = np.asarray(cols, np.int64)
    lim = N // 2 if act == "silu_mul" else N
    if c.size and (c.min() < 0 or c.max() >= lim):
        raise ValueError("column outside the output")
    return np.concatenate([c, N // 2 + c]) if act == "silu_mul" else c


def silu_mul(y: np.ndarray, limit=None) -> np.ndarray:
    """SiLU-gated product over the two halves of y [n][2I]: columns [0, I) are
    the gate g, columns [I, 2I) the up projection u; h = g / (1 + exp(-g)) * u.
    (The SiLU(gate)*up between the two GEMMs of an NVFP4 / Mixtral-style MoE
    layer.)

    limit: the clamped variant of megamoe_rm.cu's fc1_rm epilogue (the GLM
    SwiGLU), applied to the already scaled GEMM outputs before the product:
    the gate is bounded above only, g <- min(g, limit); the up projection is
    bounded on both sides, u <- min(max(u, -limit), limit).  None: no clamp."""
    I = y.shape[1] // 2
    g, u = y[:, :I], y[:, I:]
    if limit is not None:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    return g / (1.0 + np.exp(-g)) * u


def grouped_gemm_qint4(a, a_scale, a_row, w, w_scale, offsets, sorted_pair_ids, topk,
                       act="none", rows=None, cols=None):
    """W4A4 INT4 grouped GEMM with the per-token x per-channel epilogue.

    CUTLASS discussion #2855 (problem statement): activations quantized per
    token, weights per output channel, int32 accumulator, output
    scale_act * scale_weight * accumulator.
      acc[s, n] = sum_k int4(A[r, k]) * int4(W[e, n, k])
      y[s, n]   = a_scale[r] * w_scale[e, n] * acc[s, n]
    a [rows_a][K/2] bytes, a_scale [rows_a] f32, w [E][N][K/2] bytes,
    w_scale [E][N] f32.  act 'silu_mul' returns silu_mul(y).
    Returns dict(acc=int64 [n][N], y=float64 [n][N or N/2]) (with cols:
    acc over the selected weight rows, see weight_rows)."""
    s, e, r = gemm_rows(offsets, sorted_pair_ids, topk, a_row, rows)
    wr = weight_rows(w.shape[1], act, cols)
    A = int4_value(unpack_nibbles(np.asarray(a)[r])).astype(np.float64)
    acc = np.zeros((s.size, wr.size), np.float64)
    for ex in np.unique(e):
        m = e == ex
        W = int4_value(unpack_nibbles(np.asarray(w)[ex][wr])).astype(np.float64)
        acc[m] = A[m] @ W.T
    assert np.all(np.abs(acc) < 2.0 ** 31), "int32 accumulator would overflow"
    sa = np.asarray(a_scale, np.float64)[r]
    sw = np.asarray(w_scale, np.float64)[e][:, wr]
    y = sa[:, None] * sw * acc
    if act == "silu_mul":
        y = silu_mul(y)
    return dict(acc=acc.astype(np.int64), y=y)


def grouped_gemm_qfp8_block(a, a_scale, a_row, w, w_scale, offsets, sorted_pair_ids, topk,
                            rows=None, cols=None):
    """FP8 e4m3 block-scaled grouped GEMM (CUTLASS issue #2087).

    A is quantized per token per 128 columns of K: a_scale [K/128][rows_a]
    (M contiguous, the layout the issue's answer recommends so that A-scale
    loads coalesce).  W[e] is quantized per 128x128 block:
    w_scale [E][N/128][K/128].  The result is the matmul of the dequantized
    operands:
      y[s, n] = sum_k (a_scale[k//128, r] * e4m3(A[r, k]))
                    * (w_scale[e, n//128, k//128] * e4m3(W[e, n, k]))
    Returns dict(y=float64 [n][N])."""
    s, e, r = gemm_rows(offsets, sorted_pair_ids, topk, a_row, rows)
    wr = weight_rows(w.shape[1], "none", cols)
    sa = np.asarray(a_scale, np.float64)[:, r].T              # [n][K/128]
    Ad = e4m3fn_value(np.asarray(a)[r]) * np.repeat(sa, 128, axis=1)
    y = np.zeros((s.size, wr.size), np.float64)
    for ex in np.unique(e):
        m = e == ex
        sb = np.asarray(w_scale, np.float64)[ex][wr // 128]   # [n_cols][K/128]: block row of each column
        Wd = e4m3fn_value(np.asarray(w)[ex][wr]) * np.repeat(sb, 128, axis=1)
        y[m] = Ad[m] @ Wd.T
    return dict(y=y)


def grouped_gemm_qnvfp4(x, a_row, w, w_sf, w_gscale, offsets, sorted_pair_ids, topk,
                        act="none", rows=None, limit=None, x_dtype="bf16", sf_layout="rows",
                        w_layout="rows", cols=None):
    """NVFP4 W4A16 grouped GEMM (tilelang_kernels.py grouped_gemm_fp4, with the
    per-expert global scale of megamoe_rm.cu).

    x [rows_a][K] bf16 bits (x_dtype 'bf16') or IEEE binary16 bits ('f16',
    megamoe_rm.cu's fp16 activations); w [E][N][K/2] E2M1 codes packed two per byte;
    w_sf in sf_layout 'rows' ([E][N][K/16]) or 'quads' ([E][K/64][N][4]), w in
    w_layout 'rows' or 'tiled' ([E][N/16][K/64][16][32]; see oracle.layouts);
    w_sf [E][N][K/16] UE4M3 per-16 block scales; w_gscale [E] f32.
      Wd[e, n, k] = e2m1(W[e, n, k]) * ue4m3(w_sf[e, n, k // 16])
      y[s, n]     = w_gscale[e] * sum_k x[r, k] * Wd[e, n, k]
    With w_gscale = 1 this is tilelang_kernels.py's dequantize-then-linear.
    act 'silu_mul' returns silu_mul(y, limit) (megamoe_rm.cu applies the
    global scale, then the clamp, then the product).  Returns dict(y=float64)."""
    s, e, r = gemm_rows(offsets, sorted_pair_ids, topk, a_row, rows)
    if x_dtype not in ("bf16", "f16"):
        raise ValueError(x_dtype)
    if sf_layout == "quads":                       # [E][K/64][N][4] -> [E][N][K/16]
        from .layouts import rows_from_quads
        w_sf = rows_from_quads(np.asarray(w_sf))
    elif sf_layout != "rows":
        raise ValueError(sf_layout)
    if w_layout == "tiled":                        # [E][N/16][K/64][16][32] -> [E][N][K/2]
        from .layouts import rows_from_tiles
        w = rows_from_tiles(np.asarray(w))
    elif w_layout != "rows":
        raise ValueError(w_layout)
    wr = weight_rows(w.shape[1], act, cols)
    X = (bf16_value if x_dtype == "bf16" else f16_value)(np.asarray(x)[r])
    y = np.zeros((s.size, wr.size), np.float64)
    for ex in np.unique(e):
        m = e == ex
        codes = e2m1_value(unpack_nibbles(np.asarray(w)[ex][wr]))         # [n_w][K]
        sc = ue4m3_value(np.asarray(w_sf)[ex][wr])                          # [n_w][K/16]
        Wd = (codes.reshape(sc.shape + (16,)) * sc[:, :, None]).reshape(codes.shape)
        y[m] = float(np.asarray(w_gscale)[ex]) * (X[m] @ Wd.T)
    if act == "silu_mul":
        y = silu_mul(y, limit)
    elif limit is not None:
        raise ValueError("limit applies to act 'silu_mul' only")
    return dict(y=y)
