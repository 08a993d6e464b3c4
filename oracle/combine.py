"""Top-k weighted scatter back to tokens (oracle; test infrastructure only)."""
from __future__ import annotations

import numpy as np


def scatter_combine(y: np.ndarray, pair_to_sorted: np.ndarray, topk_weights: np.ndarray):
    """out[t, :] = sum over slots j with a routed pair of w[t, j] * y[pair_to_sorted[t*k+j], :]

    y holds the expert outputs in sorted order (values as stored by the
    grouped GEMM).  A pair without an expert (pair_to_sorted -1) contributes
    nothing; a token with no routed pair gets a zero row.  The output starts
    from zeros and receives each weighted expert row
    (tilelang_kernels.py: zero output, then output[tokens] += result * weight;
    megamoe_rm.cu's combine sums a token's pairs that have an expert).
    Summed in float64.  Returns float64 [T][N]."""
    w = np.asarray(topk_weights, np.float64)
    T, k = w.shape
    p2s = np.asarray(pair_to_sorted).reshape(T, k)
    y = np.asarray(y, np.float64)
    out = np.zeros((T, y.shape[1]), np.float64)
    for j in range(k):
        v = p2s[:, j] >= 0
        out[v] += w[v, j, None] * y[p2s[v, j]]
    return out


def pair_rows(y: np.ndarray, sorted_pair_ids: np.ndarray, topk_weights: np.ndarray):
    """megamoe_rm.cu's fc2_rm epilogue: each expert row, scaled by its pair's
    top-k weight, lands in its pair's row (pair id t*topk + j) rather than
    its sorted row.

    y [n][N] expert outputs in sorted order, n = offsets[E] (values as the
    GEMM computes them, before any output rounding); sorted_pair_ids the
    route table.  Returns (ypart float64 [T*topk][N], valid bool [T*topk]):
    ypart[p] = w[p] * y[s] for the sorted row s of pair p; rows of pairs
    without an expert are zero and not valid."""
    w = np.asarray(topk_weights, np.float64).reshape(-1)
    y = np.asarray(y, np.float64)
    n = y.shape[0]
    p = np.asarray(sorted_pair_ids, np.int64)[:n]
    ypart = np.zeros((w.size, y.shape[1]), np.float64)
    valid = np.zeros(w.size, bool)
    ypart[p] = w[p, None] * y
    valid[p] = True
    return ypart, valid


def sum_pairs(ypart: np.ndarray, pair_to_sorted: np.ndarray, T: int, topk: int):
    """megamoe_rm.cu's combine over pair-ordered rows: out[t, :] = sum over
    slots j, in slot order, of ypart[t*topk + j, :] for the pairs that have an
    expert (pair_to_sorted >= 0).  Summed in float64.  Returns [T][N]."""
    p2s = np.asarray(pair_to_sorted).reshape(T, topk)
    ypart = np.asarray(ypart, np.float64)
    out = np.zeros((T, ypart.shape[1]), np.float64)
    for j in range(topk):
        v = p2s[:, j] >= 0
        out[v] += ypart[np.nonzero(v)[0] * topk + j]
    return out
