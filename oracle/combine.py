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
