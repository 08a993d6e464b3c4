"""Whole routed layers built from the oracle's steps (test infrastructure only).

route -> grouped GEMM(s) -> weighted combine, with each intermediate rounded to
the element type it is stored in between steps (fp16 for INT4 layers, bf16 or
binary16 for NVFP4 layers) exactly as the GPU path stores it.

A token's output depends only on the sorted rows of its own routed pairs
(megamoe_rm.cu's combine sums a token's pairs; tilelang_kernels.py
scatter-adds each expert row into its token).  `tokens` restricts a layer to
a sample of tokens: the GEMMs then run on those tokens' rows only, with the
same arithmetic, and `out` holds the sampled tokens' rows in the given order.
"""
from __future__ import annotations

import numpy as np

from .formats import round_to, bf16_bits, f16_bits, bf16_to_f16_bits
from .route import route_prep
from .gemm import grouped_gemm_qint4, grouped_gemm_qnvfp4, grouped_gemm_qfp8_block
from .combine import scatter_combine
from .quant import quantize_int4_rows


def token_rows(pair_to_sorted, tokens, topk: int) -> np.ndarray:
    """Sorted positions of the routed pairs of `tokens`, ascending."""
    t = np.asarray(tokens, np.int64)
    p = (t[:, None] * topk + np.arange(topk)).reshape(-1)
    s = np.asarray(pair_to_sorted, np.int64)[p]
    return np.unique(s[s >= 0])


def combine_tokens(y_rows, rows, pair_to_sorted, topk_weights, tokens) -> np.ndarray:
    """scatter_combine for the tokens `tokens` when y is known only at the
    sorted positions `rows` (ascending, covering every routed pair of those
    tokens): the same weighted sum, over a y holding just those rows."""
    w = np.asarray(topk_weights)
    T, k = w.shape
    t = np.asarray(tokens, np.int64)
    p2s = np.asarray(pair_to_sorted, np.int64).reshape(T, k)[t]
    local = np.full(p2s.shape, -1, np.int64)
    v = p2s >= 0
    local[v] = np.searchsorted(rows, p2s[v])
    assert np.array_equal(np.asarray(rows)[local[v]], p2s[v]), "rows miss a routed pair of the tokens"
    return scatter_combine(y_rows, local.reshape(-1), w[t])


def _rows_and_tokens(p2s, tokens, k, n):
    if tokens is None:
        return None, np.arange(n)
    return token_rows(p2s, tokens, k), None


def int4_layer(d, act="none", y_dtype="f16"):
    """One INT4 grouped GEMM (act none, or silu_mul over [gate | up]) and the
    combine, for a problem dict from synth.int4_moe."""
    off, srt, p2s, ninv = route_prep(d["topk_ids"], d["E"])
    g = grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                           d["k"], act=act)
    y = round_to(g["y"], y_dtype)
    out = scatter_combine(np.vstack([y, np.zeros((srt.size - y.shape[0], y.shape[1]))]),
                          p2s, d["topk_weights"])
    return dict(offsets=off, sorted_pair_ids=srt, pair_to_sorted=p2s, n_invalid=ninv,
                acc=g["acc"], y=g["y"], out=out)


def int4_ffn_layer(d, tokens, chain=False):
    """The two-GEMM INT4 layer for the tokens `tokens`:
    route -> FC1 (SiLU-gated, fp16 h) -> FC2 -> fp16 y -> combine.
    chain=False: FC2 reads the synthetic SORTED int4 rows d['a2'] with scales
      d['a2_scale'] (the FC2 input of the Mixtral-sized INT4 workload).
    chain=True: the complete W4A4 layer from fp16 x (CUTLASS discussion #2855
      quantizes the fp16 activations per token): x's rows are quantized per
      row to int4, FC1 runs on those codes, h is rounded to fp16 and
      quantized per row again, and FC2 runs on h's codes.
    Returns dict(rows, h, y, out) with out [len(tokens)][H]."""
    off, srt, p2s, _ = route_prep(d["topk_ids"], d["E"])
    k = d["k"]
    rows = token_rows(p2s, tokens, k)
    if chain:
        t = np.unique(np.asarray(srt, np.int64)[rows] // k)
        qx, sx = quantize_int4_rows(d["x"][t])
        a = np.zeros((d["T"], qx.shape[1]), np.uint8)
        sa = np.ones(d["T"], np.float32)
        a[t], sa[t] = qx, sx
    else:
        a, sa = d["a"], d["a_scale"]
    h = grouped_gemm_qint4(a, sa, "token", d["w"], d["w_scale"], off, srt, k, act="silu_mul", rows=rows)["y"]
    if chain:
        qh, sh = quantize_int4_rows(round_to(h, "f16").astype(np.float16))
        a2 = np.zeros((srt.size, qh.shape[1]), np.uint8)
        sa2 = np.ones(srt.size, np.float32)
        a2[rows], sa2[rows] = qh, sh
    else:
        a2, sa2 = d["a2"], d["a2_scale"]
    y = grouped_gemm_qint4(a2, sa2, "sorted", d["w2"], d["w2_scale"], off, srt, k, rows=rows)["y"]
    out = combine_tokens(round_to(y, "f16"), rows, p2s, d["topk_weights"], tokens)
    return dict(rows=rows, h=h, y=y, out=out)


def nvfp4_layer(d, rows_dtype="bf16", tokens=None, x_dtype="bf16", sf_layout="rows", w_layout="rows"):
    """NVFP4 W4A16 MoE layer: FC1 (gate|up) with SiLU-gated product -> h -> FC2
    -> y (rows_dtype) -> weighted combine.

    x_dtype 'bf16': the bf16 activations feed FC1 and h is stored as bf16;
    'f16' (megamoe_rm.cu's fp16 activations): x is first rounded to binary16
    and h is stored as binary16.  sf_layout / w_layout name the layouts of
    d's s1, s2 / w1, w2 (see grouped_gemm_qnvfp4).  tokens: restrict the layer
    to those tokens (out then has their rows, in that order)."""
    off, srt, p2s, ninv = route_prep(d["topk_ids"], d["E"])
    rows = None if tokens is None else token_rows(p2s, tokens, d["k"])
    x = d["x"] if x_dtype == "bf16" else bf16_to_f16_bits(d["x"])
    lay = dict(x_dtype=x_dtype, sf_layout=sf_layout, w_layout=w_layout, rows=rows)
    h = grouped_gemm_qnvfp4(x, "token", d["w1"], d["s1"], d["g1"], off, srt, d["k"], act="silu_mul", **lay)["y"]
    hb = bf16_bits(h) if x_dtype == "bf16" else f16_bits(h)
    if rows is not None:                               # h's rows sit at their sorted positions
        full = np.zeros((srt.size, hb.shape[1]), np.uint16)
        full[rows] = hb
        hb = full
    y = grouped_gemm_qnvfp4(hb, "sorted", d["w2"], d["s2"], d["g2"], off, srt, d["k"], **lay)["y"]
    yr = round_to(y, rows_dtype)
    if rows is None:
        P = srt.size
        out = scatter_combine(np.vstack([yr, np.zeros((P - yr.shape[0], yr.shape[1]))]), p2s,
                              d["topk_weights"])
    else:
        out = combine_tokens(yr, rows, p2s, d["topk_weights"], tokens)
    return dict(offsets=off, sorted_pair_ids=srt, pair_to_sorted=p2s, n_invalid=ninv,
                rows=rows, h=h, y=y, out=out)


def fp8_dense(d, rows=None):
    """Dense FP8 block-scaled GEMM (E = 1, every token to expert 0)."""
    off, srt, p2s, ninv = route_prep(d["topk_ids"], d["E"])
    return grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                   d["k"], rows=rows)["y"]
