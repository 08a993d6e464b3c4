"""Whole routed layers built from the oracle's steps (test infrastructure only).

route -> grouped GEMM(s) -> weighted combine, with each intermediate rounded to
the element type it is stored in between steps (fp16 for INT4 layers, bf16 for
NVFP4 layers) exactly as the GPU path stores it.
"""
from __future__ import annotations

import numpy as np

from .formats import round_to, bf16_bits
from .route import route_prep
from .gemm import grouped_gemm_qint4, grouped_gemm_qnvfp4, grouped_gemm_qfp8_block
from .combine import scatter_combine


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


def nvfp4_layer(d, rows_dtype="bf16"):
    """NVFP4 W4A16 MoE layer: FC1 (gate|up) with SiLU-gated product -> h (bf16)
    -> FC2 -> y (bf16) -> weighted combine."""
    off, srt, p2s, ninv = route_prep(d["topk_ids"], d["E"])
    h = grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, d["k"],
                            act="silu_mul")["y"]
    hb = bf16_bits(h)
    y = grouped_gemm_qnvfp4(hb, "sorted", d["w2"], d["s2"], d["g2"], off, srt, d["k"])["y"]
    yr = round_to(y, rows_dtype)
    P = srt.size
    out = scatter_combine(np.vstack([yr, np.zeros((P - yr.shape[0], yr.shape[1]))]), p2s,
                          d["topk_weights"])
    return dict(offsets=off, sorted_pair_ids=srt, pair_to_sorted=p2s, n_invalid=ninv,
                h=h, y=y, out=out)


def fp8_dense(d, rows=None):
    """Dense FP8 block-scaled GEMM (E = 1, every token to expert 0)."""
    off, srt, p2s, ninv = route_prep(d["topk_ids"], d["E"])
    return grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                   d["k"], rows=rows)["y"]
