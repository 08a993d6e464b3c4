"""Pins for the oracle's layer compositions (route -> GEMMs -> combine): a
pure-Python brute force of the whole W4A4 chain on a tiny problem, and the
token-sampled layers against the same layers over every token."""
import math

import numpy as np
import pytest

import oracle
import synth


def _py_int4(byte_row):
    vals = []
    for b in byte_row:
        for nib in (int(b) & 15, int(b) >> 4):
            vals.append(nib - 16 if nib >= 8 else nib)
    return vals


def _py_f16(v):
    return float(np.float16(v))


def _py_quant(row):
    # per-row symmetric int4 (amax/7 scale), the rule of moe_quantize_int4,
    # each step in fp32 as numpy float32 scalars
    xs = [np.float32(v) for v in row]
    amax = max(abs(v) for v in xs)
    if amax < np.float32(2.0 ** -120):
        return [0] * len(xs), 1.0
    scale = np.float32(amax / np.float32(7))
    recip = np.float32(np.float32(7) / amax)
    codes = [int(min(7, max(-8, np.rint(np.float32(v * recip))))) for v in xs]
    return codes, float(scale)


def test_int4_chain_brute_force_per_token():
    T, E, k, H, I = 6, 3, 2, 32, 16
    d = synth.int4_chain(3, T, E, k, H, I)
    off, srt, p2s, _ = oracle.route_prep(d["topk_ids"], E)
    tokens = np.array([4, 0, 5])
    got = oracle.int4_ffn_layer(d, tokens, chain=True)["out"]
    for i, t in enumerate(tokens):
        xq, sx = _py_quant(d["x"][t].astype(np.float32))
        ref = [0.0] * H
        for j in range(k):
            e = int(d["topk_ids"][t, j])
            w = float(d["topk_weights"][t, j])
            h = []
            for c in range(I):
                gate = sum(a * b for a, b in zip(xq, _py_int4(d["w"][e, c])))
                up = sum(a * b for a, b in zip(xq, _py_int4(d["w"][e, I + c])))
                g = sx * float(d["w_scale"][e, c]) * gate
                u = sx * float(d["w_scale"][e, I + c]) * up
                h.append(_py_f16(g / (1.0 + math.exp(-g)) * u))
            hq, sh = _py_quant(h)
            for n in range(H):
                acc = sum(a * b for a, b in zip(hq, _py_int4(d["w2"][e, n])))
                ref[n] += w * _py_f16(sh * float(d["w2_scale"][e, n]) * acc)
        np.testing.assert_allclose(got[i], ref, rtol=1e-12, atol=1e-15)


def test_int4_ffn_layer_sample_equals_every_token():
    T, E, k, H, I = 40, 4, 2, 128, 64
    d = synth.int4_moe(5, T, E, k, 2 * I, H, fc2_rows=T * k, N2=H, K2=I)
    d.update(H=H, I=I)
    every = oracle.int4_ffn_layer(d, np.arange(T))
    some = oracle.int4_ffn_layer(d, np.array([7, 3, 39]))
    np.testing.assert_array_equal(some["out"], every["out"][[7, 3, 39]])
    # and the combine of all tokens is the plain scatter-combine of fp16 y
    off, srt, p2s, _ = oracle.route_prep(d["topk_ids"], E)
    y = oracle.round_to(oracle.grouped_gemm_qint4(d["a2"], d["a2_scale"], "sorted", d["w2"], d["w2_scale"],
                                                  off, srt, k)["y"], "f16")
    np.testing.assert_array_equal(every["out"], oracle.scatter_combine(y, p2s, d["topk_weights"]))


@pytest.mark.parametrize("x_dtype", ["bf16", "f16"])
def test_nvfp4_layer_sample_equals_every_token(x_dtype):
    T, E, k, H, I = 24, 5, 2, 128, 64
    d = synth.nvfp4_moe(6, T, E, k, H, I, routing="repeat")
    d["topk_ids"][3] = -1                           # a token with no expert
    full = oracle.nvfp4_layer(d, x_dtype=x_dtype)
    tok = np.array([3, 0, 23, 11])
    some = oracle.nvfp4_layer(d, x_dtype=x_dtype, tokens=tok)
    np.testing.assert_array_equal(some["out"], full["out"][tok])
    assert np.all(some["out"][0] == 0)
    # the stored layouts give the same layer
    dq = dict(d, w1=oracle.tiles_from_rows(d["w1"]), w2=oracle.tiles_from_rows(d["w2"]),
              s1=oracle.quads_from_rows(d["s1"]), s2=oracle.quads_from_rows(d["s2"]))
    lay = oracle.nvfp4_layer(dq, x_dtype=x_dtype, tokens=tok, sf_layout="quads", w_layout="tiled")
    np.testing.assert_allclose(lay["out"], some["out"], rtol=1e-12, atol=0)


def test_token_rows_and_combine_tokens():
    rng = np.random.default_rng(2)
    T, k, E, N = 30, 3, 5, 8
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    ids[rng.random((T, k)) < 0.2] = -1
    off, srt, p2s, _ = oracle.route_prep(ids, E)
    w = synth.softmax_weights(rng, T, k)
    y = rng.standard_normal((T * k, N))
    tok = np.array([29, 1, 2, 17])
    rows = oracle.token_rows(p2s, tok, k)
    assert sorted(rows.tolist()) == sorted(int(s) for t in tok for s in p2s[t * k:(t + 1) * k] if s >= 0)
    np.testing.assert_array_equal(oracle.combine_tokens(y[rows], rows, p2s, w, tok),
                                  oracle.scatter_combine(y, p2s, w)[tok])
