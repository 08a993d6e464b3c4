"""Pins for the oracle's grouped GEMMs: brute force in pure Python on tiny
inputs, library routines, a differently structured algorithm, invariants."""
import numpy as np
import pytest
import torch

import oracle
import synth


# ------------------------------------------------------------------ INT4
def _py_int4(byte_row):
    # pure-Python unpack + two's complement, element 2b = low nibble of byte b
    vals = []
    for b in byte_row:
        for nib in (int(b) & 15, int(b) >> 4):
            vals.append(nib - 16 if nib >= 8 else nib)
    return vals


@pytest.mark.parametrize("a_row", ["token", "sorted"])
def test_int4_matches_pure_python_integers(a_row):
    d = synth.int4_moe(11, T=7, E=3, k=2, N=6, K=16, routing="repeat")
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 3)
    n = int(off[-1])
    a = d["a"] if a_row == "token" else synth.uniform_bytes(np.random.default_rng(5), (n, 8))
    sa = d["a_scale"] if a_row == "token" else synth.uniform_f32(np.random.default_rng(6), (n,),
                                                                 0.005, 0.05)
    g = oracle.grouped_gemm_qint4(a, sa, a_row, d["w"], d["w_scale"], off, srt, 2)
    for s in range(n):
        e = next(x for x in range(3) if off[x] <= s < off[x + 1])
        r = int(srt[s]) // 2 if a_row == "token" else s
        av = _py_int4(a[r])
        for c in range(6):
            wv = _py_int4(d["w"][e, c])
            acc = sum(x * y for x, y in zip(av, wv))
            assert g["acc"][s, c] == acc
            assert g["y"][s, c] == pytest.approx(float(sa[r]) * float(d["w_scale"][e, c]) * acc,
                                                 rel=1e-15, abs=0)


def test_int4_fp64_blas_equals_int64_einsum_at_long_k():
    # |partial sums| <= K*64 < 2^53, so the fp64 product is exact: equal to
    # an int64 contraction (a separate library route) bit for bit.
    d = synth.int4_moe(12, T=40, E=2, k=2, N=32, K=4096)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 2)
    g = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2)
    A = oracle.int4_value(oracle.unpack_nibbles(d["a"]))
    for s in range(int(off[-1])):
        e = 0 if s < off[1] else 1
        W = oracle.int4_value(oracle.unpack_nibbles(d["w"][e]))
        ref = np.einsum("k,nk->n", A[srt[s] // 2], W, dtype=np.int64)
        assert np.array_equal(g["acc"][s], ref)


def test_int4_extreme_codes_accumulator():
    # all -8 times all -8 over K: acc = 64*K exactly
    K, N = 2048, 32
    a = np.full((3, K // 2), 0x88, np.uint8)
    w = np.full((1, N, K // 2), 0x88, np.uint8)
    off = np.array([0, 3], np.int32)
    g = oracle.grouped_gemm_qint4(a, np.ones(3, np.float32), "sorted", w, np.ones((1, N), np.float32),
                                  off, None, 1)
    assert np.all(g["acc"] == 64 * K)


def test_silu_mul_matches_torch():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((5, 8)) * 4
    h = oracle.silu_mul(y)
    t = torch.from_numpy(y)
    ref = (torch.nn.functional.silu(t[:, :4]) * t[:, 4:]).numpy()
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
    assert oracle.silu_mul(np.array([[0.0, 3.0]]))[0, 0] == 0.0


def test_silu_mul_limit_special_cases():
    # the clamp of megamoe_rm.cu's fc1_rm epilogue (gate bounded above only,
    # up bounded on both sides) pinned by limits where it reduces to known
    # results and by the shape of the clamp
    rng = np.random.default_rng(9)
    y = rng.standard_normal((6, 16)) * 8
    assert np.array_equal(oracle.silu_mul(y, np.inf), oracle.silu_mul(y))     # no clamp
    assert np.all(oracle.silu_mul(y, 0.0) == 0)                                # u clamped to 0
    big = np.abs(y).max() + 1
    assert np.array_equal(oracle.silu_mul(y, big), oracle.silu_mul(y))         # nothing reaches it
    L = 7.0
    silu7 = float(torch.nn.functional.silu(torch.tensor(L, dtype=torch.float64)))
    # gate above the limit: flat, equal to the value at the limit
    h = oracle.silu_mul(np.array([[10.0, 1e6, L, 3.0, 3.0, 3.0]]), L)[0]
    assert h[0] == h[1] == h[2] == silu7 * 3.0
    # up beyond +-limit: flat at +-limit (a gate of 0.5 keeps silu small)
    h = oracle.silu_mul(np.array([[L, L, L, 20.0, -20.0, 6.5]]), L)[0]
    assert h[0] == silu7 * L and h[1] == -silu7 * L and h[2] == silu7 * 6.5
    # gate far below -limit is NOT clamped: silu(-30) is ~ -2.8e-12, not silu(-7)
    h = oracle.silu_mul(np.array([[-30.0, 1.0]]), L)[0]
    ref = float(torch.nn.functional.silu(torch.tensor(-30.0, dtype=torch.float64)))
    assert h[0] == ref and abs(h[0]) < 1e-10


def test_nvfp4_limit_only_with_silu_mul():
    d = synth.nvfp4_moe(14, T=4, E=2, k=1, H=32, I=16)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 2)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 1, limit=1.0)
    y = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 1)["y"]
    h = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 1,
                                   act="silu_mul", limit=0.05)["y"]
    assert np.array_equal(h, oracle.silu_mul(y, 0.05))


def test_int4_silu_mul_gate_first():
    d = synth.int4_moe(13, T=6, E=2, k=1, N=8, K=32)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 2)
    y = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 1)["y"]
    h = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 1,
                                  act="silu_mul")["y"]
    g, u = y[:, :4], y[:, 4:]
    assert np.allclose(h, g * torch.sigmoid(torch.from_numpy(g)).numpy() * u, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ FP8
def _torch_e4m3(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_matches_per_group_brute_force():
    # Per-group form: y = sum_g sa[g,r] * sb[n//128, g] * sum_{k in g} a*b,
    # decoded by torch; scales vary along every index they carry so that a
    # transposed or mis-strided scale read fails.
    M, N, K, E = 5, 256, 384, 2
    rng = np.random.default_rng(9)
    d = synth.fp8_block(21, M=M, N=N, K=K, E=E, T=M, k=2)
    d["a_scale"] = synth.uniform_f32(rng, (K // 128, M), 0.25, 4.0)
    d["w_scale"] = synth.uniform_f32(rng, (E, N // 128, K // 128), 0.25, 4.0)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], E)
    y = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                       2)["y"]
    A = _torch_e4m3(d["a"])
    for s in range(int(off[-1])):
        e = 0 if s < off[1] else 1
        r = int(srt[s]) // 2
        B = _torch_e4m3(d["w"][e])
        for n in range(0, N, 37):
            acc = 0.0
            for gi in range(K // 128):
                part = sum(A[r, kk] * B[n, kk] for kk in range(128 * gi, 128 * gi + 128))
                acc += float(d["a_scale"][gi, r]) * float(d["w_scale"][e, n // 128, gi]) * part
            assert y[s, n] == pytest.approx(acc, rel=1e-12, abs=1e-12)


def test_fp8_dense_unit_scales_is_plain_matmul():
    d = synth.fp8_block(22, M=16, N=128, K=256)
    d["a_scale"][:] = 1.0
    d["w_scale"][:] = 1.0
    y = oracle.fp8_dense(d)
    ref = (torch.from_numpy(_torch_e4m3(d["a"])) @ torch.from_numpy(_torch_e4m3(d["w"][0])).T).numpy()
    assert np.array_equal(y, ref)     # sums of e4m3 products are exact in fp64


def test_fp8_rows_subset_equals_full():
    d = synth.fp8_block(23, M=20, N=128, K=256)
    full = oracle.fp8_dense(d)
    part = oracle.fp8_dense(d, rows=[0, 7, 19])
    assert np.allclose(part, full[[0, 7, 19]], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ NVFP4
def _segmented_reference(x_bits, w, sf, ids, tw):
    # The segmented algorithm of tilelang_kernels.py's grouped_gemm_fp4
    # (global scale 1): dequantize each expert, then for each expert and each
    # top-k slot, gather the tokens routed there, linear, and scatter-add
    # weighted rows into a zero output.  Float64 torch; decoders from torch.
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    E = w.shape[0]
    lut = torch.from_numpy(np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6]))
    out = torch.zeros(x.shape[0], w.shape[1], dtype=torch.float64)
    ids_t = torch.from_numpy(ids)
    for e in range(E):
        wt = torch.from_numpy(w[e]).to(torch.int64)
        codes = torch.stack([wt & 15, wt >> 4], dim=-1).reshape(wt.shape[0], -1)
        scl = torch.from_numpy(np.ascontiguousarray(sf[e])).view(torch.float8_e4m3fn).to(torch.float64)
        wd = lut[codes] * scl.repeat_interleave(16, dim=1)
        mask = ids_t == e
        for j in range(ids.shape[1]):
            tok = mask[:, j].nonzero(as_tuple=True)[0]
            if tok.numel() == 0:
                continue
            res = torch.nn.functional.linear(x[tok], wd)
            out[tok] += res * torch.from_numpy(tw)[tok, j].to(torch.float64).unsqueeze(-1)
    return out.numpy()


def test_nvfp4_gemm_plus_combine_equals_segmented_algorithm():
    d = synth.nvfp4_moe(31, T=24, E=6, k=3, H=64, I=32, routing="repeat")
    d["g1"][:] = 1.0
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 6)
    y = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 3)["y"]
    out = oracle.scatter_combine(y, inv, d["topk_weights"])
    ref = _segmented_reference(d["x"], d["w1"], d["s1"], d["topk_ids"], d["topk_weights"])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_nvfp4_brute_force_with_global_scale():
    d = synth.nvfp4_moe(32, T=5, E=3, k=2, H=32, I=16)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 3)
    y = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 2)["y"]
    xf = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for s in range(int(off[-1])):
        e = next(q for q in range(3) if off[q] <= s < off[q + 1])
        r = int(srt[s]) // 2
        for n in range(0, 32, 5):
            acc = 0.0
            for kk in range(32):
                byte = int(d["w1"][e, n, kk // 2])
                c = (byte >> 4) if kk % 2 else (byte & 15)
                sign = -1.0 if c & 8 else 1.0
                ex, m = (c >> 1) & 3, c & 1
                val = sign * (m * 0.5 if ex == 0 else 2.0 ** (ex - 1) * (1 + m / 2))
                sc = float(_torch_e4m3(d["s1"][e, n, kk // 16:kk // 16 + 1])[0])
                acc += xf[r, kk] * val * sc
            assert y[s, n] == pytest.approx(float(d["g1"][e]) * acc, rel=1e-13, abs=1e-13)


# ------------------------------------------------------------------ invariants
def test_empty_expert_weights_do_not_matter():
    d = synth.nvfp4_moe(33, T=16, E=5, k=2, H=32, I=16, routing="repeat")
    d["topk_ids"][d["topk_ids"] == 3] = 1       # expert 3 gets no rows
    a = oracle.nvfp4_layer(d)
    d2 = dict(d)
    d2["w1"] = d["w1"].copy(); d2["w1"][3] ^= 0x5A
    d2["w2"] = d["w2"].copy(); d2["w2"][3] ^= 0xA5
    d2["s1"] = d["s1"].copy(); d2["s1"][3] = 0x40
    b = oracle.nvfp4_layer(d2)
    assert np.array_equal(a["out"], b["out"])


def test_token_permutation_permutes_output_rows():
    d = synth.int4_moe(34, T=20, E=4, k=2, N=32, K=64)
    base = oracle.int4_layer(d)["out"]
    perm = np.random.default_rng(0).permutation(20)
    d2 = dict(d, a=d["a"][perm], a_scale=d["a_scale"][perm], topk_ids=d["topk_ids"][perm],
              topk_weights=d["topk_weights"][perm])
    out = oracle.int4_layer(d2)["out"]
    assert np.allclose(out, base[perm], rtol=1e-12, atol=1e-12)


def test_scaling_a_scale_scales_rows_exactly():
    d = synth.int4_moe(35, T=10, E=3, k=2, N=32, K=64)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 3)
    y1 = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2)["y"]
    sa = d["a_scale"].copy(); sa[4] *= 2
    y2 = oracle.grouped_gemm_qint4(d["a"], sa, "token", d["w"], d["w_scale"], off, srt, 2)["y"]
    rows4 = (srt[: off[-1]] // 2) == 4
    assert np.array_equal(y2[rows4], 2 * y1[rows4]) and np.array_equal(y2[~rows4], y1[~rows4])


def test_nvfp4_f16_activations_equal_bf16_when_exact():
    # bf16 activations in the binary16 normal range convert exactly, so the
    # fp16 form of the GEMM gives the same fp64 result; a value below 2^-14
    # rounds and changes it by at most its rounding error
    d = synth.nvfp4_moe(15, T=6, E=2, k=1, H=64, I=32)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 2)
    x = d["x"].copy()
    v = oracle.bf16_value(x)
    x[np.abs(v) < 2.0 ** -14] = 0x3F80                     # 1.0: keep every value exact
    xh = oracle.bf16_to_f16_bits(x)
    yb = oracle.grouped_gemm_qnvfp4(x, "token", d["w1"], d["s1"], d["g1"], off, srt, 1)["y"]
    yh = oracle.grouped_gemm_qnvfp4(xh, "token", d["w1"], d["s1"], d["g1"], off, srt, 1, x_dtype="f16")["y"]
    assert np.array_equal(yb, yh)
    x[0, 0] = 0x3300                                       # bf16 2^-25: an fp16 tie, rounds to 0
    xh = oracle.bf16_to_f16_bits(x)
    assert xh[0, 0] == 0
    with pytest.raises(ValueError):
        oracle.grouped_gemm_qnvfp4(xh, "token", d["w1"], d["s1"], d["g1"], off, srt, 1, x_dtype="f32")


# ------------------------------------------------------------------ column selection
def test_column_selection_is_the_same_contraction():
    # `cols` picks the weight rows of the selected outputs before the matmul:
    # integers bit-exact, floats equal up to fp64 summation order (the BLAS
    # may block a narrower product differently)
    d = synth.int4_moe(13, T=30, E=3, k=2, N=96, K=256, routing="repeat")
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 3)
    full = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2)
    cols = np.array([0, 5, 31, 32, 95])
    part = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2,
                                     cols=cols)
    assert np.array_equal(part["acc"], full["acc"][:, cols])
    assert np.array_equal(part["y"], full["y"][:, cols])
    fs = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2,
                                   act="silu_mul")["y"]
    hc = np.array([0, 7, 47])
    ps = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 2,
                                   act="silu_mul", cols=hc)
    assert np.array_equal(ps["y"], fs[:, hc])
    # the gate rows come first, then the matching up rows
    assert np.array_equal(oracle.weight_rows(96, "silu_mul", hc), np.array([0, 7, 47, 48, 55, 95]))
    with pytest.raises(ValueError):
        oracle.weight_rows(96, "silu_mul", [48])

    f = synth.fp8_block(14, 0, 384, 256, E=2, T=20, k=2)
    off, srt, inv, _ = oracle.route_prep(f["topk_ids"], 2)
    full = oracle.grouped_gemm_qfp8_block(f["a"], f["a_scale"], "token", f["w"], f["w_scale"], off, srt, 2)["y"]
    c = np.array([1, 127, 128, 300, 383])      # three 128-column scale blocks
    part = oracle.grouped_gemm_qfp8_block(f["a"], f["a_scale"], "token", f["w"], f["w_scale"], off, srt, 2,
                                          cols=c)["y"]
    np.testing.assert_allclose(part, full[:, c], rtol=1e-12, atol=0)

    n = synth.nvfp4_moe(15, 24, 3, 2, 128, 64, routing="repeat")
    off, srt, inv, _ = oracle.route_prep(n["topk_ids"], 3)
    for sfl, wl in (("rows", "rows"), ("quads", "tiled")):
        w = n["w1"] if wl == "rows" else oracle.tiles_from_rows(n["w1"])
        s = n["s1"] if sfl == "rows" else oracle.quads_from_rows(n["s1"])
        full = oracle.grouped_gemm_qnvfp4(n["x"], "token", w, s, n["g1"], off, srt, 2, act="silu_mul",
                                          sf_layout=sfl, w_layout=wl)["y"]
        hc = np.array([0, 15, 16, 63])
        part = oracle.grouped_gemm_qnvfp4(n["x"], "token", w, s, n["g1"], off, srt, 2, act="silu_mul",
                                          sf_layout=sfl, w_layout=wl, cols=hc)["y"]
        np.testing.assert_allclose(part, full[:, hc], rtol=1e-12, atol=0)
