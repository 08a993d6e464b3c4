"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (bench.Workload issues the calls).

Coverage: route tables equal; every sorted row of every GEMM is compared,
in full where the oracle is cheap and otherwise on a column sample with one
column in every 16 (NVFP4) or 32 (INT4) consecutive output columns, so that
every (expert, m-tile, n-tile) work item of every schedule and every wave's
column slice is checked.  End to end, the oracle's own chain (route -> FC1 ->
rounded h -> FC2 -> rounded y -> combine) is compared with the GPU's output
on every token (decode) or on a token sample that includes the tokens of the
largest and the smallest expert."""
import functools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import host, bf16_bits, assert_rows_close

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@functools.lru_cache(maxsize=3)
def _run(idx, fc2="sorted", act="f16", sfl="quads", wlay="tiled"):
    """One bench step of workload idx (cached: each test reads its outputs)."""
    import bench
    print(f"[workload {idx} fc2={fc2} act={act} sf={sfl} w={wlay}]", flush=True)
    wl = bench.Workload(idx, fc2, act, sfl, wlay)
    wl.step()
    torch.cuda.synchronize()
    return wl


def _check_route(wl):
    offs, srt, p2s, ninv = (host(t) for t in wl.route_out)
    ref = oracle.route_prep(wl.d["topk_ids"], wl.E)
    assert np.array_equal(offs, ref[0]) and np.array_equal(srt, ref[1]) and np.array_equal(p2s, ref[2])
    assert int(ninv[0]) == ref[3] == 0
    return ref


def _stratified_cols(n_out, block, seed):
    """One random column in each run of `block` consecutive output columns."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, n_out, block)
    return starts + rng.integers(0, np.minimum(block, n_out - starts))


def _assert_cols_close(gpu_rows, cols, ref_cols, full_ref, what):
    """The per-row tolerance on a column sample.  The bound is 2e-3 times the
    L2 norm of the whole oracle row, which is at least the norm over the
    sampled columns; rows that pass against the sampled norm pass, and any
    other row is recomputed by the oracle over all its columns
    (full_ref(row_indices) -> rows) and judged against its full norm."""
    gpu_rows = np.asarray(gpu_rows)
    sel = gpu_rows if cols is None else gpu_rows[:, cols]
    ref_cols = np.asarray(ref_cols, np.float64)
    assert np.all(np.isfinite(sel)), f"{what}: non-finite output"
    err = np.abs(sel - ref_cols).max(axis=1)
    norm = np.linalg.norm(ref_cols, axis=1)
    unsure = np.nonzero(err > 2e-3 * norm)[0]
    if cols is None or unsure.size == 0:
        assert_rows_close(sel, ref_cols, what=what)
        return
    assert unsure.size <= 0.05 * sel.shape[0], f"{what}: {unsure.size} rows exceed the sampled-norm bound"
    assert_rows_close(gpu_rows[unsure], full_ref(unsure), what=what + " (whole rows)")


def _token_sample(off, srt, k, T, n_rand, seed):
    """Tokens of the largest and the smallest non-empty expert, the first
    and last token, and n_rand random ones."""
    rng = np.random.default_rng(seed)
    sizes = np.diff(off)
    ne = np.nonzero(sizes)[0]
    big, small = ne[np.argmax(sizes[ne])], ne[np.argmin(sizes[ne])]
    pick = [srt[off[big]] // k, srt[off[big + 1] - 1] // k, srt[off[small]] // k, 0, T - 1]
    pick += list(rng.choice(T, n_rand, replace=False))
    return np.array(list(dict.fromkeys(int(t) for t in pick)))


# ------------------------------------------------------------------ W4A4 tiny (64 tokens, E=4)
def test_workload0_w4a4_tiny_end_to_end():
    wl = _run(0)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    ref = oracle.int4_layer(d)
    assert_rows_close(host(wl.y)[: ref["y"].shape[0]], ref["y"], what="y")
    assert_rows_close(host(wl.out), ref["out"], what="layer")
    acc = wl.mq.grouped_gemm_qint4(wl.a, wl.sa, wl.w, wl.sw, wl.route_out[0], wl.route_out[1], wl.k,
                                   out_dtype=torch.int32)
    assert np.array_equal(host(acc), ref["acc"])


# ------------------------------------------------------------------ FP8 dense 1024x4096x7168
def test_workload1_fp8_dense_every_output():
    wl = _run(1)
    off, srt, _, _ = _check_route(wl)
    d = wl.d
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, 1)["y"]
    assert_rows_close(host(wl.y), ref, what="fp8 1024x4096x7168")


# ------------------------------------------------------------------ NVFP4 decode (8 tokens) and Zipf prefill (4096)
def _nvfp4_rows_layout(wl):
    """The workload's weights in the oracle's row-major layouts (one
    conversion per test instead of one per oracle call)."""
    w1 = oracle.rows_from_tiles(wl.w1_host) if wl.wl == "tiled" else wl.w1_host
    w2 = oracle.rows_from_tiles(wl.w2_host) if wl.wl == "tiled" else wl.w2_host
    s1 = oracle.rows_from_quads(wl.s1_host) if wl.sfl == "quads" else wl.s1_host
    s2 = oracle.rows_from_quads(wl.s2_host) if wl.sfl == "quads" else wl.s2_host
    return w1, s1, w2, s2


def _x_bits(wl):
    d = wl.d
    if wl.act == "f16":
        xb = oracle.bf16_to_f16_bits(d["x"])
        assert np.array_equal(host(wl.xh.view(torch.int16)).view(np.uint16), xb)
        return xb
    return d["x"]


def _h_bits(wl):
    return host(wl.h.view(torch.int16)).view(np.uint16) if wl.act == "f16" else bf16_bits(wl.h)


def _nvfp4_per_call(wl, block_h, block_y):
    """FC1 and FC2 on every sorted row (FC2 on the GPU's own h), on a
    stratified column sample when block_* > 1; the combine on every token
    against the oracle applied to the GPU's own y."""
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    w1, s1, w2, s2 = _nvfp4_rows_layout(wl)
    n = int(off[-1])
    xb, hb = _x_bits(wl), _h_bits(wl)
    fc1 = lambda cols=None, rows=None: oracle.grouped_gemm_qnvfp4(
        xb, "token", w1, s1, d["g1"], off, srt, d["k"], act="silu_mul", x_dtype=wl.act, cols=cols, rows=rows)["y"]
    fc2 = lambda cols=None, rows=None: oracle.grouped_gemm_qnvfp4(
        hb, "sorted", w2, s2, d["g2"], off, srt, d["k"], x_dtype=wl.act, cols=cols, rows=rows)["y"]
    ch = None if block_h == 1 else _stratified_cols(d["I"], block_h, 31)
    _assert_cols_close(host(wl.h)[:n], ch, fc1(cols=ch), lambda r: fc1(rows=r), "FC1 h")
    cy = None if block_y == 1 else _stratified_cols(d["H"], block_y, 32)
    _assert_cols_close(host(wl.y)[:n], cy, fc2(cols=cy), lambda r: fc2(rows=r), "FC2 y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine (GPU y)")


def _nvfp4_end_to_end(wl, tokens):
    w1, s1, w2, s2 = _nvfp4_rows_layout(wl)
    d = dict(wl.d, w1=w1, s1=s1, w2=w2, s2=s2)
    ref = oracle.nvfp4_layer(d, rows_dtype="bf16", tokens=tokens, x_dtype=wl.act)
    assert_rows_close(host(wl.out)[tokens], ref["out"], what="layer (oracle chain)")


def test_workload2_nvfp4_decode_every_row():
    _nvfp4_per_call(_run(2), block_h=1, block_y=1)


def test_workload2_nvfp4_decode_end_to_end_every_token():
    wl = _run(2)
    _nvfp4_end_to_end(wl, np.arange(wl.T))


def test_workload3_nvfp4_prefill_zipf_every_row():
    wl = _run(3)
    sizes = np.diff(host(wl.route_out[0]))
    assert sizes.min() == 0 and sizes.max() > 1000      # skewed, with empty experts
    _nvfp4_per_call(wl, block_h=16, block_y=16)


def test_workload3_nvfp4_prefill_end_to_end_token_sample():
    wl = _run(3)
    off, srt, _, _ = _check_route(wl)
    _nvfp4_end_to_end(wl, _token_sample(off, srt, wl.k, wl.T, 3, 33))


@pytest.mark.parametrize("idx", [2, 3])
def test_nvfp4_workloads_with_bf16_activations_rows_scales(idx):
    wl = _run(idx, act="bf16", sfl="rows", wlay="rows")
    _nvfp4_per_call(wl, block_h=1 if idx == 2 else 16, block_y=1 if idx == 2 else 16)


@pytest.mark.parametrize("idx", [2, 3])
def test_nvfp4_workloads_with_fc2_pair_epilogue(idx):
    # the step with the top-k weight in FC2's epilogue: every pair row (on
    # the column sample at prefill size), then the whole pair sum against
    # the oracle on the GPU's rows
    wl = _run(idx, fc2="pair")
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    _, _, w2, s2 = _nvfp4_rows_layout(wl)
    n = int(off[-1])
    cy = None if idx == 2 else _stratified_cols(d["H"], 16, 34)
    hb = _h_bits(wl)
    fc2 = lambda cols=None, rows=None: oracle.grouped_gemm_qnvfp4(
        hb, "sorted", w2, s2, d["g2"], off, srt, d["k"], x_dtype="f16", cols=cols, rows=rows)["y"]
    pairs = srt[:n]
    w = d["topk_weights"].reshape(-1)[pairs]
    yp = host(wl.y)
    _assert_cols_close(yp[pairs], cy, w[:, None] * fc2(cols=cy), lambda r: w[r, None] * fc2(rows=r),
                       "FC2 pair rows")
    yp[p2s < 0] = 0
    assert_rows_close(host(wl.out), oracle.sum_pairs(yp, p2s, wl.T, wl.k), what="pair sum")


# ------------------------------------------------------------------ W4A4 Mixtral-sized (8192 tokens, E=8)
def test_workload4_w4a4_mixtral_every_row():
    wl = _run(4)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    n = int(off[-1])
    ch = _stratified_cols(d["N"] // 2, 32, 41)
    fc1 = lambda cols=None, rows=None: oracle.grouped_gemm_qint4(
        d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt, d["k"], act="silu_mul", cols=cols,
        rows=rows)["y"]
    _assert_cols_close(host(wl.h)[:n], ch, fc1(cols=ch), lambda r: fc1(rows=r), "FC1 h")
    # FC2 raw accumulators at full size, bit-exact on every row
    acc = wl.mq.grouped_gemm_qint4(wl.a2, wl.sa2, wl.w2, wl.sw2, wl.route_out[0], wl.route_out[1],
                                   wl.k, a_row="sorted", out_dtype=torch.int32)
    cy = _stratified_cols(d["N2"], 32, 42)
    fc2 = lambda cols=None, rows=None: oracle.grouped_gemm_qint4(
        d["a2"], d["a2_scale"], "sorted", d["w2"], d["w2_scale"], off, srt, d["k"], cols=cols, rows=rows)
    ref2 = fc2(cols=cy)
    assert np.array_equal(host(acc)[:n][:, cy], ref2["acc"])
    _assert_cols_close(host(wl.y)[:n], cy, ref2["y"], lambda r: fc2(rows=r)["y"], "FC2 y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine (GPU y)")


def test_workload4_w4a4_mixtral_end_to_end_token_sample():
    wl = _run(4)
    off, srt, _, _ = _check_route(wl)
    tok = _token_sample(off, srt, wl.k, wl.T, 3, 43)
    d = dict(wl.d, H=wl.d["K"], I=wl.d["N"] // 2)
    ref = oracle.int4_ffn_layer(d, tok)
    assert_rows_close(host(wl.h)[ref["rows"]], ref["h"], what="FC1 h (oracle chain)")
    assert_rows_close(host(wl.out)[tok], ref["out"], what="layer (oracle chain)")


# ------------------------------------------------------------------ next-row workloads
def test_workload5_int4_quantizer_every_row():
    wl = _run(5)
    ref_q, ref_s = oracle.quantize_int4_rows(wl.d["x"])
    assert np.array_equal(host(wl.qs), ref_s)
    assert np.array_equal(host(wl.q), ref_q)


def test_workload6_fp8_moe_decode_every_row():
    # the FP8 block-scaled kernel under routing, weight-streaming schedule
    wl = _run(6)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                         d["k"])["y"]
    assert_rows_close(host(wl.y)[: ref.shape[0]], ref, what="fp8 decode full size")


def test_workload7_nvfp4_repack_every_expert():
    wl = _run(7)
    d = wl.d
    rw, rs = oracle.repack_nvfp4(d["w"], d["sf"], bool(wl.cfg["swap"]))
    assert np.array_equal(host(wl.w_out), rw)
    assert np.array_equal(host(wl.sf_out).reshape(rs.shape), rs)


def test_workload8_w4a4_chain_from_fp16_every_row():
    # every step of the chain against the oracle applied to the GPU's own
    # input of that step; both quantizations bit-exact on every row
    wl = _run(8)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    n = int(off[-1])
    ref_q, ref_s = oracle.quantize_int4_rows(d["x"])
    assert np.array_equal(host(wl.qx), ref_q) and np.array_equal(host(wl.sx), ref_s)
    ch = _stratified_cols(d["I"], 32, 81)
    qx, sx = host(wl.qx), host(wl.sx)
    fc1 = lambda cols=None, rows=None: oracle.grouped_gemm_qint4(
        qx, sx, "token", d["w"], d["w_scale"], off, srt, d["k"], act="silu_mul", cols=cols, rows=rows)["y"]
    _assert_cols_close(host(wl.h)[:n], ch, fc1(cols=ch), lambda r: fc1(rows=r), "FC1 h")
    hq_ref, hs_ref = oracle.quantize_int4_rows(host(wl.h)[:n].astype(np.float16))
    assert np.array_equal(host(wl.qh)[:n], hq_ref) and np.array_equal(host(wl.sh)[:n], hs_ref)
    cy = _stratified_cols(d["H"], 32, 82)
    qh, sh = host(wl.qh), host(wl.sh)
    fc2 = lambda cols=None, rows=None: oracle.grouped_gemm_qint4(
        qh, sh, "sorted", d["w2"], d["w2_scale"], off, srt, d["k"], cols=cols, rows=rows)["y"]
    _assert_cols_close(host(wl.y)[:n], cy, fc2(cols=cy), lambda r: fc2(rows=r), "FC2 y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine (GPU y)")


def test_workload8_w4a4_chain_end_to_end_token_sample():
    wl = _run(8)
    off, srt, _, _ = _check_route(wl)
    tok = _token_sample(off, srt, wl.k, wl.T, 3, 83)
    ref = oracle.int4_ffn_layer(wl.d, tok, chain=True)
    assert_rows_close(host(wl.out)[tok], ref["out"], what="W4A4 layer (oracle chain)")


def test_workload9_w4a4_chain_decode_every_row_and_token():
    # the layer at one 8-token decode step: both GEMMs on the weight-streaming
    # schedule; every element of every step against the oracle, both
    # quantizations bit-exact, and the oracle's own chain on every token
    wl = _run(9)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    n = int(off[-1])
    assert n == wl.T * wl.k < 16 * wl.E
    ref_q, ref_s = oracle.quantize_int4_rows(d["x"])
    assert np.array_equal(host(wl.qx), ref_q) and np.array_equal(host(wl.sx), ref_s)
    h_ref = oracle.grouped_gemm_qint4(host(wl.qx), host(wl.sx), "token", d["w"], d["w_scale"], off, srt,
                                      d["k"], act="silu_mul")["y"]
    assert_rows_close(host(wl.h)[:n], h_ref, what="FC1 h")
    hq_ref, hs_ref = oracle.quantize_int4_rows(host(wl.h)[:n].astype(np.float16))
    assert np.array_equal(host(wl.qh)[:n], hq_ref) and np.array_equal(host(wl.sh)[:n], hs_ref)
    y_ref = oracle.grouped_gemm_qint4(host(wl.qh), host(wl.sh), "sorted", d["w2"], d["w2_scale"], off, srt,
                                      d["k"])["y"]
    assert_rows_close(host(wl.y)[:n], y_ref, what="FC2 y")
    ref = oracle.int4_ffn_layer(d, np.arange(wl.T), chain=True)
    assert_rows_close(host(wl.out), ref["out"], what="W4A4 decode layer (oracle chain)")
