"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (bench.Workload issues the calls).  Route tables must be
equal; expert outputs are checked on sampled rows that the oracle computes
one by one; the combine is checked in full against the oracle applied to the
GPU's own expert rows."""
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


def _run(idx, fc2="sorted", act="f16", sfl="quads", wlay="tiled"):
    import bench
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


def _sample_rows(offs, n_per=2, max_experts=6, seed=0):
    """A few sorted rows from the largest, the smallest and random non-empty experts."""
    rng = np.random.default_rng(seed)
    sizes = np.diff(offs)
    ne = np.nonzero(sizes)[0]
    order = ne[np.argsort(sizes[ne])]
    pick = list(dict.fromkeys([order[-1], order[0]] + list(rng.permutation(ne)[: max_experts - 2])))
    rows = []
    for e in pick[:max_experts]:
        lo, hi = offs[e], offs[e + 1]
        rows += list(rng.choice(np.arange(lo, hi), size=min(n_per, hi - lo), replace=False))
        rows.append(hi - 1)
    return np.unique(np.array(rows, np.int64))


def test_workload0_w4a4_tiny_end_to_end():
    wl = _run(0)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    ref = oracle.int4_layer(d)
    assert_rows_close(host(wl.y), ref["y"], what="y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine (GPU y)")
    assert_rows_close(host(wl.out), ref["out"], what="layer")
    acc = wl.mq.grouped_gemm_qint4(wl.a, wl.sa, wl.w, wl.sw, wl.route_out[0], wl.route_out[1], wl.k,
                                   out_dtype=torch.int32)
    assert np.array_equal(host(acc), ref["acc"])


def test_workload1_fp8_dense_sampled_rows():
    wl = _run(1)
    _check_route(wl)
    d = wl.d
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 511, 1023],
                                     np.random.default_rng(1).choice(1024, 40, replace=False)]))
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                         host(wl.route_out[0]), host(wl.route_out[1]), 1, rows=rows)["y"]
    assert_rows_close(host(wl.y)[rows], ref, what="fp8 full size")


def _nvfp4_checks(wl, n_per):
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    rows = _sample_rows(off, n_per=n_per)
    xdt = wl.act
    if xdt == "f16":
        xb = oracle.bf16_to_f16_bits(d["x"])
        assert np.array_equal(host(wl.xh.view(torch.int16)).view(np.uint16), xb)
    else:
        xb = d["x"]
    h_ref = oracle.grouped_gemm_qnvfp4(xb, "token", wl.w1_host, wl.s1_host, d["g1"], off, srt, d["k"],
                                       act="silu_mul", rows=rows, x_dtype=xdt, sf_layout=wl.sfl,
                                       w_layout=wl.wl)["y"]
    assert_rows_close(host(wl.h)[rows], h_ref, what="FC1 h")
    # FC2 consumes the GPU's h (per-call parity)
    hb = host(wl.h.view(torch.int16)).view(np.uint16) if xdt == "f16" else bf16_bits(wl.h)
    y_ref = oracle.grouped_gemm_qnvfp4(hb, "sorted", wl.w2_host, wl.s2_host, d["g2"], off, srt, d["k"],
                                       rows=rows, x_dtype=xdt, sf_layout=wl.sfl, w_layout=wl.wl)["y"]
    assert_rows_close(host(wl.y)[rows], y_ref, what="FC2 y")
    out_ref = oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"])
    assert_rows_close(host(wl.out), out_ref, what="combine")


def test_workload2_nvfp4_decode():
    _nvfp4_checks(_run(2), n_per=1)


def test_workload3_nvfp4_prefill_zipf():
    wl = _run(3)
    sizes = np.diff(host(wl.route_out[0]))
    assert sizes.min() == 0 and sizes.max() > 1000      # skewed, with empty experts
    _nvfp4_checks(wl, n_per=2)


@pytest.mark.parametrize("idx", [2, 3])
def test_nvfp4_workloads_with_bf16_activations_rows_scales(idx):
    wl = _run(idx, act="bf16", sfl="rows", wlay="rows")
    _nvfp4_checks(wl, n_per=1 if idx == 2 else 2)


@pytest.mark.parametrize("idx", [2, 3])
def test_nvfp4_workloads_with_fc2_pair_epilogue(idx):
    # the step with the top-k weight in FC2's epilogue: pair rows of sampled
    # sorted rows, then the whole pair sum against the oracle on the GPU's rows
    wl = _run(idx, fc2="pair")
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    rows = _sample_rows(off, n_per=1 if idx == 2 else 2)
    hb = host(wl.h.view(torch.int16)).view(np.uint16)
    y_ref = oracle.grouped_gemm_qnvfp4(hb, "sorted", wl.w2_host, wl.s2_host, d["g2"], off, srt, d["k"], rows=rows,
                                       x_dtype="f16", sf_layout="quads", w_layout="tiled")["y"]
    pairs = srt[rows]
    w = d["topk_weights"].reshape(-1)[pairs]
    assert_rows_close(host(wl.y)[pairs], w[:, None] * y_ref, what="FC2 pair rows")
    yp = host(wl.y)
    yp[p2s < 0] = 0
    assert_rows_close(host(wl.out), oracle.sum_pairs(yp, p2s, wl.T, wl.k), what="pair sum")


def test_workload4_w4a4_mixtral():
    wl = _run(4)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    rows = _sample_rows(off, n_per=2, max_experts=3)
    h_ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                      d["k"], act="silu_mul", rows=rows)["y"]
    assert_rows_close(host(wl.h)[rows], h_ref, what="FC1 h")
    # FC2 raw accumulators at full size, bit-exact on the sampled rows
    acc = wl.mq.grouped_gemm_qint4(wl.a2, wl.sa2, wl.w2, wl.sw2, wl.route_out[0], wl.route_out[1],
                                   wl.k, a_row="sorted", out_dtype=torch.int32)
    ref2 = oracle.grouped_gemm_qint4(d["a2"], d["a2_scale"], "sorted", d["w2"], d["w2_scale"], off,
                                     srt, d["k"], rows=rows)
    assert np.array_equal(host(acc)[rows], ref2["acc"])
    assert_rows_close(host(wl.y)[rows], ref2["y"], what="FC2 y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine")


def test_workload5_int4_quantizer_sampled_rows():
    wl = _run(5)
    x = wl.d["x"]
    rows = np.unique(np.concatenate([[0, x.shape[0] - 1],
                                     np.random.default_rng(5).integers(0, x.shape[0], 62)]))
    ref_q, ref_s = oracle.quantize_int4_rows(x[rows])
    assert np.array_equal(host(wl.qs)[rows], ref_s)
    assert np.array_equal(host(wl.q)[rows], ref_q)


def test_workload6_fp8_moe_decode_sampled_rows():
    # the FP8 block-scaled kernel under routing, weight-streaming schedule
    wl = _run(6)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    rows = _sample_rows(off, n_per=2, max_experts=6)
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                         d["k"], rows=rows)["y"]
    assert_rows_close(host(wl.y)[rows], ref, what="fp8 decode full size")


def test_workload7_nvfp4_repack_sampled_experts():
    wl = _run(7)
    d = wl.d
    experts = np.unique(np.concatenate([[0, 1, d["E"] - 1],
                                        np.random.default_rng(7).integers(0, d["E"], 3)]))
    for e in experts:
        rw, rs = oracle.repack_nvfp4(d["w"][e:e + 1], d["sf"][e:e + 1], bool(wl.cfg["swap"]))
        assert np.array_equal(host(wl.w_out[int(e)]), rw[0]), e
        assert np.array_equal(host(wl.sf_out[int(e)]), rs[0]), e


def test_workload8_w4a4_chain_from_fp16():
    # every step of the chain against the oracle applied to the GPU's own
    # input of that step; both quantizations bit-exact on sampled rows
    wl = _run(8)
    off, srt, p2s, _ = _check_route(wl)
    d = wl.d
    rows = _sample_rows(off, n_per=2, max_experts=3)
    toks = np.unique(np.concatenate([[0, wl.T - 1], srt[rows] // wl.k]))
    ref_q, ref_s = oracle.quantize_int4_rows(d["x"][toks])
    assert np.array_equal(host(wl.qx)[toks], ref_q) and np.array_equal(host(wl.sx)[toks], ref_s)
    qx, sx = host(wl.qx), host(wl.sx)
    h_ref = oracle.grouped_gemm_qint4(qx, sx, "token", d["w"], d["w_scale"], off, srt, d["k"],
                                      act="silu_mul", rows=rows)["y"]
    assert_rows_close(host(wl.h)[rows], h_ref, what="FC1 h")
    hq_ref, hs_ref = oracle.quantize_int4_rows(host(wl.h)[rows].astype(np.float16))
    assert np.array_equal(host(wl.qh)[rows], hq_ref) and np.array_equal(host(wl.sh)[rows], hs_ref)
    y_ref = oracle.grouped_gemm_qint4(host(wl.qh), host(wl.sh), "sorted", d["w2"], d["w2_scale"], off, srt,
                                      d["k"], rows=rows)["y"]
    assert_rows_close(host(wl.y)[rows], y_ref, what="FC2 y")
    assert_rows_close(host(wl.out), oracle.scatter_combine(host(wl.y), p2s, d["topk_weights"]),
                      what="combine")
