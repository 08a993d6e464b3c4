"""Seeded random sweeps.  Whole layer steps: route prep -> one grouped GEMM ->
weighted combine, over random shapes (ragged, single-expert, single-token),
routings with -1 and out-of-range ids, activation-row modes, output types,
NVFP4 layouts and schedules.  Each step is compared with the oracle: the
routing tables and raw INT4 accumulators exactly, each GEMM's f32 output
within max_j |gpu - oracle| <= 2e-3 * ||oracle_row||_2 and its 16-bit
outputs as that output rounded, the combine against the oracle's combine of
the stored GEMM output.  Also the INT4 activation quantizer and the NVFP4
weight repack over random shapes, types and layouts, bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev, dev_f16, host, assert_rows_close

pytestmark = pytest.mark.gpu

mq = pytest.importorskip("quantized_moe_grouped_route_amd")

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}
N_CASES = 24


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _ids(rng, T, k, E):
    """Independent uniform ids with about 8 % -1 and 4 % ids in [E, E+5)."""
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    u = rng.random((T, k))
    ids = np.where(u < 0.08, -1, ids)
    ids = np.where((u >= 0.08) & (u < 0.12), rng.integers(E, E + 5, size=(T, k)), ids)
    return ids.astype(np.int32)


def _route(ids, E):
    """GPU tables (device tensors), checked against the oracle's."""
    offs, srt, p2s, ninv = mq.moe_route_prep(dev(ids), E)
    ref = oracle.route_prep(ids, E)
    for g, r in zip((offs, srt, p2s), ref[:3]):
        assert np.array_equal(host(g), r)
    assert int(host(ninv)[0]) == ref[3]
    return (offs, srt, p2s), ref


def _check_gemm(call, y_ref, odt, what):
    """The GEMM's f32 output against the oracle; a 16-bit output against the
    f32 output rounded (a single bf16 rounding can exceed the row tolerance
    on rows one element dominates): bf16 exactly, binary16 within one ulp
    (the last multiply may be fused with the conversion)."""
    n = y_ref.shape[0]
    y32 = call(torch.float32)
    assert_rows_close(host(y32)[:n], y_ref, what=what)
    if odt == "f32":
        return y32
    y = call(DT[odt])
    if odt == "bf16":
        assert torch.equal(y[:n], y32[:n].to(torch.bfloat16)), what
    else:
        h = host(y)[:n].astype(np.float32)
        f = host(y32)[:n].astype(np.float32)
        assert np.all(np.abs(h - f) <= np.spacing(np.abs(h).astype(np.float16)).astype(np.float32)), what
    return y


def _check_combine(y_gpu, n, p2s_gpu, ref_tables, tw, what):
    """The GPU combine of the GPU's y (its first n rows are the routed ones)
    against the oracle's combine of the same stored values."""
    y_host = np.zeros((y_gpu.shape[0], y_gpu.shape[1]))
    y_host[:n] = host(y_gpu)[:n]
    out = mq.moe_scatter_combine(y_gpu, p2s_gpu, dev(tw), out_dtype=torch.float32)
    ref = oracle.scatter_combine(y_host, ref_tables[2], tw)
    assert_rows_close(host(out), ref, what=f"{what} combine")


def _int4_case(i):
    rng = np.random.default_rng(3100 + i)
    T = int(rng.choice([1, 5, 33, 64, 130, 257]))
    E = int(rng.choice([1, 2, 5, 8, 17]))
    k = int(rng.integers(1, min(4, E) + 1))
    act = str(rng.choice(["none", "silu_mul"]))
    N = 32 * int(rng.integers(1, 10))
    K = 128 * int(rng.integers(1, 6))
    odt = str(rng.choice(["f16", "bf16", "f32"] + (["i32"] if act == "none" else [])))
    sched = str(rng.choice(["auto", "prefill"] + (["decode"] if K % 256 == 0 else [])))
    a_row = str(rng.choice(["token", "sorted"]))
    return dict(T=T, E=E, k=k, act=act, N=N, K=K, odt=odt, sched=sched, a_row=a_row, seed=3100 + i)


@pytest.mark.parametrize("case", [_int4_case(i) for i in range(N_CASES)],
                         ids=lambda c: "T{T}-E{E}-k{k}-N{N}-K{K}-{act}-{odt}-{sched}-{a_row}".format(**c))
def test_sweep_int4_layer_step(case):
    c = case
    d = synth.int4_moe(c["seed"], c["T"], c["E"], c["k"], c["N"], c["K"], routing="repeat")
    rng = np.random.default_rng(c["seed"] + 7)
    ids = _ids(rng, c["T"], c["k"], c["E"])
    (offs, srt, p2s), ref_t = _route(ids, c["E"])
    P = c["T"] * c["k"]
    if c["a_row"] == "sorted":
        a = synth.uniform_bytes(rng, (P, c["K"] // 2))
        sa = synth.uniform_f32(rng, (P,), 0.005, 0.05)
    else:
        a, sa = d["a"], d["a_scale"]
    args = (dev(a), dev(sa), dev(d["w"]), dev(d["w_scale"]), offs, srt, c["k"])
    call = lambda odt: mq.grouped_gemm_qint4(*args, a_row=c["a_row"], act=c["act"], out_dtype=odt,
                                             sched=c["sched"])
    ref = oracle.grouped_gemm_qint4(a, sa, c["a_row"], d["w"], d["w_scale"], ref_t[0], ref_t[1], c["k"],
                                    act=c["act"])
    n = ref["y"].shape[0]
    if c["odt"] == "i32":
        assert np.array_equal(host(call(torch.int32))[:n], ref["acc"])
        return
    y = _check_gemm(call, ref["y"], c["odt"], "int4 sweep")
    _check_combine(y, n, p2s, ref_t, d["topk_weights"], "int4 sweep")


def _fp8_case(i):
    rng = np.random.default_rng(3200 + i)
    T = int(rng.choice([1, 7, 40, 96, 201]))
    E = int(rng.choice([1, 3, 6, 9]))
    k = int(rng.integers(1, min(3, E) + 1))
    N = 128 * int(rng.integers(1, 4))
    K = 128 * int(rng.integers(1, 6))
    odt = str(rng.choice(["f16", "bf16", "f32"]))
    sched = str(rng.choice(["auto", "decode", "prefill"]))
    a_row = str(rng.choice(["token", "sorted"]))
    return dict(T=T, E=E, k=k, N=N, K=K, odt=odt, sched=sched, a_row=a_row, seed=3200 + i)


@pytest.mark.parametrize("case", [_fp8_case(i) for i in range(N_CASES)],
                         ids=lambda c: "T{T}-E{E}-k{k}-N{N}-K{K}-{odt}-{sched}-{a_row}".format(**c))
def test_sweep_fp8_layer_step(case):
    c = case
    d = synth.fp8_block(c["seed"], c["T"], c["N"], c["K"], c["E"], T=c["T"], k=c["k"])
    rng = np.random.default_rng(c["seed"] + 7)
    ids = _ids(rng, c["T"], c["k"], c["E"])
    (offs, srt, p2s), ref_t = _route(ids, c["E"])
    P = c["T"] * c["k"]
    if c["a_row"] == "sorted":
        a, sa = synth.fp8_quant_1x128(rng.standard_normal((P, c["K"]), dtype=np.float32))
    else:
        a, sa = d["a"], d["a_scale"]
    args = (dev(a), dev(sa), dev(d["w"]), dev(d["w_scale"]), offs, srt, c["k"])
    call = lambda odt: mq.grouped_gemm_qfp8_block(*args, a_row=c["a_row"], out_dtype=odt, sched=c["sched"])
    ref = oracle.grouped_gemm_qfp8_block(a, sa, c["a_row"], d["w"], d["w_scale"], ref_t[0], ref_t[1],
                                         c["k"])["y"]
    y = _check_gemm(call, ref, c["odt"], "fp8 sweep")
    _check_combine(y, ref.shape[0], p2s, ref_t, d["topk_weights"], "fp8 sweep")


def _nvfp4_case(i):
    rng = np.random.default_rng(3300 + i)
    T = int(rng.choice([1, 6, 31, 80, 150]))
    E = int(rng.choice([1, 4, 7, 12]))
    k = int(rng.integers(1, min(4, E) + 1))
    act = str(rng.choice(["none", "silu_mul"]))
    H = 128 * int(rng.integers(1, 7))
    I = 16 * int(rng.integers(2, 9))
    xdt = str(rng.choice(["bf16", "f16"]))
    sfl, wl = [("rows", "rows"), ("quads", "rows"), ("quads", "tiled")][int(rng.integers(0, 3))]
    odt = str(rng.choice(["f16", "bf16", "f32"]))
    sched = str(rng.choice(["auto", "decode", "prefill"]))
    a_row = str(rng.choice(["token", "sorted"]))
    return dict(T=T, E=E, k=k, act=act, H=H, I=I, xdt=xdt, sfl=sfl, wl=wl, odt=odt, sched=sched,
                a_row=a_row, seed=3300 + i)


@pytest.mark.parametrize("case", [_nvfp4_case(i) for i in range(N_CASES)],
                         ids=lambda c: "T{T}-E{E}-k{k}-H{H}-I{I}-{act}-{xdt}-{sfl}-{wl}-{odt}-{sched}-{a_row}".format(**c))
def test_sweep_nvfp4_layer_step(case):
    c = case
    d = synth.nvfp4_moe(c["seed"], c["T"], c["E"], c["k"], c["H"], c["I"], routing="repeat")
    rng = np.random.default_rng(c["seed"] + 7)
    ids = _ids(rng, c["T"], c["k"], c["E"])
    (offs, srt, p2s), ref_t = _route(ids, c["E"])
    P = c["T"] * c["k"]
    xb = synth.normal_bf16(rng, (P, c["H"])) if c["a_row"] == "sorted" else d["x"]
    if c["xdt"] == "f16":
        xo = oracle.bf16_to_f16_bits(xb)
        xg = dev_f16(xo)
    else:
        xo, xg = xb, dev(xb)
    sf = d["s1"] if c["sfl"] == "rows" else oracle.quads_from_rows(d["s1"])
    w = d["w1"] if c["wl"] == "rows" else oracle.tiles_from_rows(d["w1"])
    wg, sg, gg = dev(w), dev(sf), dev(d["g1"])
    call = lambda odt: mq.grouped_gemm_qnvfp4(xg, wg, sg, gg, offs, srt, c["k"], a_row=c["a_row"],
                                              act=c["act"], out_dtype=odt, sched=c["sched"])
    ref = oracle.grouped_gemm_qnvfp4(xo, c["a_row"], w, sf, d["g1"], ref_t[0], ref_t[1], c["k"], act=c["act"],
                                     x_dtype=c["xdt"], sf_layout=c["sfl"], w_layout=c["wl"])["y"]
    y = _check_gemm(call, ref, c["odt"], "nvfp4 sweep")
    _check_combine(y, ref.shape[0], p2s, ref_t, d["topk_weights"], "nvfp4 sweep")


def _quant_case(i):
    rng = np.random.default_rng(3400 + i)
    rows = int(rng.choice([1, 2, 9, 64, 257]))
    K = 16 * int(rng.choice([1, 3, 8, 65, 300, 1024, 1100]))
    dt = str(rng.choice(["f16", "bf16", "f32"]))
    scale = float(rng.choice([1e-3, 1.0, 300.0]))
    return dict(rows=rows, K=K, dt=dt, scale=scale, seed=3400 + i)


@pytest.mark.parametrize("case", [_quant_case(i) for i in range(N_CASES)],
                         ids=lambda c: "rows{rows}-K{K}-{dt}-x{scale}".format(**c))
def test_sweep_int4_quantizer(case):
    # per-row int4 codes and scales, bit-exact; some rows all zero, some with
    # a single nonzero element
    c = case
    rng = np.random.default_rng(c["seed"])
    x = (rng.standard_normal((c["rows"], c["K"])) * c["scale"]).astype(np.float32)
    x[rng.random(c["rows"]) < 0.1] = 0.0
    one = rng.random(c["rows"]) < 0.1
    x[one] = 0.0
    x[one, rng.integers(0, c["K"], size=int(one.sum()))] = -c["scale"]
    xt = torch.from_numpy(x).to(DT[c["dt"]]).cuda()
    q, s = mq.quantize_int4_rows(xt)
    ref_q, ref_s = oracle.quantize_int4_rows(xt.float().cpu().numpy())
    assert np.array_equal(host(q), ref_q)
    assert np.array_equal(host(s).astype(np.float32), ref_s)


def _repack_case(i):
    rng = np.random.default_rng(3500 + i)
    E = int(rng.choice([1, 2, 3]))
    N = 128 * int(rng.integers(1, 4))
    K = 64 * int(rng.choice([1, 2, 3, 5, 8]))
    swap = bool(rng.integers(0, 2)) and N % 256 == 0
    sfl = str(rng.choice(["rows", "quads"]))
    wl = str(rng.choice(["rows", "tiled"]))
    return dict(E=E, N=N, K=K, swap=swap, sfl=sfl, wl=wl, seed=3500 + i)


@pytest.mark.parametrize("case", [_repack_case(i) for i in range(N_CASES)],
                         ids=lambda c: "E{E}-N{N}-K{K}-swap{swap}-{sfl}-{wl}".format(**c))
def test_sweep_nvfp4_repack(case):
    # a pure byte permutation: bit-exact against the oracle's layouts
    c = case
    d = synth.nvfp4_stored_weights(c["seed"], c["E"], c["N"], c["K"])
    w_out, sf_out = mq.nvfp4_repack(dev(d["w"]), dev(d["sf"]), swap_halves=c["swap"],
                                    sf_layout=c["sfl"], w_layout=c["wl"])
    ref_w, ref_sf = oracle.repack_nvfp4(d["w"], d["sf"], c["swap"], out_layout=c["sfl"], w_layout=c["wl"])
    assert np.array_equal(host(w_out), ref_w)
    assert np.array_equal(host(sf_out), ref_sf)
