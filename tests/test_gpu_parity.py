"""GPU parity: every entry point of the HIP library against the CPU oracle on
the same seeded inputs.  Tables and integer accumulators must be equal;
floating outputs must satisfy max_j |gpu - oracle| <= 2e-3 * ||oracle_row||_2
per row."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev, dev_f16, host, bf16_bits, assert_rows_close

pytestmark = pytest.mark.gpu

mq = pytest.importorskip("quantized_moe_grouped_route_amd")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mq.lib()


def _route_gpu(ids, E):
    offs, srt, p2s, ninv = mq.moe_route_prep(dev(ids.astype(np.int32)), E)
    return host(offs), host(srt), host(p2s), int(host(ninv)[0])


# ------------------------------------------------------------------ route
ROUTE_CASES = [
    ("tiny", lambda r: synth.distinct_uniform_ids(r, 5, 2, 4), 4),
    ("repeats", lambda r: synth.uniform_ids_with_repeats(r, 300, 3, 7), 7),
    ("minus1_and_invalid", lambda r: np.where(r.random((333, 3)) < 0.2, -1,
                                              r.integers(-3, 12, size=(333, 3))).astype(np.int32), 9),
    ("E1", lambda r: np.zeros((1024, 1), np.int32), 1),
    ("T0", lambda r: np.zeros((0, 2), np.int32), 4),
    ("all_minus1", lambda r: -np.ones((70, 2), np.int32), 3),
    ("multi_chunk", lambda r: synth.uniform_ids_with_repeats(r, 1500, 4, 33), 33),
    ("multi_chunk_ragged", lambda r: np.where(r.random((2049, 3)) < 0.1, -1,
                                              synth.uniform_ids_with_repeats(r, 2049, 3, 5)), 5),
    ("E1024", lambda r: synth.uniform_ids_with_repeats(r, 700, 8, 1024), 1024),
    ("zipf_T4096", lambda r: synth.zipf_ids(r, 4096, 8, 256), 256),
    ("mixtral_T8192", lambda r: synth.distinct_uniform_ids(r, 8192, 2, 8), 8),
    ("decode_T8", lambda r: synth.distinct_uniform_ids(r, 8, 8, 256), 256),
    # E > 16 ranks by the 64-step scan: with -1 and out-of-range ids, and
    # with every pair of a wave on one expert
    ("minus1_and_invalid_E64", lambda r: np.where(r.random((333, 3)) < 0.2, -1,
                                                  r.integers(-3, 70, size=(333, 3))).astype(np.int32), 64),
    ("one_expert_E256", lambda r: np.full((300, 3), 17, np.int32), 256),
    ("one_expert_E256_multi_chunk", lambda r: np.full((700, 3), 200, np.int32), 256),
    # the 4-wave workgroup (P <= 256) and its boundary
    ("minus1_and_invalid_P240_E40", lambda r: np.where(r.random((80, 3)) < 0.2, -1,
                                                       r.integers(-3, 45, size=(80, 3))).astype(np.int32), 40),
    ("boundary_P256", lambda r: synth.uniform_ids_with_repeats(r, 128, 2, 20), 20),
    ("boundary_P257", lambda r: synth.uniform_ids_with_repeats(r, 257, 1, 20), 20),
]


@pytest.mark.parametrize("name,make,E", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_prep_exact(name, make, E):
    ids = make(np.random.default_rng(11)).astype(np.int32)
    ref = oracle.route_prep(ids, E)
    got = _route_gpu(ids, E) if ids.size else None
    if ids.size == 0:
        offs, srt, p2s, ninv = mq.moe_route_prep(torch.zeros((0, ids.shape[1]), dtype=torch.int32,
                                                             device="cuda"), E)
        assert host(offs).tolist() == [0] * (E + 1) and int(host(ninv)[0]) == 0
        return
    for g, r in zip(got[:3], ref[:3]):
        assert np.array_equal(g, r)
    assert got[3] == ref[3]


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("ydt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16),
                                     (torch.float32, torch.float32), (torch.float32, torch.bfloat16)])
def test_combine(ydt, odt):
    rng = np.random.default_rng(5)
    T, k, E, N = 97, 4, 6, 520
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    ids[3] = -1
    ids[10, 2] = -1
    w = synth.softmax_weights(rng, T, k)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    y = torch.randn(T * k, N, device="cuda").to(ydt)
    out = mq.moe_scatter_combine(y, p2s, dev(w), out_dtype=odt)
    ref = oracle.scatter_combine(host(y), host(p2s), w)
    assert_rows_close(host(out), ref, what="combine")
    assert torch.all(out[3] == 0)


# ------------------------------------------------------------------ INT4
def _int4_case(seed, T, E, k, N, K, routing="distinct"):
    d = synth.int4_moe(seed, T, E, k, N, K, routing=routing)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    return d, offs, srt, p2s


@pytest.mark.parametrize("sched", ["prefill", "auto"])
@pytest.mark.parametrize("T,E,k,N,K", [(300, 5, 2, 384, 512), (64, 4, 2, 256, 256),
                                       (37, 3, 3, 128, 128), (5, 8, 2, 256, 384)])
def test_int4_raw_accumulator_bit_exact(sched, T, E, k, N, K):
    d, offs, srt, p2s = _int4_case(21, T, E, k, N, K, routing="repeat")
    acc = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                                offs, srt, k, out_dtype=torch.int32, sched=sched)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), k)
    n = int(host(offs)[-1])
    assert np.array_equal(host(acc)[:n], ref["acc"])


@pytest.mark.parametrize("sched", ["prefill", "auto"])
@pytest.mark.parametrize("odt", [torch.float16, torch.bfloat16, torch.float32])
def test_int4_scaled(sched, odt):
    d, offs, srt, p2s = _int4_case(22, 300, 5, 2, 384, 512)
    y = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                              offs, srt, 2, out_dtype=odt, sched=sched)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), 2)
    assert_rows_close(host(y)[: ref["y"].shape[0]], ref["y"], what="int4")


@pytest.mark.parametrize("sched", ["prefill", "auto"])
def test_int4_silu_mul_and_sorted_rows(sched):
    d, offs, srt, p2s = _int4_case(23, 200, 4, 2, 512, 256)
    h = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                              offs, srt, 2, act="silu_mul", out_dtype=torch.float16, sched=sched)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), 2, act="silu_mul")
    assert_rows_close(host(h)[: ref["y"].shape[0]], ref["y"], what="int4 silu")
    # SORTED rows: A already in sorted order
    rng = np.random.default_rng(3)
    P = 400
    a2 = synth.uniform_bytes(rng, (P, 128))
    s2 = synth.uniform_f32(rng, (P,), 0.005, 0.05)
    y2 = mq.grouped_gemm_qint4(dev(a2), dev(s2), dev(d["w"][:, :, :128].copy()),
                               dev(d["w_scale"]), offs, srt, 2, a_row="sorted",
                               out_dtype=torch.int32, sched=sched)
    ref2 = oracle.grouped_gemm_qint4(a2, s2, "sorted", d["w"][:, :, :128], d["w_scale"],
                                     host(offs), host(srt), 2)
    assert np.array_equal(host(y2)[: ref2["acc"].shape[0]], ref2["acc"])


@pytest.mark.parametrize("sched", ["prefill", "auto"])
def test_int4_rows_past_offsets_untouched_and_empty_experts(sched):
    T, E, k, N, K = 50, 6, 2, 256, 256
    d = synth.int4_moe(24, T, E, k, N, K)
    d["topk_ids"][d["topk_ids"] >= 3] = -1          # experts 3..5 empty, some pairs skipped
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    n = int(host(offs)[-1])
    out = torch.full((T * k, N), 12345, dtype=torch.int32, device="cuda")
    mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                          offs, srt, k, out_dtype=torch.int32, out=out, sched=sched)
    assert torch.all(out[n:] == 12345)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), k)
    assert np.array_equal(host(out)[:n], ref["acc"])


@pytest.mark.parametrize("sched", ["prefill", "auto"])
def test_int4_extreme_codes(sched):
    # all codes -8: acc = 64*K per element, the largest magnitude
    T, E, N, K = 40, 2, 128, 4096
    ids = np.zeros((T, 1), np.int32)
    ids[::2] = 1
    a = np.full((T, K // 2), 0x88, np.uint8)
    w = np.full((E, N, K // 2), 0x88, np.uint8)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    acc = mq.grouped_gemm_qint4(dev(a), dev(np.ones(T, np.float32)), dev(w),
                                dev(np.ones((E, N), np.float32)), offs, srt, 1,
                                out_dtype=torch.int32, sched=sched)
    assert torch.all(acc == 64 * K)


# INT4 weight-streaming schedule (few rows per expert).  AUTO takes it for
# P < 16 E with K % 256 == 0; its arithmetic is the tiled schedule's, so the
# two schedules must give identical outputs as well as meet the oracle.
INT4_DECODE_CASES = [
    (8, 8, 2, 256, 512),      # Mixtral-like decode routing, tiny shapes
    (5, 16, 4, 96, 256),      # N not a multiple of 64, one K group
    (33, 4, 1, 160, 768),     # several 4-row tiles per expert, ragged last tile
    (1, 3, 1, 32, 256),       # one row, one 32-row weight block
    (60, 8, 2, 4096, 4096),   # more items than waves: two rounds per wave
]


@pytest.mark.parametrize("sched", ["decode", "auto"])
@pytest.mark.parametrize("T,E,k,N,K", INT4_DECODE_CASES)
def test_int4_decode_raw_accumulator_bit_exact(sched, T, E, k, N, K):
    d, offs, srt, p2s = _int4_case(31, T, E, k, N, K, routing="repeat")
    assert T * k < 16 * E  # AUTO must pick the streaming schedule here
    acc = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                                offs, srt, k, out_dtype=torch.int32, sched=sched)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), k)
    n = int(host(offs)[-1])
    assert np.array_equal(host(acc)[:n], ref["acc"])


@pytest.mark.parametrize("act", ["none", "silu_mul"])
@pytest.mark.parametrize("T,E,k,N,K", [INT4_DECODE_CASES[0], INT4_DECODE_CASES[2], INT4_DECODE_CASES[4]])
def test_int4_decode_scaled_matches_oracle_and_tiled_schedule(act, T, E, k, N, K):
    d, offs, srt, p2s = _int4_case(32, T, E, k, N, K)
    args = (dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), k, act=act)
    n = ref["y"].shape[0]
    y32 = mq.grouped_gemm_qint4(*args, act=act, out_dtype=torch.float32, sched="decode")
    assert_rows_close(host(y32)[:n], ref["y"], what=f"int4 decode {act}")
    for odt in (torch.float32, torch.float16, torch.bfloat16):
        y_dec = mq.grouped_gemm_qint4(*args, act=act, out_dtype=odt, sched="decode")
        y_til = mq.grouped_gemm_qint4(*args, act=act, out_dtype=odt, sched="prefill")
        assert torch.equal(y_dec[:n], y_til[:n]), odt
        if odt == torch.float16:
            # the last multiply may be fused with the conversion (one rounding
            # of the exact product straight to binary16), so a binary16 output
            # is the f32 output rounded, or its neighbour where rounding twice
            # would differ: within one binary16 ulp
            h = host(y_dec)[:n].astype(np.float32)
            f = host(y32)[:n]
            assert np.all(np.abs(h - f) <= np.spacing(np.abs(h).astype(np.float16)).astype(np.float32)), odt
            assert np.mean(h == f.astype(np.float16).astype(np.float32)) > 0.999
        else:
            assert torch.equal(y_dec[:n], y32[:n].to(odt)), odt


def test_int4_decode_sorted_rows_invalid_ids_and_untouched_rows():
    T, E, k, N, K = 40, 12, 2, 320, 1024
    d = synth.int4_moe(33, T, E, k, N, K, routing="repeat")
    ids = d["topk_ids"].copy()
    ids[ids >= 9] = -1                               # experts 9..11 empty, some pairs skipped
    ids[::7, 0] = 99                                 # out-of-range ids are skipped too
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    n = int(host(offs)[-1])
    # TOKEN rows, I32, rows past the routed ones untouched
    out = torch.full((T * k, N), 12345, dtype=torch.int32, device="cuda")
    mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                          offs, srt, k, out_dtype=torch.int32, out=out, sched="decode")
    assert torch.all(out[n:] == 12345)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                    host(offs), host(srt), k)
    assert np.array_equal(host(out)[:n], ref["acc"])
    # SORTED rows with SiLU: A holds one row per routed pair
    rng = np.random.default_rng(34)
    a2 = synth.uniform_bytes(rng, (T * k, K // 2))
    s2 = synth.uniform_f32(rng, (T * k,), 0.005, 0.05)
    h = torch.full((T * k, N // 2), -7.0, dtype=torch.float32, device="cuda")
    mq.grouped_gemm_qint4(dev(a2), dev(s2), dev(d["w"]), dev(d["w_scale"]), offs, srt, k, a_row="sorted",
                          act="silu_mul", out_dtype=torch.float32, out=h, sched="decode")
    ref2 = oracle.grouped_gemm_qint4(a2, s2, "sorted", d["w"], d["w_scale"], host(offs), host(srt), k,
                                     act="silu_mul")
    assert_rows_close(host(h)[:n], ref2["y"], what="int4 decode sorted silu")
    assert torch.all(h[n:] == -7.0)


def test_int4_decode_extreme_codes_and_no_rows():
    # all codes -8 at the largest K the streaming schedule is given here
    T, E, N, K = 6, 2, 64, 8192
    ids = np.zeros((T, 1), np.int32)
    ids[::2] = 1
    a = np.full((T, K // 2), 0x88, np.uint8)
    w = np.full((E, N, K // 2), 0x88, np.uint8)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    acc = mq.grouped_gemm_qint4(dev(a), dev(np.ones(T, np.float32)), dev(w),
                                dev(np.ones((E, N), np.float32)), offs, srt, 1,
                                out_dtype=torch.int32, sched="decode")
    assert torch.all(acc == 64 * K)
    # every id -1: no routed rows, the output is left as it was
    ids = -np.ones((T, 1), np.int32)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    out = torch.full((T, N), 77, dtype=torch.int32, device="cuda")
    mq.grouped_gemm_qint4(dev(a), dev(np.ones(T, np.float32)), dev(w), dev(np.ones((E, N), np.float32)),
                          offs, srt, 1, out_dtype=torch.int32, out=out, sched="decode")
    assert torch.all(out == 77)


# ------------------------------------------------------------------ FP8
@pytest.mark.parametrize("M,N,K", [(300, 256, 512), (128, 128, 128), (1, 384, 256)])
def test_fp8_dense(M, N, K):
    d = synth.fp8_block(31, M, N, K)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), 1)
    y = mq.grouped_gemm_qfp8_block(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                                   offs, srt, 1, out_dtype=torch.float32)
    ref = oracle.fp8_dense(d)
    assert_rows_close(host(y), ref, what="fp8")


def test_fp8_routed_scales_vary_on_every_index():
    rng = np.random.default_rng(9)
    d = synth.fp8_block(32, 0, 256, 384, E=3, T=150, k=2)
    d["a_scale"] = synth.uniform_f32(rng, d["a_scale"].shape, 0.25, 4.0)
    d["w_scale"] = synth.uniform_f32(rng, d["w_scale"].shape, 0.25, 4.0)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), 3)
    y = mq.grouped_gemm_qfp8_block(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]),
                                   offs, srt, 2, out_dtype=torch.bfloat16)
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                         host(offs), host(srt), 2)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what="fp8 routed")


@pytest.mark.parametrize("sched", ["auto", "decode", "prefill"])
@pytest.mark.parametrize("T,E,k,N,K,odt", [(8, 16, 4, 256, 512, torch.bfloat16),
                                           (37, 5, 2, 384, 128, torch.float32),
                                           (3, 64, 8, 128, 1152, torch.float16)])
def test_fp8_decode_schedule(sched, T, E, k, N, K, odt):
    # AUTO picks the weight-streaming decode schedule for all three (P < 16 E);
    # both forced schedules must agree with the oracle.  K = 128 is one K
    # group, K = 1152 is nine (past the ring depth, not a multiple of it);
    # tiles of 1..4 rows; rows past offsets[E] stay untouched.
    d = synth.fp8_block(33, 0, N, K, E=E, T=T, k=k)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    P = T * k
    out = torch.full((P + 5, N), 7.0, dtype=odt, device="cuda")
    mq.grouped_gemm_qfp8_block(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k,
                               out_dtype=odt, sched=sched, out=out[:P])
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"],
                                         host(offs), host(srt), k)["y"]
    n = ref.shape[0]
    assert_rows_close(host(out)[:n].astype(np.float64), ref, what=f"fp8 {sched}")
    assert (host(out)[P:] == 7.0).all()


def test_fp8_decode_sorted_rows_and_empty_experts():
    # SORTED A (row = sorted position), experts 0 and 3 empty, tiles with 1..4 rows.
    rng = np.random.default_rng(34)
    E, N, K = 5, 256, 640
    counts = np.array([0, 3, 9, 0, 6])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = int(offs[-1])
    a, sa = synth.fp8_quant_1x128(rng.standard_normal((P, K)).astype(np.float32))
    d = synth.fp8_block(35, 0, N, K, E=E, T=4, k=2)
    y = mq.grouped_gemm_qfp8_block(dev(a), dev(sa), dev(d["w"]), dev(d["w_scale"]), dev(offs), None, 1,
                                   a_row="sorted", out_dtype=torch.float32, sched="decode")
    ref = oracle.grouped_gemm_qfp8_block(a, sa, "sorted", d["w"], d["w_scale"], offs, None, 1)["y"]
    assert_rows_close(host(y), ref, what="fp8 decode sorted")


# ------------------------------------------------------------------ NVFP4
def _xin(x_bf16_bits, xdt):
    """Activations for the GEMM in the form xdt ('bf16' or 'f16'): (device
    tensor, the bits the oracle reads).  The f16 form is the oracle's
    rounding of the bf16 values (exact for these inputs' magnitudes except
    the rare |x| < 2^-14)."""
    if xdt == "bf16":
        return dev(x_bf16_bits), x_bf16_bits
    bits = oracle.bf16_to_f16_bits(x_bf16_bits)
    return dev_f16(bits), bits


def _sf(s_rows, sfl):
    """Scales in layout sfl ('rows' or 'quads'): (device tensor, oracle array)."""
    a = s_rows if sfl == "rows" else oracle.quads_from_rows(s_rows)
    return dev(a), a


def _w(w_rows, wl):
    """Codes in layout wl ('rows' or 'tiled'): (device tensor, oracle array)."""
    a = w_rows if wl == "rows" else oracle.tiles_from_rows(w_rows)
    return dev(a), a


@pytest.mark.parametrize("I", [128, 256])
@pytest.mark.parametrize("wl,sfl", [("rows", "rows"), ("rows", "quads"), ("tiled", "quads")])
@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("sched", ["prefill", "decode"])
@pytest.mark.parametrize("act", ["none", "silu_mul"])
def test_nvfp4(sched, act, xdt, wl, sfl, I):
    # N = 2I = 256: the 256-row prefill tile; N = 512: the 512-row tile
    T, E, k, H = 150, 5, 2, 256
    d = synth.nvfp4_moe(41, T, E, k, H, I, routing="repeat")
    xg, xb = _xin(d["x"], xdt)
    sg, sa = _sf(d["s1"], sfl)
    wg, wa = _w(d["w1"], wl)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(xg, wg, sg, dev(d["g1"]), offs, srt, k,
                               act=act, out_dtype=torch.float32, sched=sched)
    ref = oracle.grouped_gemm_qnvfp4(xb, "token", wa, sa, d["g1"], host(offs),
                                     host(srt), k, act=act, x_dtype=xdt, sf_layout=sfl, w_layout=wl)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 {sched} {act} {xdt} {wl} {sfl}")


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("sched", ["prefill", "decode"])
def test_nvfp4_sorted_rows_full_code_range(sched, xdt):
    # every scale byte 0x00..0x7E occurs; SORTED activation rows
    T, E, k, H, I = 64, 3, 2, 512, 128
    d = synth.nvfp4_moe(42, T, E, k, H, I, scale_lo=0x00, scale_hi=0x7E)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    P = T * k
    xg, xb = _xin(synth.normal_bf16(np.random.default_rng(1), (P, I)), xdt)
    y = mq.grouped_gemm_qnvfp4(xg, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k,
                               a_row="sorted", out_dtype=torch.float32, sched=sched)
    ref = oracle.grouped_gemm_qnvfp4(xb, "sorted", d["w2"], d["s2"], d["g2"], host(offs),
                                     host(srt), k, x_dtype=xdt)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 sorted {sched} {xdt}")


@pytest.mark.parametrize("xdt,sfl,wl", [("bf16", "rows", "rows"), ("f16", "rows", "rows"), ("f16", "quads", "rows"),
                                        ("f16", "quads", "tiled")])
@pytest.mark.parametrize("H", [1024, 1536, 2176, 3200])
def test_nvfp4_decode_chunk_counts(H, xdt, sfl, wl):
    # K / 128 = 8, 12, 17, 25 weight chunks per lane: exactly the in-flight
    # depth, a partial refill, one steady pass plus a tail, several passes
    # plus a ragged tail.
    T, E, k, I = 20, 3, 2, 128
    d = synth.nvfp4_moe(45, T, E, k, H, I, routing="repeat")
    xg, xb = _xin(d["x"], xdt)
    sg, sa = _sf(d["s1"], sfl)
    wg, wa = _w(d["w1"], wl)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(xg, wg, sg, dev(d["g1"]), offs, srt, k,
                               act="silu_mul", out_dtype=torch.float32, sched="decode")
    ref = oracle.grouped_gemm_qnvfp4(xb, "token", wa, sa, d["g1"], host(offs),
                                     host(srt), k, act="silu_mul", x_dtype=xdt, sf_layout=sfl, w_layout=wl)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 decode H={H} {xdt}")


@pytest.mark.parametrize("I", [64, 192])
@pytest.mark.parametrize("sched", ["prefill", "auto"])
def test_nvfp4_n_not_multiple_of_prefill_tile(I, sched):
    # N = 2I = 128 or 384 is not a multiple of the 256-wide prefill tile:
    # every column must still be computed.
    T, E, k, H = 150, 5, 2, 256
    d = synth.nvfp4_moe(46, T, E, k, H, I, routing="repeat")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k,
                               act="silu_mul", out_dtype=torch.float32, sched=sched)
    ref = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs),
                                     host(srt), k, act="silu_mul")["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 N={2 * I} {sched}")


@pytest.mark.parametrize("xdt,sfl,wl", [("bf16", "rows", "rows"), ("f16", "rows", "rows"), ("f16", "quads", "rows"),
                                        ("f16", "quads", "tiled")])
@pytest.mark.parametrize("act", ["silu_mul", "none"])
def test_nvfp4_decode_several_items_per_wave(act, xdt, sfl, wl):
    # More 4-row tiles x column blocks than the streaming schedule has waves,
    # so each wave runs several items back to back, with K / 512 = 3 (an odd
    # number of 4-chunk groups per item) and ragged last tiles.
    T, E, k, H, I = 203, 4, 2, 1536, 512
    d = synth.nvfp4_moe(47, T, E, k, H, I, routing="repeat")
    xg, xb = _xin(d["x"], xdt)
    sg, sa = _sf(d["s1"], sfl)
    wg, wa = _w(d["w1"], wl)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(xg, wg, sg, dev(d["g1"]), offs, srt, k,
                               act=act, out_dtype=torch.float32, sched="decode")
    ref = oracle.grouped_gemm_qnvfp4(xb, "token", wa, sa, d["g1"], host(offs),
                                     host(srt), k, act=act, x_dtype=xdt, sf_layout=sfl, w_layout=wl)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 decode many items {act}")


@pytest.mark.parametrize("H", [512, 384])
def test_nvfp4_decode_more_than_64_items_per_wave(H):
    # 8192 pairs over 8 experts x 128 column blocks: about 128 items per
    # streaming wave, so each wave reloads its per-lane item metadata table
    # (64 items per table) while its copy ring is running.  H = 512 takes
    # the 512-K stream, H = 384 the 128-K one.
    T, E, k, I = 4096, 8, 2, 2048
    d = synth.nvfp4_moe(48, T, E, k, H, I, routing="repeat")
    xg, xb = _xin(d["x"], "f16")
    sg, sa = _sf(d["s1"], "quads")
    wg, wa = _w(d["w1"], "tiled")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(xg, wg, sg, dev(d["g1"]), offs, srt, k,
                               act="silu_mul", out_dtype=torch.float32, sched="decode")
    ref = oracle.grouped_gemm_qnvfp4(xb, "token", wa, sa, d["g1"], host(offs), host(srt), k,
                                     act="silu_mul", x_dtype="f16", sf_layout="quads", w_layout="tiled")["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"nvfp4 decode >64 items H={H}")


def test_both_schedules_meet_tolerance():
    # decode and prefill both sum exact bf16 products in fp32; they may round
    # differently, but both must meet the tolerance on the same input.
    T, E, k, H, I = 24, 4, 2, 256, 128
    d = synth.nvfp4_moe(43, T, E, k, H, I)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    ys = [host(mq.grouped_gemm_qnvfp4(dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs,
                                      srt, k, out_dtype=torch.float32, sched=s))
          for s in ("prefill", "decode")]
    ref = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs),
                                     host(srt), k)["y"]
    for y in ys:
        assert_rows_close(y[: ref.shape[0]], ref, what="nvfp4 schedules")


def test_repeat_runs_bitwise_identical():
    d = synth.nvfp4_moe(44, 100, 4, 2, 256, 128)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), 4)
    args = (dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, 2)
    a = mq.grouped_gemm_qnvfp4(*args, act="silu_mul")
    b = mq.grouped_gemm_qnvfp4(*args, act="silu_mul")
    assert torch.equal(a, b)


@pytest.mark.parametrize("I", [512, 384])       # 512-row tiles (8 waves), 256-row tiles (4 waves)
@pytest.mark.parametrize("pair", [False, True])
def test_nvfp4_work_queue_same_outputs_and_left_zero(I, pair):
    # skewed routing: many partial m-tiles of unequal cost, more tiles than
    # workgroups; the queue only changes which workgroup computes a tile
    T, E, k, H = 600, 40, 4, 1024
    d = synth.nvfp4_moe(45, T, E, k, H, I, routing="zipf")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    x = dev(d["x"])
    wq = mq.work_queue()
    fc1 = dict(act="silu_mul", out_dtype=torch.bfloat16, sched="prefill")
    h0 = mq.grouped_gemm_qnvfp4(x, dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k, **fc1)
    for _ in range(3):  # the queue is left zero by each call, so every call sees all tiles
        h1 = mq.grouped_gemm_qnvfp4(x, dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k, **fc1,
                                    work_queue=wq)
        assert torch.equal(h0, h1)
        assert torch.all(wq == 0)
    tw = dev(d["topk_weights"].reshape(-1).astype(np.float32)) if pair else None
    fc2 = dict(a_row="sorted", out_dtype=torch.float32, sched="prefill", pair_weights=tw, P=T * k)
    y0 = mq.grouped_gemm_qnvfp4(h0, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, **fc2)
    y1 = mq.grouped_gemm_qnvfp4(h0, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, **fc2,
                                work_queue=wq)
    n = int(host(offs)[-1])
    rows = host(srt)[:n] if pair else np.arange(n)
    assert torch.equal(y0[rows], y1[rows]) and torch.all(wq == 0)
    ref = oracle.grouped_gemm_qnvfp4(bf16_bits(h0), "sorted", d["w2"], d["s2"], d["g2"], host(offs),
                                     host(srt), k)["y"]
    if pair:
        ref = ref * d["topk_weights"].reshape(-1)[host(srt)[:n]][:, None]
    assert_rows_close(host(y1)[rows], ref, what=f"nvfp4 work queue FC2 pair={pair}")


# ------------------------------------------------------------------ INT4 activation quantizer
def _quant_check(x_np, torch_dtype):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(torch_dtype)
    q, s = mq.quantize_int4_rows(x.cuda())
    ref_q, ref_s = oracle.quantize_int4_rows(x.float().numpy())
    assert np.array_equal(host(s), ref_s), "scales differ"
    assert np.array_equal(host(q), ref_q), "codes differ"


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,K", [(1, 16), (33, 256), (7, 14336), (130, 528), (3, 32784)])
def test_quantize_int4_bit_exact(dt, rows, K):
    rng = np.random.default_rng(rows * 131 + K)
    x = rng.standard_normal((rows, K)) * rng.uniform(1e-2, 1e2, (rows, 1))
    _quant_check(x, dt)


def test_quantize_int4_ties_zero_and_tiny_rows():
    K = 64
    x = np.zeros((4, K), np.float32)
    # amax 7 -> multiplier 1: exact halves round to even
    x[0, :8] = [7.0, -7.0, 2.5, 3.5, -0.5, 0.5, -2.5, 1.5]
    x[1, 3] = 2.0 ** -125                      # below the tiny threshold
    x[3, :] = np.linspace(-3.0, 3.0, K)        # every row value distinct
    _quant_check(x, torch.float32)
    q, s = mq.quantize_int4_rows(torch.from_numpy(x).cuda())
    codes = oracle.int4_value(oracle.unpack_nibbles(host(q)))
    assert list(codes[0, :8]) == [7, -7, 2, 4, 0, 0, -2, 2]
    assert np.all(codes[1:3] == 0) and host(s)[1] == 1 and host(s)[2] == 1


def test_w4a4_chain_with_quantized_activations():
    # fp16 x -> per-token int4 -> FC1 (SiLU-gated, fp16 h) -> per-row int4
    # of h -> FC2 on sorted rows -> combine; each GPU step checked against
    # the oracle applied to the GPU's own inputs of that step, and the codes
    # of both quantizations bit-exact.
    T, E, k, H, I = 96, 4, 2, 256, 384
    rng = np.random.default_rng(21)
    d = synth.int4_moe(22, T, E, k, 2 * I, H, routing="distinct")
    x = (rng.standard_normal((T, H)) * 2).astype(np.float16)
    w2 = synth.uniform_bytes(np.random.default_rng(23), (E, H, I // 2))
    sw2 = synth.uniform_f32(np.random.default_rng(24), (E, H), 0.005, 0.05)
    ids = dev(d["topk_ids"])
    offs, srt, p2s, _ = mq.moe_route_prep(ids, E)
    qa, sa = mq.quantize_int4_rows(torch.from_numpy(x).cuda())
    ref_qa, ref_sa = oracle.quantize_int4_rows(x)
    assert np.array_equal(host(qa), ref_qa) and np.array_equal(host(sa), ref_sa)
    h = mq.grouped_gemm_qint4(qa, sa, dev(d["w"]), dev(d["w_scale"]), offs, srt, k, act="silu_mul",
                              out_dtype=torch.float16)
    ref_h = oracle.grouped_gemm_qint4(ref_qa, ref_sa, "token", d["w"], d["w_scale"], host(offs),
                                      host(srt), k, act="silu_mul")["y"]
    n = ref_h.shape[0]
    assert_rows_close(host(h)[:n].astype(np.float64), ref_h, what="chain FC1")
    qh, sh = mq.quantize_int4_rows(h[:n].contiguous())
    ref_qh, ref_sh = oracle.quantize_int4_rows(host(h)[:n])
    assert np.array_equal(host(qh), ref_qh) and np.array_equal(host(sh), ref_sh)
    y = mq.grouped_gemm_qint4(qh, sh, dev(w2), dev(sw2), offs, srt, k, a_row="sorted",
                              out_dtype=torch.float16)
    ref_y = oracle.grouped_gemm_qint4(ref_qh, ref_sh, "sorted", w2, sw2, host(offs), host(srt), k)["y"]
    assert_rows_close(host(y)[:n].astype(np.float64), ref_y, what="chain FC2")
    out = mq.moe_scatter_combine(y, p2s, dev(d["topk_weights"]), out_dtype=torch.float32)
    ref_out = oracle.scatter_combine(host(y).astype(np.float64), host(p2s), d["topk_weights"])
    assert_rows_close(host(out), ref_out, what="chain combine")


# ------------------------------------------------------- NVFP4 layout repack
@pytest.mark.parametrize("E,N,K", [(1, 128, 64), (3, 256, 128), (2, 384, 1216), (2, 512, 2176),
                                   (1, 256, 4096)])
@pytest.mark.parametrize("swap", [False, True])
@pytest.mark.parametrize("wl,sfl", [("rows", "rows"), ("rows", "quads"), ("tiled", "quads")])
def test_nvfp4_repack_bit_exact(E, N, K, swap, wl, sfl):
    # K/64 = 1, 2, 19, 34, 64 scale quads per row: a partial 16-tile group,
    # ragged tails and whole groups; N/128 = 1..4 row blocks.
    d = synth.nvfp4_stored_weights(60 + N + K, E, N, K)
    w_out, sf_out = mq.nvfp4_repack(dev(d["w"]), dev(d["sf"]), swap_halves=swap, sf_layout=sfl, w_layout=wl)
    rw, rs = oracle.repack_nvfp4(d["w"], d["sf"], swap, out_layout=sfl, w_layout=wl)
    assert np.array_equal(host(w_out), rw)
    assert np.array_equal(host(sf_out), rs)


def test_nvfp4_repack_leaves_bytes_outside_untouched():
    E, N, K = 2, 256, 256
    d = synth.nvfp4_stored_weights(70, E, N, K)
    w_big = torch.full((E + 1, N, K // 2), 0xA5, dtype=torch.uint8, device="cuda")
    s_big = torch.full((E + 1, N, K // 16), 0x5A, dtype=torch.uint8, device="cuda")
    mq.nvfp4_repack(dev(d["w"]), dev(d["sf"]), swap_halves=True, w_out=w_big[:E], sf_out=s_big[:E])
    rw, rs = oracle.repack_nvfp4(d["w"], d["sf"], True)
    assert np.array_equal(host(w_big[:E]), rw) and np.array_equal(host(s_big[:E]), rs)
    assert bool((w_big[E] == 0xA5).all()) and bool((s_big[E] == 0x5A).all())


def test_nvfp4_repacked_layer_matches_gate_first_layer():
    # Weights generated gate-first (the library's layout) are put into the
    # up-first, swizzled layout on the host, repacked on the GPU, and must
    # give back the original bytes and the same FC1 (SiLU-gated) and FC2
    # outputs as the original layout.
    T, E, k, H, I = 96, 4, 2, 384, 256
    d = synth.nvfp4_moe(61, T, E, k, H, I, routing="repeat")
    up_first = np.concatenate([d["w1"][:, I:], d["w1"][:, :I]], axis=1)
    s_up_first = oracle.swizzle_scales(np.concatenate([d["s1"][:, I:], d["s1"][:, :I]], axis=1))
    s2_swz = oracle.swizzle_scales(d["s2"])
    w1, s1 = mq.nvfp4_repack(dev(up_first), dev(s_up_first), swap_halves=True)
    w2, s2 = mq.nvfp4_repack(dev(d["w2"]), dev(s2_swz), swap_halves=False)
    assert np.array_equal(host(w1), d["w1"]) and np.array_equal(host(s1), d["s1"])
    assert np.array_equal(host(w2), d["w2"]) and np.array_equal(host(s2), d["s2"])
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    h = mq.grouped_gemm_qnvfp4(dev(d["x"]), w1, s1, dev(d["g1"]), offs, srt, k, act="silu_mul")
    ref_h = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt),
                                       k, act="silu_mul")["y"]
    assert_rows_close(host(h)[: ref_h.shape[0]], ref_h, what="FC1 on repacked weights")
    y = mq.grouped_gemm_qnvfp4(h, w2, s2, dev(d["g2"]), offs, srt, k, a_row="sorted",
                               out_dtype=torch.float32)
    ref_y = oracle.grouped_gemm_qnvfp4(bf16_bits(h), "sorted", d["w2"], d["s2"], d["g2"], host(offs),
                                       host(srt), k)["y"]
    assert_rows_close(host(y)[: ref_y.shape[0]], ref_y, what="FC2 on repacked weights")


def test_nvfp4_u32_packed_scales_are_the_same_bytes():
    # [TLK]'s packed form: word g of a row holds blocks 4g..4g+3, block 4g+j
    # in bits 8j..8j+7; built here with explicit shifts, not a memory view
    T, E, k, H, I = 40, 3, 2, 256, 128
    d = synth.nvfp4_moe(62, T, E, k, H, I)
    b = d["s1"].astype(np.uint32).reshape(E, 2 * I, H // 64, 4)
    packed = (b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)).astype(np.uint32)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qnvfp4(dev(d["x"]), dev(d["w1"]), dev(packed.view(np.int32)), dev(d["g1"]), offs, srt,
                               k, act="silu_mul", out_dtype=torch.float32)
    ref = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt), k,
                                     act="silu_mul")["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what="nvfp4 u32-packed scales")


@pytest.mark.parametrize("sched", ["prefill", "decode"])
@pytest.mark.parametrize("I", [128, 256])
def test_nvfp4_silu_mul_limit(sched, I):
    # megamoe_rm.cu's clamped SwiGLU: a limit of 0.15 clamps about a quarter
    # of the gates and half of the up values of this input (I = 256: the
    # 512-row prefill tile)
    T, E, k, H = 150, 5, 2, 256
    lim = float(np.float32(0.15))
    d = synth.nvfp4_moe(41, T, E, k, H, I, routing="repeat")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    args = (dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k)
    h = mq.grouped_gemm_qnvfp4(*args, act="silu_mul", limit=lim, out_dtype=torch.float32, sched=sched)
    ref = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt), k,
                                     act="silu_mul", limit=lim)["y"]
    assert_rows_close(host(h)[: ref.shape[0]], ref, what=f"nvfp4 limit {sched}")
    plain = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt), k,
                                       act="silu_mul")["y"]
    assert np.abs(plain - ref).max() > 0.05 * np.abs(plain).max()     # the clamp is active
    # an infinite limit is the plain product, bit for bit
    h_inf = mq.grouped_gemm_qnvfp4(*args, act="silu_mul", limit=float("inf"), out_dtype=torch.float32,
                                   sched=sched)
    h_plain = mq.grouped_gemm_qnvfp4(*args, act="silu_mul", out_dtype=torch.float32, sched=sched)
    assert torch.equal(h_inf, h_plain)


def _pair_case(seed, T, E, k, H, I, drop=0.1):
    d = synth.nvfp4_moe(seed, T, E, k, H, I, routing="repeat")
    rng = np.random.default_rng(seed)
    d["topk_ids"][rng.random((T, k)) < drop] = -1          # pairs without an expert
    return d


@pytest.mark.parametrize("sched", ["prefill", "decode"])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("H", [256, 512])
def test_nvfp4_fc2_pair_weighted_epilogue(sched, odt, H):
    # megamoe_rm.cu's fc2_rm epilogue: w[p] * y in pair row p; rows of pairs
    # without an expert keep their previous contents.  H = 512 takes the
    # 512-row prefill tile.
    T, E, k, I = 120, 5, 3, 256
    d = _pair_case(63, T, E, k, H, I)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    P = T * k
    hs = synth.normal_bf16(np.random.default_rng(2), (P, I))
    tw = dev(d["topk_weights"].reshape(-1))
    out = torch.full((P, H), float("nan"), dtype=odt, device="cuda")
    mq.grouped_gemm_qnvfp4(dev(hs), dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, a_row="sorted",
                           pair_weights=tw, out=out, out_dtype=odt, sched=sched)
    y = oracle.grouped_gemm_qnvfp4(hs, "sorted", d["w2"], d["s2"], d["g2"], host(offs), host(srt), k)["y"]
    ypart, valid = oracle.pair_rows(y, host(srt), d["topk_weights"])
    got = host(out)
    assert valid.sum() < P and np.all(np.isnan(got[~valid]))
    assert_rows_close(got[valid], ypart[valid], what=f"fc2 pair epilogue {sched} H={H}")


@pytest.mark.parametrize("ydt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.float16, torch.bfloat16)])
def test_sum_pairs(ydt, odt):
    T, k, E, N = 77, 4, 6, 264
    rng = np.random.default_rng(4)
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    ids[rng.random((T, k)) < 0.15] = -1
    ids[5] = -1                                                 # a token with no expert
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    yp = torch.from_numpy(rng.standard_normal((T * k, N)).astype(np.float32)).to(ydt).cuda()
    yp[torch.from_numpy(host(p2s) < 0).cuda()] = float("nan")    # unrouted rows hold garbage
    out = mq.moe_sum_pairs(yp, p2s, T, k, out_dtype=odt)
    ref = oracle.sum_pairs(np.nan_to_num(host(yp)), host(p2s), T, k)
    assert_rows_close(host(out), ref, what="sum_pairs")
    assert bool((out[5] == 0).all())


@pytest.mark.parametrize("sched", ["prefill", "decode"])
def test_nvfp4_layer_with_fc2_pair_epilogue(sched):
    # FC1 -> FC2 with the top-k weight in its epilogue -> pair sum, against
    # the oracle; the same layer through the sorted FC2 and the weighted
    # scatter-combine meets the same bar
    T, E, k, H, I = 90, 4, 2, 512, 256
    d = _pair_case(64, T, E, k, H, I)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    h = mq.grouped_gemm_qnvfp4(dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k,
                               act="silu_mul", sched=sched)
    tw = dev(d["topk_weights"])
    yp = mq.grouped_gemm_qnvfp4(h, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, a_row="sorted",
                                pair_weights=tw.reshape(-1), sched=sched)
    out = mq.moe_sum_pairs(yp, p2s, T, k)
    y = oracle.grouped_gemm_qnvfp4(bf16_bits(h), "sorted", d["w2"], d["s2"], d["g2"], host(offs), host(srt),
                                   k)["y"]
    ref = oracle.scatter_combine(y, host(p2s), d["topk_weights"])
    assert_rows_close(host(out), ref, what=f"layer, pair epilogue {sched}")
    ys = mq.grouped_gemm_qnvfp4(h, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, a_row="sorted",
                                sched=sched)
    out2 = mq.moe_scatter_combine(ys, p2s, tw)
    assert_rows_close(host(out2), ref, what=f"layer, sorted FC2 {sched}")



def test_cast_bf16_to_f16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = dev(bits)
    y = mq.cast_bf16_to_f16(x)
    got = host(y.view(torch.int16)).view(np.uint16)
    ref = oracle.bf16_to_f16_bits(bits)
    nan = np.isnan(oracle.bf16_value(bits))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.f16_value(got[nan])))
    # in place, on a 2-D tensor whose size is not a multiple of the 2048
    # values one workgroup converts
    x2 = dev(bits[: 8 * 1000].reshape(80, 100))
    mq.cast_bf16_to_f16(x2, out=x2.view(torch.float16))
    got2 = host(x2.view(torch.int16)).reshape(-1).view(np.uint16)
    assert np.array_equal(got2[~nan[:8000]], ref[:8000][~nan[:8000]])


@pytest.mark.parametrize("sched", ["prefill", "decode"])
def test_nvfp4_f16_layer_with_gpu_cast(sched):
    # bf16 x -> GPU cast -> FC1 (f16, SiLU, f16 h) -> FC2 (f16) -> combine:
    # megamoe_rm.cu's fp16 activation path, against the oracle step by step
    T, E, k, H, I = 100, 4, 2, 512, 256
    d = synth.nvfp4_moe(65, T, E, k, H, I, routing="repeat")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    xh = mq.cast_bf16_to_f16(dev(d["x"]))
    xb = oracle.bf16_to_f16_bits(d["x"])
    assert np.array_equal(host(xh.view(torch.int16)).view(np.uint16), xb)
    h = mq.grouped_gemm_qnvfp4(xh, dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k, act="silu_mul",
                               out_dtype=torch.float16, sched=sched)
    ref_h = oracle.grouped_gemm_qnvfp4(xb, "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt), k,
                                       act="silu_mul", x_dtype="f16")["y"]
    n = ref_h.shape[0]
    assert_rows_close(host(h)[:n], ref_h, what=f"f16 FC1 {sched}")
    y = mq.grouped_gemm_qnvfp4(h, dev(d["w2"]), dev(d["s2"]), dev(d["g2"]), offs, srt, k, a_row="sorted",
                               sched=sched)
    hb = host(h.view(torch.int16)).view(np.uint16)
    ref_y = oracle.grouped_gemm_qnvfp4(hb, "sorted", d["w2"], d["s2"], d["g2"], host(offs), host(srt), k,
                                       x_dtype="f16")["y"]
    assert_rows_close(host(y)[:n], ref_y, what=f"f16 FC2 {sched}")


# ------------------------------------------------------------------ N % 32 shapes
def _guarded(P, ncols, dtype, fill):
    """out [P][ncols] as the head of a longer buffer whose tail holds `fill`,
    so a write past column ncols of the last row, or past row P, shows."""
    buf = torch.full((P * ncols + 4096,), fill, dtype=dtype, device="cuda")
    return buf, buf[: P * ncols].view(P, ncols)


@pytest.mark.parametrize("N,act", [(160, "none"), (96, "none"), (96, "silu_mul"), (288, "silu_mul")])
@pytest.mark.parametrize("sched", ["decode", "prefill", "auto"])
@pytest.mark.parametrize("xdt,sfl,wl", [("bf16", "rows", "rows"), ("f16", "quads", "tiled")])
def test_nvfp4_n_multiple_of_32(N, act, sched, xdt, sfl, wl):
    # N % 32 == 0 but not a multiple of 128 (SILU_MUL: I = 48, 144, a
    # multiple of 16): PREFILL falls back to the streaming schedule; every
    # column is computed and nothing past the output is written.
    T, E, k, H = 90, 5, 2, 256
    d = synth.nvfp4_moe(49, T, E, k, H, N // 2, routing="repeat")
    xg, xb = _xin(d["x"], xdt)
    sg, sa = _sf(d["s1"], sfl)
    wg, wa = _w(d["w1"], wl)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    P = T * k
    ncols = N // 2 if act == "silu_mul" else N
    buf, out = _guarded(P, ncols, torch.float32, 3.0)
    mq.grouped_gemm_qnvfp4(xg, wg, sg, dev(d["g1"]), offs, srt, k, act=act, out_dtype=torch.float32,
                           sched=sched, out=out)
    ref = oracle.grouped_gemm_qnvfp4(xb, "token", wa, sa, d["g1"], host(offs), host(srt), k, act=act,
                                     x_dtype=xdt, sf_layout=sfl, w_layout=wl)["y"]
    n = ref.shape[0]
    assert_rows_close(host(out)[:n], ref, what=f"nvfp4 N={N} {act} {sched}")
    assert torch.all(buf[n * ncols:] == 3.0), "written past the routed rows or the last column"


# raw int32 accumulators exist for act none only
@pytest.mark.parametrize("N,act,odt", [(160, "none", torch.int32), (96, "none", torch.int32),
                                       (160, "none", torch.float16), (96, "none", torch.float16),
                                       (96, "silu_mul", torch.float16), (288, "silu_mul", torch.float16)])
def test_int4_n_multiple_of_32(N, act, odt):
    # a partial last column tile: masked columns of the int8-MFMA tile are
    # neither stored nor allowed to read past the weights
    T, E, k, K = 300, 5, 2, 384
    d = synth.int4_moe(25, T, E, k, N, K, routing="repeat")
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    P = T * k
    ncols = N // 2 if act == "silu_mul" else N
    fill = 777 if odt == torch.int32 else 3.0
    buf, out = _guarded(P, ncols, odt, fill)
    mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k,
                          act=act, out_dtype=odt, out=out)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], host(offs),
                                    host(srt), k, act=act)
    n = ref["y"].shape[0]
    if odt == torch.int32:
        assert np.array_equal(host(out)[:n], ref["acc"])
    else:
        assert_rows_close(host(out)[:n], ref["y"], what=f"int4 N={N} {act}")
    assert torch.all(buf[n * ncols:] == fill), "written past the routed rows or the last column"


# ------------------------------------------------------------------ no routed pair at all
def test_every_id_minus_one_gemms_write_nothing_and_combine_writes_zeros():
    # CUTLASS discussion #2855 returns early with no problem to run; here the
    # route table is empty, every GEMM (both schedules) leaves its output
    # untouched and the combine writes zero rows.
    T, k, E = 37, 2, 4
    ids = -np.ones((T, k), np.int32)
    offs, srt, p2s, ninv = mq.moe_route_prep(dev(ids), E)
    assert host(offs).tolist() == [0] * (E + 1) and int(host(ninv)[0]) == 0
    assert np.all(host(srt) == -1) and np.all(host(p2s) == -1)
    P = T * k
    i4 = synth.int4_moe(26, T, E, k, 256, 256)
    f8 = synth.fp8_block(36, 0, 256, 256, E=E, T=T, k=k)
    nv = synth.nvfp4_moe(50, T, E, k, 256, 128)
    for sched in ("auto", "decode", "prefill"):
        out = torch.full((P, 256), 5, dtype=torch.int32, device="cuda")
        mq.grouped_gemm_qint4(dev(i4["a"]), dev(i4["a_scale"]), dev(i4["w"]), dev(i4["w_scale"]), offs, srt, k,
                              out_dtype=torch.int32, out=out, sched=sched)
        assert torch.all(out == 5)
        out = torch.full((P, 256), 5.0, dtype=torch.bfloat16, device="cuda")
        mq.grouped_gemm_qfp8_block(dev(f8["a"]), dev(f8["a_scale"]), dev(f8["w"]), dev(f8["w_scale"]), offs, srt,
                                   k, out=out, sched=sched)
        assert torch.all(out == 5.0)
        for act in ("none", "silu_mul"):
            out = torch.full((P, 256 if act == "none" else 128), 5.0, dtype=torch.bfloat16, device="cuda")
            mq.grouped_gemm_qnvfp4(dev(nv["x"]), dev(nv["w1"]), dev(nv["s1"]), dev(nv["g1"]), offs, srt, k,
                                   act=act, out=out, sched=sched)
            assert torch.all(out == 5.0)
    y = torch.full((P, 256), 9.0, dtype=torch.float16, device="cuda")
    comb = mq.moe_scatter_combine(y, p2s, dev(synth.softmax_weights(np.random.default_rng(0), T, k)))
    pairs = mq.moe_sum_pairs(y, p2s, T, k)
    torch.cuda.synchronize()
    assert torch.all(comb == 0) and torch.all(pairs == 0)


# ------------------------------------------------------------------ the boundary's largest sizes
@pytest.mark.parametrize("sched", ["decode", "prefill"])
def test_int4_largest_k_extreme_codes(sched):
    # K = 2^17 - 256, the largest K both INT4 schedules take, every code -8:
    # each output is 64 K exactly, the accumulator's largest magnitude
    T, E, N, K = 6, 2, 32, (1 << 17) - 256
    ids = np.zeros((T, 1), np.int32)
    ids[1::2] = 1
    a = np.full((T, K // 2), 0x88, np.uint8)
    w = np.full((E, N, K // 2), 0x88, np.uint8)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), E)
    acc = mq.grouped_gemm_qint4(dev(a), dev(np.ones(T, np.float32)), dev(w), dev(np.ones((E, N), np.float32)),
                                offs, srt, 1, out_dtype=torch.int32, sched=sched)
    assert torch.all(acc == 64 * K)


@pytest.mark.parametrize("sched", ["decode", "prefill"])
def test_int4_1024_experts_top64(sched):
    # E = 1024 and topk = 64, the boundary's limits: 2048 pairs, about two
    # per expert, some experts empty
    T, E, k, N, K = 32, 1024, 64, 64, 256
    d = synth.int4_moe(71, T, E, k, N, K)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    assert (np.diff(host(offs)) == 0).any()
    acc = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k,
                                out_dtype=torch.int32, sched=sched)
    ref = oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], host(offs), host(srt), k)
    assert np.array_equal(host(acc)[: int(host(offs)[-1])], ref["acc"])
    y = mq.grouped_gemm_qint4(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k,
                              out_dtype=torch.float16, sched=sched)
    out = mq.moe_scatter_combine(y, p2s, dev(d["topk_weights"]))
    ref_out = oracle.scatter_combine(oracle.round_to_f16(ref["y"]), host(p2s), d["topk_weights"])
    assert_rows_close(host(out), ref_out, what=f"int4 E=1024 top-64 {sched} combine")


@pytest.mark.parametrize("sched", ["decode", "prefill"])
def test_nvfp4_1024_experts_top64(sched):
    T, E, k, H, I = 16, 1024, 64, 256, 256
    d = synth.nvfp4_moe(72, T, E, k, H, I)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    h = mq.grouped_gemm_qnvfp4(dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k,
                               act="silu_mul", out_dtype=torch.float32, sched=sched, work_queue=mq.work_queue())
    ref = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], host(offs), host(srt), k,
                                     act="silu_mul")["y"]
    assert_rows_close(host(h)[: ref.shape[0]], ref, what=f"nvfp4 E=1024 top-64 {sched}")


@pytest.mark.parametrize("sched", ["decode", "prefill"])
def test_fp8_1024_experts_top64(sched):
    T, E, k, N, K = 16, 1024, 64, 128, 256
    d = synth.fp8_moe(73, T, E, k, N, K)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    y = mq.grouped_gemm_qfp8_block(dev(d["a"]), dev(d["a_scale"]), dev(d["w"]), dev(d["w_scale"]), offs, srt, k,
                                   out_dtype=torch.float32, sched=sched)
    ref = oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], host(offs),
                                         host(srt), k)["y"]
    assert_rows_close(host(y)[: ref.shape[0]], ref, what=f"fp8 E=1024 top-64 {sched}")


def test_nvfp4_work_queue_grid_not_a_multiple_of_8():
    # few tiles: the grid is smaller than the chip and not a multiple of 8,
    # so one counter hands out every tile
    T, E, k, H, I = 50, 3, 1, 512, 256
    d = synth.nvfp4_moe(74, T, E, k, H, I)
    offs, srt, p2s, _ = mq.moe_route_prep(dev(d["topk_ids"]), E)
    args = (dev(d["x"]), dev(d["w1"]), dev(d["s1"]), dev(d["g1"]), offs, srt, k)
    wq = mq.work_queue()
    h0 = mq.grouped_gemm_qnvfp4(*args, act="silu_mul", out_dtype=torch.float32, sched="prefill")
    for _ in range(2):
        h1 = mq.grouped_gemm_qnvfp4(*args, act="silu_mul", out_dtype=torch.float32, sched="prefill", work_queue=wq)
        assert torch.equal(h0, h1) and torch.all(wq == 0)


@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_combine_streaming_size(ydt):
    # y past 256 MB: the combine takes its nontemporal (streaming) path
    T, k, N = 8192 if ydt == torch.float32 else 16384, 2, 4096
    rng = np.random.default_rng(75)
    ids = synth.uniform_ids_with_repeats(rng, T, k, 64)
    ids[::97, 1] = -1
    offs, srt, p2s, _ = mq.moe_route_prep(dev(ids), 64)
    y = torch.randn(T * k, N, device="cuda").to(ydt)
    assert y.numel() * y.element_size() >= 256 << 20
    w = synth.softmax_weights(rng, T, k)
    out = mq.moe_scatter_combine(y, p2s, dev(w), out_dtype=torch.float32)
    rows = np.r_[0:64, T - 64:T, rng.integers(0, T, 256)]
    y_h = host(y)
    ref = oracle.scatter_combine(y_h, host(p2s), w)
    assert_rows_close(host(out)[rows], ref[rows], what=f"combine streaming {ydt}")
