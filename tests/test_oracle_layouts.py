"""Pins of oracle/layouts.py (the FlashInfer/megamoe_rm.cu NVFP4 layout and
its repack into the library's linear layout)."""
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import layouts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_scale_swizzle_offsets.txt")


def test_hand_worked_offsets():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    for r, c, off in rows:
        assert layouts.scale_swizzle_offset(int(r), int(c), 8) == int(off), (r, c)


@pytest.mark.parametrize("R,C", [(128, 4), (256, 12), (384, 28)])
def test_offsets_are_a_permutation(R, C):
    rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    off = layouts.scale_swizzle_offset(rr, cc, C).ravel()
    assert np.array_equal(np.sort(off), np.arange(R * C))


def test_each_tile_holds_128_rows_by_4_columns():
    R, C = 256, 12
    rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    tile = layouts.scale_swizzle_offset(rr, cc, C) // 512
    for t in range(R * C // 512):
        r, c = rr[tile == t], cc[tile == t]
        assert r.size == 512
        assert np.array_equal(np.unique(r), np.arange(128) + 128 * (t // (C // 4)))
        assert np.array_equal(np.unique(c), np.arange(4) + 4 * (t % (C // 4)))


def test_swizzle_round_trip():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 256, (2, 256, 20), dtype=np.uint8)
    sw = layouts.swizzle_scales(s)
    assert sw.shape == (2, 256 * 20)
    assert np.array_equal(layouts.unswizzle_scales(sw, 256, 20), s)


def test_rejects_shapes_outside_the_tiling():
    with pytest.raises(ValueError):
        layouts.unswizzle_scales(np.zeros((1, 100 * 8), np.uint8), 100, 8)
    with pytest.raises(ValueError):
        layouts.swizzle_scales(np.zeros((1, 128, 6), np.uint8))


def test_repacked_silu_layer_matches_the_page_layout_brute_force():
    # w13 with up rows first and swizzled scales -> repack -> the oracle's
    # gate-first SiLU-gated GEMM; against a per-element computation that reads
    # the page's layout directly (up = rows [0, I), gate = rows [I, 2I), each
    # scale found through the offset of its (row, block)).
    rng = np.random.default_rng(4)
    I, K, T = 64, 64, 3
    R, C = 2 * I, K // 16
    w = rng.integers(0, 256, (1, R, K // 2), dtype=np.uint8)
    s_lin = rng.integers(0x30, 0x48, (1, R, C), dtype=np.uint8)
    s_swz = layouts.swizzle_scales(s_lin)
    x = oracle.round_to_bf16(rng.standard_normal((T, K)))
    xb = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gs = np.array([0.75], np.float32)
    w2, s2 = layouts.repack_nvfp4(w, s_swz, swap_halves=True)
    offs = np.array([0, T], np.int32)
    h = oracle.grouped_gemm_qnvfp4(xb, "sorted", w2, s2, gs, offs, None, 1, act="silu_mul")["y"]

    def e2m1(code):
        sgn, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        return -mag if sgn else mag

    def ue4m3(b):
        e, m = (b >> 3) & 15, b & 7
        return 2.0 ** -6 * m / 8 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)

    flat = s_swz[0]
    for t in range(T):
        for j in range(I):
            acc = {}
            for name, row in (("up", j), ("gate", I + j)):
                total = 0.0
                for k in range(K):
                    byte = int(w[0, row, k // 2])
                    code = byte & 15 if k % 2 == 0 else byte >> 4
                    sc = ue4m3(int(flat[layouts.scale_swizzle_offset(row, k // 16, C)]))
                    total += float(x[t, k]) * e2m1(code) * sc
                acc[name] = 0.75 * total
            g, u = acc["gate"], acc["up"]
            want = g / (1 + np.exp(-g)) * u
            assert abs(h[t, j] - want) <= 1e-12 * max(1.0, abs(want))


def test_quad_layout_hand_worked_offsets():
    # R=3 rows, C=8 block columns: byte (n, c) of the row-major matrix sits
    # at ((c // 4) * R + n) * 4 + c % 4 of the quad-major one
    R, C = 3, 8
    s = np.arange(R * C, dtype=np.uint8).reshape(1, R, C)           # value = n*C + c
    q = oracle.quads_from_rows(s).reshape(-1)
    for n, c in [(0, 0), (0, 5), (2, 3), (1, 7), (2, 4)]:
        assert q[((c // 4) * R + n) * 4 + c % 4] == n * C + c
    assert list(q[:12]) == [0, 1, 2, 3, 8, 9, 10, 11, 16, 17, 18, 19]  # quad 0 of rows 0, 1, 2
    assert np.array_equal(oracle.rows_from_quads(oracle.quads_from_rows(s)), s)


def test_repack_to_quads_and_gemm_on_quads():
    rng = np.random.default_rng(5)
    E, R, K = 2, 256, 128
    w = rng.integers(0, 256, (E, R, K // 2), dtype=np.uint8)
    s_lin = rng.integers(0x30, 0x48, (E, R, K // 16), dtype=np.uint8)
    s_swz = oracle.swizzle_scales(s_lin)
    w_r, s_r = oracle.repack_nvfp4(w, s_swz, True)
    w_q, s_q = oracle.repack_nvfp4(w, s_swz, True, out_layout="quads")
    assert np.array_equal(w_q, w_r) and s_q.shape == (E, K // 64, R, 4)
    assert np.array_equal(oracle.rows_from_quads(s_q), s_r)
    # the GEMM reads the quad layout as the same scales
    x = synth.normal_bf16(rng, (5, K))
    off = np.array([0, 3, 5], np.int32)
    g = np.ones(E, np.float32)
    y_r = oracle.grouped_gemm_qnvfp4(x, "sorted", w_r, s_r, g, off, None, 1)["y"]
    y_q = oracle.grouped_gemm_qnvfp4(x, "sorted", w_q, s_q, g, off, None, 1, sf_layout="quads")["y"]
    assert np.array_equal(y_r, y_q)


def test_tiled_weight_layout_hand_worked_offsets():
    # R=32 rows, K/2=96 bytes (K=192, 3 blocks of 32 bytes per row): byte
    # (n, b) sits at ((n // 16) * 3 + b // 32) * 512 + (n % 16) * 32 + b % 32
    R, KB = 32, 96
    n_ = np.arange(R)[:, None]
    b_ = np.arange(KB)[None, :]
    w = ((n_ * 7 + b_ * 3) % 251).astype(np.uint8)[None]          # distinct enough to locate
    t = oracle.tiles_from_rows(w).reshape(-1)
    for n, b in [(0, 0), (0, 33), (15, 31), (16, 0), (17, 95), (31, 64), (5, 70)]:
        assert t[((n // 16) * 3 + b // 32) * 512 + (n % 16) * 32 + b % 32] == w[0, n, b]
    assert np.array_equal(t[32:64], w[0, 1, :32])                    # row 1 follows row 0 in block 0
    assert np.array_equal(t[512:544], w[0, 0, 32:64])                # block 1 is row 0's next 32 bytes
    assert np.array_equal(oracle.rows_from_tiles(oracle.tiles_from_rows(w)), w)
    with pytest.raises(ValueError):
        oracle.tiles_from_rows(np.zeros((1, 24, 32), np.uint8))


def test_gemm_on_tiled_weights_and_quad_scales():
    rng = np.random.default_rng(6)
    d = synth.nvfp4_moe(16, T=7, E=2, k=1, H=128, I=64)
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 2)
    y = oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, 1)["y"]
    y2 = oracle.grouped_gemm_qnvfp4(d["x"], "token", oracle.tiles_from_rows(d["w1"]),
                                    oracle.quads_from_rows(d["s1"]), d["g1"], off, srt, 1,
                                    sf_layout="quads", w_layout="tiled")["y"]
    assert np.array_equal(y, y2)
    w_t, s_q = oracle.repack_nvfp4(d["w1"], oracle.swizzle_scales(d["s1"]), False, out_layout="quads",
                                   w_layout="tiled")
    assert np.array_equal(oracle.rows_from_tiles(w_t), d["w1"])
