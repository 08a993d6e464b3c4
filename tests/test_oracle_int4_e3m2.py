"""Pins for the e3m2 storage of int4 values (oracle.int4_e3m2): the FP6 E3M2
decoder against the format's defining values, the exact code of every int4
value, the block layout against hand-computed words, and the INT4 GEMM over
e3m2 rows against the same GEMM over packed rows."""
import numpy as np
import pytest

import oracle
import synth


def test_e3m2_decoder_defining_values():
    v = oracle.e3m2_value(np.arange(64))
    # smallest subnormal, smallest normal, one, largest, and the sign bit
    assert v[0b000001] == 2.0 ** -4 and v[0b000100] == 0.25 and v[0b001100] == 1.0
    assert v[0b011111] == 28.0 and v[0b111111] == -28.0 and v[0b100000] == 0.0
    # positive codes are strictly increasing, negatives mirror them
    assert np.all(np.diff(v[:32]) > 0) and np.array_equal(v[32:], -v[:32])
    # each binade (exponent e >= 1) holds 2^(e-3) * {1, 1.25, 1.5, 1.75}
    for e in range(1, 8):
        np.testing.assert_array_equal(v[4 * e:4 * e + 4], 2.0 ** (e - 3) * np.array([1, 1.25, 1.5, 1.75]))


def test_every_int4_value_has_its_exact_code():
    vals = np.arange(-8, 8)
    codes = oracle.e3m2_code_of_int(vals)
    np.testing.assert_array_equal(oracle.e3m2_value(codes), vals)
    # by hand: 1 = 2^0 (exponent 3, code 0b001100), 3 = 2 * 1.5 (0b010010),
    # 7 = 4 * 1.75 (0b010111), -8 = -2^3 (0b111000)
    assert list(oracle.e3m2_code_of_int([1, 3, 7, -8])) == [0b001100, 0b010010, 0b010111, 0b111000]


def test_block_layout_hand_computed_words():
    # a row of 64 ones: every code is 12, so the low word of each half's
    # stream is 12 * (1 + 2^6 + 2^12 + 2^18 + 2^24) plus code 5's low bits (0)
    row = np.full((1, 32), 0x11, np.uint8)                  # 64 values of 1
    words = oracle.int4_to_e3m2_rows(row).view("<u4")[0]
    assert words[0] == words[4] == 0x0C30C30C
    # the value at position k of a block sits in half h = k // 32, bit 6 i of
    # that half's stream (i = k % 32); stream word j < 4 is block word 4h + j,
    # j >= 4 is block word 8 + 2h + (j - 4)
    for k in range(64):
        vals = np.zeros(64, np.int64)
        vals[k] = 7                                          # code 0b010111
        nib = (vals & 15).astype(np.uint8)
        packed = (nib[0::2] | (nib[1::2] << 4)).reshape(1, 32)
        w = oracle.int4_to_e3m2_rows(packed).view("<u4")[0].astype(np.uint64)
        h, i = divmod(k, 32)
        bit = 6 * i
        expect = np.zeros(12, np.uint64)
        for part, (j, o) in enumerate([(bit // 32, bit % 32), (bit // 32 + 1, 0)]):
            if part == 1 and bit % 32 <= 26:
                break
            word = 4 * h + j if j < 4 else 8 + 2 * h + (j - 4)
            expect[word] |= np.uint64((0b010111 << o) & 0xFFFFFFFF if part == 0 else 0b010111 >> (32 - bit % 32))
        np.testing.assert_array_equal(w, expect, err_msg=f"k={k}")


def test_round_trip_random_rows():
    rng = np.random.default_rng(3)
    packed = synth.uniform_bytes(rng, (5, 3, 96))           # K = 192
    e = oracle.int4_to_e3m2_rows(packed)
    assert e.shape == (5, 3, 144)
    np.testing.assert_array_equal(oracle.e3m2_rows_values(e),
                                  oracle.int4_value(oracle.unpack_nibbles(packed)))


@pytest.mark.parametrize("a_row", ["token", "sorted"])
def test_int4_gemm_over_e3m2_rows_equals_packed(a_row):
    d = synth.int4_moe(17, T=20, E=3, k=2, N=96, K=128, routing="repeat")
    off, srt, inv, _ = oracle.route_prep(d["topk_ids"], 3)
    n = int(off[-1])
    a = d["a"] if a_row == "token" else synth.uniform_bytes(np.random.default_rng(4), (n, 64))
    sa = d["a_scale"] if a_row == "token" else synth.uniform_f32(np.random.default_rng(5), (n,), 0.005, 0.05)
    ref = oracle.grouped_gemm_qint4(a, sa, a_row, d["w"], d["w_scale"], off, srt, 2, act="silu_mul")
    got = oracle.grouped_gemm_qint4(oracle.int4_to_e3m2_rows(a), sa, a_row, oracle.int4_to_e3m2_rows(d["w"]),
                                    d["w_scale"], off, srt, 2, act="silu_mul", layout="e3m2")
    np.testing.assert_array_equal(got["acc"], ref["acc"])
    np.testing.assert_array_equal(got["y"], ref["y"])
