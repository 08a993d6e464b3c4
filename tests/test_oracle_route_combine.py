"""Pins for the oracle's route table and combine: brute force and invariants."""
import numpy as np
import pytest

import oracle
import synth


def _brute_route(ids, E):
    # Append each pair to its expert's list while walking the pairs in order.
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    lists = [[] for _ in range(E)]
    bad = 0
    for p, e in enumerate(flat):
        if 0 <= e < E:
            lists[e].append(p)
        elif e != -1:
            bad += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(lists[e]))
    srt = [p for e in range(E) for p in lists[e]]
    srt += [-1] * (len(flat) - len(srt))
    inv = [-1] * len(flat)
    for s, p in enumerate(srt):
        if p >= 0:
            inv[p] = s
    return offsets, srt, inv, bad


CASES = [
    ("uniform", lambda r: synth.distinct_uniform_ids(r, 50, 4, 9), 9),
    ("repeats", lambda r: synth.uniform_ids_with_repeats(r, 40, 3, 5), 5),
    ("minus1", lambda r: np.where(r.random((30, 2)) < 0.3, -1,
                                  synth.uniform_ids_with_repeats(r, 30, 2, 6)), 6),
    ("out_of_range", lambda r: r.integers(-3, 9, size=(25, 3)).astype(np.int32), 6),
    ("E1", lambda r: np.zeros((17, 1), np.int32), 1),
    ("T0", lambda r: np.zeros((0, 2), np.int32), 4),
    ("all_minus1", lambda r: -np.ones((6, 2), np.int32), 3),
    ("empty_experts", lambda r: synth.distinct_uniform_ids(r, 20, 2, 3) * 3, 11),
    ("zipf", lambda r: synth.zipf_ids(r, 64, 8, 64, n_zero=4), 64),
]


@pytest.mark.parametrize("name,make,E", CASES, ids=[c[0] for c in CASES])
def test_route_matches_brute_force(name, make, E):
    ids = make(np.random.default_rng(7))
    off, srt, inv, bad = oracle.route_prep(ids, E)
    b_off, b_srt, b_inv, b_bad = _brute_route(ids, E)
    assert off.tolist() == b_off and srt.tolist() == b_srt and inv.tolist() == b_inv
    assert bad == b_bad
    # invariants
    flat = ids.reshape(-1)
    n = off[-1]
    valid = (flat >= 0) & (flat < E)
    assert n == valid.sum()
    assert np.all(np.diff(off) >= 0)
    assert sorted(srt[:n].tolist()) == np.nonzero(valid)[0].tolist()
    for e in range(E):
        seg = srt[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.all(inv[srt[:n]] == np.arange(n))


def test_combine_brute_force_and_edge_rows():
    rng = np.random.default_rng(3)
    T, k, E, N = 12, 3, 4, 5
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    ids[2, :] = -1                      # token with no routed pair
    ids[5, 1] = -1
    w = synth.softmax_weights(rng, T, k)
    off, srt, inv, _ = oracle.route_prep(ids, E)
    y = rng.standard_normal((T * k, N))
    out = oracle.scatter_combine(y, inv, w)
    for t in range(T):
        ref = [0.0] * N
        for j in range(k):
            e = ids[t, j]
            if e < 0:
                continue
            s = int(inv[t * k + j])
            for c in range(N):
                ref[c] += float(w[t, j]) * float(y[s, c])
        assert np.allclose(out[t], ref, rtol=0, atol=1e-15)
    assert np.all(out[2] == 0)


def test_combine_one_hot_weights_select_one_expert():
    rng = np.random.default_rng(4)
    T, k, E, N = 9, 2, 3, 6
    ids = synth.distinct_uniform_ids(rng, T, k, E)
    w = np.zeros((T, k), np.float32)
    w[:, 1] = 1.0
    off, srt, inv, _ = oracle.route_prep(ids, E)
    y = rng.standard_normal((T * k, N))
    out = oracle.scatter_combine(y, inv, w)
    assert np.array_equal(out, y[inv.reshape(T, k)[:, 1]])


def test_route_worked_example():
    # Worked by hand from the stable-rank rule of megamoe_rm.cu's route_prep:
    # pairs p = t*k + j: 0->e2, 1->e0, 2->e0, 3->e2, 4->none(-1), 5->e2.
    ids = np.array([[2, 0], [0, 2], [-1, 2]], np.int32)
    off, srt, inv, bad = oracle.route_prep(ids, 3)
    assert off.tolist() == [0, 2, 2, 5]
    assert srt.tolist() == [1, 2, 0, 3, 5, -1]
    assert inv.tolist() == [2, 0, 1, 3, -1, 4]
    assert bad == 0
    assert oracle.route_prep(np.array([[7, -2]], np.int32), 3)[3] == 2


def test_pair_rows_and_sum_pairs_worked_example():
    # T=2, k=2, E=2; token 1 slot 0 has no expert.  Sorted order: expert 0
    # holds pair 1, expert 1 holds pairs 0 and 3 (ascending pair id).
    ids = np.array([[1, 0], [-1, 1]], np.int32)
    off, srt, p2s, _ = oracle.route_prep(ids, 2)
    assert list(srt[:3]) == [1, 0, 3]
    y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    w = np.array([[0.5, 0.25], [0.9, 2.0]], np.float32)
    ypart, valid = oracle.pair_rows(y, srt, w)
    assert list(valid) == [True, True, False, True]
    assert np.array_equal(ypart, [[1.5, 2.0], [0.25, 0.5], [0.0, 0.0], [10.0, 12.0]])
    out = oracle.sum_pairs(ypart, p2s, 2, 2)
    assert np.array_equal(out, [[1.75, 2.5], [10.0, 12.0]])


def test_pair_path_equals_scatter_combine():
    # weighting in the FC2 epilogue then summing pair rows is the same sum,
    # in the same slot order, as the weighted scatter-combine
    rng = np.random.default_rng(3)
    T, k, E, N = 37, 4, 6, 24
    ids = synth.uniform_ids_with_repeats(rng, T, k, E)
    ids[rng.random((T, k)) < 0.1] = -1
    off, srt, p2s, _ = oracle.route_prep(ids, E)
    y = rng.standard_normal((int(off[-1]), N))
    w = synth.softmax_weights(rng, T, k)
    ypart, valid = oracle.pair_rows(y, srt, w)
    assert np.array_equal(valid, p2s >= 0)
    assert np.array_equal(oracle.sum_pairs(ypart, p2s, T, k), oracle.scatter_combine(y, p2s, w))
