"""Pins for oracle.cs4a: block scores against a library route, top-p against
brute force over subsets and hand-derived fixtures, mapping against closed
forms, hand fixtures and monotonicity."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import cs4a, geometry as G
from varsparse_inputs import gaussian_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cs4a_hand.json")


def test_scores_match_membership_matmul_route():
    """Second route: P from torch.softmax, pooled by one-hot tile-membership
    matrices (score = Mq^T P Mk / |Q|)."""
    sides, D, t = (1, 2, 4, 6, 8), 4, 2
    nqb, nkb, nq, nk = G.counts(sides, D, t)
    q, k, _ = gaussian_qkv(3, 11, 2, 2, nq, nk, 16)
    sc = cs4a.block_scores(q, k, sides, D, t, 0.25)
    mq = np.zeros((nq, nqb))
    for i, qt in enumerate(G.query_tiles(sides, D, t)):
        mq[qt.tokens(), i] = 1.0 / qt.tokens().size
    mk = np.zeros((nk, nkb))
    for j, kt in enumerate(G.key_tiles(sides, D, t)):
        mk[kt.tokens(), j] = 1.0
    for b in range(2):
        for h in range(2):
            p = torch.softmax(torch.from_numpy(q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T * 0.25),
                              dim=1).numpy()
            assert np.abs(sc[b, h] - mq.T @ p @ mk).max() < 1e-12
    assert np.abs(sc.sum(axis=-1) - 1).max() < 1e-12


def test_scores_each_query_normalised_by_its_own_maximum():
    """Every query's softmax over the keys sums to 1 whatever the other
    queries' score ranges: with one query's scores ~2000 above another's, a
    maximum shared across queries would underflow the lower query's weights
    to zero (and its normalisation to 0/0)."""
    sides, D, t = (1, 2, 4), 2, 2
    nk = 1 + 4 + 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 16, 8))
    k = rng.standard_normal((1, 1, nk, 8))
    q[0, 0, 3] = 4000.0 * k[0, 0, 7] / np.dot(k[0, 0, 7], k[0, 0, 7])   # query 3 scores key 7 at 4000
    sc = cs4a.block_scores(q, k, sides, D, t, 0.5)
    assert np.isfinite(sc).all()
    np.testing.assert_allclose(sc.sum(axis=-1), 1.0, rtol=0, atol=1e-12)


def test_top_p_hand_fixture():
    fx = json.load(open(GOLDEN))["top_p"]
    for case in fx["cases"]:
        assert list(cs4a.top_p_row(np.array(case["scores"], np.float32), case["p"])) == case["kept"], case


def _f32_exact(num, exp):
    """The float32 value num * 2^exp (asserted exact)."""
    v = np.float32(num * 2.0 ** exp)
    assert float(v) == num * 2.0 ** exp
    return v


def test_quantise_floors_non_dyadic_scores():
    """quantise takes the floor of score * 2^24: hand cases whose product has a
    fractional part (round and ceil give one more)."""
    fx = json.load(open(GOLDEN))["quantise"]
    for case in fx["cases"]:
        got = int(cs4a.quantise(np.array([_f32_exact(case["num"], case["exp"])], np.float32))[0])
        assert got == case["m"], case


def test_top_p_non_dyadic_fixture():
    """Top-p on scores that are not exact multiples of 2^-24: the threshold
    uses the float32 value of p (case A) and the floored quantisation decides
    the order (case B)."""
    fx = json.load(open(GOLDEN))["top_p_nondyadic"]
    for case in fx["cases"]:
        sc = np.array([_f32_exact(n, e) for n, e in zip(case["nums"], case["exps"])], np.float32)
        assert list(cs4a.top_p_row(sc, case["p"])) == case["kept"], case
        cnt, idx = cs4a.top_p_select(sc[None, :], case["p"])
        assert list(idx[0, : cnt[0]]) == case["kept"]


def _brute_force_min_size(m, thr):
    n = len(m)
    for size in range(n + 1):
        if any(sum(m[j] for j in c) >= thr for c in itertools.combinations(range(n), size)):
            return size
    return None


@pytest.mark.parametrize("seed", range(12))
def test_top_p_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    raw = rng.random(n) ** 3
    if seed % 3 == 0:
        raw[rng.integers(0, n, size=n // 2)] = raw[0]          # ties
    sc = (raw / raw.sum()).astype(np.float32)
    p = float(rng.choice([0.3, 0.5, 0.9, 0.99, 1.0]))
    kept = cs4a.top_p_row(sc, p)
    m = [int(x) for x in np.floor(sc.astype(np.float64) * 2 ** 24)]
    thr = math.ceil(float(np.float32(p)) * sum(m))
    mass = sum(m[j] for j in kept)
    assert mass >= thr
    assert len(kept) == _brute_force_min_size(m, thr)
    # the kept set is the top-|kept| in (mass desc, id asc) order
    order = sorted(range(n), key=lambda j: (-m[j], j))
    assert sorted(order[: len(kept)]) == list(kept)


def test_top_p_special_cases():
    sc = np.array([0.1, 0.4, 0.2, 0.3], np.float32)
    assert list(cs4a.top_p_row(sc, 1e-9)) == [1]                 # just the heaviest tile
    assert list(cs4a.top_p_row(sc, 1.0)) == [0, 1, 2, 3]
    uniform = np.full(10, 0.1, np.float32)
    # every m equal: ceil(p * 10 m) needs ceil(10 p) tiles (lowest ids on ties)
    assert list(cs4a.top_p_row(uniform, 0.55)) == [0, 1, 2, 3, 4, 5]
    assert cs4a.top_p_row(np.zeros(5, np.float32), 0.9).size == 0


def test_map_hand_fixture():
    fx = json.load(open(GOLDEN))["map"]
    g = fx["geometry"]
    nqbD = G.counts(g["sides"], g["d_scale"], g["tile"])[0]
    nkbD = G.counts(g["sides"], g["d_scale"], g["tile"])[1]
    cnt = np.zeros(nqbD, np.int32)
    idx = np.full((nqbD, nkbD), -1, np.int32)
    for q, sel in fx["selected"].items():
        cnt[int(q)] = len(sel)
        idx[int(q), : len(sel)] = sel
    oc, oi = cs4a.map_indices(cnt, idx, g["sides"], g["d_scale"], g["t_scale"], g["tile"], g["n_sink"])
    for q, want in fx["lists"].items():
        q = int(q)
        assert list(oi[q, : oc[q]]) == want, q


def test_map_same_scale_is_identity():
    sides, t = (1, 2, 4, 8, 16), 4
    nqb, nkb, _, _ = G.counts(sides, 4, t)
    rng = np.random.default_rng(5)
    keep = rng.random((nqb, nkb)) < 0.3
    cnt = keep.sum(1).astype(np.int32)
    idx = np.full((nqb, nkb), -1, np.int32)
    for r in range(nqb):
        idx[r, : cnt[r]] = np.flatnonzero(keep[r])
    oc, oi = cs4a.map_indices(cnt, idx, sides, 4, 4, t, 0)
    assert (oc == cnt).all() and (oi == idx).all()


def test_map_doubling_closed_form():
    """Side 4 -> side 8 with t = 2 and no scale in between: parent (i//2, j//2);
    decision tile (a,b) maps to itself on the decision scale and to
    {2a, 2a+1} x {2b, 2b+1} on the target scale."""
    sides, t, D, T = (2, 4, 8), 2, 1, 2
    nqbD, nkbD, _, _ = G.counts(sides, D, t)
    rng = np.random.default_rng(6)
    keep = rng.random((nqbD, nkbD)) < 0.5
    cnt = keep.sum(1).astype(np.int32)
    idx = np.full((nqbD, nkbD), -1, np.int32)
    for r in range(nqbD):
        idx[r, : cnt[r]] = np.flatnonzero(keep[r])
    oc, oi = cs4a.map_indices(cnt, idx, sides, D, T, t, 0)
    for i in range(4):
        for j in range(4):
            parent = (i // 2) * 2 + (j // 2)
            want = set()
            for tid in idx[parent, : cnt[parent]]:
                if tid == 0:
                    want.add(0)
                    continue
                a, b = divmod(int(tid) - 1, 2)
                want.add(int(tid))
                for da in (0, 1):
                    for db in (0, 1):
                        want.add(5 + (2 * a + da) * 4 + (2 * b + db))
            q = i * 4 + j
            assert list(oi[q, : oc[q]]) == sorted(want)


def test_map_monotone_and_sinks():
    from varsparse_inputs import SCHEDULE_13
    sides, t, D, T = SCHEDULE_13, 8, 9, 12
    nqbD, nkbD, _, _ = G.counts(sides, D, t)
    rng = np.random.default_rng(7)
    small = rng.random((nqbD, nkbD)) < 0.1
    big = small | (rng.random((nqbD, nkbD)) < 0.1)

    def lists(m):
        c = m.sum(1).astype(np.int32)
        x = np.full(m.shape, -1, np.int32)
        for r in range(m.shape[0]):
            x[r, : c[r]] = np.flatnonzero(m[r])
        return c, x
    c1, i1 = cs4a.map_indices(*lists(small), sides, D, T, t, 5)
    c2, i2 = cs4a.map_indices(*lists(big), sides, D, T, t, 5)
    for q in range(c1.shape[0]):
        s1, s2 = set(i1[q, : c1[q]]), set(i2[q, : c2[q]])
        assert s1 <= s2
        assert {0, 1, 2, 3, 4} <= s1


# ---- Top-K-fraction selector


def test_top_k_count():
    from oracle import cs4a as OC
    assert OC.top_k_count(47, 0.2) == 10            # ceil(9.4)
    assert OC.top_k_count(160, 0.2) == 32            # float32 product 32.0 exactly
    assert OC.top_k_count(5, 0.0001) == 1            # at least one tile
    assert OC.top_k_count(5, 0.0) == 1               # even for a zero fraction
    assert OC.top_k_count(5, 1.0) == 5
    # the product is taken in float32 (the precision of the fraction), not in
    # double: float32(0.07) * 100 = 7.0000000298 rounds to 7.0 in float32 -> 7,
    # while 0.07 * 100 in double is 7.000000000000001 -> 8; float32(0.09) * 300
    # = 27.00000107 rounds up to 27.0000019 (27 + 2^-19) in float32 -> 28,
    # while 0.09 * 300 in double is exactly 27 -> 27
    assert OC.top_k_count(100, 0.07) == 7
    assert OC.top_k_count(300, 0.09) == 28


def test_top_k_full_fraction_keeps_all_and_argmax():
    from oracle import cs4a as OC
    rng = np.random.default_rng(11)
    row = rng.random(31).astype(np.float32)
    assert np.array_equal(OC.top_k_row(row, 1.0), np.arange(31))
    one = OC.top_k_row(row, 1e-6)
    assert one.tolist() == [int(np.argmax(OC.quantise(row)))]


def test_top_k_ties_go_to_lower_ids_and_set_is_a_top_set():
    from oracle import cs4a as OC
    row = np.array([0.1, 0.3, 0.3, 0.05, 0.3, 0.25], np.float32)
    # three equal maxima; keep 2 -> the two lowest ids among them
    assert OC.top_k_row(row, 2 / 6).tolist() == [1, 2]
    rng = np.random.default_rng(12)
    for _ in range(20):
        r = rng.random(40).astype(np.float32)
        kept = OC.top_k_row(r, 0.2)
        m = OC.quantise(r)
        rest = np.setdiff1d(np.arange(40), kept)
        assert m[kept].min() >= m[rest].max()
        assert kept.size == OC.top_k_count(40, 0.2)
