"""Pins of the oracle's k-means (semantic-aware smoothing) against SciPy,
brute force, exact rational means and Lloyd's invariants."""
import itertools
import warnings
from fractions import Fraction

import numpy as np
import pytest
from scipy.cluster.vq import kmeans2, vq

from oracle import assign, bf16_round, lloyd, update, forgy_indices


def _blobs(rng, centers, per, jitter, d):
    pts = [np.asarray(c, float)[None, :] + jitter * rng.standard_normal((per, d)) for c in centers]
    return np.concatenate(pts)


@pytest.mark.parametrize("seed", range(6))
def test_exact_mode_equals_scipy_kmeans2(seed):
    rng = np.random.default_rng(seed)
    N, d, K, I = 300, 8, 12, 6
    X = _blobs(rng, rng.standard_normal((6, d)) * 4, N // 6, 1.0, d)
    C0 = X[forgy_indices(len(X), K, seed, 0, 1)]
    C, lab, _ = lloyd(X, C0, I, mode="exact")
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        Cs, lab_before = kmeans2(X, C0.copy(), iter=I, minit="matrix")
    lab_s, _ = vq(X, Cs)
    np.testing.assert_allclose(C, Cs, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(lab, lab_s)
    # the labels scipy returns are those of the last round, before its update
    Cp, lab_p, _ = lloyd(X, C0, I - 1, mode="exact")
    np.testing.assert_array_equal(lab_p, lab_before)


def test_parity_assign_equals_vq_on_rounded_operands():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((2000, 64)).astype(np.float32) * 3
    C = rng.standard_normal((100, 64)).astype(np.float32) * 3
    lab = assign(X, C, "parity")
    ref, _ = vq(bf16_round(X), bf16_round(C))
    np.testing.assert_array_equal(lab, ref)


def test_ties_go_to_lowest_index():
    C = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0], [0.0, 1.0]])
    X = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.5], [3.0, 3.0]])
    np.testing.assert_array_equal(assign(X, C, "exact"), [0, 1, 0, 0])
    np.testing.assert_array_equal(assign(X, C, "parity"), [0, 1, 0, 0])


def test_near_tie_decided_on_exact_distance():
    # D = |c|^2 - 2<x,c>: D0 - D1 = eps^2 = 2^-10, far below the re-check
    # window (1e-12 * 2^41), so the exactly summed distances decide
    big = 2.0 ** 20
    x = np.array([[big, 1.0]])
    C = np.array([[big, 1.0 + 2.0 ** -5], [big, 1.0]])   # the second is the exact match
    assert assign(x, C, "exact")[0] == 1
    # below float64 resolution of D (eps^2 = 2^-14 < ulp(2^40) = 2^-12) it is a tie
    C2 = np.array([[big, 1.0 + 2.0 ** -7], [big, 1.0]])
    assert assign(x, C2, "exact")[0] == 0


def test_empty_cluster_keeps_previous_centroid():
    X = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    C0 = np.array([[0.2, 0.2], [100.0, 100.0]])
    lab = assign(X, C0, "exact")
    C, counts = update(X, lab, C0, "exact")
    assert counts.tolist() == [3, 0]
    np.testing.assert_array_equal(C[1], C0[1])
    np.testing.assert_allclose(C[0], [1 / 3, 1 / 3])


def _rounded_mean(rows):
    """fp32(fp64(fp64(exact sum) / n)) from rational arithmetic."""
    exact = sum((Fraction(float(v)) for v in rows), Fraction(0))
    return np.float32(np.float64(float(exact)) / np.float64(len(rows)))


@pytest.mark.parametrize("kind", ["bf16", "fp32-cancelling"])
def test_parity_update_is_the_rounded_exact_mean(kind):
    rng = np.random.default_rng(3)
    if kind == "bf16":
        X = bf16_round(rng.standard_normal((500, 16)) * np.array([1.0] * 15 + [300.0]))
    else:
        # fp32 rows whose sums cancel: big values of both signs plus tiny ones
        X = (rng.standard_normal((500, 16)) * rng.choice([1e-6, 1.0, 1e4], size=(500, 16))).astype(np.float32)
        X = X.astype(np.float64)
    lab = rng.integers(0, 7, size=500)
    C, counts = update(X, lab, np.zeros((7, 16)), "parity")
    for k in range(7):
        rows = X[lab == k]
        for j in range(16):
            assert np.float32(C[k, j]) == _rounded_mean(rows[:, j]), (k, j)


def test_update_does_not_depend_on_row_order():
    rng = np.random.default_rng(4)
    X = (rng.standard_normal((300, 8)) * rng.choice([1e-7, 1.0, 1e5], size=(300, 8))).astype(np.float32)
    lab = rng.integers(0, 3, size=300)
    perm = rng.permutation(300)
    a, _ = update(X.astype(np.float64), lab, np.zeros((3, 8)), "parity")
    b, _ = update(X[perm].astype(np.float64), lab[perm], np.zeros((3, 8)), "parity")
    np.testing.assert_array_equal(a, b)


def test_brute_force_optimum_on_separated_blobs():
    rng = np.random.default_rng(11)
    X = _blobs(rng, [[0, 0], [10, 0], [0, 10]], 3, 0.3, 2)
    N, K = len(X), 3
    labs = np.array(list(itertools.product(range(K), repeat=N)))
    onehot = (labs[:, :, None] == np.arange(K)[None, None, :]).astype(float)   # [L][N][K]
    cnt = onehot.sum(1)
    sums = np.einsum("lnk,nd->lkd", onehot, X)
    sq = (X ** 2).sum(1)
    sse = sq.sum() - ((sums ** 2).sum(2) / np.maximum(cnt, 1)).sum(1)
    best = sse.min()
    blob = np.repeat(np.arange(3), 3)
    hit = 0
    for seed in range(40):
        C0 = X[forgy_indices(N, K, seed, 0, 1)]
        C, lab, _ = lloyd(X, C0, 8, mode="exact")
        got = ((X - C[lab]) ** 2).sum()
        if len(set(blob[forgy_indices(N, K, seed, 0, 1)])) == 3:
            hit += 1
            assert got == pytest.approx(best, rel=1e-12)
        assert got >= best - 1e-9
    assert hit >= 5


def test_result_is_a_lloyd_fixed_point():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((400, 6))
    C, lab, _ = lloyd(X, X[:10], 60, mode="exact")
    # every label is the nearest centroid; every used centroid is its cluster's mean
    D = ((X[:, None, :] - C[None, :, :]) ** 2).sum(2)
    np.testing.assert_array_equal(lab, D.argmin(1))
    for k in np.unique(lab):
        np.testing.assert_allclose(C[k], X[lab == k].mean(0), rtol=1e-12, atol=1e-12)


def test_sse_never_increases_in_exact_mode():
    rng = np.random.default_rng(9)
    X = rng.standard_normal((800, 16)) * np.linspace(0.5, 4, 16)
    _, _, hist = lloyd(X, X[forgy_indices(800, 32, 1, 0, 1)], 15, mode="exact")
    assert all(b <= a * (1 + 1e-12) for a, b in zip(hist, hist[1:]))
