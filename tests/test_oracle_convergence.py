"""Pins of the oracle's convergence-driven k-means (the stop rule behind the
pages' claim that k-means needs fewer rounds with the streaming centroid
cache: 163.com article, section 5; German summary, section 2C).

* c = 1 stops at a fixed point of Lloyd's iteration, so the result must equal
  the fixed-count result for every larger count, and be a fixed point by
  brute-force check (every label nearest, every non-empty centroid the mean).
* c > 1: the number of updates run must be the first round, counted from an
  independent fixed-count run's label history, whose assignment moved fewer
  than c tokens; the result must equal the fixed-count run stopped there."""
import numpy as np
import pytest

import synthkv
from oracle import CodecConfig, encode_chunk, lloyd
from oracle.rng import forgy_indices


def _blobs(seed, N=900, d=16, K=12):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((K, d)) * 6
    lab = rng.integers(0, K, N)
    return (centers[lab] + rng.standard_normal((N, d))).astype(np.float32)


@pytest.mark.parametrize("mode", ["exact", "parity"])
def test_stop_on_unchanged_labels_is_exact(mode):
    X = _blobs(1)
    C0 = X[forgy_indices(len(X), 12, 7, 0, 1)]
    Cc, lc, hc = lloyd(X, C0, 80, mode, converge=1)
    r = len(hc)
    assert 0 < r < 80
    for iters in (r, r + 1, r + 7, 80):
        Cf, lf, _ = lloyd(X, C0, iters, mode)
        np.testing.assert_array_equal(Cf, Cc)
        np.testing.assert_array_equal(lf, lc)
    # one round fewer is not the fixed point yet (the stop is not late either)
    Cm, lm, _ = lloyd(X, C0, r - 1, mode)
    assert not (np.array_equal(Cm, Cc) and np.array_equal(lm, lc))


def test_converged_result_is_a_fixed_point_by_brute_force():
    X = _blobs(2, N=300, d=6, K=5).astype(np.float64)
    C0 = X[:5].copy()
    C, lab, _ = lloyd(X, C0, 100, "exact", converge=1)
    D = ((X[:, None, :] - C[None, :, :]) ** 2).sum(axis=2)
    np.testing.assert_array_equal(lab, D.argmin(axis=1))
    for k in range(5):
        if (lab == k).any():
            np.testing.assert_allclose(C[k], X[lab == k].mean(axis=0), rtol=0, atol=1e-12)


@pytest.mark.parametrize("c", [2, 5, 20])
def test_threshold_stop_matches_the_label_history(c):
    X = synthkv.gen_numpy(synthkv.PRESETS[2], "V", heads=1, n_tokens=1500)[0]
    C0 = X[forgy_indices(len(X), 64, 3, 0, 1)]
    hist_labels = []
    lloyd(X, C0, 40, "parity", labels_history=hist_labels)
    moved = [int((b != a).sum()) for a, b in zip(hist_labels, hist_labels[1:])]
    first = next((i + 1 for i, m in enumerate(moved) if m < c), 40)
    Cc, lc, hc = lloyd(X, C0, 40, "parity", converge=c)
    assert len(hc) == first, (moved, first, len(hc))
    Cf, lf, _ = lloyd(X, C0, first, "parity")
    np.testing.assert_array_equal(Cc, Cf)
    np.testing.assert_array_equal(lc, lf)


def test_encode_records_rounds_and_warm_chunks_start_converged_sooner_or_equal():
    p = synthkv.PRESETS[2]
    X = synthkv.gen_numpy(p, "K", heads=2, n_tokens=1200)
    cfg = CodecConfig(d=p.d, n_centroids=32, n_stages=2, group_size=p.group_size, iters_cold=40, iters_warm=40,
                      seed=5, dtype="bf16", converge=1)
    a = encode_chunk(X[:, :600], cfg)
    fixed = encode_chunk(X[:, :600], CodecConfig(**{**cfg.__dict__, "converge": 0}))
    assert a.rounds.shape == (2, 2) and np.all(a.rounds <= 40)
    assert np.all(fixed.rounds == 40)
    for k in ("codes", "scales", "assign", "centroids", "cache"):
        if np.all(a.rounds < 40):   # converged within the budget: identical to the fixed count
            np.testing.assert_array_equal(getattr(a, k), getattr(fixed, k))
    b = encode_chunk(X[:, 600:], cfg, cache=a.cache)
    assert b.rounds.shape == (2, 2)
