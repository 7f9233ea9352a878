"""Pins of the seeded cold-start draw: published SplitMix64 outputs, the
Fisher-Yates definition applied by hand to them, and distribution checks."""
import numpy as np

from conftest import golden
from oracle import forgy_indices, forgy_key, shuffle_prefix, splitmix64_next


def test_splitmix64_published_outputs():
    g = golden("splitmix64_seed0.json")
    s = g["state0"]
    for want in g["outputs_hex"]:
        s, z = splitmix64_next(s)
        assert z == int(want, 16)


def test_shuffle_prefix_by_hand_from_published_draws():
    # key 0 draws the three published values r0, r1, r2 (decimal r0 =
    # 16294208416658607535).  For n = 10: r0 mod 10 = 5 -> swap a[0], a[5];
    # r1 mod 9 = 0 -> a[1] stays; r2 mod 8 = 7 -> swap a[2], a[9].
    # a = [5, 1, 9, 3, 4, 0, 6, 7, 8, 2]
    assert shuffle_prefix(10, 3, 0) == [5, 1, 9]
    assert shuffle_prefix(10, 10, 0)[:3] == [5, 1, 9]


def test_forgy_key_layout():
    assert forgy_key(0, 0, 1) == 1
    assert forgy_key(1, 0, 1) == 65536 * 64 + 1
    assert forgy_key(2, 3, 4) == (2 * 65536 + 3) * 64 + 4
    assert forgy_key(1 << 60, 0, 0) == ((1 << 60) * 65536 * 64) % (1 << 64)


def test_forgy_distinct_and_in_range():
    for n, k in [(4680, 256), (560, 256), (257, 256), (128, 16)]:
        idx = forgy_indices(n, k, 2000, 3, 1)
        assert len(set(idx)) == k and min(idx) >= 0 and max(idx) < n


def test_forgy_fewer_tokens_than_centroids_cycles():
    idx = forgy_indices(5, 12, 7, 0, 2)
    assert sorted(idx[:5]) == [0, 1, 2, 3, 4]
    assert idx[5:10] == idx[:5] and idx[10:] == idx[:2]


def test_forgy_first_index_uniform():
    n, trials = 10, 20000
    counts = np.bincount([shuffle_prefix(n, 1, forgy_key(s, 0, 1))[0] for s in range(trials)],
                         minlength=n)
    chi2 = (((counts - trials / n) ** 2) / (trials / n)).sum()
    assert chi2 < 27.9        # chi-square, 9 dof, p = 0.001


def test_forgy_pairs_uniform():
    # second index given the first: all ordered pairs of distinct values equally likely
    n, trials = 5, 20000
    counts = np.zeros((n, n))
    for s in range(trials):
        i, j = shuffle_prefix(n, 2, forgy_key(s, 1, 2))
        counts[i, j] += 1
    assert np.all(np.diag(counts) == 0)
    off = counts[~np.eye(n, dtype=bool)]
    chi2 = (((off - trials / 20) ** 2) / (trials / 20)).sum()
    assert chi2 < 43.8        # 19 dof, p = 0.001
