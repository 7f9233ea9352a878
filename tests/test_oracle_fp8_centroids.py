"""Pins of the oracle's FP8 centroid storage (the storage-format variant with
the centroid tables in E4M3 like the scales: 163.com article, sections 5-7).

* The table exponent is the smallest e with max|C| <= 448 * 2^e, checked by
  scanning every e in a range.
* Every stored value is the nearest point of the E4M3 grid scaled by 2^e,
  checked by brute force over all 253 finite grid points (ties to the even
  code), and is exactly representable in bf16.
* A chunk of at most K distinct rows on that grid, started from one copy of
  each, is reconstructed exactly (the FP8 analogue of the lossless case).
* The residual chain stays pinned with FP8 tables (error bound and fp32
  residuals), and every stage's labels are nearest under the stored values.
* Byte accounting: each table costs K d bytes plus a 16-byte header; the
  compression ratio of the bench layer's format rises from 4.00x to 5.12x."""
import math

import numpy as np
import pytest

import oracle
from oracle import CodecConfig, bf16_round, e4m3_values, store_e4m3

from test_oracle_residual_chain import _chunk, _pin


@pytest.mark.parametrize("amax", [448.0, 448.0001, 3584.0, 1000.0, 224.0, 224.1, 1e-3, 7.5, 2.0 ** -20])
def test_table_exponent_is_the_smallest_that_fits(amax):
    C = np.array([[amax, -0.5 * amax], [0.25, 0.0]])
    e = oracle.e4m3_table_exponent(C)
    fits = [k for k in range(-80, 40) if np.abs(C).max() <= 448.0 * 2.0 ** k]
    assert e == min(fits)


def test_stored_values_are_the_nearest_scaled_grid_points():
    rng = np.random.default_rng(4)
    C = (rng.standard_normal((64, 32)) * rng.lognormal(0, 3, (64, 1))).astype(np.float32)
    C[0, 0] = 0.0
    C[1, 1] = -0.0
    e, codes, vals = store_e4m3(C)
    grid = np.concatenate([-e4m3_values()[::-1], e4m3_values()]) * 2.0 ** e
    x = C.astype(np.float64).ravel()
    d = np.abs(x[:, None] - grid[None, :])
    best = d.min(axis=1)
    np.testing.assert_array_equal(np.abs(vals.ravel() - x), best)          # nearest
    assert np.all(np.isin(vals.ravel(), grid))
    np.testing.assert_array_equal(bf16_round(vals), vals)                   # bf16 holds them
    # ties: a value half way between two grid points takes the even code
    C2 = np.array([[448.0, 1.0 + 1.0 / 16, 1.0 + 3.0 / 16]])
    _, c2, v2 = store_e4m3(C2)
    assert list(v2.ravel()) == [448.0, 1.0, 1.25]


def test_lossless_when_rows_are_on_the_scaled_grid():
    rng = np.random.default_rng(1)
    K, d, N = 12, 64, 400
    g = e4m3_values()
    V = rng.choice(g, size=(K, d)) * np.where(rng.random((K, d)) < 0.5, -1, 1) * 8.0
    V[0, 0] = 448.0 * 8.0                                                  # table exponent 3
    X = V[rng.integers(0, K, N)][None].astype(np.float32)
    cfg = CodecConfig(d=d, n_centroids=K, n_stages=1, group_size=16, iters_cold=2, iters_warm=2, seed=1,
                      dtype="bf16", centroid_format="e4m3")
    enc = oracle.encode_chunk(X, cfg, init=V[None, None], keep_residuals=True)
    assert enc.cent_exp[0, 0] == 3
    assert np.all(enc.residuals[1] == 0)
    np.testing.assert_array_equal(oracle.decode(enc, 16, "f32"), X)


def test_residual_chain_and_labels_with_fp8_tables():
    X = _chunk(seed=6)
    cfg = CodecConfig(d=64, n_centroids=8, n_stages=2, group_size=16, iters_cold=4, iters_warm=2, seed=9,
                      dtype="bf16", centroid_format="e4m3")
    enc = oracle.encode_chunk(X, cfg, keep_residuals=True)
    assert _pin(enc, X, cfg.group_size) == []
    for t in range(2):
        for h in range(X.shape[0]):
            R = enc.residuals[t][h]
            Cs = enc.centroids[t, h].astype(np.float64)
            D = ((R[:, None, :] - Cs[None]) ** 2).sum(axis=2)      # no near ties on this data
            np.testing.assert_array_equal(enc.assign[t, h], D.argmin(axis=1))
            e, _, vals = store_e4m3(enc.cache[t, h])
            assert e == enc.cent_exp[t, h]
            np.testing.assert_array_equal(vals.astype(np.float32), enc.centroids[t, h])


def test_fp8_table_bytes_and_ratio():
    cfg = CodecConfig(d=128, n_centroids=256, n_stages=2, group_size=64, iters_cold=10, iters_warm=3, seed=1,
                      dtype="bf16", centroid_format="e4m3")
    b = oracle.chunk_bytes(cfg, 1, 4680)
    assert b["centroids"] == 2 * (256 * 128 + 16)
    r = oracle.compression_ratio(cfg, 1, 4680)
    d, G, T, K, N = 128, 64, 2, 256, 4680
    assert r == pytest.approx(16 * d / (2 * d + 8 * d / G + 8 * T + 8 * T * (K * d + 16) / N), rel=1e-12)
    assert round(r, 2) == 5.12
    assert round(oracle.compression_ratio(CodecConfig(**{**cfg.__dict__, "centroid_format": "native"}), 1, 4680), 2) == 4.0
