"""Pins of the oracle's two-level scales (a per-(chunk, head) power of two
times the E4M3 group scale, for value residuals whose groups exceed E4M3's
range: 163.com article, section 2 for value outliers near 1e3, section 5 for
the E4M3 scales).

* The exponent is the smallest f >= 0 with no saturating group (scan).
* Without saturation f = 0 and the result equals the plain quantiser.
* Lossless groups far above E4M3's range ({+-0.5, +-1.5} x 2^k with k >= 9,
  where the plain scale saturates) are reconstructed exactly.
* The per-element bound max(s/2, a - 1.5 s) holds with the true scale, and the
  worst error on saturating groups is below the saturated one (the mean square
  error need not be: the larger step also applies to the group's small
  values)."""
import math

import numpy as np
import pytest

import oracle
from oracle import CodecConfig, dequant, group_quant, two_level_exponent


@pytest.mark.parametrize("amax", [1.0, 671.9, 672.0, 672.1, 1344.0, 1344.5, 5000.0, 1e6])
def test_exponent_is_the_smallest_without_saturation(amax):
    R = np.array([[amax] + [0.5] * 15], np.float32)
    f = two_level_exponent(R)
    a15 = float(np.float32(np.float32(amax) / np.float32(1.5)))
    ok = [k for k in range(0, 40) if a15 <= 448.0 * 2.0 ** k]
    assert f == min(ok)


def test_no_saturation_means_the_plain_quantiser():
    rng = np.random.default_rng(0)
    R = (rng.standard_normal((200, 64)) * 100).astype(np.float32)
    assert two_level_exponent(R) == 0
    a = group_quant(R, 16)
    b = group_quant(R, 16, 0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_lossless_far_above_the_e4m3_range():
    rng = np.random.default_rng(1)
    N, d, G, k = 40, 64, 16, 11                       # values up to 1.5 x 2^11 = 3072
    vals = np.array([-1.5, -0.5, 0.5, 1.5]) * 2.0 ** k
    R = rng.choice(vals, size=(N, d)).astype(np.float32)
    R[:, ::G] = 1.5 * 2.0 ** k                         # every group holds its outer level
    f = two_level_exponent(R)
    assert f == 3                                      # 2^11 / 2^3 = 256 <= 448
    _, packed, s = group_quant(R, G, f)
    np.testing.assert_array_equal(dequant(packed, s, G, f), R)
    _, p0, s0 = group_quant(R, G, 0)                   # the plain scale saturates at 448
    assert np.abs(dequant(p0, s0, G, 0) - R).max() > 100


def test_error_bound_and_gain_on_saturating_groups():
    rng = np.random.default_rng(2)
    R = (rng.standard_normal((300, 64)) * 200).astype(np.float32)
    R[:30, 3] = rng.uniform(800, 3000, 30)             # saturating groups in 30 tokens
    f = two_level_exponent(R)
    assert f >= 1
    _, p2, s2 = group_quant(R, 16, f)
    y2 = dequant(p2, s2, 16, f)
    a = np.abs(R.reshape(300, 4, 16)).max(axis=2)
    sf = np.ldexp(oracle.e4m3_decode(s2), f)
    bound = np.maximum(sf / 2, a - 1.5 * sf)
    err2 = np.abs(y2 - R).reshape(300, 4, 16).max(axis=2)
    assert np.all(err2 <= bound * (1 + 1e-6) + 1e-6)
    _, p0, s0 = group_quant(R, 16, 0)
    err0 = np.abs(dequant(p0, s0, 16, 0) - R).reshape(300, 4, 16).max(axis=2)
    assert err2[:30, 0].max() < err0[:30, 0].max()


def test_encode_records_the_exponent_and_decode_uses_it():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((2, 300, 64)) * 3).astype(np.float32)
    X[1, :5, 7] = [1000.0, 2000.0, 3000.0, 4000.0, 5000.0]   # head 1: residual groups above 672
    cfg = CodecConfig(d=64, n_centroids=8, n_stages=1, group_size=16, iters_cold=2, iters_warm=2, seed=1,
                      dtype="f32", scale_mode="two_level")
    enc = oracle.encode_chunk(X, cfg)
    assert enc.scale_exp[0] == 0 and enc.scale_exp[1] >= 1
    y = oracle.decode(enc, 16, "f32")
    plain = oracle.encode_chunk(X, CodecConfig(**{**cfg.__dict__, "scale_mode": "e4m3"}))
    np.testing.assert_array_equal(enc.codes[0], plain.codes[0])
    # the worst element error drops (saturation leaves a - 672); the mean
    # square error of the group's small values may rise with the larger step
    y0 = oracle.decode(plain, 16, "f32")
    assert np.abs(y[1] - X[1]).max() < np.abs(y0[1] - X[1]).max()
