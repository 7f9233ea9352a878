"""Pins of the oracle's 2-bit group quantiser, packing and reconstruction:
a hand-worked example, lossless special cases and the closed-form error bound."""
import numpy as np
import pytest

from conftest import golden
from oracle import (CodecConfig, decode, dequant, e4m3_decode, encode_chunk, group_quant,
                    pack2, unpack2)


def _hand_cfg(g):
    c = g["config"]
    return CodecConfig(d=c["d"], n_centroids=c["n_centroids"], n_stages=c["n_stages"],
                       group_size=c["group_size"], iters_cold=c["iters"], iters_warm=c["iters"],
                       seed=0, dtype=c["dtype"])


def test_hand_worked_example():
    g = golden("hand_example_t1.json")
    cfg = _hand_cfg(g)
    X = np.array(g["x"], np.float32)[None]
    init = np.array(g["init"], np.float32)[None, None]
    enc = encode_chunk(X, cfg, init=init)
    np.testing.assert_array_equal(enc.assign[0, 0], g["labels"])
    np.testing.assert_array_equal(enc.centroids[0, 0], g["centroids"])
    np.testing.assert_array_equal(enc.cache[0, 0], g["centroids"])
    np.testing.assert_array_equal(enc.scales[0, :, 0], g["scale_codes"])
    np.testing.assert_array_equal(enc.codes[0, :, 0], g["packed"])
    for out in ("f32", "f64"):
        np.testing.assert_array_equal(decode(enc, cfg.group_size, out)[0], g["decoded"])
    np.testing.assert_array_equal(decode(enc, cfg.group_size, "bf16")[0], g["decoded_bf16"])


def test_codes_in_range_and_pack_roundtrip():
    rng = np.random.default_rng(0)
    R = (rng.standard_normal((300, 128)) * rng.uniform(0.01, 50, (300, 1))).astype(np.float32)
    q, packed, s = group_quant(R, 64)
    assert q.min() >= 0 and q.max() <= 3
    np.testing.assert_array_equal(unpack2(packed), q)
    np.testing.assert_array_equal(pack2(unpack2(packed)), packed)
    # lowest channel in the lowest bits
    one = np.zeros((1, 8), np.uint8)
    one[0, :4] = [1, 2, 3, 0]
    assert pack2(one)[0, 0] == 1 + (2 << 2) + (3 << 4)


def test_lossless_when_values_sit_on_the_levels():
    # T = 0: each group holds values in {+-0.5, +-1.5} * 2^e and contains +-1.5 * 2^e,
    # so the scale 2^e is exact in E4M3 and every value is a level
    rng = np.random.default_rng(1)
    N, d, G = 64, 128, 16
    e = rng.integers(-9, 9, size=(N, d // G, 1))
    lv = rng.choice(np.array([-1.5, -0.5, 0.5, 1.5]), size=(N, d // G, G))
    lv[..., 0] = rng.choice([-1.5, 1.5], size=(N, d // G))
    X = (lv * np.ldexp(1.0, e)).reshape(N, d).astype(np.float32)
    cfg = CodecConfig(d=d, n_centroids=4, n_stages=0, group_size=G, iters_cold=1, iters_warm=1,
                      seed=0, dtype="f32")
    enc = encode_chunk(X[None], cfg)
    np.testing.assert_array_equal(decode(enc, G, "f32")[0], X)
    np.testing.assert_array_equal(e4m3_decode(enc.scales[0]), np.ldexp(1.0, e[..., 0]))


def test_zero_groups_give_zero_scale():
    R = np.zeros((3, 32), np.float32)
    R[1, 16:] = -0.0
    q, packed, s = group_quant(R, 16)
    assert np.all(s == 0) and np.all(q == 3)
    np.testing.assert_array_equal(dequant(packed, s, 16), 0.0)


@pytest.mark.parametrize("G", [16, 64])
def test_error_bound(G):
    rng = np.random.default_rng(G)
    N, d = 2000, 128
    R = (rng.standard_normal((N, d)) * rng.lognormal(0, 3, (N, 1))).astype(np.float32)
    R[:5, :3] = [[900.0, -1200.0, 5.0]] * 5                  # saturating scales (a > 672)
    q, packed, s = group_quant(R, G)
    y = dequant(packed, s, G).astype(np.float64)
    sf = e4m3_decode(s)[:, :, None]
    a = np.abs(R.reshape(N, d // G, G)).max(2)[:, :, None].astype(np.float64)
    bound = np.maximum(sf / 2, a - 1.5 * sf)
    err = np.abs(R.reshape(N, d // G, G) - y.reshape(N, d // G, G))
    assert np.all(err <= bound * (1 + 1e-7))
    assert np.any(s[:5] == 0x7E)
    # the outer level never overshoots the group maximum by more than E4M3 rounding
    assert np.all(1.5 * sf <= a * (1 + 2.0 ** -4) + 1.5 * 2.0 ** -10)


def test_nearest_level_with_ties_going_up():
    s = 1.0                              # E4M3(1.5 / 1.5) = 1.0 exactly
    R = np.array([[1.5, -1.5, 0.0, -0.0, 1.0, -1.0, 0.999, -1.001,
                   0.5, -0.5, 1.2, -0.2, 0.0, 0.0, 0.0, 0.0]], np.float32)
    q, packed, sc = group_quant(R, 16)
    assert e4m3_decode(sc)[0, 0] == s
    np.testing.assert_array_equal(q[0], [3, 0, 2, 2, 3, 1, 2, 0, 2, 1, 3, 1, 2, 2, 2, 2])
