"""Pins of the oracle's whole encode/decode: lossless special cases, the
progressive-stage invariants, warm starts and error against round-to-nearest
on the redundant generator."""
import numpy as np
import pytest

import synthkv
from oracle import (CodecConfig, bf16_round, decode, encode_chunk, mse, rtn_reconstruct)


def _cfg(p, tensor, **kw):
    c = dict(d=p.d, n_centroids=p.n_centroids, n_stages=p.n_stages, group_size=p.group_size,
             iters_cold=p.iters_cold, iters_warm=p.iters_warm, seed=p.codec_seed(tensor),
             dtype=p.dtype)
    c.update(kw)
    return CodecConfig(**c)


def test_lossless_when_chunk_has_at_most_k_distinct_rows():
    rng = np.random.default_rng(0)
    K, d, N = 16, 64, 300
    V = bf16_round(rng.standard_normal((K, d)) * 30).astype(np.float32)
    V[3, 5] = 250.0                                  # an outlier channel
    X = V[rng.integers(0, K, size=N)][None]
    cfg = CodecConfig(d=d, n_centroids=K, n_stages=1, group_size=16, iters_cold=3,
                      iters_warm=3, seed=1, dtype="bf16")
    enc = encode_chunk(X, cfg, init=V[None, None], keep_residuals=True)
    assert np.all(enc.residuals[1] == 0)
    assert np.all(enc.scales == 0)
    np.testing.assert_array_equal(decode(enc, 16, "bf16"), X)
    np.testing.assert_array_equal(decode(enc, 16, "f32"), X)


def test_stage_prefix_property():
    p = synthkv.PRESETS[1]
    X = synthkv.gen_numpy(p, "K")
    e1 = encode_chunk(X, _cfg(p, "K", n_stages=1))
    e3 = encode_chunk(X, _cfg(p, "K", n_stages=3))
    np.testing.assert_array_equal(e1.assign[0], e3.assign[0])
    np.testing.assert_array_equal(e1.centroids[0], e3.centroids[0])
    np.testing.assert_array_equal(e1.cache[0], e3.cache[0])


def test_warm_start_uses_previous_chunk_centroids():
    p = synthkv.PRESETS[2]
    X = synthkv.gen_numpy(p, "K", n_tokens=1200)
    cfg = _cfg(p, "K", n_centroids=32, iters_cold=4, iters_warm=2)
    a, b = X[:, :600], X[:, 600:]
    ea = encode_chunk(a, cfg)
    assert [len(h) for h in ea.sse[0]] == [4]
    eb = encode_chunk(b, cfg, cache=ea.cache)
    assert [len(h) for h in eb.sse[0]] == [2]
    eb2 = encode_chunk(b, cfg, init=ea.cache)
    np.testing.assert_array_equal(eb.assign, eb2.assign)
    # the cache holds the unrounded fp32 centroids, the stream holds bf16 ones
    assert ea.cache.dtype == np.float32
    np.testing.assert_array_equal(bf16_round(ea.cache).astype(np.float32), ea.centroids)
    assert not np.array_equal(ea.cache, ea.centroids)


def test_stage_energy_never_increases_exact_mode():
    p = synthkv.PRESETS[1]
    X = synthkv.gen_numpy(p, "K")
    enc = encode_chunk(X, _cfg(p, "K", n_stages=3), mode="exact", keep_residuals=True)
    e = [float((r.astype(np.float64) ** 2).sum()) for r in enc.residuals]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(e, e[1:])), e


@pytest.mark.parametrize("tensor", ["K", "V"])
def test_qvg_beats_rtn_on_redundant_data(tensor):
    p = synthkv.PRESETS[2]
    X = synthkv.gen_numpy(p, tensor)
    cfg = _cfg(p, tensor)
    y = decode(encode_chunk(X, cfg), cfg.group_size, "bf16")
    m_q, m_r = mse(y, X), mse(rtn_reconstruct(X, cfg.group_size), X)
    assert m_q < m_r / 10, (m_q, m_r)


def test_per_stage_error_decreases_aggressive_setting():
    p = synthkv.PRESETS[4]
    X = synthkv.gen_numpy(p, "K", heads=2, n_tokens=2000)
    errs = []
    for T in range(0, 5):
        cfg = _cfg(p, "K", n_stages=T)
        errs.append(mse(decode(encode_chunk(X, cfg), cfg.group_size, "f32"), X))
    assert all(b < a for a, b in zip(errs, errs[1:])), errs


def test_decode_orders_agree_and_bf16_is_rounded_fp32():
    p = synthkv.PRESETS[1]
    X = synthkv.gen_numpy(p, "K")
    cfg = _cfg(p, "K", n_stages=2)
    enc = encode_chunk(X, cfg)
    y32, y64 = decode(enc, 16, "f32"), decode(enc, 16, "f64")
    mag = np.abs(y64) + np.abs(enc.centroids).max()
    assert np.all(np.abs(y32 - y64) <= 4 * np.finfo(np.float32).eps * mag)
    np.testing.assert_array_equal(decode(enc, 16, "bf16"), bf16_round(y32).astype(np.float32))
