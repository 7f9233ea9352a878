"""Pins of the oracle's attention over the decoded cache (the consumer the
fused decode feeds: the pages' fused dequantisation kernel keeps the rebuilt
keys and values out of memory, 163.com article, section 5; German summary,
section 2C).

* A hand-derived 2-query, 2-key case (closed-form softmax weights).
* Special cases: one key gives its value; equal keys give the mean of the
  values; a per-query constant added to every score leaves the output alone.
* The log-sum-exp merges: attention over two halves of the keys, combined by
  their log-sum-exps, equals attention over all keys.
* Lossless inputs: a chunk encoded without loss (at most K distinct rows, one
  of each in the start) decodes to the input, so attention over the decoded
  cache equals attention over the original keys and values exactly."""
import math

import numpy as np
import pytest

import oracle
from oracle import CodecConfig, bf16_round


def test_hand_derived_two_by_two():
    # q1 = (1, 0), q2 = (0, 2); k1 = (ln 3, 0), k2 = (0, 0); scale 1
    # scores: q1: (ln 3, 0) -> weights (3/4, 1/4); q2: (0, 0) -> (1/2, 1/2)
    Q = np.array([[[1.0, 0.0], [0.0, 2.0]]])
    K = np.array([[[math.log(3.0), 0.0], [0.0, 0.0]]])
    V = np.array([[[4.0, -8.0], [0.0, 8.0]]])
    O, lse = oracle.attention(Q, K, V, 1.0)
    np.testing.assert_allclose(O[0], [[3.0, -4.0], [2.0, 0.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], [math.log(4.0), math.log(2.0)], rtol=0, atol=1e-15)


def test_special_cases():
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((2, 5, 8))
    K1, V1 = rng.standard_normal((2, 1, 8)), rng.standard_normal((2, 1, 8))
    np.testing.assert_allclose(oracle.attention(Q, K1, V1, 0.3)[0], np.broadcast_to(V1, (2, 5, 8)), atol=1e-15)
    Ke = np.repeat(K1, 7, axis=1)
    Ve = rng.standard_normal((2, 7, 8))
    np.testing.assert_allclose(oracle.attention(Q, Ke, Ve, 0.3)[0],
                               np.broadcast_to(Ve.mean(axis=1, keepdims=True), (2, 5, 8)), atol=1e-14)
    K, V = rng.standard_normal((2, 9, 8)), rng.standard_normal((2, 9, 8))
    O, lse = oracle.attention(Q, K, V, 0.5)
    # a shift of every score of a query: append a channel of value c to q and 1 to every key
    c = 3.7
    Qs = np.concatenate([Q, np.full((2, 5, 1), c / 0.5)], axis=2)
    Ks = np.concatenate([K, np.ones((2, 9, 1))], axis=2)
    Os, lses = oracle.attention(Qs, Ks, V, 0.5)
    np.testing.assert_allclose(Os, O, atol=1e-13)
    np.testing.assert_allclose(lses, lse + c, atol=1e-12)


def test_halves_merge_by_log_sum_exp():
    rng = np.random.default_rng(1)
    Q, K, V = rng.standard_normal((3, 4, 16)), rng.standard_normal((3, 20, 16)), rng.standard_normal((3, 20, 16))
    O, lse = oracle.attention(Q, K, V, 0.25)
    Oa, la = oracle.attention(Q, K[:, :7], V[:, :7], 0.25)
    Ob, lb = oracle.attention(Q, K[:, 7:], V[:, 7:], 0.25)
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M)[..., None], np.exp(lb - M)[..., None]
    np.testing.assert_allclose((wa * Oa + wb * Ob) / (wa + wb), O, atol=1e-14)
    np.testing.assert_allclose(M + np.log(np.exp(la - M) + np.exp(lb - M)), lse, atol=1e-14)


def test_lossless_cache_gives_the_exact_attention():
    rng = np.random.default_rng(2)
    Kc, d, N = 16, 64, 300
    rows = {}
    for t in ("K", "V"):
        Vd = bf16_round(rng.standard_normal((Kc, d)) * 3).astype(np.float32)
        X = Vd[rng.integers(0, Kc, N)][None]
        cfg = CodecConfig(d=d, n_centroids=Kc, n_stages=1, group_size=16, iters_cold=2, iters_warm=2, seed=1,
                          dtype="bf16")
        enc = oracle.encode_chunk(X, cfg, init=Vd[None, None])
        np.testing.assert_array_equal(oracle.decode(enc, 16, "bf16"), X)
        rows[t] = (X, oracle.decode(enc, 16, "bf16"))
    Q = bf16_round(rng.standard_normal((1, 10, d))).astype(np.float32)
    Oa, la = oracle.attention(Q, rows["K"][0], rows["V"][0], d ** -0.5)
    Ob, lb = oracle.attention(Q, rows["K"][1], rows["V"][1], d ** -0.5)
    np.testing.assert_array_equal(Oa, Ob)
    np.testing.assert_array_equal(la, lb)


def test_tolerance_covers_bf16_rounded_weights():
    """The stated tolerance holds for an emulation that rounds the weights to
    bf16 and accumulates in float32 (the kernel's arithmetic order)."""
    rng = np.random.default_rng(3)
    Q = bf16_round(rng.standard_normal((2, 8, 32)) * 4)
    K = bf16_round(rng.standard_normal((2, 50, 32)) * 4)
    V = bf16_round(rng.standard_normal((2, 50, 32)) * 100)
    O, _ = oracle.attention(Q, K, V, 32 ** -0.5)
    S = (32 ** -0.5) * np.einsum("hqd,hkd->hqk", Q, K)
    E = np.exp(S - S.max(axis=2, keepdims=True))
    Pb = bf16_round(E).astype(np.float32)
    Oe = np.einsum("hqk,hkd->hqd", Pb, V.astype(np.float32)) / E.sum(axis=2, keepdims=True)
    assert np.all(np.abs(Oe - O) <= oracle.attention_tolerance(Q, K, V, 32 ** -0.5))
