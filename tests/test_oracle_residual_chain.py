"""Pin of the oracle's residual chain (163.com article, section 4: each stage
works on what the earlier stages left, and reconstruction adds the stored
centroids back stage by stage in reverse).

The chain is R(t) = fp32(R(t-1) - C_stored(t)[pi(t)]): the residual is taken
against the centroids as stored (bf16 for a bf16 tensor), and it is held in
fp32.  Two facts that do not restate that formula pin it:

* whatever the oracle quantised, the reconstruction from the *stored* encoding,
  summed exactly, must lie within the quantiser's error bound of the input:
  |x - (deq + sum_t C_stored(t)[pi(t)])| <= max(s/2, a - 1.5 s) of the group,
  plus the T fp32 roundings of the chain;
* every residual the oracle hands to the next stage is an fp32 number.

The chunk is bf16 with 1e2 / 1e3 outlier channels, so the fp32 means differ
from their bf16-stored values by up to 2 there, far above the final residual's
quantisation step; a few tokens hold tiny values in an outlier channel, so the
differences against 1e3-sized centroids are not fp32 numbers.  The test also
plants each plausible mistake in a copy of the oracle (subtracting the unrounded
fp32 centroids; keeping R in float64) and checks that the pin catches it."""
import os
import sys
import types

import numpy as np
import pytest

import oracle
from oracle import CodecConfig, bf16_round, e4m3_decode

F32 = np.float32
ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "qvg.py")


def _chunk(seed=3, H=2, N=600, d=64, K=8):
    rng = np.random.default_rng(seed)
    X = np.empty((H, N, d), np.float32)
    for h in range(H):
        centers = rng.standard_normal((K, d)) * 4.0
        centers[:, 3] = 100.0 * (1 + 0.1 * rng.standard_normal(K))       # key-like outlier channel
        centers[:, 17] = -1000.0 * (1 + 0.1 * rng.standard_normal(K))    # value-like outlier channel
        lab = rng.integers(0, K, N)
        rows = centers[lab] + 0.05 * rng.standard_normal((N, d))
        odd = rng.choice(N, size=N // 40, replace=False)                   # outlier moved away
        rows[odd, 17] = rng.uniform(-1e-3, 1e-3, size=len(odd))
        X[h] = bf16_round(rows)
    return X


def _pin(enc, X, G):
    """The two facts above; returns the failures (empty when the pin holds)."""
    bad = []
    T = enc.assign.shape[0]
    for t in range(1, T + 1):
        r = enc.residuals[t]
        if not np.array_equal(r, r.astype(F32).astype(np.float64)):
            bad.append(f"R({t}) holds values that are not fp32 numbers")
    H, N, d = X.shape
    RT = enc.residuals[T].astype(F32)
    a = np.abs(RT.reshape(H, N, d // G, G)).max(axis=3).astype(np.float64)
    s = e4m3_decode(enc.scales).astype(np.float64)
    bound = np.maximum(s / 2, a - 1.5 * s)[..., None] * np.ones((1, 1, 1, G))
    bound = bound.reshape(H, N, d)
    mag = np.abs(X).astype(np.float64)
    for t in range(T):
        for h in range(H):
            mag[h] += np.abs(enc.centroids[t, h].astype(np.float64))[enc.assign[t, h]]
    slack = T * 2.0 ** -23 * mag
    err = np.abs(X.astype(np.float64) - oracle.decode(enc, G, "f64"))
    over = err > bound + slack
    if over.any():
        bad.append(f"{int(over.sum())} values outside the quantiser bound (worst excess "
                   f"{float((err - bound - slack).max()):.4g})")
    return bad


def _mutant(old: str, new: str) -> types.ModuleType:
    """A copy of oracle/qvg.py with one line changed (CPU only, never used elsewhere)."""
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"the line to mutate is no longer in the oracle: {old!r}"
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    sys.modules[mod.__name__] = mod          # dataclasses look their module up there
    try:
        exec(compile(src.replace(old, new), ORACLE_SRC + " (mutant)", "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


CFG = CodecConfig(d=64, n_centroids=8, n_stages=2, group_size=16, iters_cold=4, iters_warm=2, seed=9,
                  dtype="bf16")


def test_stored_centroids_differ_from_fp32_means():
    """Premise of the pin: the data makes bf16 storage matter."""
    X = _chunk()
    enc = oracle.encode_chunk(X, CFG, keep_residuals=True)
    gap = np.abs(enc.cache.astype(np.float64) - enc.centroids.astype(np.float64))
    assert gap[..., 17].max() >= 0.5          # the 1e3 channel: bf16 spacing is 4 there
    assert _pin(enc, X, CFG.group_size) == []


def test_residual_chain_pinned_cold_and_warm():
    X = _chunk(seed=4, N=1200)
    a = oracle.encode_chunk(X[:, :600], CFG, keep_residuals=True)
    assert _pin(a, X[:, :600], CFG.group_size) == []
    b = oracle.encode_chunk(X[:, 600:], CFG, cache=a.cache, keep_residuals=True)
    assert _pin(b, X[:, 600:], CFG.group_size) == []


@pytest.mark.parametrize("old,new,why", [
    ("R = R - Cs.astype(np.float64)[lab]", "R = R - C.astype(np.float64)[lab]",
     "residual against the unrounded fp32 centroids"),
    ("R = R.astype(F32).astype(np.float64)", "R = R", "residual kept in float64"),
])
def test_pin_catches_planted_mistakes(old, new, why):
    X = _chunk()
    enc = _mutant(old, new).encode_chunk(X, CFG, keep_residuals=True)
    assert _pin(enc, X, CFG.group_size), f"a broken oracle ({why}) passed the pin"
