"""Convergence-driven k-means on the device (config field `converge`): each
head's Lloyd rounds of a stage stop at the first assignment that moves fewer
than `converge` tokens, decided on the device without a host
synchronisation.  Through the C ABI, against the oracle's same rule: labels,
centroids, codes, scales and the streaming cache bit for bit, and the number
of rounds every (stage, head) ran."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, check_chunk, fetch, gcfg, lib, ocfg, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _encode_with_rounds(oc, X, chunk_tokens):
    q = lib()
    H, Ntot, d = X.shape
    cfg = q.config(oc.d, oc.n_centroids, oc.n_stages, oc.group_size, oc.iters_cold, oc.iters_warm, oc.seed,
                   oc.dtype, oc.converge)
    xd = to_dev(X, oc.dtype)
    dst = q.CompressedKV(cfg, H, Ntot, chunk_tokens, DEV)
    enc = q.Encoder(cfg, H, chunk_tokens, DEV)
    cache = q.CentroidCache(cfg, H)
    rounds = []
    for c in range(-(-Ntot // chunk_tokens)):
        b, e = c * chunk_tokens, min((c + 1) * chunk_tokens, Ntot)
        enc.encode(xd[:, b:e], dst, c, cache=cache)
        rounds.append(to_np(enc.rounds()))
    torch.cuda.synchronize()
    return dst, rounds


@pytest.mark.parametrize("converge,tensor,N,chunk", [(1, "K", 4000, 2000), (1, "V", 4000, 2000),
                                                     (6, "V", 4000, 2000), (180, "K", 18000, 18000)])
def test_converged_encode_matches_oracle(converge, tensor, N, chunk):
    say(f"convergence mode c={converge} {tensor} N={N} chunk={chunk}")
    p = synthkv.PRESETS[2]
    oc = ocfg(p, tensor, n_centroids=48, iters_cold=25, iters_warm=25, converge=converge)
    H = 3 if N <= 4000 else 1
    X = synthkv.gen_numpy(p, tensor, heads=H, n_tokens=N)
    dst, rounds = _encode_with_rounds(oc, X, chunk)
    cache = {}
    for c in range(-(-N // chunk)):
        b, e = c * chunk, min((c + 1) * chunk, N)
        g = fetch(dst, c, oc)
        for h in range(H):
            ora = oracle.encode_chunk(X[h:h + 1, b:e], oc, cache=cache.get(h), head_offset=h)
            cache[h] = ora.cache
            say(f"  chunk {c} head {h}: rounds per stage GPU {rounds[c][:, h].tolist()} "
                f"oracle {ora.rounds[:, 0].tolist()}")
            np.testing.assert_array_equal(rounds[c][:, h], ora.rounds[:, 0])
            assert check_chunk(oc, X[:, b:e], g, ora, 0, h, f"chunk {c}") == 0


def test_stop_on_unchanged_labels_equals_the_fixed_count():
    """c = 1 stops at a fixed point: where every head settles within the budget,
    the encoding equals the fixed-count encoding with that budget."""
    say("convergence mode c=1 against the fixed count")
    p = synthkv.PRESETS[2]
    X = synthkv.gen_numpy(p, "K", heads=4, n_tokens=1500)
    oc_c = ocfg(p, "K", n_centroids=32, iters_cold=60, iters_warm=60, converge=1)
    oc_f = ocfg(p, "K", n_centroids=32, iters_cold=60, iters_warm=60)
    dc, rounds = _encode_with_rounds(oc_c, X, 1500)
    assert np.all(rounds[0] < 60), rounds[0]
    from gpu_util import gpu_encode_chunks
    df, _ = gpu_encode_chunks(oc_f, X, 1500)
    a, b = fetch(dc, 0, oc_c), fetch(df, 0, oc_f)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
