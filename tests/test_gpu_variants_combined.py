"""The variants together in one encode: FP8 (E4M3) centroid tables, two-level
group scales and the convergence stop, against the oracle through the C ABI.
Each is tested on its own elsewhere; here the FP8 store (which also writes the
table later stages and the quantiser read), the two-pass quantiser and the
device-side stop run in the same stage loop.  Labels, stored tables, codes,
scales, second-level exponents, rounds per (stage, head) and the decode bit
for bit."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, check_chunk, fetch, gcfg, lib, ocfg, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,sm,conv,tensor,T,G", [("e4m3", "two_level", 0, "V", 2, 64), ("e4m3", "e4m3", 2, "K", 2, 64),
                                                    ("native", "two_level", 1, "V", 2, 64),
                                                    ("e4m3", "two_level", 3, "V", 2, 64),
                                                    ("e4m3", "two_level", 2, "K", 4, 16)])
def test_variants_together_match_oracle(fmt, sm, conv, tensor, T, G):
    say(f"variants together: tables {fmt}, scales {sm}, converge {conv}, {tensor}, T={T}, G={G}")
    p = synthkv.PRESETS[2]
    rounds_cap = 12 if conv else 3
    oc = ocfg(p, tensor, n_centroids=48, iters_cold=rounds_cap, iters_warm=rounds_cap if conv else 2,
              centroid_format=fmt, scale_mode=sm, converge=conv, n_stages=T, group_size=G)
    H, N, chunk = 2, 2000, 1000
    X = synthkv.gen_numpy(p, tensor, heads=H, n_tokens=N)
    if sm == "two_level":   # residual groups past E4M3's range (a power of two: exact in bf16)
        X = X * np.float32(8.0)
    X = oracle.bf16_round(X).astype(np.float32)
    q = lib()
    cfg = gcfg(oc)
    xd = to_dev(X, oc.dtype)
    dst = q.CompressedKV(cfg, H, N, chunk, DEV)
    enc = q.Encoder(cfg, H, chunk, DEV)
    cache_d = q.CentroidCache(cfg, H)
    rounds = []
    for c in range(N // chunk):
        enc.encode(xd[:, c * chunk:(c + 1) * chunk], dst, c, cache=cache_d)
        if conv:
            rounds.append(to_np(enc.rounds()))
    y = to_np(q.decode(cfg, dst, 0, N, out_dtype="f32"))
    torch.cuda.synchronize()
    cache = {}
    for c in range(N // chunk):
        b, e = c * chunk, (c + 1) * chunk
        g = fetch(dst, c, oc)
        for h in range(H):
            ora = oracle.encode_chunk(X[h:h + 1, b:e], oc, cache=cache.get(h), head_offset=h)
            cache[h] = ora.cache
            if conv:
                say(f"  chunk {c} head {h}: rounds GPU {rounds[c][:, h].tolist()} oracle {ora.rounds[:, 0].tolist()}")
                np.testing.assert_array_equal(rounds[c][:, h], ora.rounds[:, 0])
            if sm == "two_level":
                assert int(g["scale_exp"][h]) == int(ora.scale_exp[0])
            assert check_chunk(oc, X[:, b:e], g, ora, 0, h, f"chunk {c}") == 0
            np.testing.assert_array_equal(y[h, b:e], oracle.decode(ora, oc.group_size, "f32")[0])
