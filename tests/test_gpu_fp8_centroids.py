"""FP8 (E4M3) centroid storage on the device, against the oracle, through the
C ABI: every stored table's exponent and codes, labels, codes and scales of the
chunk bit for bit (cold and warm chunks, bf16 and fp32 tensors, 1-3 stages),
and the fused decode of FP8 tables by both decode kernels."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, check_chunk, fetch, fp8_tables, gcfg, gpu_encode_chunks, lib, ocfg, say, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tensor", ["K", "V"])
def test_fp8_tables_encode_matches_oracle(tensor):
    say(f"FP8 centroid tables, {tensor}, 2 heads x 2 chunks of 4,680 tokens")
    p = synthkv.PRESETS[2]
    oc = ocfg(p, tensor, centroid_format="e4m3", iters_cold=6)
    X = synthkv.gen_numpy(p, tensor, heads=2, n_tokens=2 * p.chunk_tokens)
    dst, _ = gpu_encode_chunks(oc, X, p.chunk_tokens)
    q = lib()
    y = to_np(q.decode(gcfg(oc), dst, 0, X.shape[1], out_dtype="bf16"))
    cache = {}
    for c in range(2):
        b, e = c * p.chunk_tokens, (c + 1) * p.chunk_tokens
        g = fetch(dst, c, oc)
        _, exps = fp8_tables(to_np(dst.centroids[c]), oc.n_centroids, oc.d)
        for h in range(2):
            ora = oracle.encode_chunk(X[h:h + 1, b:e], oc, cache=cache.get(h), head_offset=h)
            cache[h] = ora.cache
            np.testing.assert_array_equal(exps[:, h], ora.cent_exp[:, 0])
            assert check_chunk(oc, X[:, b:e], g, ora, 0, h, f"chunk {c}") == 0
            np.testing.assert_array_equal(y[h, b:e], oracle.decode(ora, oc.group_size, "bf16")[0])
    # quality and bytes next to bf16 tables (printed)
    on = ocfg(p, tensor, iters_cold=6)
    dn, _ = gpu_encode_chunks(on, X, p.chunk_tokens)
    yn = to_np(q.decode(gcfg(on), dn, 0, X.shape[1], out_dtype="bf16"))
    m8, mn = oracle.mse(y, X), oracle.mse(yn, X)
    rtn = oracle.mse(oracle.rtn_reconstruct(X, oc.group_size), X)
    say(f"  MSE with FP8 tables {m8:.4g}, bf16 tables {mn:.4g}, RTN {rtn:.4g}; "
        f"ratio {oracle.compression_ratio(oc, 2, p.chunk_tokens):.2f}x vs {oracle.compression_ratio(on, 2, p.chunk_tokens):.2f}x")
    assert m8 < rtn


@pytest.mark.parametrize("T", [1, 3])
def test_fp8_tables_fp32_input(T):
    say(f"FP8 centroid tables, fp32 tiny chunk, T={T}, cold then warm")
    p = synthkv.PRESETS[1]
    oc = ocfg(p, "K", centroid_format="e4m3", n_stages=T)
    X = synthkv.gen_numpy(p, "K", n_tokens=2 * p.chunk_tokens)
    dst, _ = gpu_encode_chunks(oc, X, p.chunk_tokens)
    q = lib()
    y = to_np(q.decode(gcfg(oc), dst, 0, X.shape[1], out_dtype="f32"))
    cache = None
    for c in range(2):
        b, e = c * p.chunk_tokens, (c + 1) * p.chunk_tokens
        ora = oracle.encode_chunk(X[:, b:e], oc, cache=cache)
        cache = ora.cache
        assert check_chunk(oc, X[:, b:e], fetch(dst, c, oc), ora, 0, 0, f"chunk {c}") == 0
        np.testing.assert_array_equal(y[:, b:e], oracle.decode(ora, oc.group_size, "f32"))


@pytest.mark.parametrize("T,d,G", [(1, 128, 64), (2, 128, 64), (4, 128, 16), (2, 64, 32), (5, 128, 32)])
def test_decode_of_fp8_tables(T, d, G):
    """Random FP8 tables with random exponents; T = 5 takes the kernel that
    reads the tables through L2."""
    say(f"decode of FP8 tables T={T} d={d} G={G}")
    q = lib()
    rng = np.random.default_rng(T * 100 + d + G)
    H, N, K = 3, 777, 256
    codes = rng.integers(0, 256, (H, N, d // 4), dtype=np.uint8)
    scales = rng.integers(0, 0x70, (H, N, d // G), dtype=np.uint8)
    asg = rng.integers(0, K, (T, H, N), dtype=np.uint8)
    raw = rng.integers(0, 256, (T, H, 16 + K * d), dtype=np.uint8)
    raw[..., 16:][(raw[..., 16:] & 0x7F) == 0x7F] = 0x11             # no NaN codes
    raw[..., :16] = 0
    raw[..., :4] = rng.integers(-12, 8, (T, H)).astype(np.int32).view(np.uint8).reshape(T, H, 4)
    vals, _ = fp8_tables(raw, K, d)
    cfg = q.config(d, K, T, G, 2, 2, 1, "bf16", 0, "e4m3")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    for out_dtype in ("f32", "bf16"):
        out = torch.empty((H, N, d), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=DEV)
        q.qvg_dequant_reconstruct(cfg, H, N, dev(codes), dev(scales), dev(asg), dev(raw), out,
                                  q.QVG_F32 if out_dtype == "f32" else q.QVG_BF16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out), oracle.decode_chunk(codes, scales, asg, vals, G, out_dtype))
