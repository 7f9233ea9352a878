"""End-to-end parity of the HIP encode/decode against the oracle, chunk by
chunk with the streaming centroid cache, through the C ABI.

Where every assignment agrees with the oracle, codes, scales, centroids and the
decoded tensor must be bit-exact.  Where an assignment differs (a near tie
decided differently by fp32 accumulation), the disagreement rate must stay
below the rule's bound, the HIP labels must be nearest under the HIP path's own
centroids within the relative-gap rule, and its codes must equal the oracle's
quantiser applied to the HIP path's own residual."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, check_chunk as _check_chunk, fetch, gcfg, gpu_encode_chunks, lib, ocfg, say, to_np
from gpu_util import oracle_chunks as _oracle_chunks

pytestmark = pytest.mark.gpu


def _run(p, tensor, heads=None, n_tokens=None, oracle_heads=None, **kw):
    oc = ocfg(p, tensor, **kw)
    X = synthkv.gen_numpy(p, tensor, heads=heads, n_tokens=n_tokens)
    dst, cache = gpu_encode_chunks(oc, X, p.chunk_tokens)
    ora = _oracle_chunks(oc, X, p.chunk_tokens, oracle_heads)
    hs = list(range(X.shape[0])) if oracle_heads is None else oracle_heads
    total_mis = 0
    for c, per_head in enumerate(ora):
        b, e = c * p.chunk_tokens, min((c + 1) * p.chunk_tokens, X.shape[1])
        g = fetch(dst, c, oc)
        for i, h in enumerate(hs):
            total_mis += _check_chunk(oc, X[:, b:e], g, per_head[i], i, h, f"chunk {c}")
    return oc, X, dst, ora, total_mis


def test_tiny_fp32_chunk():
    say("e2e tiny fp32 chunk")
    p = synthkv.PRESETS[1]
    oc, X, dst, ora, mis = _run(p, "K")
    assert mis == 0
    q = lib()
    y = q.decode(gcfg(oc), dst, 0, X.shape[1], out_dtype="f32")
    np.testing.assert_array_equal(to_np(y), oracle.decode(ora[0][0], oc.group_size, "f32"))


def test_fp32_three_stages_cold_then_warm():
    """fp32 tensor, three stages, a cold and a warm chunk: the general operand
    loader rebuilds R(1) and R(2) from fp32 tables (no stored bf16 operand), and
    the update's run certificate uses the fp32 stored-table statistics."""
    say("e2e fp32, T = 3, cold then warm")
    p = synthkv.PRESETS[1]
    oc, X, dst, ora, mis = _run(p, "V", n_tokens=2 * p.chunk_tokens, n_stages=3)
    assert mis == 0
    q = lib()
    y = q.decode(gcfg(oc), dst, 0, X.shape[1], out_dtype="f32")
    ref = np.concatenate([oracle.decode(ora[c][0], oc.group_size, "f32") for c in range(2)], axis=1)
    np.testing.assert_array_equal(to_np(y), ref)


@pytest.mark.parametrize("tensor", ["K", "V"])
def test_single_head_chunk(tensor):
    say(f"e2e single-head chunk {tensor}")
    p = synthkv.PRESETS[2]
    oc, X, dst, ora, mis = _run(p, tensor)
    assert mis == 0
    q = lib()
    cfg = gcfg(oc)
    y = to_np(q.decode(cfg, dst, 0, X.shape[1], out_dtype="bf16"))
    if mis == 0:
        np.testing.assert_array_equal(y, oracle.decode(ora[0][0], oc.group_size, "bf16")[0][None])
    m_q, m_r = oracle.mse(y, X), oracle.mse(oracle.rtn_reconstruct(X, oc.group_size), X)
    say(f"  MSE qvg {m_q:.4g}  rtn {m_r:.4g}")
    assert m_q < m_r / 10


def test_aggressive_setting_two_chunks_warm():
    say("e2e aggressive setting, 3 heads, 2 chunks (cold then warm)")
    p = synthkv.PRESETS[4]
    assert _run(p, "V", heads=3)[-1] == 0


def test_ragged_tail_and_reset_is_cold():
    say("e2e ragged chunks; cache reset gives the cold result")
    p = synthkv.PRESETS[2]
    oc = ocfg(p, "K", n_centroids=64, iters_cold=4, iters_warm=2)
    X = synthkv.gen_numpy(p, "K", heads=2, n_tokens=2 * 1000 + 333)
    q = lib()
    cfg = gcfg(oc)
    xd = torch.from_numpy(X).to(torch.bfloat16).to(DEV)
    dst = q.CompressedKV(cfg, 2, X.shape[1], 1000, DEV)
    enc = q.Encoder(cfg, 2, 1000, DEV)
    cache = q.CentroidCache(cfg, 2)
    for c in range(3):
        enc.encode(xd[:, c * 1000:(c + 1) * 1000], dst, c, cache=cache)
    torch.cuda.synchronize()
    ora = _oracle_chunks(oc, X, 1000)
    for c in range(3):
        g = fetch(dst, c, oc)
        for h in range(2):
            _check_chunk(oc, X[:, c * 1000:(c + 1) * 1000], g, ora[c][h], h, h, f"chunk {c}")
    # export / import round trip of the streaming state
    saved = cache.export(DEV)
    np.testing.assert_array_equal(to_np(saved)[:, 0], ora[2][0].cache[:, 0])
    # reset: the next encode is cold and equals a cache-less encode
    cache.reset()
    dst2 = q.CompressedKV(cfg, 2, X.shape[1], 1000, DEV)
    enc.encode(xd[:, 1000:2000], dst2, 1, cache=cache)
    dst3 = q.CompressedKV(cfg, 2, X.shape[1], 1000, DEV)
    enc.encode(xd[:, 1000:2000], dst3, 1, cache=None)
    torch.cuda.synchronize()
    a, b = fetch(dst2, 1, oc), fetch(dst3, 1, oc)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # import: warm start from a saved state equals the explicit-init hook
    cache.load(saved)
    dst4 = q.CompressedKV(cfg, 2, X.shape[1], 1000, DEV)
    enc.encode(xd[:, 1000:2000], dst4, 1, cache=cache)
    dst5 = q.CompressedKV(cfg, 2, X.shape[1], 1000, DEV)
    enc.encode(xd[:, 1000:2000], dst5, 1, init=saved)
    torch.cuda.synchronize()
    a, b = fetch(dst4, 1, oc), fetch(dst5, 1, oc)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_run_twice_is_deterministic():
    say("e2e determinism")
    p = synthkv.PRESETS[2]
    oc = ocfg(p, "V", iters_cold=3)
    X = synthkv.gen_numpy(p, "V", heads=4, n_tokens=3000)
    d1, _ = gpu_encode_chunks(oc, X, 3000)
    d2, _ = gpu_encode_chunks(oc, X, 3000)
    a, b = fetch(d1, 0, oc), fetch(d2, 0, oc)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_tiny_values_need_exact_sums():
    """bf16 input where channel 5 of one well-separated cluster holds 1, 2^-80
    and -1 in three tokens and zero in the rest: the exact column sum is 2^-80,
    while an fp64 sum that adds 1 + 2^-80 first returns 0.  The input's value
    statistics (gathered by the first assign) must rule out the run-level
    exactness certificate, so the update sums that cluster exactly; centroids,
    codes and the decode must equal the oracle's."""
    say("e2e bf16 input with values 2^80 apart inside one cluster")
    rng = np.random.default_rng(11)
    K, N, d = 16, 480, 128
    centers = oracle.bf16_round(rng.standard_normal((K, d)) * 50).astype(np.float32)
    lab = np.arange(N) % K
    X = oracle.bf16_round(centers[lab] + rng.standard_normal((N, d)) * 0.5).astype(np.float32)
    members = np.nonzero(lab == 3)[0]
    X[members, 5] = 0.0
    X[members[:3], 5] = [1.0, 2.0 ** -80, -1.0]
    X = X.reshape(1, N, d).copy()   # (a fresh head axis: numpy's X[None] has stride 0 there)
    oc = oracle.CodecConfig(d=d, n_centroids=K, n_stages=1, group_size=64, iters_cold=3, iters_warm=3, seed=5,
                            dtype="bf16")
    init = centers.reshape(1, 1, K, d).copy()        # [T][H][K][d]
    dst, _ = gpu_encode_chunks(oc, X, N, use_cache=False, init=init)
    ora = oracle.encode_chunk(X, oc, init=init.astype(np.float64))
    assert abs(float(ora.cache[0, 0, 3, 5])) > 0     # the exact mean is 2^-80 / 30, not 0
    g = fetch(dst, 0, oc)
    assert check_chunk_exact(oc, X, g, ora) == 0
    q = lib()
    y = to_np(q.decode(gcfg(oc), dst, 0, N, out_dtype="bf16"))
    np.testing.assert_array_equal(y, oracle.decode(ora, oc.group_size, "bf16"))


def check_chunk_exact(oc, X, g, ora):
    return _check_chunk(oc, X, g, ora, 0, 0, "chunk 0")


def test_chunk_over_16384_tokens_uses_the_global_sort_update():
    """A chunk longer than the LDS token list (16,384): inside the stage loop
    every update orders the tokens by label in global memory (scatter) and sums
    one centroid per wave; the encoding must equal the oracle's bit for bit."""
    say("e2e chunk of 20,000 tokens (global-sort update), 2 heads, K and V")
    p = synthkv.PRESETS[2]
    for tensor in ("K", "V"):
        oc = ocfg(p, tensor, iters_cold=3)
        X = synthkv.gen_numpy(p, tensor, heads=2, n_tokens=20000)
        dst, _ = gpu_encode_chunks(oc, X, 20000)
        g = fetch(dst, 0, oc)
        q = lib()
        y = to_np(q.decode(gcfg(oc), dst, 0, 20000, out_dtype="bf16"))
        for h in range(2):
            ora = oracle.encode_chunk(X[h:h + 1], oc, head_offset=h)
            assert _check_chunk(oc, X, g, ora, 0, h, f"{tensor} chunk 0") == 0
            np.testing.assert_array_equal(y[h], oracle.decode(ora, oc.group_size, "bf16")[0])
