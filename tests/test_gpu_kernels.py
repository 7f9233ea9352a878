"""Per-kernel parity of the HIP path against the oracle, through the C ABI.

Each kernel gets inputs produced by the oracle (or the seeded generator) and its
output is compared element by element: codes, scales, centroids and decoded
values bit-exact; assignments under the near-tie rule (agreement >= 99.99% and a
relative distance gap < 1e-4 wherever the labels differ)."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, distance_table, gap_ok, lib, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _residuals(rng, H, N, d, G):
    R = rng.standard_normal((H, N, d)) * rng.lognormal(0, 2.5, (H, N, 1))
    R = R.astype(np.float32)
    special = [lambda r: r.__setitem__(slice(0, G), 0.0),                 # all-zero group
               lambda r: r.__setitem__(slice(0, 3), [900.0, -1200.0, 3.0]),  # saturating scale
               lambda r: r.__setitem__(slice(0, G), 1.5),                  # values on the outer level
               lambda r: r.__setitem__(slice(0, G), np.float32(2.0 ** -12)),  # scale rounds to zero
               lambda r: r.__setitem__(slice(0, G), -0.0)]
    for i, f in enumerate(special[:N]):
        for h in range(H):
            f(R[h, i])
    return R


@pytest.mark.parametrize("d,G,N,H", [(128, 64, 1000, 2), (128, 16, 777, 3), (64, 16, 130, 1),
                                     (128, 128, 65, 1), (64, 32, 301, 2), (128, 32, 1, 1)])
def test_group_quant_bit_exact(d, G, N, H):
    say(f"group_quant d={d} G={G} N={N} H={H}")
    q = lib()
    R = _residuals(np.random.default_rng(d + G + N), H, N, d, G)
    codes = torch.empty((H, N, d // 4), dtype=torch.uint8, device=DEV)
    scales = torch.empty((H, N, d // G), dtype=torch.uint8, device=DEV)
    q.qvg_group_quant(to_dev(R, "f32"), N * d, H, N, d, G, codes, scales)
    torch.cuda.synchronize()
    for h in range(H):
        _, packed, s = oracle.group_quant(R[h], G)
        np.testing.assert_array_equal(to_np(scales[h]), s)
        np.testing.assert_array_equal(to_np(codes[h]), packed)


def _oracle_encoding(rng, H, N, d, K, T, G, dtype):
    oc = oracle.CodecConfig(d=d, n_centroids=K, n_stages=T, group_size=G, iters_cold=2, iters_warm=2,
                            seed=7, dtype=dtype)
    X = (rng.standard_normal((H, N, d)) * 3).astype(np.float32)
    X[:, :, 5] += 80.0
    if dtype == "bf16":
        X = oracle.bf16_round(X).astype(np.float32)
    return oc, X, oracle.encode_chunk(X, oc)


@pytest.mark.parametrize("H,N,d,K,T,G,dtype", [(2, 700, 128, 32, 2, 64, "bf16"), (1, 333, 128, 256, 4, 16, "bf16"),
                                               (2, 200, 64, 16, 1, 16, "f32"), (1, 97, 128, 8, 0, 64, "bf16"),
                                               (3, 129, 64, 20, 3, 32, "bf16"), (2, 257, 128, 16, 6, 32, "bf16"),
                                               (1, 95, 64, 12, 5, 16, "f32")])
def test_dequant_reconstruct_bit_exact(H, N, d, K, T, G, dtype):
    say(f"dequant_reconstruct H={H} N={N} d={d} K={K} T={T} G={G} {dtype}")
    q = lib()
    oc, X, enc = _oracle_encoding(np.random.default_rng(N), H, N, d, K, T, G, dtype)
    cfg = q.config(d, K, T, G, 2, 2, 7, dtype)
    dev = lambda a, dt=torch.uint8: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)
    codes, scales = dev(enc.codes), dev(enc.scales)
    asg = dev(enc.assign if T else np.zeros((1, H, N), np.uint8))
    cent = to_dev(enc.centroids if T else np.zeros((1, H, K, d), np.float32), dtype)
    for out_dtype, ref in (("f32", oracle.decode(enc, G, "f32")), ("bf16", oracle.decode(enc, G, "bf16"))):
        out = torch.empty((H, N, d), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=DEV)
        q.qvg_dequant_reconstruct(cfg, H, N, codes, scales, asg, cent, out,
                                  q.QVG_F32 if out_dtype == "f32" else q.QVG_BF16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out), ref)


def test_decode_every_scale_code():
    """All 256 E4M3FN scale bytes (subnormal, normal, 448, NaN and negative
    codes) with random 2-bit codes and one stage of random centroids."""
    say("dequant_reconstruct over every scale code")
    q = lib()
    rng = np.random.default_rng(11)
    H, N, d, G, K = 1, 256, 64, 16, 8
    codes = rng.integers(0, 256, (H, N, d // 4), dtype=np.uint8)
    scales = ((np.arange(N)[:, None] * (d // G) + np.arange(d // G)[None, :]) % 256).astype(np.uint8)[None]
    asg = rng.integers(0, K, (1, H, N), dtype=np.uint8)
    cent = oracle.bf16_round(rng.standard_normal((1, H, K, d))).astype(np.float32)
    cfg = q.config(d, K, 1, G, 2, 2, 7, "bf16")
    dev = lambda a, dt=torch.uint8: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)
    for out_dtype in ("f32", "bf16"):
        ref = oracle.decode_chunk(codes, scales, asg, cent, G, out_dtype)
        out = torch.empty((H, N, d), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device=DEV)
        q.qvg_dequant_reconstruct(cfg, H, N, dev(codes), dev(scales), dev(asg), to_dev(cent, "bf16"), out,
                                  q.QVG_F32 if out_dtype == "f32" else q.QVG_BF16)
        torch.cuda.synchronize()
        got = to_np(out)
        np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
        np.testing.assert_array_equal(got.view(np.uint32)[~np.isnan(got)], ref.view(np.uint32)[~np.isnan(ref)])


def _assign_case(rng, which):
    p = synthkv.PRESETS[2]
    if which == "kv":
        X = synthkv.gen_numpy(p, "V", heads=1, n_tokens=4680)
        oc = oracle.CodecConfig(d=128, n_centroids=256, n_stages=1, group_size=64, iters_cold=3, iters_warm=3,
                                seed=3, dtype="bf16")
        enc = oracle.encode_chunk(X, oc)
        C = enc.cache[0]
        return X, C, 128
    if which == "dups":
        X = oracle.bf16_round(rng.standard_normal((1, 515, 64)) * 4).astype(np.float32)
        C = X[0, rng.integers(0, 515, 20)].copy()[None]
        C[0, 7] = C[0, 3]                    # duplicated centroids: the lower index wins
        C[0, 11] = C[0, 3]                   # three copies: still the lowest
        C[0, 19] = C[0, 0]
        X[0, 5] = C[0, 3]                    # tokens at distance zero from the copies
        X[0, 400] = C[0, 3]
        return X, C, 64
    if which == "many_heads":
        # two tiles per head: one workgroup's run spans five heads, taken in
        # windows of two tables
        X = oracle.bf16_round(rng.standard_normal((5, 40, 128))).astype(np.float32)
        C = rng.standard_normal((5, 45, 128)).astype(np.float32)
        return X, C, 128
    # fewer tokens than centroids, K not a multiple of 16
    X = oracle.bf16_round(rng.standard_normal((2, 37, 128))).astype(np.float32)
    C = rng.standard_normal((2, 45, 128)).astype(np.float32)
    return X, C, 128


@pytest.mark.parametrize("which", ["kv", "dups", "small", "many_heads"])
def test_assign_matches_oracle_within_tie_rule(which):
    say(f"kmeans_assign {which}")
    q = lib()
    X, C, d = _assign_case(np.random.default_rng(5), which)
    H, N, _ = X.shape
    K = C.shape[1]
    ws_bytes = q.qvg_stage_workspace_bytes(H, N, d, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((H, N), dtype=torch.uint8, device=DEV)
    q.qvg_kmeans_assign(to_dev(X, "bf16"), q.QVG_BF16, N * d, to_dev(C, "f32"), H, N, d, K, out, N, ws, ws_bytes)
    torch.cuda.synchronize()
    got = to_np(out).astype(int)
    for h in range(H):
        ref = oracle.assign(X[h], C[h], "parity")
        n_mis, worst = gap_ok(X[h], C[h], got[h], ref)
        say(f"  head {h}: mismatches {n_mis}/{N}, worst relative gap {worst:.3g}")
        assert worst < 1e-4
        np.testing.assert_array_equal(got[h], ref)
    if which == "dups":
        assert not np.any(np.isin(got, [7, 19]))


def test_assign_three_centroids_inside_the_fp32_band():
    """Each token has three candidate centroids whose exact distances differ by
    2^-14 .. 9 * 2^-14 while |x|^2 is about 2e6 (value-like outlier channels),
    far inside the matrix cores' fp32 error band, and the exact nearest has the
    highest index of the three.  The fp32 ranking of the three is then noise.
    The fp64 re-decision sees the best two of each lane's quarter of the
    centroids, merged into the token's best three, so the exact nearest can be
    missed when all three candidates fall in one quarter (centroid numbers
    with equal (k mod 16) / 4).  Whatever the kernel returns must obey the
    near-tie rule (relative gap < 1e-4) and be one of the three; the outcome
    is printed."""
    say("kmeans_assign, three centroids within the fp32 error band")
    q = lib()
    rng = np.random.default_rng(21)
    d, B, K = 128, 64, 256
    base = oracle.bf16_round(rng.standard_normal((B, d))).astype(np.float32)
    base[:, 7] = oracle.bf16_round(1000.0 * (1 + 0.1 * rng.standard_normal(B)))
    base[:, 99] = oracle.bf16_round(-1000.0 * (1 + 0.1 * rng.standard_normal(B)))
    base[:, 10:13] = 1.0 + np.float32(2.0 ** -7) * rng.integers(0, 64, (B, 3))
    C = np.empty((1, K, d), np.float32)
    C[0, 3 * B:] = oracle.bf16_round(rng.standard_normal((K - 3 * B, d)) * 30)
    for b in range(B):
        for j in range(3):                       # distances (3 - j)^2 2^-14: index 3b + 2 is nearest
            C[0, 3 * b + j] = base[b]
            C[0, 3 * b + j, 10 + j] += np.float32((3 - j) * 2.0 ** -7)
    X = np.repeat(base, 16, axis=0)[None].copy()   # 16 tokens per base, all equal to it
    N = X.shape[1]
    ws_bytes = q.qvg_stage_workspace_bytes(1, N, d, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((1, N), dtype=torch.uint8, device=DEV)
    q.qvg_kmeans_assign(to_dev(X, "bf16"), q.QVG_BF16, N * d, to_dev(C, "f32"), 1, N, d, K, out, N, ws, ws_bytes)
    torch.cuda.synchronize()
    got = to_np(out)[0].astype(int)
    ref = oracle.assign(X[0], C[0], "parity")
    np.testing.assert_array_equal(ref, 3 * (np.arange(N) // 16) + 2)
    n_mis, worst = gap_ok(X[0], C[0], got, ref)
    say(f"  tokens {N}: exact nearest returned for {N - n_mis}, another of the three for {n_mis} "
        f"(worst relative gap {worst:.3g})")
    assert worst < 1e-4
    assert np.all(got // 3 == np.arange(N) // 16)


def test_assign_from_fp32_input_rounds_operands():
    say("kmeans_assign fp32 input")
    q = lib()
    rng = np.random.default_rng(9)
    X = (rng.standard_normal((1, 300, 64)) * 2).astype(np.float32)
    C = X[0, :16].copy()[None] + np.float32(0.01)
    ws_bytes = q.qvg_stage_workspace_bytes(1, 300, 64, 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty((1, 300), dtype=torch.uint8, device=DEV)
    q.qvg_kmeans_assign(to_dev(X, "f32"), q.QVG_F32, 300 * 64, to_dev(C, "f32"), 1, 300, 64, 16, out, 300, ws,
                        ws_bytes)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out)[0], oracle.assign(X[0], C[0], "parity"))


def _run_update(X, lab, C0, dtype):
    """qvg_centroid_update on the device; returns (centroids, counts) as numpy."""
    q = lib()
    H, N, d = X.shape
    K = C0.shape[1]
    cd = torch.from_numpy(C0).to(DEV)
    counts = torch.empty((H, K), dtype=torch.int32, device=DEV)
    ws_bytes = q.qvg_stage_workspace_bytes(H, N, d, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    labd = torch.from_numpy(lab.astype(np.uint8)).to(DEV)
    q.qvg_centroid_update(to_dev(X, dtype), q.QVG_BF16 if dtype == "bf16" else q.QVG_F32, N * d, labd, N, H, N,
                          d, K, cd, counts, ws, ws_bytes)
    torch.cuda.synchronize()
    return to_np(cd), to_np(counts)


def _check_update(X, lab, C0, dtype):
    got, cnt_got = _run_update(X, lab, C0, dtype)
    for h in range(X.shape[0]):
        ref, cnt = oracle.update(X[h].astype(np.float64), lab[h], C0[h].astype(np.float64), "parity")
        np.testing.assert_array_equal(cnt_got[h], cnt)
        np.testing.assert_array_equal(got[h], ref.astype(np.float32))
    return got


# N up to 16384 runs the LDS token-list kernel, longer chunks the global sort
@pytest.mark.parametrize("dtype,d,K,N,H", [("bf16", 128, 256, 4680, 1), ("f32", 128, 256, 2000, 2),
                                           ("f32", 64, 16, 128, 1), ("bf16", 64, 40, 1001, 3),
                                           ("bf16", 128, 256, 16384, 1), ("bf16", 128, 256, 20000, 1),
                                           ("f32", 64, 200, 17000, 2)])
def test_update_bit_exact(dtype, d, K, N, H):
    say(f"centroid_update {dtype} d={d} K={K} N={N} H={H}")
    q = lib()
    rng = np.random.default_rng(K + N)
    X = (rng.standard_normal((H, N, d)) * rng.lognormal(0, 2, (H, N, 1))).astype(np.float32)
    X[:, :, 3] *= 100.0
    if dtype == "bf16":
        X = oracle.bf16_round(X).astype(np.float32)
    lab = rng.integers(0, K, (H, N))
    lab[:, : N // 3] = rng.integers(0, 3, (H, N // 3))   # a few big clusters
    lab[lab == K - 1] = 0                                 # one empty cluster
    C0 = rng.standard_normal((H, K, d)).astype(np.float32)
    cd = torch.from_numpy(C0).to(DEV)
    counts = torch.empty((H, K), dtype=torch.int32, device=DEV)
    ws_bytes = q.qvg_stage_workspace_bytes(H, N, d, K)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    labd = torch.from_numpy(lab.astype(np.uint8)).to(DEV)
    q.qvg_centroid_update(to_dev(X, dtype), q.QVG_BF16 if dtype == "bf16" else q.QVG_F32, N * d, labd, N, H, N,
                          d, K, cd, counts, ws, ws_bytes)
    torch.cuda.synchronize()
    for h in range(H):
        ref, cnt = oracle.update(X[h].astype(np.float64), lab[h], C0[h].astype(np.float64), "parity")
        np.testing.assert_array_equal(to_np(counts[h]), cnt)
        np.testing.assert_array_equal(to_np(cd[h]), ref.astype(np.float32))
        np.testing.assert_array_equal(to_np(cd[h])[K - 1], C0[h, K - 1])


@pytest.mark.parametrize("N", [300, 16384])
def test_update_one_cluster_holds_every_token(N):
    """The whole chunk in one centroid: the token list of one workgroup is full."""
    say(f"centroid_update, all {N} tokens in centroid 37")
    rng = np.random.default_rng(N)
    X = oracle.bf16_round(rng.standard_normal((1, N, 128)) * 3).astype(np.float32)
    lab = np.full((1, N), 37)
    C0 = rng.standard_normal((1, 256, 128)).astype(np.float32)
    got = _check_update(X, lab, C0, "bf16")
    np.testing.assert_array_equal(np.delete(got[0], 37, axis=0), np.delete(C0[0], 37, axis=0))


@pytest.mark.parametrize("N", [1000, 17000])
def test_update_cancellation_needs_exact_sums(N):
    """Rows that cancel at 2^24 around tiny values: the plain fp64 sum loses the
    tiny part, so neither the lowest-bit certificate nor the interval test holds
    and the exact two-sum pass decides (its result is the oracle's exactly rounded
    mean).  Other centroids hold values 2^40 apart in magnitude, which fail the
    certificate but pass the interval test."""
    say(f"centroid_update cancellation, N={N}")
    rng = np.random.default_rng(7)
    d, K = 64, 20
    X = rng.standard_normal((1, N, d)).astype(np.float32)
    lab = rng.integers(2, K, (1, N))
    big = np.float32(2.0 ** 24)
    tiny = (rng.integers(1, 1 << 20, d) * 2.0 ** -52).astype(np.float32)
    X[0, 0], X[0, 1], X[0, 2] = big, -big, tiny          # centroid 0: exact mean tiny / 5
    X[0, 3], X[0, 4] = big * 0.5, -big * 0.5
    lab[0, :5] = 0
    X[0, 5:9] = rng.standard_normal((4, d)) * 2.0 ** 20   # centroid 1: magnitudes 2^40 apart
    X[0, 9:13] = rng.standard_normal((4, d)) * 2.0 ** -20
    lab[0, 5:13] = 1
    C0 = rng.standard_normal((1, K, d)).astype(np.float32)
    got = _check_update(X, lab, C0, "f32")
    np.testing.assert_array_equal(got[0, 0], (tiny.astype(np.float64) / 5).astype(np.float32))


@pytest.mark.parametrize("N,K,dtype", [(4680, 256, "bf16"), (128, 16, "f32"), (100, 256, "bf16"), (257, 256, "f32")])
def test_cold_start_rows_match_oracle_draw(N, K, dtype):
    say(f"forgy N={N} K={K}")
    from gpu_util import gpu_encode_chunks

    H, d = 3, 64
    rng = np.random.default_rng(N)
    X = (rng.standard_normal((H, N, d)) * 5).astype(np.float32)
    if dtype == "bf16":
        X = oracle.bf16_round(X).astype(np.float32)
    oc = oracle.CodecConfig(d=d, n_centroids=K, n_stages=1, group_size=16, iters_cold=0, iters_warm=0,
                            seed=123456789, dtype=dtype)
    dst, _ = gpu_encode_chunks(oc, X, N, use_cache=False)
    got = to_np(dst.centroids[0, 0])
    for h in range(H):
        idx = oracle.forgy_indices(N, K, oc.seed, h, 1)
        np.testing.assert_array_equal(got[h], X[h][idx])
