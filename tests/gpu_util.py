"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and bring results back as NumPy arrays; compare with the oracle under the
parity rules."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synthkv

DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def lib():
    import bit_vector_quantization_amd as q

    return q


def ocfg(p: synthkv.Preset, tensor: str, **kw) -> oracle.CodecConfig:
    c = dict(d=p.d, n_centroids=p.n_centroids, n_stages=p.n_stages, group_size=p.group_size,
             iters_cold=p.iters_cold, iters_warm=p.iters_warm, seed=p.codec_seed(tensor), dtype=p.dtype)
    c.update(kw)
    return oracle.CodecConfig(**c)


def gcfg(oc: oracle.CodecConfig):
    q = lib()
    return q.config(oc.d, oc.n_centroids, oc.n_stages, oc.group_size, oc.iters_cold, oc.iters_warm,
                    oc.seed, oc.dtype, oc.converge, oc.centroid_format, oc.scale_mode)


def fp8_tables(raw: np.ndarray, K: int, d: int):
    """Stored FP8 tables [..][16 + K d] bytes -> (values [..][K][d] fp32, exponents [..])."""
    e = raw[..., :4].copy().view(np.int32)[..., 0]
    vals = oracle.e4m3_decode(raw[..., 16:]).reshape(raw.shape[:-1] + (K, d))
    return np.ldexp(vals, e[..., None, None]).astype(np.float32), e


def to_dev(X: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def gpu_encode_chunks(oc: oracle.CodecConfig, X: np.ndarray, chunk_tokens: int, use_cache=True,
                      init: np.ndarray | None = None):
    """Encode X [H][Ntot][d] chunk by chunk on the GPU; returns the CompressedKV."""
    q = lib()
    H, Ntot, d = X.shape
    cfg = gcfg(oc)
    xd = to_dev(X, oc.dtype)
    dst = q.CompressedKV(cfg, H, Ntot, chunk_tokens, DEV)
    enc = q.Encoder(cfg, H, min(chunk_tokens, Ntot), DEV)
    cache = q.CentroidCache(cfg, H) if use_cache else None
    ini = None if init is None else torch.from_numpy(np.ascontiguousarray(init, np.float32)).to(DEV)
    for c in range(-(-Ntot // chunk_tokens)):
        b, e = c * chunk_tokens, min((c + 1) * chunk_tokens, Ntot)
        enc.encode(xd[:, b:e], dst, c, cache=cache, init=ini)
    torch.cuda.synchronize()
    return dst, cache


def fetch(dst, chunk: int, oc: oracle.CodecConfig):
    """Chunk `chunk` of a CompressedKV as oracle-shaped arrays."""
    b, e = chunk * dst.chunk_tokens, min((chunk + 1) * dst.chunk_tokens, dst.cap)
    T = oc.n_stages
    cent = to_np(dst.centroids[chunk, :T])
    if oc.centroid_format == "e4m3":
        cent, _ = fp8_tables(cent, oc.n_centroids, oc.d)
    return dict(codes=to_np(dst.codes[:, b:e]), scales=to_np(dst.scales[:, b:e]),
                assign=to_np(dst.assign[:T, :, b:e]), centroids=cent,
                scale_exp=None if dst.scale_exp is None else to_np(dst.scale_exp[chunk]).astype(np.int32))


def distance_table(Xop: np.ndarray, C: np.ndarray) -> np.ndarray:
    """|c|^2 - 2<x, c> in float64 on bf16-rounded operands."""
    xb, cb = oracle.bf16_round(Xop), oracle.bf16_round(C)
    return (cb * cb).sum(1)[None, :] - 2.0 * xb @ cb.T


def gap_ok(Xop: np.ndarray, C: np.ndarray, got: np.ndarray, ref: np.ndarray, rel=1e-4):
    """Where labels differ, the two choices' distances must be within `rel` of
    |x_b|^2 + max(|c_g|^2, |c_o|^2).  Returns (n_mismatch, worst relative gap)."""
    mis = np.nonzero(got != ref)[0]
    if len(mis) == 0:
        return 0, 0.0
    xb, cb = oracle.bf16_round(Xop[mis]), oracle.bf16_round(C)
    cn = (cb * cb).sum(1)
    D = cn[None, :] - 2.0 * xb @ cb.T
    g, o = got[mis].astype(int), ref[mis].astype(int)
    r = np.arange(len(mis))
    gap = np.abs(D[r, g] - D[r, o])
    scale = (xb * xb).sum(1) + np.maximum(cn[g], cn[o])
    return len(mis), float((gap / scale).max())


def oracle_chunks(oc, X, chunk_tokens, heads=None):
    heads = list(range(X.shape[0])) if heads is None else heads
    out, cache = [], None
    for c in range(-(-X.shape[1] // chunk_tokens)):
        b, e = c * chunk_tokens, min((c + 1) * chunk_tokens, X.shape[1])
        per_head = []
        for h in heads:
            hc = None if cache is None else cache[h]
            per_head.append(oracle.encode_chunk(X[h:h + 1, b:e], oc, cache=hc, head_offset=h))
        out.append(per_head)
        cache = {h: per_head[i].cache for i, h in enumerate(heads)}
    return out


def check_chunk(oc, Xc, g, ora, h_local, h_global, tag):
    """g: GPU chunk arrays (all heads); ora: oracle Encoded for one head."""
    T = oc.n_stages
    stats = {}
    exact = True
    for t in range(T):
        mis = int((g["assign"][t, h_global] != ora.assign[t, 0]).sum())
        stats[t + 1] = mis
        exact &= mis == 0
    say(f"  {tag} head {h_global}: assignment mismatches per stage {stats}")
    N = Xc.shape[1]
    if exact:
        np.testing.assert_array_equal(g["centroids"][:, h_global], ora.centroids[:, 0])
        np.testing.assert_array_equal(g["scales"][h_global], ora.scales[0])
        np.testing.assert_array_equal(g["codes"][h_global], ora.codes[0])
        return 0
    # the assignment re-decides the two best candidates on exact distances, so a
    # disagreement needs the true nearest centroid outside the fp32 top two
    assert stats[1] <= int(1e-4 * N), stats
    # validity of the HIP result on its own residual chain
    R = Xc[h_global].astype(np.float64)
    for t in range(T):
        Ct = g["centroids"][t, h_global].astype(np.float64)
        lab = g["assign"][t, h_global].astype(int)
        ref = oracle.assign(R, Ct, "parity")
        n_mis, worst = gap_ok(R, Ct, lab, ref)
        assert worst < 1e-4, (t, n_mis, worst)
        R = (R - Ct[lab]).astype(np.float32).astype(np.float64)
    _, packed, s = oracle.group_quant(R.astype(np.float32), oc.group_size)
    np.testing.assert_array_equal(g["scales"][h_global], s)
    np.testing.assert_array_equal(g["codes"][h_global], packed)
    return sum(stats.values())


def check_chunk_properties(oc: oracle.CodecConfig, Xc: np.ndarray, g, h: int, tag: str) -> None:
    """Checks that hold for any chunk without replaying the centroid chain:
    every stage's labels are nearest under the HIP path's own stored centroids
    on the residual they define (at least 99.99% exactly; any other label
    within the 1e-4 relative-gap rule), the codes and scales are the oracle's
    quantiser of the last residual."""
    R = Xc[h].astype(np.float64)
    for t in range(oc.n_stages):
        Ct = g["centroids"][t, h].astype(np.float64)
        lab = g["assign"][t, h].astype(int)
        ref = oracle.assign(R, Ct, "parity")
        n_mis, worst = gap_ok(R, Ct, lab, ref)
        say(f"  {tag} head {h} stage {t + 1}: labels not nearest {n_mis} (worst relative gap {worst:.3g})")
        assert n_mis <= int(1e-4 * len(lab)) and worst < 1e-4, (n_mis, worst)
        R = (R - Ct[lab]).astype(np.float32).astype(np.float64)
    _, packed, s = oracle.group_quant(R.astype(np.float32), oc.group_size)
    np.testing.assert_array_equal(g["scales"][h], s)
    np.testing.assert_array_equal(g["codes"][h], packed)


def layer_on_device(p: synthkv.Preset) -> torch.Tensor:
    """K and V of a layer as one [2H][N][d] bf16 tensor on the device (the
    benchmark's layout: a [2][H][N][d] buffer viewed as 2H heads)."""
    X = torch.empty((2, p.heads, p.n_tokens, p.d), dtype=torch.bfloat16, device=DEV)
    for i, t in enumerate(("K", "V")):
        X[i] = torch.cat(list(synthkv.gen_torch(p, t, DEV, frames_per_call=p.chunk_frames)), dim=1)
    return X.view(2 * p.heads, p.n_tokens, p.d)
