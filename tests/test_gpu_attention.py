"""Attention that reads the compressed cache (qvg_attention), through the C
ABI, against the oracle: fp64 softmax(scale Q K^T) V over the oracle's decode
of the same compressed cache (keys rotated by the same table when one is
given), within the oracle's stated tolerance for bf16 softmax weights; the
log-sum-exp to 1e-5 relative."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, fetch, gcfg, gpu_encode_chunks, lib, ocfg, say, to_np

pytestmark = pytest.mark.gpu


def _decoded(oc, dst, b, e, chunk, heads, rope=None):
    """bf16 rows of tokens [b, e) of the given heads, from the oracle's decode of each chunk."""
    out = []
    for c in range(b // chunk, (e - 1) // chunk + 1):
        g = fetch(dst, c, oc)
        cb, ce = c * chunk, min((c + 1) * chunk, dst.cap)
        lo, hi = max(b, cb), min(e, ce)
        rp = None if rope is None else rope[cb - b:ce - b] if cb >= b else None
        sl = slice(lo - cb, hi - cb)
        rows = []
        for h in heads:
            r = None
            if rope is not None:
                # the table's rows cover [b, e): pad the chunk's rows before b
                full = np.zeros((ce - cb, oc.d // 2, 2), np.float32)
                full[lo - cb:hi - cb] = rope[lo - b:hi - b]
                r = full
            y = oracle.decode_chunk(g["codes"][h:h + 1], g["scales"][h:h + 1], g["assign"][:, h:h + 1],
                                    g["centroids"][:, h:h + 1], oc.group_size, "bf16", rope=r,
                                    scale_exp=None if g["scale_exp"] is None else g["scale_exp"][h:h + 1])[0]
            rows.append(y[sl])
        out.append(np.stack(rows))
    return np.concatenate(out, axis=1)


@pytest.mark.parametrize("fmt,use_rope,b,e,Nq,sm", [("native", False, 0, 2000, 300, "e4m3"),
                                                    ("native", True, 137, 1931, 256, "e4m3"),
                                                    ("e4m3", True, 700, 2000, 77, "e4m3"),
                                                    ("native", False, 0, 64, 1, "e4m3"),
                                                    ("native", True, 0, 2000, 100, "two_level"),
                                                    ("e4m3", True, 300, 1800, 90, "two_level")])
def test_attention_over_compressed_cache(fmt, use_rope, b, e, Nq, sm):
    _attention_case(fmt, use_rope, b, e, Nq, sm)


@pytest.mark.parametrize("T,fmt,use_rope,b,e,Nq", [(1, "native", True, 5, 2000, 129),
                                                   (3, "e4m3", False, 0, 1999, 260),
                                                   (4, "native", True, 300, 1700, 40)])
def test_attention_stage_counts(T, fmt, use_rope, b, e, Nq):
    """The kernel's instances for 1, 3 and 4 stages (the other cases run 2)."""
    _attention_case(fmt, use_rope, b, e, Nq, "e4m3", T=T)


@pytest.mark.parametrize("b,e,Nq", [(999, 1000, 17), (999, 1001, 33), (1, 2000, 257)])
def test_attention_edge_ranges(b, e, Nq):
    """One key; two keys on either side of a chunk boundary; query counts that
    leave partial 16-query groups and a partial 256-query block."""
    _attention_case("native", True, b, e, Nq, "e4m3")


@pytest.mark.parametrize("chunk,b,e,Nq", [(48, 0, 2000, 100), (48, 37, 1500, 20), (128, 5, 2000, 64)])
def test_attention_chunk_lengths(chunk, b, e, Nq):
    """Chunks shorter than a 128-key tile (a tile spans several chunks, each with
    its own tables) and chunks of exactly one tile (tiles that start inside a
    chunk span two)."""
    _attention_case("native", True, b, e, Nq, "e4m3", chunk=chunk)


def _attention_case(fmt, use_rope, b, e, Nq, sm, T=None, chunk=1000):
    say(f"attention fmt={fmt} rope={use_rope} keys [{b}, {e}) Nq={Nq} scales {sm} T={T} chunk={chunk}")
    q = lib()
    p = synthkv.PRESETS[2]
    H = 2
    extra = {} if T is None else {"n_stages": T}
    oc = ocfg(p, "K", n_centroids=64, iters_cold=3, iters_warm=2, centroid_format=fmt, scale_mode=sm, **extra)
    # K and V of H heads as one 2H-head tensor (keys first)
    X = np.concatenate([synthkv.gen_numpy(p, t, heads=H, n_tokens=2000) for t in ("K", "V")])
    dst, _ = gpu_encode_chunks(oc, X, chunk)
    rng = np.random.default_rng(Nq + b)
    Q = oracle.bf16_round(rng.standard_normal((H, Nq, 128)) * 0.1).astype(np.float32)
    rope = None
    if use_rope:
        ang = rng.uniform(-50, 50, (e - b, 64))
        rope = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    qd = torch.from_numpy(Q).to(torch.bfloat16).to(DEV)
    out, lse = q.attention(gcfg(oc), dst, dst, qd, b, e, k_head0=0, v_head0=H,
                           rope=None if rope is None else torch.from_numpy(rope).to(DEV), want_lse=True)
    torch.cuda.synchronize()
    Kr = _decoded(oc, dst, b, e, chunk, range(H), rope)
    Vr = _decoded(oc, dst, b, e, chunk, range(H, 2 * H))
    scale = 128 ** -0.5
    O, L = oracle.attention(Q, Kr, Vr, scale)
    tol = oracle.attention_tolerance(Q, Kr, Vr, scale)
    got = to_np(out).astype(np.float64)
    err = np.abs(got - O)
    say(f"  max |err| {err.max():.3g}, max err / tol {float((err / tol).max()):.3g}")
    assert np.all(err <= tol)
    np.testing.assert_allclose(to_np(lse), L, rtol=1e-5, atol=1e-5)


def test_attention_argument_errors():
    q = lib()
    p = synthkv.PRESETS[2]
    oc = ocfg(p, "K", n_centroids=16)
    cfg = gcfg(oc)
    dst = q.CompressedKV(cfg, 2, 100, 100, DEV)
    qd = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device=DEV)
    for kw, st in ((dict(tok_begin=0, tok_end=101), q.QVG_ERR_INVALID_ARG),
                   (dict(tok_begin=5, tok_end=5), q.QVG_ERR_INVALID_ARG),
                   (dict(tok_begin=0, tok_end=50, v_head0=2), q.QVG_ERR_INVALID_ARG)):
        b, e = kw.pop("tok_begin"), kw.pop("tok_end")
        with pytest.raises(q.QvgError) as ex:
            q.attention(cfg, dst, dst, qd, b, e, **kw)
        assert ex.value.status == st
    cfg64 = q.config(64, 16, 2, 16, 2, 2, 1, "bf16")
    with pytest.raises(q.QvgError) as ex:
        q.attention(cfg64, dst, dst, qd, 0, 50)
    assert ex.value.status == q.QVG_ERR_UNSUPPORTED
