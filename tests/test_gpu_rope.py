"""Parity of the decode with the rotary position embedding applied in the same
pass (qvg_decode_rope), through the C ABI, against the oracle's decode +
rotation: bit-exact, fp32 and bf16 outputs.

Keys are cached before the rotation (163.com article, section 5,
implementation details).  The stored arrays are drawn at random (every 2-bit
code, E4M3 scale byte and label value occurs) and laid out as a cache of
several chunks with a ragged last one; decoded ranges start and end inside
chunks.  Both kernels are covered: the one that stages the tables in LDS
(1 to 4 stages with small enough tables) and the one that reads them through
L2 (no stages, more than 4, or tables too large for LDS), with native and FP8
(E4M3) centroid tables and with plain and two-level scales."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import DEV, lib, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _cache(rng, H, cap, chunk, d, K, T, G, dtype):
    C = -(-cap // chunk)
    codes = rng.integers(0, 256, (H, cap, d // 4), dtype=np.uint8)
    scales = rng.integers(0, 256, (H, cap, d // G), dtype=np.uint8)
    asg = rng.integers(0, K, (max(T, 1), H, cap), dtype=np.uint8)
    cent = (rng.standard_normal((C, max(T, 1), H, K, d)) * rng.lognormal(0, 1, (C, max(T, 1), H, K, 1)) * 4)
    cent = cent.astype(np.float32)
    if dtype == "bf16":
        cent = oracle.bf16_round(cent).astype(np.float32)
    return codes, scales, asg, cent


def _table(rng, n, d):
    ang = rng.uniform(-np.pi, np.pi, (n, d // 2)) * rng.choice([1.0, 1e-3, 100.0], (n, 1))
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def _reference(arrs, chunk, T, G, tb, te, out, rope, rope_heads):
    codes, scales, asg, cent = arrs
    parts = []
    for c in range(tb // chunk, (te - 1) // chunk + 1):
        b, e = max(tb, c * chunk), min(te, (c + 1) * chunk)
        a = asg[:T, :, b:e] if T else np.zeros((0, codes.shape[0], e - b), np.uint8)
        parts.append(oracle.decode_chunk(codes[:, b:e], scales[:, b:e], a, cent[c, :T], G, out,
                                         rope=None if rope is None else rope[b - tb:e - tb], rope_heads=rope_heads))
    return np.concatenate(parts, axis=1)


def _same(got, ref):
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got.view(np.uint32)[~np.isnan(got)], ref.view(np.uint32)[~np.isnan(ref)])


def _run(q, arrs, H, cap, chunk, d, K, T, G, dtype, tb, te, rope, rope_heads, out_dtype, pad=0):
    codes, scales, asg, cent = arrs
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    keep = [dev(codes), dev(scales), dev(asg), to_dev(cent, dtype)]
    view = q.qvg_cache_view(keep[0].data_ptr(), keep[1].data_ptr(), keep[2].data_ptr(), keep[3].data_ptr(),
                            cap, chunk, H)
    cfg = q.config(d, K, T, G, 2, 2, 7, dtype)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    # pad > 0: heads pad rows apart in a larger buffer whose gaps must stay untouched
    big = torch.full((H, te - tb + pad, d), 7.0, dtype=dt, device=DEV)
    out = big[:, :te - tb]
    odt = q.QVG_F32 if out_dtype == "f32" else q.QVG_BF16
    if rope is None:
        q.qvg_decode(cfg, view, tb, te, out, out.stride(0), odt)
    else:
        keep.append(to_dev(rope, "f32"))
        q.qvg_decode_rope(cfg, view, tb, te, keep[-1], rope_heads, out, out.stride(0), odt)
    torch.cuda.synchronize()
    if pad:
        assert (big[:, te - tb:] == 7.0).all()
    return to_np(out)


CASES = [
    # H, cap, chunk, d, K, T, G, dtype, tb, te, rope_heads
    (3, 777, 300, 128, 32, 2, 64, "bf16", 123, 700, 2),     # LDS tables, three chunks, ragged range
    (4, 3100, 1500, 128, 256, 2, 64, "bf16", 0, 3100, 2),   # several trips per workgroup
    (2, 500, 250, 64, 16, 1, 16, "f32", 0, 500, 2),         # d = 64, fp32 centroids
    (2, 700, 350, 128, 256, 4, 16, "bf16", 349, 351, 1),    # four stages, a range across one boundary
    (1, 300, 300, 128, 16, 3, 32, "bf16", 299, 300, 1),     # one token
    (2, 300, 300, 128, 8, 0, 64, "bf16", 7, 290, 1),        # no stages: L2 kernel
    (1, 260, 130, 128, 16, 5, 32, "bf16", 1, 259, 1),       # five stages: L2 kernel
    (2, 600, 300, 128, 256, 3, 64, "f32", 50, 600, 2),      # fp32 tables too large for LDS: L2 kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}_T{c[5]}_d{c[3]}_{c[7]}" for c in CASES])
def test_decode_rope_bit_exact(case):
    H, cap, chunk, d, K, T, G, dtype, tb, te, rh = case
    say(f"decode_rope {case}")
    q = lib()
    rng = np.random.default_rng(cap + T)
    arrs = _cache(rng, H, cap, chunk, d, K, T, G, dtype)
    rope = _table(rng, te - tb, d)
    for out in ("f32", "bf16"):
        got = _run(q, arrs, H, cap, chunk, d, K, T, G, dtype, tb, te, rope, rh, out)
        _same(got, _reference(arrs, chunk, T, G, tb, te, out, rope, rh))


def test_decode_rope_zero_heads_and_3d_table():
    """rope_heads = 0 is the plain decode, bit for bit; the 3-D position table
    of the 13B layer's latent grid on a two-chunk cache."""
    say("decode_rope: rope_heads 0, 3-D table")
    q = lib()
    p = synthkv.PRESETS[3]
    H, cap, chunk, d, K, T, G = 2, 2 * 4680, 4680, 128, 256, 2, 64
    rng = np.random.default_rng(5)
    arrs = _cache(rng, H, cap, chunk, d, K, T, G, "bf16")
    tb, te = 1000, cap
    rope = synthkv.rope_table(p, tb, te)
    plain = _run(q, arrs, H, cap, chunk, d, K, T, G, "bf16", tb, te, None, 0, "bf16")
    zero = _run(q, arrs, H, cap, chunk, d, K, T, G, "bf16", tb, te, rope, 0, "bf16")
    _same(zero, plain)
    got = _run(q, arrs, H, cap, chunk, d, K, T, G, "bf16", tb, te, rope, 1, "bf16")
    _same(got, _reference(arrs, chunk, T, G, tb, te, "bf16", rope, 1))
    _same(got[1], plain[1])


def test_decode_rope_head_stride_with_gaps():
    """Heads written out_head_stride elements apart with gaps between them (the
    gaps keep their contents), a range that starts and ends inside chunks."""
    say("decode_rope: output heads with gaps")
    q = lib()
    H, cap, chunk, d, K, T, G = 3, 1000, 400, 128, 64, 2, 64
    rng = np.random.default_rng(9)
    arrs = _cache(rng, H, cap, chunk, d, K, T, G, "bf16")
    tb, te = 37, 911
    rope = _table(rng, te - tb, d)
    for out in ("bf16", "f32"):
        got = _run(q, arrs, H, cap, chunk, d, K, T, G, "bf16", tb, te, rope, 2, out, pad=24)
        _same(got, _reference(arrs, chunk, T, G, tb, te, out, rope, 2))


FMT_CASES = [
    # H, cap, chunk, K, T, G, tb, te, rope_heads, centroid format, two-level scales
    (3, 777, 300, 32, 2, 64, 123, 700, 2, "e4m3", False),   # LDS kernel, FP8 tables
    (2, 600, 300, 64, 2, 64, 0, 600, 1, "native", True),     # LDS kernel, two-level scales
    (2, 700, 350, 256, 4, 16, 349, 351, 2, "e4m3", True),    # both, four stages, across a boundary
    (1, 260, 130, 16, 5, 32, 1, 259, 1, "e4m3", True),       # both, five stages: L2 kernel
]


@pytest.mark.parametrize("case", FMT_CASES, ids=[f"H{c[0]}_T{c[4]}_{c[9]}_{'2l' if c[10] else '1l'}" for c in FMT_CASES])
def test_decode_rope_fp8_tables_and_two_level_scales(case):
    """The rotated decode over FP8 (E4M3) centroid tables (a power-of-two
    exponent per table in a 16-byte header, then K x d codes) and over two-level
    scales (a second-level exponent per (chunk, head)), against the oracle's
    decode of the same stored values."""
    H, cap, chunk, K, T, G, tb, te, rh, fmt, two = case
    d = 128
    say(f"decode_rope formats {case}")
    q = lib()
    rng = np.random.default_rng(cap + 17 * T)
    codes, scales, asg, cent = _cache(rng, H, cap, chunk, d, K, T, G, "bf16")
    C = -(-cap // chunk)
    if fmt == "e4m3":
        ok = np.array([v for v in range(256) if v & 0x7F != 0x7F], np.uint8)   # every E4M3 byte but NaN
        raw = np.zeros((C, T, H, 16 + K * d), np.uint8)
        raw[..., 16:] = rng.choice(ok, (C, T, H, K * d))
        raw[..., :4] = rng.integers(-6, 7, (C, T, H), dtype=np.int32)[..., None].view(np.uint8).reshape(C, T, H, 4)
        cent = oracle.e4m3_decode(raw[..., 16:]).reshape(C, T, H, K, d)
        cent = np.ldexp(cent, raw[..., :4].copy().view(np.int32)[..., 0][..., None, None]).astype(np.float32)
        dev_cent = torch.from_numpy(raw).to(DEV)
    else:
        dev_cent = to_dev(cent, "bf16")
    sexp = rng.integers(0, 4, (C, H)).astype(np.int8) if two else None
    rope = _table(rng, te - tb, d)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    keep = [dev(codes), dev(scales), dev(asg), dev_cent, dev(rope)]
    if two:
        keep.append(dev(sexp))
    view = q.qvg_cache_view(keep[0].data_ptr(), keep[1].data_ptr(), keep[2].data_ptr(), keep[3].data_ptr(), cap,
                            chunk, H, keep[5].data_ptr() if two else None)
    cfg = q.config(d, K, T, G, 2, 2, 7, "bf16", 0, fmt, "two_level" if two else "e4m3")
    for out_dtype in ("f32", "bf16"):
        dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = torch.empty((H, te - tb, d), dtype=dt, device=DEV)
        q.qvg_decode_rope(cfg, view, tb, te, keep[4], rh, out, out.stride(0),
                          q.QVG_F32 if out_dtype == "f32" else q.QVG_BF16)
        torch.cuda.synchronize()
        parts = []
        for c in range(tb // chunk, (te - 1) // chunk + 1):
            b, e = max(tb, c * chunk), min(te, (c + 1) * chunk)
            parts.append(oracle.decode_chunk(codes[:, b:e], scales[:, b:e], asg[:T, :, b:e], cent[c, :T], G, out_dtype,
                                             rope=rope[b - tb:e - tb], rope_heads=rh,
                                             scale_exp=None if sexp is None else sexp[c]))
        _same(to_np(out), np.concatenate(parts, axis=1))
