"""The C ABI without a GPU: the library loads, exports every function the header
declares, and its host-only calls (byte counts, workspace sizes, validation)
behave as documented.  No kernel is launched here: every call below returns
before touching the device."""
import ctypes
import os
import re

import pytest

import oracle
import synthkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qvg.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qvg_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def q():
    import bit_vector_quantization_amd as q

    return q


def test_every_declared_function_is_exported(q):
    names = _declared()
    assert len(names) >= 20
    # RTLD_NOW: every symbol the library needs must resolve at load time
    lib = ctypes.CDLL(q._lib.LIB_PATH, mode=os.RTLD_NOW)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding wraps every one of them under the same name
    for n in names:
        assert callable(getattr(q, n)), n


def test_struct_layouts_match_the_header(q):
    assert ctypes.sizeof(q.qvg_config) == 48
    assert q.qvg_config.seed.offset == 24 and q.qvg_config.dtype.offset == 32
    assert q.qvg_config.converge.offset == 36 and q.qvg_config.centroid_format.offset == 40
    assert ctypes.sizeof(q.qvg_cache_view) == 56
    assert q.qvg_cache_view.cap_tokens.offset == 32 and q.qvg_cache_view.heads.offset == 44
    assert ctypes.sizeof(q.qvg_kernel_stat) == 64


def _cfg(q, p, **kw):
    c = dict(d=p.d, n_centroids=p.n_centroids, n_stages=p.n_stages, group_size=p.group_size,
             iters_cold=p.iters_cold, iters_warm=p.iters_warm, seed=p.codec_seed("K"), dtype=p.dtype)
    c.update(kw)
    return q.config(**c), oracle.CodecConfig(**c)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_chunk_bytes_equal_the_closed_form(q, idx):
    p = synthkv.PRESETS[idx]
    g, o = _cfg(q, p)
    for N in (p.chunk_tokens, 1, 560):
        want = oracle.chunk_bytes(o, p.heads, N)
        assert q.qvg_chunk_bytes(g, p.heads, N) == (want["codes"], want["scales"], want["assign"],
                                                   want["centroids"])


def test_cache_view_bytes(q):
    p = synthkv.PRESETS[5]
    g, o = _cfg(q, p)
    v = q.qvg_cache_view_bytes(g, p.heads, p.n_tokens, p.chunk_tokens)
    per = oracle.chunk_bytes(o, p.heads, p.n_tokens)
    assert v[:3] == (per["codes"], per["scales"], per["assign"])
    assert v[3] == p.n_chunks * oracle.chunk_bytes(o, p.heads, 1)["centroids"]
    # the long-horizon cache: about 1.68 GB for K+V against 6.7 GB raw
    assert 1.6e9 < 2 * sum(v) < 1.75e9


def test_workspace_sizes(q):
    p = synthkv.PRESETS[3]
    g, _ = _cfg(q, p)
    ws = q.qvg_encode_workspace_bytes(g, p.heads, p.chunk_tokens)
    H, N, d, K = p.heads, p.chunk_tokens, p.d, p.n_centroids
    # token order + centroid tables + one bf16 copy of R(1) (the stage-2 assign
    # operand of a bf16 tensor); no fp32 residual is ever stored
    assert H * N * 4 + H * K * d * 6 + H * N * d * 2 <= ws < H * N * d * 3
    g1, _ = _cfg(q, p, n_stages=1)   # one stage: nothing to carry to a next stage
    assert q.qvg_encode_workspace_bytes(g1, H, N) < H * N * d
    g0, _ = _cfg(q, p, n_stages=0)
    assert q.qvg_encode_workspace_bytes(g0, H, N) <= 4096
    assert q.qvg_stage_workspace_bytes(H, N, d, 256) >= H * N * 4


def _attention_splits(q, g, H, Nq, Nk):
    """The split count behind qvg_attention_workspace_bytes: its partial outputs
    take round_up(splits x H x Nq x d x 4, 256) bytes and its (max, sum) pairs
    splits x H x Nq x 8."""
    ws = q.qvg_attention_workspace_bytes(g, H, Nq, Nk)
    per = H * Nq * 128 * 4
    for sp in range(1, 65):
        if ws == (sp * per + 255) // 256 * 256 + sp * H * Nq * 8:
            return sp
    raise AssertionError(f"workspace {ws} matches no split count")


@pytest.mark.parametrize("H,Nq,Nk", [(12, 4680, 1_092_000), (12, 4680, 9360), (40, 4680, 38_000), (2, 300, 19_017),
                                     (12, 1, 1_092_000), (1, 1, 10), (7, 1000, 500_000), (3, 257, 70_000)])
def test_attention_splits_fill_their_rounds(q, H, Nq, Nk):
    """One attention workgroup runs per CU (256) and the splits are equal, so the
    workgroups run in rounds of 256: the split count never fills its rounds worse
    than the plain rule (enough workgroups to fill the chip twice), stays within
    1..64 and keeps at least 256 keys per split."""
    p = synthkv.PRESETS[3]
    g, _ = _cfg(q, p)
    sp = _attention_splits(q, g, H, Nq, Nk)
    w = (Nq + 255) // 256 * H
    most = max(1, min(64, Nk // 256))
    plain = min(most, (512 + w - 1) // w)

    def fill(s):
        return w * s / (-(-w * s // 256) * 256)

    assert 1 <= sp <= most
    assert fill(sp) >= fill(plain) - 1e-12
    if (H, Nq, Nk) == (12, 4680, 1_092_000):   # the long-horizon attention: 2,280 workgroups in 9 rounds
        assert sp == 10
    if (H, Nq, Nk) == (40, 4680, 38_000):      # already 760 of 768 slots with one split
        assert sp == 1


@pytest.mark.parametrize("field,value,status", [
    ("n_centroids", 0, -1), ("n_centroids", 257, -1), ("n_stages", -1, -1), ("n_stages", 9, -1),
    ("group_size", 48, -1), ("group_size", 0, -1), ("iters_cold", -1, -1), ("dtype", 7, -1),
    ("converge", -1, -1), ("centroid_format", 2, -1), ("scale_mode", 2, -1), ("d", 192, -2), ("d", 256, -2), ("group_size", 8, -2)])
def test_config_validation(q, field, value, status):
    g, _ = _cfg(q, synthkv.PRESETS[2])
    setattr(g, field, value)
    assert q.qvg_config_validate(g) == status
    with pytest.raises(q.QvgError) as e:
        q.qvg_chunk_bytes(g, 1, 10)
    assert e.value.status == status


def _view(q, heads=2, cap=100, chunk=50, ptr=4096):
    return q.qvg_cache_view(ptr, ptr, ptr, ptr, cap, chunk, heads, None)


def test_encode_argument_errors_launch_nothing(q):
    g, _ = _cfg(q, synthkv.PRESETS[2])
    v = _view(q)
    good = dict(x=4096, hs=50 * 128, H=2, N=50, init=None, cache=None, dst=v, c=0, ws=4096, wsb=1 << 40)

    def call(**kw):
        a = dict(good, **kw)
        return q.LIB.qvg_encode_chunk(ctypes.byref(g), a["x"], a["hs"], a["H"], a["N"], a["init"], a["cache"],
                                      ctypes.byref(a["dst"]), a["c"], a["ws"], a["wsb"], None)

    assert call(x=None) == q.QVG_ERR_INVALID_ARG
    assert call(x=4100) == q.QVG_ERR_INVALID_ARG                  # misaligned
    assert call(hs=50 * 128 - 8) == q.QVG_ERR_INVALID_ARG         # rows would overlap
    assert call(N=0) == q.QVG_ERR_INVALID_ARG
    assert call(N=51) == q.QVG_ERR_INVALID_ARG                    # longer than a chunk
    assert call(c=2) == q.QVG_ERR_INVALID_ARG                     # past the capacity
    assert call(H=3) == q.QVG_ERR_INVALID_ARG                     # view holds 2 heads
    assert call(ws=None) == q.QVG_ERR_INVALID_ARG
    assert call(wsb=1024) == q.QVG_ERR_WORKSPACE
    assert call(dst=_view(q, ptr=0)) == q.QVG_ERR_INVALID_ARG


def test_decode_argument_errors_launch_nothing(q):
    g, _ = _cfg(q, synthkv.PRESETS[2])
    v = _view(q)

    def call(b=0, e=100, out=4096, hs=100 * 128, dt=q.QVG_BF16, view=v):
        return q.LIB.qvg_decode(ctypes.byref(g), ctypes.byref(view), b, e, out, hs, dt, None)

    assert call(b=-1) == q.QVG_ERR_INVALID_ARG
    assert call(b=10, e=10) == q.QVG_ERR_INVALID_ARG
    assert call(e=101) == q.QVG_ERR_INVALID_ARG
    assert call(out=None) == q.QVG_ERR_INVALID_ARG
    assert call(hs=100 * 128 - 1) == q.QVG_ERR_INVALID_ARG
    assert call(dt=5) == q.QVG_ERR_INVALID_ARG
    assert call(view=_view(q, ptr=0)) == q.QVG_ERR_INVALID_ARG


def test_decode_rope_argument_errors_launch_nothing(q):
    g, _ = _cfg(q, synthkv.PRESETS[2])
    v = _view(q)

    def call(rope=8192, rh=1, b=0, e=100, out=4096, view=v):
        return q.LIB.qvg_decode_rope(ctypes.byref(g), ctypes.byref(view), b, e, rope, rh, out, 100 * 128,
                                     q.QVG_BF16, None)

    assert call(rope=None) == q.QVG_ERR_INVALID_ARG
    assert call(rope=8200) == q.QVG_ERR_INVALID_ARG               # misaligned
    assert call(rh=-1) == q.QVG_ERR_INVALID_ARG
    assert call(rh=3) == q.QVG_ERR_INVALID_ARG                    # view holds 2 heads
    assert call(view=_view(q, ptr=0)) == q.QVG_ERR_INVALID_ARG    # then qvg_decode's own checks
    assert call(e=101) == q.QVG_ERR_INVALID_ARG
    assert call(out=None) == q.QVG_ERR_INVALID_ARG


def test_stage_entry_point_errors(q):
    L = q.LIB
    assert L.qvg_kmeans_assign(4096, q.QVG_BF16, 128, 4096, 1, 1, 96, 4, 4096, 1, 4096, 1 << 30, None) == -2
    assert L.qvg_kmeans_assign(4096, q.QVG_BF16, 128, 4096, 1, 1, 128, 300, 4096, 1, 4096, 1 << 30, None) == -1
    assert L.qvg_kmeans_assign(4096, q.QVG_BF16, 128, 4096, 1, 1, 128, 4, 4096, 1, 4096, 16, None) == -3
    assert L.qvg_centroid_update(4096, 3, 128, 4096, 1, 1, 1, 128, 4, 4096, None, 4096, 1 << 30, None) == -1
    assert L.qvg_group_quant(4096, 128, 1, 1, 128, 48, 4096, 4096, None) == -1
    assert L.qvg_group_quant(4100, 128, 1, 1, 128, 64, 4096, 4096, None) == -1
    assert L.qvg_centroid_cache_reset(None) == -1
    assert L.qvg_centroid_cache_destroy(None) == 0
    assert L.qvg_profile_read(None, 0, None) == -1
    assert q.status_string(-4) == "QVG_ERR_STATE"
