"""ctypes binding of libqvg.so: the C ABI declared in include/qvg.h, one Python
function per C entry point with the same name.

Argument marshalling only: device buffers are passed as raw pointers (ints) or
torch tensors (their ``data_ptr()``), streams as ``hipStream_t`` handles (ints)
or ``torch.cuda.Stream`` objects; every computation runs in the library.  A
non-zero status raises :class:`QvgError`.  There is no fallback: if the library
is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqvg.so")

QVG_OK = 0
QVG_ERR_INVALID_ARG = -1
QVG_ERR_UNSUPPORTED = -2
QVG_ERR_WORKSPACE = -3
QVG_ERR_STATE = -4
QVG_ERR_HIP = -5
QVG_ERR_OOM = -6

QVG_F32 = 0
QVG_BF16 = 1

QVG_CENT_NATIVE = 0
QVG_CENT_E4M3 = 1

QVG_SCALE_E4M3 = 0
QVG_SCALE_TWO_LEVEL = 1


class QvgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class qvg_config(ctypes.Structure):
    _fields_ = [("d", c_int32), ("n_centroids", c_int32), ("n_stages", c_int32),
                ("group_size", c_int32), ("iters_cold", c_int32), ("iters_warm", c_int32),
                ("seed", c_uint64), ("dtype", c_int32), ("converge", c_int32),
                ("centroid_format", c_int32), ("scale_mode", c_int32)]


class qvg_cache_view(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("scales", c_void_p), ("assign", c_void_p),
                ("centroids", c_void_p), ("cap_tokens", c_int64), ("chunk_tokens", c_int32),
                ("heads", c_int32), ("scale_exp", c_void_p)]


class qvg_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


_CFG = POINTER(qvg_config)
_VIEW = POINTER(qvg_cache_view)
_U64x4 = c_uint64 * 4

_SIGNATURES = {
    "qvg_status_string": (c_char_p, [c_int32]),
    "qvg_config_validate": (c_int32, [_CFG]),
    "qvg_chunk_bytes": (c_int32, [_CFG, c_int32, c_int32, _U64x4]),
    "qvg_cache_view_bytes": (c_int32, [_CFG, c_int32, c_int64, c_int32, _U64x4]),
    "qvg_encode_workspace_bytes": (c_int32, [_CFG, c_int32, c_int32, POINTER(c_uint64)]),
    "qvg_stage_workspace_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, POINTER(c_uint64)]),
    "qvg_centroid_cache_create": (c_int32, [_CFG, c_int32, POINTER(c_void_p)]),
    "qvg_centroid_cache_reset": (c_int32, [c_void_p]),
    "qvg_centroid_cache_destroy": (c_int32, [c_void_p]),
    "qvg_centroid_cache_data": (c_int32, [c_void_p, POINTER(c_void_p), POINTER(c_int32)]),
    "qvg_centroid_cache_export": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "qvg_centroid_cache_import": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "qvg_encode_chunk": (c_int32, [_CFG, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                   _VIEW, c_int32, c_void_p, c_uint64, c_void_p]),
    "qvg_attention_workspace_bytes": (c_int32, [_CFG, c_int32, c_int32, c_int64, POINTER(c_uint64)]),
    "qvg_attention": (c_int32, [_CFG, _VIEW, c_int32, _VIEW, c_int32, c_int64, c_int64, c_void_p, c_void_p,
                                c_int64, c_int32, c_int32, ctypes.c_float, c_void_p, c_int64, c_void_p, c_void_p,
                                c_uint64, c_void_p]),
    "qvg_encode_rounds": (c_int32, [_CFG, c_int32, c_int32, c_void_p, c_uint64, c_void_p, c_void_p]),
    "qvg_encode_chunk_static": (c_int32, [_CFG, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p,
                                          _VIEW, c_int32, c_void_p]),
    "qvg_decode": (c_int32, [_CFG, _VIEW, c_int64, c_int64, c_void_p, c_int64, c_int32, c_void_p]),
    "qvg_decode_rope": (c_int32, [_CFG, _VIEW, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int64,
                                  c_int32, c_void_p]),
    "qvg_kmeans_assign": (c_int32, [c_void_p, c_int32, c_int64, c_void_p, c_int32, c_int32, c_int32,
                                    c_int32, c_void_p, c_int64, c_void_p, c_uint64, c_void_p]),
    "qvg_centroid_update": (c_int32, [c_void_p, c_int32, c_int64, c_void_p, c_int64, c_int32, c_int32,
                                      c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_uint64, c_void_p]),
    "qvg_group_quant": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                  c_void_p, c_void_p]),
    "qvg_profile_enable": (c_int32, [c_int32]),
    "qvg_profile_read": (c_int32, [POINTER(qvg_kernel_stat), c_int32, POINTER(c_int32)]),
    "qvg_dequant_reconstruct": (c_int32, [_CFG, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_int32, c_void_p]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bit_vector_quantization_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def qvg_status_string(status: int) -> str:
    return LIB.qvg_status_string(status).decode()


status_string = qvg_status_string


def _check(status: int, what: str) -> None:
    if status != QVG_OK:
        raise QvgError(status, what)


def _ptr(x) -> int | None:
    """Device pointer of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_config(d: int, n_centroids: int, n_stages: int, group_size: int, iters_cold: int,
                iters_warm: int, seed: int, dtype: int, converge: int = 0,
                centroid_format: int = QVG_CENT_NATIVE, scale_mode: int = QVG_SCALE_E4M3) -> qvg_config:
    return qvg_config(d, n_centroids, n_stages, group_size, iters_cold, iters_warm, seed, dtype, converge,
                      centroid_format, scale_mode)


# ---- entry points (same names as the C ABI) --------------------------------

def qvg_config_validate(cfg: qvg_config) -> int:
    return LIB.qvg_config_validate(ctypes.byref(cfg))


def qvg_chunk_bytes(cfg: qvg_config, heads: int, n_tokens: int):
    out = _U64x4()
    _check(LIB.qvg_chunk_bytes(ctypes.byref(cfg), heads, n_tokens, out), "qvg_chunk_bytes")
    return tuple(out)


def qvg_cache_view_bytes(cfg: qvg_config, heads: int, cap_tokens: int, chunk_tokens: int):
    out = _U64x4()
    _check(LIB.qvg_cache_view_bytes(ctypes.byref(cfg), heads, cap_tokens, chunk_tokens, out),
           "qvg_cache_view_bytes")
    return tuple(out)


def qvg_encode_workspace_bytes(cfg: qvg_config, heads: int, n_tokens: int) -> int:
    out = c_uint64()
    _check(LIB.qvg_encode_workspace_bytes(ctypes.byref(cfg), heads, n_tokens, ctypes.byref(out)),
           "qvg_encode_workspace_bytes")
    return out.value


def qvg_stage_workspace_bytes(heads: int, n_tokens: int, d: int, n_centroids: int) -> int:
    out = c_uint64()
    _check(LIB.qvg_stage_workspace_bytes(heads, n_tokens, d, n_centroids, ctypes.byref(out)),
           "qvg_stage_workspace_bytes")
    return out.value


def qvg_centroid_cache_create(cfg: qvg_config, heads: int) -> int:
    h = c_void_p()
    _check(LIB.qvg_centroid_cache_create(ctypes.byref(cfg), heads, ctypes.byref(h)),
           "qvg_centroid_cache_create")
    return h.value


def qvg_centroid_cache_reset(cache: int) -> None:
    _check(LIB.qvg_centroid_cache_reset(cache), "qvg_centroid_cache_reset")


def qvg_centroid_cache_destroy(cache: int | None) -> None:
    _check(LIB.qvg_centroid_cache_destroy(cache), "qvg_centroid_cache_destroy")


def qvg_centroid_cache_data(cache: int):
    p, v = c_void_p(), c_int32()
    _check(LIB.qvg_centroid_cache_data(cache, ctypes.byref(p), ctypes.byref(v)),
           "qvg_centroid_cache_data")
    return p.value, v.value


def qvg_centroid_cache_export(cache: int, dst, stream=None) -> None:
    _check(LIB.qvg_centroid_cache_export(cache, _ptr(dst), _stream(stream)), "qvg_centroid_cache_export")


def qvg_centroid_cache_import(cache: int, src, stream=None) -> None:
    _check(LIB.qvg_centroid_cache_import(cache, _ptr(src), _stream(stream)), "qvg_centroid_cache_import")


def qvg_encode_chunk(cfg: qvg_config, x, x_head_stride: int, heads: int, n_tokens: int,
                     init_centroids, cache, dst: qvg_cache_view, chunk_index: int, workspace,
                     workspace_bytes: int, stream=None) -> None:
    _check(LIB.qvg_encode_chunk(ctypes.byref(cfg), _ptr(x), x_head_stride, heads, n_tokens,
                                _ptr(init_centroids), cache, ctypes.byref(dst), chunk_index,
                                _ptr(workspace), workspace_bytes, _stream(stream)),
           "qvg_encode_chunk")


def qvg_encode_rounds(cfg: qvg_config, heads: int, n_tokens: int, workspace, workspace_bytes: int, rounds_out,
                      stream=None) -> None:
    _check(LIB.qvg_encode_rounds(ctypes.byref(cfg), heads, n_tokens, _ptr(workspace), workspace_bytes,
                                 _ptr(rounds_out), _stream(stream)), "qvg_encode_rounds")


def qvg_attention_workspace_bytes(cfg: qvg_config, heads: int, n_queries: int, n_keys: int) -> int:
    out = c_uint64()
    _check(LIB.qvg_attention_workspace_bytes(ctypes.byref(cfg), heads, n_queries, n_keys, ctypes.byref(out)),
           "qvg_attention_workspace_bytes")
    return out.value


def qvg_attention(cfg: qvg_config, k_src: qvg_cache_view, k_head0: int, v_src: qvg_cache_view, v_head0: int,
                  tok_begin: int, tok_end: int, rope, q, q_head_stride: int, heads: int, n_queries: int,
                  scale: float, out, out_head_stride: int, lse, workspace, workspace_bytes: int, stream=None) -> None:
    _check(LIB.qvg_attention(ctypes.byref(cfg), ctypes.byref(k_src), k_head0, ctypes.byref(v_src), v_head0,
                             tok_begin, tok_end, _ptr(rope), _ptr(q), q_head_stride, heads, n_queries, scale,
                             _ptr(out), out_head_stride, _ptr(lse), _ptr(workspace), workspace_bytes,
                             _stream(stream)), "qvg_attention")


QVG_STATIC_SCRATCH_BYTES = 64 << 20   # the fixed scratch array of qvg_encode_chunk_static


def qvg_encode_chunk_static(cfg: qvg_config, x, x_head_stride: int, heads: int, n_tokens: int,
                            init_centroids, cache, dst: qvg_cache_view, chunk_index: int, stream=None) -> None:
    _check(LIB.qvg_encode_chunk_static(ctypes.byref(cfg), _ptr(x), x_head_stride, heads, n_tokens,
                                       _ptr(init_centroids), cache, ctypes.byref(dst), chunk_index,
                                       _stream(stream)),
           "qvg_encode_chunk_static")


def qvg_decode(cfg: qvg_config, src: qvg_cache_view, tok_begin: int, tok_end: int, out,
               out_head_stride: int, out_dtype: int, stream=None) -> None:
    _check(LIB.qvg_decode(ctypes.byref(cfg), ctypes.byref(src), tok_begin, tok_end, _ptr(out),
                          out_head_stride, out_dtype, _stream(stream)), "qvg_decode")


def qvg_decode_rope(cfg: qvg_config, src: qvg_cache_view, tok_begin: int, tok_end: int, rope,
                    rope_heads: int, out, out_head_stride: int, out_dtype: int, stream=None) -> None:
    _check(LIB.qvg_decode_rope(ctypes.byref(cfg), ctypes.byref(src), tok_begin, tok_end, _ptr(rope),
                               rope_heads, _ptr(out), out_head_stride, out_dtype, _stream(stream)),
           "qvg_decode_rope")


def qvg_kmeans_assign(x, x_dtype: int, x_head_stride: int, centroids, heads: int, n_tokens: int,
                      d: int, n_centroids: int, assign_out, assign_head_stride: int, workspace,
                      workspace_bytes: int, stream=None) -> None:
    _check(LIB.qvg_kmeans_assign(_ptr(x), x_dtype, x_head_stride, _ptr(centroids), heads, n_tokens,
                                 d, n_centroids, _ptr(assign_out), assign_head_stride,
                                 _ptr(workspace), workspace_bytes, _stream(stream)),
           "qvg_kmeans_assign")


def qvg_centroid_update(x, x_dtype: int, x_head_stride: int, assign, assign_head_stride: int,
                        heads: int, n_tokens: int, d: int, n_centroids: int, centroids, counts_out,
                        workspace, workspace_bytes: int, stream=None) -> None:
    _check(LIB.qvg_centroid_update(_ptr(x), x_dtype, x_head_stride, _ptr(assign), assign_head_stride,
                                   heads, n_tokens, d, n_centroids, _ptr(centroids), _ptr(counts_out),
                                   _ptr(workspace), workspace_bytes, _stream(stream)),
           "qvg_centroid_update")


def qvg_group_quant(r, r_head_stride: int, heads: int, n_tokens: int, d: int, group_size: int,
                    codes, scales, stream=None) -> None:
    _check(LIB.qvg_group_quant(_ptr(r), r_head_stride, heads, n_tokens, d, group_size, _ptr(codes),
                               _ptr(scales), _stream(stream)), "qvg_group_quant")


def qvg_dequant_reconstruct(cfg: qvg_config, heads: int, n_tokens: int, codes, scales, assign,
                            centroids, out, out_dtype: int, stream=None) -> None:
    _check(LIB.qvg_dequant_reconstruct(ctypes.byref(cfg), heads, n_tokens, _ptr(codes), _ptr(scales),
                                       _ptr(assign), _ptr(centroids), _ptr(out), out_dtype,
                                       _stream(stream)), "qvg_dequant_reconstruct")


def qvg_profile_enable(on: bool) -> None:
    _check(LIB.qvg_profile_enable(1 if on else 0), "qvg_profile_enable")


def qvg_profile_read() -> dict:
    """{kernel name: {launches, total_ms, avg_ms, flops, bytes}} since enabling."""
    n = c_int32()
    _check(LIB.qvg_profile_read(None, 0, ctypes.byref(n)), "qvg_profile_read")
    buf = (qvg_kernel_stat * max(n.value, 1))()
    _check(LIB.qvg_profile_read(buf, n.value, ctypes.byref(n)), "qvg_profile_read")
    out = {}
    for i in range(n.value):
        e = buf[i]
        out[e.name.decode()] = dict(launches=e.launches, total_ms=e.total_ms,
                                   avg_ms=e.total_ms / max(e.launches, 1), flops=e.flops, bytes=e.bytes)
    return out
