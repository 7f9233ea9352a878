"""Device-buffer plumbing around the C ABI: torch allocates the compressed cache,
the workspace and the outputs; every step of the codec runs in libqvg.so."""
from __future__ import annotations

import torch

from . import _lib as L


def config(d: int, n_centroids: int, n_stages: int, group_size: int, iters_cold: int,
           iters_warm: int, seed: int, dtype: str, converge: int = 0,
           centroid_format: str = "native", scale_mode: str = "e4m3") -> L.qvg_config:
    dt = {"bf16": L.QVG_BF16, "f32": L.QVG_F32}[dtype]
    cf = {"native": L.QVG_CENT_NATIVE, "e4m3": L.QVG_CENT_E4M3}[centroid_format]
    sm = {"e4m3": L.QVG_SCALE_E4M3, "two_level": L.QVG_SCALE_TWO_LEVEL}[scale_mode]
    return L.make_config(d, n_centroids, n_stages, group_size, iters_cold, iters_warm, seed, dt, converge, cf, sm)


def _dtype_of(cfg: L.qvg_config) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == L.QVG_BF16 else torch.float32


def _contiguous_for(t: torch.Tensor, stream) -> torch.Tensor:
    """t itself when contiguous; otherwise a contiguous copy that the caching
    allocator will not hand out again before the work enqueued on `stream` is
    done (the library reads it asynchronously there)."""
    if t.is_contiguous():
        return t
    c = t.contiguous()
    if stream is None or isinstance(stream, torch.cuda.Stream):
        if stream is not None and stream != torch.cuda.current_stream(c.device):
            c.record_stream(stream)
        return c
    raise ValueError("a non-contiguous tensor needs a torch.cuda.Stream (or none): a raw stream "
                     "handle cannot keep its contiguous copy alive")


class CompressedKV:
    """The compressed cache of one tensor of one layer: codes, scales,
    assignments and per-chunk centroids, plus the qvg_cache_view over them."""

    def __init__(self, cfg: L.qvg_config, heads: int, cap_tokens: int, chunk_tokens: int, device):
        self.cfg, self.heads, self.cap, self.chunk_tokens = cfg, heads, cap_tokens, chunk_tokens
        nb = L.qvg_cache_view_bytes(cfg, heads, cap_tokens, chunk_tokens)
        d, G, T, K = cfg.d, cfg.group_size, cfg.n_stages, cfg.n_centroids
        self.n_chunks = -(-cap_tokens // chunk_tokens)
        self.codes = torch.empty((heads, cap_tokens, d // 4), dtype=torch.uint8, device=device)
        self.scales = torch.empty((heads, cap_tokens, d // G), dtype=torch.uint8, device=device)
        self.assign = torch.empty((max(T, 1), heads, cap_tokens), dtype=torch.uint8, device=device)
        if cfg.centroid_format == L.QVG_CENT_E4M3:   # per table: 16-byte exponent header + K*d codes
            self.centroids = torch.empty((self.n_chunks, max(T, 1), heads, 16 + K * d), dtype=torch.uint8,
                                         device=device)
        else:
            self.centroids = torch.empty((self.n_chunks, max(T, 1), heads, K, d), dtype=_dtype_of(cfg),
                                         device=device)
        assert self.codes.numel() == nb[0] and self.scales.numel() == nb[1]
        assert T == 0 or (self.assign.numel() == nb[2]
                          and self.centroids.numel() * self.centroids.element_size() == nb[3])
        # second-level scale exponents, [n_chunks][H] (two-level scales only)
        self.scale_exp = (torch.zeros((self.n_chunks, heads), dtype=torch.int8, device=device)
                          if cfg.scale_mode == L.QVG_SCALE_TWO_LEVEL else None)
        self.view = L.qvg_cache_view(self.codes.data_ptr(), self.scales.data_ptr(),
                                     self.assign.data_ptr(), self.centroids.data_ptr(),
                                     cap_tokens, chunk_tokens, heads,
                                     None if self.scale_exp is None else self.scale_exp.data_ptr())

    def bytes(self) -> int:
        return sum(L.qvg_cache_view_bytes(self.cfg, self.heads, self.cap, self.chunk_tokens))


class CentroidCache:
    """Owner of a qvg_centroid_cache handle."""

    def __init__(self, cfg: L.qvg_config, heads: int):
        self.cfg, self.heads = cfg, heads
        self.handle = L.qvg_centroid_cache_create(cfg, heads)

    def reset(self) -> None:
        L.qvg_centroid_cache_reset(self.handle)

    def export(self, device, stream=None) -> torch.Tensor:
        c = self.cfg
        out = torch.empty((c.n_stages, self.heads, c.n_centroids, c.d), dtype=torch.float32, device=device)
        L.qvg_centroid_cache_export(self.handle, out, stream or torch.cuda.current_stream())
        return out

    def load(self, src: torch.Tensor, stream=None) -> None:
        L.qvg_centroid_cache_import(self.handle, _contiguous_for(src, stream), stream or torch.cuda.current_stream())

    def close(self) -> None:
        if self.handle is not None:
            L.qvg_centroid_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Encoder:
    """Holds a workspace sized for (heads, max chunk tokens) and encodes chunks."""

    def __init__(self, cfg: L.qvg_config, heads: int, max_tokens: int, device):
        self.cfg, self.heads = cfg, heads
        self.ws_bytes = L.qvg_encode_workspace_bytes(cfg, heads, max_tokens)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.last_tokens = None

    def rounds(self, stream=None) -> torch.Tensor:
        """[T][H] int32 Lloyd rounds of the last encode (convergence mode only)."""
        out = torch.empty((self.cfg.n_stages, self.heads), dtype=torch.int32, device=self.ws.device)
        L.qvg_encode_rounds(self.cfg, self.heads, self.last_tokens, self.ws, self.ws_bytes, out,
                            stream or torch.cuda.current_stream())
        return out

    def encode(self, x: torch.Tensor, dst: CompressedKV, chunk_index: int,
               cache: CentroidCache | None = None, init: torch.Tensor | None = None, stream=None):
        """x: [H][N][d] view whose rows are contiguous (a token slice of a larger
        [H][Ntot][d] tensor is fine)."""
        H, N, d = x.shape
        assert x.stride(2) == 1 and x.stride(1) == d and x.dtype == _dtype_of(self.cfg)
        self.last_tokens = N
        L.qvg_encode_chunk(self.cfg, x, x.stride(0), H, N,
                           None if init is None else _contiguous_for(init, stream),
                           None if cache is None else cache.handle, dst.view, chunk_index,
                           self.ws, self.ws_bytes, stream or torch.cuda.current_stream())


def decode(cfg: L.qvg_config, src: CompressedKV, tok_begin: int, tok_end: int,
           out: torch.Tensor | None = None, out_dtype: str = "bf16", stream=None,
           rope: torch.Tensor | None = None, rope_heads: int | None = None) -> torch.Tensor:
    """Tokens [tok_begin, tok_end) of every head.  With ``rope`` (fp32
    [tok_end - tok_begin][d/2][2] of (cos, sin), contiguous, on the device) the
    first ``rope_heads`` heads (all by default) come out rotated."""
    if out is None:
        dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        out = torch.empty((src.heads, tok_end - tok_begin, cfg.d), dtype=dt, device=src.codes.device)
    odt = L.QVG_BF16 if out.dtype == torch.bfloat16 else L.QVG_F32
    assert out.stride(2) == 1 and out.stride(1) == cfg.d
    if rope is None:
        L.qvg_decode(cfg, src.view, tok_begin, tok_end, out, out.stride(0), odt,
                     stream or torch.cuda.current_stream())
    else:
        assert rope.dtype == torch.float32 and rope.is_contiguous()
        assert tuple(rope.shape) == (tok_end - tok_begin, cfg.d // 2, 2)
        L.qvg_decode_rope(cfg, src.view, tok_begin, tok_end, rope, src.heads if rope_heads is None else rope_heads,
                          out, out.stride(0), odt, stream or torch.cuda.current_stream())
    return out


def attention(cfg: L.qvg_config, k_src: CompressedKV, v_src: CompressedKV, q: torch.Tensor, tok_begin: int,
              tok_end: int, k_head0: int = 0, v_head0: int = 0, rope: torch.Tensor | None = None,
              scale: float | None = None, stream=None, want_lse: bool = False):
    """softmax(scale q k^T) v over the compressed keys and values of tokens
    [tok_begin, tok_end), rebuilt inside the kernel (q: bf16 [H][Nq][d] with
    contiguous rows).  Returns fp32 [H][Nq][d] (and the lse [H][Nq])."""
    H, Nq, d = q.shape
    assert q.dtype == torch.bfloat16 and q.stride(2) == 1 and q.stride(1) == d
    if rope is not None:
        assert rope.dtype == torch.float32 and rope.is_contiguous()
        assert tuple(rope.shape) == (tok_end - tok_begin, d // 2, 2)
    out = torch.empty((H, Nq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((H, Nq), dtype=torch.float32, device=q.device) if want_lse else None
    ws_bytes = L.qvg_attention_workspace_bytes(cfg, H, Nq, tok_end - tok_begin)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    L.qvg_attention(cfg, k_src.view, k_head0, v_src.view, v_head0, tok_begin, tok_end, rope, q, q.stride(0), H,
                    Nq, d ** -0.5 if scale is None else scale, out, out.stride(0), lse, ws, ws_bytes,
                    stream or torch.cuda.current_stream())
    return (out, lse) if want_lse else out
