"""Quant VideoGen (QVG) 2-bit KV-cache codec for AMD MI355X (gfx950).

The codec's hot path (k-means smoothing on bf16 matrix cores, progressive
residual stages, 2-bit group quantisation with FP8 E4M3 scales, fused
dequantise + reconstruct) runs in the hand-written HIP kernels of libqvg.so,
reached through the C ABI of include/qvg.h.  ``_lib`` binds that ABI name for
name; ``codec`` allocates device buffers with torch around it.
"""
from . import _lib
from ._lib import *  # noqa: F401,F403  (the C entry points, same names)
from .codec import CentroidCache, CompressedKV, Encoder, attention, config, decode  # noqa: F401
