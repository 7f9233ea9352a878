"""qvg_encode_chunk_static, the encode entry point that allocates nothing (its
workspace is the library's fixed device array), against qvg_encode_chunk with
a caller-given workspace, through the C ABI: two calls in a row on the same
array, the second with a smaller chunk, every output byte equal; a call over
the array's limit is rejected before anything is launched.  The variants'
workspace regions (the FP8 operand table, the per-head stop state) come from the
array too."""
import numpy as np
import pytest
import torch

import synthkv
from gpu_util import DEV, fetch, gcfg, lib, ocfg, say, to_np

pytestmark = pytest.mark.gpu


def _encode_pair(q, oc, X, cache_a, cache_b, chunk, dst_a, dst_b, enc):
    """The same chunk through both entry points; each has its own streaming cache."""
    H, N, _ = X.shape
    cfg = gcfg(oc)
    enc.encode(X, dst_a, chunk, cache=cache_a)
    q.qvg_encode_chunk_static(cfg, X, X.stride(0), H, N, None, cache_b.handle, dst_b.view, chunk,
                              torch.cuda.current_stream())


def test_static_scratch_encode_equals_workspace_encode():
    q = lib()
    p = synthkv.PRESETS[3]
    say("no-allocation encode: 12 heads x 4,680 tokens, then 5 heads x 1,000 tokens, then 4 heads x 1,500 "
        "tokens with FP8 tables, two-level scales and the convergence stop")
    variants = dict(centroid_format="e4m3", scale_mode="two_level", converge=2, iters_cold=8, iters_warm=8)
    for H, N, tensor, extra in ((12, p.chunk_tokens, "V", {}), (5, 1000, "K", {}), (4, 1500, "V", variants)):
        oc = ocfg(p, tensor, **extra)
        cfg = gcfg(oc)
        assert q.qvg_encode_workspace_bytes(cfg, H, N) <= q.QVG_STATIC_SCRATCH_BYTES
        X = torch.from_numpy(synthkv.gen_numpy(p, tensor, heads=H, n_tokens=2 * N)).to(torch.bfloat16).to(DEV)
        dst_a = q.CompressedKV(cfg, H, 2 * N, N, DEV)
        dst_b = q.CompressedKV(cfg, H, 2 * N, N, DEV)
        enc = q.Encoder(cfg, H, N, DEV)
        ca, cb = q.CentroidCache(cfg, H), q.CentroidCache(cfg, H)
        for c in range(2):   # cold, then warm from each path's own cache
            _encode_pair(q, oc, X[:, c * N:(c + 1) * N], ca, cb, c, dst_a, dst_b, enc)
        torch.cuda.synchronize()
        for c in range(2):
            a, b = fetch(dst_a, c, oc), fetch(dst_b, c, oc)
            for k in a:
                np.testing.assert_array_equal(a[k], b[k], err_msg=f"{H}x{N} chunk {c} {k}")
        np.testing.assert_array_equal(to_np(ca.export(DEV)), to_np(cb.export(DEV)))
        say(f"  {H} heads x {N} tokens: codes, scales, assignments, centroids and cache equal")


def test_static_scratch_rejects_oversized_calls():
    q = lib()
    p = synthkv.PRESETS[3]
    oc = ocfg(p, "K")
    cfg = gcfg(oc)
    H, N = 80, p.chunk_tokens
    assert q.qvg_encode_workspace_bytes(cfg, H, N) > q.QVG_STATIC_SCRATCH_BYTES
    X = torch.zeros((H, N, p.d), dtype=torch.bfloat16, device=DEV)
    dst = q.CompressedKV(cfg, H, N, N, DEV)
    with pytest.raises(q.QvgError) as e:
        q.qvg_encode_chunk_static(cfg, X, X.stride(0), H, N, None, None, dst.view, 0, torch.cuda.current_stream())
    assert e.value.status == q.QVG_ERR_WORKSPACE
