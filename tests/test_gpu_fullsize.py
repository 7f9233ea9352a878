"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole tensor (all heads, every chunk, the streaming
centroid cache) goes through the HIP path; the oracle replays sampled heads
from the same inputs.

* 13B-shaped layer: K and V of 40 heads as one 80-head tensor, 38,000 tokens
  in 9 chunks (the last 560 tokens).  Two sampled heads (one key, one value)
  are replayed by the oracle over all 9 chunks, warm starts included, and
  compared bit for bit, decoded rows too.  The whole cache is then decoded
  with the 40 key heads rotated by the latent grid's 3-D position table;
  sampled heads and chunks match the oracle's decode + rotation bit for bit.
* Aggressive setting: 24 heads, 4 stages, groups of 16, 2 chunks, keys and
  values; three heads of each replayed.
* Long-horizon cache: 24 heads x 1,092,000 tokens (234 chunks).  The oracle
  replays chunks 0-1 of two heads.  Two late chunks of the same heads are
  replayed by the oracle from the streaming cache the HIP path held just
  before them (exported through the C ABI), and also checked through
  properties that hold for any chunk (labels nearest under the HIP path's own
  centroids, codes the oracle's quantiser of the resulting residual, decoded
  rows the oracle's reconstruction).

Inputs come from the device generator; the sampled heads' rows are copied to
the host for the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synthkv
from gpu_util import (DEV, check_chunk, check_chunk_properties, fetch, gcfg, layer_on_device, lib, ocfg, say,
                      to_np)

pytestmark = pytest.mark.gpu


def _encode_all(p, oc, X, export_before=()):
    """The benchmark's loop: one encode call per chunk over all heads.  With
    export_before, also returns the streaming cache's content (fp32, on the
    host) just before each of those chunks was encoded."""
    q = lib()
    cfg = gcfg(oc)
    H, N, _ = X.shape
    dst = q.CompressedKV(cfg, H, N, p.chunk_tokens, DEV)
    enc = q.Encoder(cfg, H, p.chunk_tokens, DEV)
    cache = q.CentroidCache(cfg, H)
    saved = {}
    for c in range(p.n_chunks):
        b, e = p.chunk_range(c)
        if c in export_before:
            saved[c] = to_np(cache.export(DEV))
        enc.encode(X[:, b:e], dst, c, cache=cache)
    torch.cuda.synchronize()
    return (dst, saved) if export_before else dst


def _host_heads(X, heads):
    return {h: X[h].float().cpu().numpy()[None] for h in heads}


def _replay(p, oc, X, dst, heads, chunks):
    """Oracle over chunks [0, chunks) of each sampled head; bit-exact comparison."""
    q = lib()
    hx = _host_heads(X, heads)
    total = 0
    for h in heads:
        say(f"  oracle replay of head {h}, chunks 0..{chunks - 1}")
        Xh = hx[h][:, :p.chunk_range(chunks - 1)[1]]
        cache = None
        for c in range(chunks):
            b, e = p.chunk_range(c)
            ora = oracle.encode_chunk(Xh[:, b:e], oc, cache=cache, head_offset=h)
            cache = ora.cache
            g = fetch(dst, c, oc)
            total += check_chunk(oc, _slice(hx, h, b, e, X.shape[0]), g, ora, 0, h, f"chunk {c}")
            y = q.decode(gcfg(oc), dst, b, e, out_dtype="bf16")
            np.testing.assert_array_equal(to_np(y)[h], oracle.decode(ora, oc.group_size, "bf16")[0])
    return total


def _slice(hx, h, b, e, H):
    """A [H][e-b][d] array whose row h holds the sampled head's chunk (other
    heads are never read by the checks)."""
    out = np.zeros((H, e - b, hx[h].shape[2]), np.float32)
    out[h] = hx[h][0, b:e]
    return out


def test_layer_13b_full_size():
    p = synthkv.PRESETS[3]
    say("full size: 13B-shaped layer, K and V as one 80-head tensor, 9 chunks")
    X = layer_on_device(p)
    oc = ocfg(p, "K")   # one codec seed for the layer; the draw is keyed per head
    dst = _encode_all(p, oc, X)
    assert _replay(p, oc, X, dst, heads=[7, 40 + 29], chunks=p.n_chunks) == 0
    # the whole cache decoded with the keys (heads 0-39) rotated by the latent
    # grid's 3-D position table, as the benchmark's rotated decode runs it
    say("  decode with the rotation of the 40 key heads, whole cache")
    q = lib()
    rope = synthkv.rope_table(p, 0, p.n_tokens)
    rope_d = torch.from_numpy(rope).to(DEV)
    y = q.decode(gcfg(oc), dst, 0, p.n_tokens, out_dtype="bf16", rope=rope_d, rope_heads=p.heads)
    torch.cuda.synchronize()
    for c in (0, 4, p.n_chunks - 1):
        b, e = p.chunk_range(c)
        g = fetch(dst, c, oc)
        for h in (0, 7, 39, 40, 69):
            ref = oracle.decode_chunk(g["codes"][h:h + 1], g["scales"][h:h + 1], g["assign"][:, h:h + 1],
                                      g["centroids"][:, h:h + 1], oc.group_size, "bf16",
                                      rope=rope[b:e] if h < p.heads else None)[0]
            np.testing.assert_array_equal(to_np(y[h, b:e]), ref)


@pytest.mark.parametrize("tensor", ["K", "V"])
def test_aggressive_full_24_heads(tensor):
    p = synthkv.PRESETS[4]
    say(f"full size: aggressive setting, {tensor}, 24 heads, 4 stages, G=16, 2 chunks")
    X = torch.cat(list(synthkv.gen_torch(p, tensor, DEV, frames_per_call=p.chunk_frames)), dim=1)
    oc = ocfg(p, tensor)
    dst = _encode_all(p, oc, X)
    assert _replay(p, oc, X, dst, heads=[0, 11, 23], chunks=p.n_chunks) == 0


def test_long_horizon_sampled_chunks():
    p = synthkv.PRESETS[5]
    say("full size: long-horizon cache, 24 heads x 1,092,000 tokens, 234 chunks")
    X = layer_on_device(p)
    oc = ocfg(p, "K")
    late = (117, p.n_chunks - 1)
    dst, saved = _encode_all(p, oc, X, export_before=late)
    heads = [3, 12 + 8]
    assert _replay(p, oc, X, dst, heads=heads, chunks=2) == 0
    q = lib()
    hx = _host_heads(X, heads)
    for c in late:
        b, e = p.chunk_range(c)
        g = fetch(dst, c, oc)
        y = to_np(q.decode(gcfg(oc), dst, b, e, out_dtype="bf16"))
        for h in heads:
            xs = _slice(hx, h, b, e, X.shape[0])
            check_chunk_properties(oc, xs, g, h, f"chunk {c}")
            # the whole chunk replayed by the oracle from the HIP path's own
            # streaming state: every Lloyd round (labels, exact means, empty
            # clusters), the stored tables, codes and scales must agree bit for bit
            say(f"  oracle replay of head {h}, chunk {c}, from the exported cache")
            ora = oracle.encode_chunk(hx[h][:, b:e], oc, cache=saved[c][:, h:h + 1], head_offset=h)
            assert check_chunk(oc, xs, g, ora, 0, h, f"chunk {c}") == 0
            ref = oracle.decode_chunk(g["codes"][h:h + 1], g["scales"][h:h + 1], g["assign"][:, h:h + 1],
                                      g["centroids"][:, h:h + 1], oc.group_size, "bf16")[0]
            np.testing.assert_array_equal(y[h], ref)
    # the whole cache decodes in one call; spot rows against the per-chunk decode
    full = q.decode(gcfg(oc), dst, 0, p.n_tokens, out_dtype="bf16")
    for c in (0, 117, p.n_chunks - 1):
        b, e = p.chunk_range(c)
        part = q.decode(gcfg(oc), dst, b, e, out_dtype="bf16")
        torch.testing.assert_close(full[:, b:e], part, rtol=0, atol=0)
