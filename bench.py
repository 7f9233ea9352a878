#!/usr/bin/env python3
"""Throughput of the QVG KV-cache codec hot path on one MI355X.

One step = the whole hot path over one 13B-video-model-shaped layer: K and V,
40 heads x 128 dims each, 38,000 tokens (about 5 s of 480p video) in 9 chunks
of 3 latent frames (the last one 560 tokens).  The layer's KV cache is one
[2][40][38000][128] buffer, so K and V form one 80-head tensor with a uniform
head stride: each chunk is encoded by one call through the streaming centroid
cache (first chunk cold: Forgy start, 10 Lloyd rounds; later chunks warm: 3
rounds; 256 centroids, 2 progressive stages, 2-bit codes in groups of 64 with
E4M3 scales), then one fused decode rebuilds the whole cache in bf16.  The
centroid cache is reset at the start of every step.

`value` is KV vectors encoded per second of step time (a vector = one head's
128-dim key or value row of one token; 3.04 M per step).  The inputs are
generated on the device before timing and stay resident in HBM.

Also reported on the same line: encode-only and warm-chunk rates, the fused
decode's algorithmic GB/s (timed with HIP events around each decode launch on
its stream), a per-kernel breakdown from the library's event profiler, the
roofline of the dominant kernel, the same decode with the 40 key heads
rotated by a 3-D rotary position table in the same pass (keys are cached
before the rotation) next to the rotation run as a separate pass, one step of
the aggressive setting (4 stages, groups of 16), the long-horizon decode stress (12 heads, 700 frames, 1.09 M tokens) and the CPU
oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix, TFLOP/s
METRIC = "KV tokens encoded/s (d=128, 256 centroids) + fused decode GB/s vs HBM peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--profile-steps", type=int, default=2,
                    help="extra steps run with the library's per-kernel event profiler")
    ap.add_argument("--stress-reps", type=int, default=20,
                    help="timed decodes of the 1.09M-token cache (0 skips the stress part)")
    ap.add_argument("--rope-reps", type=int, default=10,
                    help="timed decodes of the layer's cache with the key heads rotated (0 skips)")
    ap.add_argument("--aggressive-reps", type=int, default=5,
                    help="timed steps of the aggressive setting (4 stages, G=16; 0 skips)")
    ap.add_argument("--share-reps", type=int, default=5,
                    help="timed steps of one GPU's share of the layer when its heads are split over 8 GPUs "
                         "(5 key + 5 value heads; 0 skips)")
    ap.add_argument("--attn-reps", type=int, default=3,
                    help="timed attention calls over the long-horizon cache (0 skips)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-stage error, convergence, FP8-table and latency reports")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=2, help="heads of K and of V in the oracle's warm-chunk leg")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def hbm_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads
    for a copy kernel of known size), or None when the kernels' source has
    changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "hbm_traffic.json")
    src = os.path.join(root, "bit_vector_quantization_amd", "csrc", "qvg_kernels.hip")
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("kernels_source_sha256") != sha or not k:
        return None
    return round(k["fetch_bytes"] * rec["copy_scale"]["fetch"] + k["write_bytes"] * rec["copy_scale"]["write"])


def decode_bytes(H, ntok, d, G, T, K, chunks, out_bytes=2, cent_bytes=2):
    """Algorithmic HBM bytes of one fused decode: codes, scales, assignments and
    every touched chunk's centroid tables read once, the output written once."""
    return H * ntok * (d // 4 + d // G + T + d * out_bytes) + chunks * T * H * K * d * cent_bytes


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this codec shards by head with no exchange, "
              "so only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_vector_quantization_amd as q
    import synthkv

    assert torch.cuda.is_available(), "no GPU visible"
    dev = "cuda:0"
    p = synthkv.PRESETS[3]
    H, Ntot, d = p.heads, p.n_tokens, p.d
    K, T, G = p.n_centroids, p.n_stages, p.group_size
    stream = torch.cuda.current_stream()

    log("generating the layer's K and V on the device")
    # the layer's KV cache as one [2][H][N][d] buffer: K and V form one tensor of
    # 2H heads with a uniform head stride, encoded and decoded by single calls
    X = torch.empty((2, H, Ntot, d), dtype=torch.bfloat16, device=dev)
    for i, t in enumerate(("K", "V")):
        X[i] = torch.cat(list(synthkv.gen_torch(p, t, dev)), dim=1)
    X = X.view(2 * H, Ntot, d)
    torch.cuda.synchronize()
    HK = 2 * H
    cfg = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype)
    dst = q.CompressedKV(cfg, HK, Ntot, p.chunk_tokens, dev)
    cache = q.CentroidCache(cfg, HK)
    enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
    out = torch.empty((HK, Ntot, d), dtype=torch.bfloat16, device=dev)
    n_chunks = p.n_chunks

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step(marks):
        cache.reset()
        marks.append(("enc", -1, ev()))
        for c in range(n_chunks):
            b, e = p.chunk_range(c)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)
            marks.append(("enc", c, ev()))
        marks.append(("dec0", 0, ev()))
        q.decode(cfg, dst, 0, Ntot, out=out, stream=stream)
        marks.append(("dec1", 0, ev()))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step([])
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    all_marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m = []
        step(m)
        all_marks.append(m)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # event breakdown of the timed steps
    cold_ms = warm_ms = rag_ms = enc_ms = dec_ms = 0.0
    dec_launches = 0
    for m in all_marks:
        idx = {(k, c): e for k, c, e in m}
        prev = idx[("enc", -1)]
        for c in range(n_chunks):
            cur = idx[("enc", c)]
            dt = prev.elapsed_time(cur)
            b, e = p.chunk_range(c)
            if c == 0:
                cold_ms += dt
            elif e - b == p.chunk_tokens:
                warm_ms += dt
            else:
                rag_ms += dt
            enc_ms += dt
            prev = cur
        dec_ms += idx[("dec0", 0)].elapsed_time(idx[("dec1", 0)])
        dec_launches += 1
    S = args.steps
    vec_step = HK * Ntot
    n_warm = sum(1 for c in range(n_chunks) if p.chunk_range(c)[1] - p.chunk_range(c)[0] == p.chunk_tokens) - 1
    dec_b = decode_bytes(HK, Ntot, d, G, T, K, n_chunks)
    dec_avg_ms = dec_ms / dec_launches
    decode_gbs = dec_b / (dec_avg_ms * 1e-3) / 1e9

    # reference copy bandwidth on the same tensors (torch copy kernel)
    src, cpy = out, torch.empty_like(out)
    for _ in range(3):
        cpy.copy_(src)
    e0 = ev()
    for _ in range(10):
        cpy.copy_(src)
    e1 = ev()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 2 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9

    # the same whole-cache decode with the 40 key heads rotated by the latent
    # grid's 3-D position table in the same pass, and for comparison the
    # rotation as a separate pass of torch ops over the decoded keys
    rope_rec = None
    if args.rope_reps > 0:
        rope_rec = run_rope(q, synthkv, torch, p, cfg, dst, out, stream, ev, args.rope_reps, H, dec_b,
                            dec_avg_ms)

    # per-kernel breakdown with the library's event profiler
    kernels, raw_stats = {}, {}
    if args.profile_steps > 0:
        log(f"profiling {args.profile_steps} steps with per-launch events")
        q.qvg_profile_enable(True)
        t1 = time.perf_counter()
        for _ in range(args.profile_steps):
            step([])
        torch.cuda.synchronize()
        prof_ms_step = (time.perf_counter() - t1) * 1e3 / args.profile_steps
        q.qvg_profile_enable(False)
        raw = q.qvg_profile_read()
        raw_stats.update(raw)
        for name, r in raw.items():
            kernels[name] = dict(launches_per_step=r["launches"] / args.profile_steps,
                                 avg_us=round(r["avg_ms"] * 1e3, 3),
                                 ms_per_step=round(r["total_ms"] / args.profile_steps, 4),
                                 tflops=round(r["flops"] / (r["total_ms"] * 1e-3) / 1e12, 2) if r["flops"] else 0.0,
                                 gbs=round(r["bytes"] / (r["total_ms"] * 1e-3) / 1e9, 1))
    else:
        prof_ms_step = None

    # rooflines: assign against the bf16 matrix peak, update, quantiser and decode against HBM
    roofs = {}
    dec_roof = dict(kernel="decode", bound="hbm", achieved=round(decode_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(decode_gbs / HBM_PEAK_GBS, 4), traffic=hbm_traffic("decode"),
                    avg_launch_us=round(dec_avg_ms * 1e3, 2), algorithmic_per_launch=int(dec_b),
                    timed="HIP events around every decode launch of the timed steps, on its stream")
    roofs["decode"] = dec_roof
    if rope_rec is not None:
        roofs["decode_rope"] = rope_rec.pop("roofline")
    for name, key in (("assign", "assign"), ("update", "update"), ("residual_quant", "quant")):
        if name not in raw_stats:
            continue
        r = raw_stats[name]
        per = (r["flops"] if name == "assign" else r["bytes"]) / r["launches"]
        secs = r["total_ms"] * 1e-3 / r["launches"]
        if name == "assign":
            ach = per / secs / 1e12
            roofs[key] = dict(kernel=key, bound="mfma", achieved=round(ach, 2), peak=MFMA_BF16_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4))
        else:
            ach = per / secs / 1e9
            roofs[key] = dict(kernel=key, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(ach / HBM_PEAK_GBS, 4))
        roofs[key].update(traffic=hbm_traffic(key), avg_launch_us=round(secs * 1e6, 2),
                          algorithmic_per_launch=per,
                          timed="HIP events around every launch of the profiled steps, on the launch stream")
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"]) if kernels else "decode"
    roof = roofs.get(dom, dec_roof)

    # one GPU's share when the layer's 40 heads are split over 8 GPUs by head
    share = None
    if args.share_reps > 0:
        share = run_share(q, synthkv, torch, dev, stream, args.share_reps, H // 8)

    # the aggressive setting: 4 stages, groups of 16 (24 heads, 2 chunks)
    aggressive = None
    if args.aggressive_reps > 0:
        aggressive = run_aggressive(q, synthkv, torch, dev, stream, args.aggressive_reps)

    # long-horizon decode stress: 12 heads x 128, 700 frames (1,092,000 tokens)
    stress = attention = None
    if args.stress_reps > 0:
        stress, attention = run_stress(q, synthkv, torch, dev, stream, args.stress_reps, args.attn_reps)

    extras = {}
    if not args.no_extras:
        extras["stage_errors"] = run_stage_errors(q, synthkv, torch, dev, stream)
        extras["convergence"] = run_convergence(q, synthkv, torch, dev, stream, X, p, HK)
        extras["fp8_tables"] = run_fp8_tables(q, synthkv, torch, dev, stream, X, p, HK, out)
        extras["latency_single_head_chunk"] = run_latency(q, synthkv, torch, dev, stream)

    cpu = None if args.no_cpu_baseline else cpu_baseline(p, args.cpu_heads, ms_per_step, vec_step)

    line = {
        "metric": METRIC,
        "value": round(vec_step / (ms_per_step * 1e-3), 1),
        "unit": "KV vectors/s (vector = one head's 128-dim key or value row of one token)",
        "n_gpus": 1, "steps": S, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded spatio-temporally redundant KV, generated on the device)",
        "config": {"workload": "13B-shaped layer: K and V (one [2][40][38000][128] buffer, 80 heads x 128), "
                               "38,000 tokens in 9 chunks of 3 frames (last 560), streaming centroid cache, "
                               "then full-cache fused decode",
                   "heads": HK, "tokens": Ntot, "d": d, "centroids": K, "stages": T, "group_size": G,
                   "chunk_tokens": p.chunk_tokens, "iters_cold": p.iters_cold, "iters_warm": p.iters_warm},
        "tokens_per_s": round(Ntot / (ms_per_step * 1e-3), 1),
        "roofline": roof,
        "rooflines": roofs,
        "cpu_baseline": cpu,
        "encode": {"ms_per_step": round(enc_ms / S, 4),
                   "vectors_per_s": round(vec_step / (enc_ms / S * 1e-3), 1),
                   "warm_chunk_ms": round(warm_ms / (S * n_warm), 4),
                   "warm_vectors_per_s": round(HK * p.chunk_tokens / (warm_ms / (S * n_warm) * 1e-3), 1),
                   "cold_chunk_ms": round(cold_ms / S, 4),
                   "ragged_chunk_ms": round(rag_ms / S, 4)},
        "decode": {"launch_us": round(dec_avg_ms * 1e3, 2), "algorithmic_bytes": int(dec_b),
                   "gbs": round(decode_gbs, 1), "frac_hbm_peak": round(decode_gbs / HBM_PEAK_GBS, 4),
                   "copy_kernel_gbs": round(copy_gbs, 1)},
        "decode_rope": rope_rec,
        "aggressive": aggressive,
        "head_share_of_8": share,
        "decode_stress": stress,
        "attention": attention,
        **extras,
        "kernels": kernels,
        "profiled_ms_per_step": None if prof_ms_step is None else round(prof_ms_step, 4),
    }
    print(json.dumps(line), flush=True)


def run_rope(q, synthkv, torch, p, cfg, dst, out, stream, ev, reps, n_rot, dec_b, dec_avg_ms):
    Ntot, d = p.n_tokens, p.d
    rope = torch.from_numpy(synthkv.rope_table(p, 0, Ntot)).to(out.device)
    log(f"rotated decode: {reps} timed decodes of the whole cache, heads 0..{n_rot - 1} rotated")
    # before each timed launch a read of 1 GiB evicts the inputs from the
    # caches (L2 and the 256 MB last-level cache), as the encode's traffic does
    # before the step's decode
    flush = torch.empty(1 << 28, dtype=torch.float32, device=out.device).fill_(1.0)

    def timed(**kw):
        for _ in range(2):
            q.decode(cfg, dst, 0, Ntot, out=out, stream=stream, **kw)
        t = 0.0
        for _ in range(reps):
            flush.sum()
            e0 = ev()
            q.decode(cfg, dst, 0, Ntot, out=out, stream=stream, **kw)
            e1 = ev()
            torch.cuda.synchronize()
            t += e0.elapsed_time(e1)
        return t / reps

    ms = timed(rope=rope, rope_heads=n_rot)
    plain_ms = timed()   # the plain decode timed the same way
    del flush
    b = dec_b + Ntot * d * 4   # plus the table, read once
    gbs = b / (ms * 1e-3) / 1e9

    # unfused: the rotation as its own pass over the decoded bf16 keys
    c, s = rope[..., 0], rope[..., 1]

    def rotate():
        k = out[:n_rot].float().view(n_rot, Ntot, d // 2, 2)
        a, bb = k[..., 0], k[..., 1]
        out[:n_rot] = torch.stack((a * c - bb * s, a * s + bb * c), dim=-1).view(n_rot, Ntot, d).to(out.dtype)

    rotate()
    e0 = ev()
    for _ in range(3):
        rotate()
    e1 = ev()
    torch.cuda.synchronize()
    sep_ms = e0.elapsed_time(e1) / 3
    return {"launch_us": round(ms * 1e3, 2), "algorithmic_bytes": int(b), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "rotated_heads": n_rot,
            "plain_decode_us": round(plain_ms * 1e3, 2),
            "plain_decode_in_step_us": round(dec_avg_ms * 1e3, 2),
            "separate_rotation_pass_us": round(sep_ms * 1e3, 2),
            "table": "3-D (frame, row, col) rotary table of the 30x52 latent grid, fp32 (cos, sin) per pair",
            "roofline": dict(kernel="decode_rope", bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS,
                             unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4), traffic=hbm_traffic("decode_rope"),
                             avg_launch_us=round(ms * 1e3, 2), algorithmic_per_launch=int(b),
                             timed="HIP events around each rotated decode launch, on its stream")}


def run_share(q, synthkv, torch, dev, stream, reps, heads):
    """The bench step on one GPU's share of the 13B layer when its heads are
    split over 8 GPUs (the codec shards by head with no exchange): K and V of
    `heads` heads, the same 38,000 tokens, 9 chunks, cache, decode."""
    p = synthkv.PRESETS[3]
    Ntot, d = p.n_tokens, p.d
    HK = 2 * heads
    log(f"one GPU's share of 8: {HK} heads x {Ntot} tokens")
    X = torch.empty((2, heads, Ntot, d), dtype=torch.bfloat16, device=dev)
    for i, t in enumerate(("K", "V")):
        X[i] = torch.cat(list(synthkv.gen_torch(p, t, dev, heads=heads)), dim=1)
    X = X.view(HK, Ntot, d)
    cfg = q.config(d, p.n_centroids, p.n_stages, p.group_size, p.iters_cold, p.iters_warm, p.codec_seed("K"),
                   p.dtype)
    dst = q.CompressedKV(cfg, HK, Ntot, p.chunk_tokens, dev)
    cache = q.CentroidCache(cfg, HK)
    enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
    out = torch.empty((HK, Ntot, d), dtype=torch.bfloat16, device=dev)

    def step():
        cache.reset()
        for c in range(p.n_chunks):
            b, e = p.chunk_range(c)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)
        q.decode(cfg, dst, 0, Ntot, out=out, stream=stream)

    step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"workload": f"13B layer, K and V of {heads} heads ({HK} heads), 38,000 tokens in 9 chunks, then the "
                        "decode: one GPU's share when the 40 heads are split over 8 GPUs",
            "ms_per_step": round(ms, 4), "vectors_per_s": round(HK * Ntot / (ms * 1e-3), 1), "reps": reps}


def run_aggressive(q, synthkv, torch, dev, stream, reps):
    """One step of the aggressive setting: K and V of 24 heads as one 48-head
    tensor, 9,360 tokens in 2 chunks (cold, then warm), 4 stages, groups of
    16, then the decode of both chunks."""
    p = synthkv.PRESETS[4]
    H, Ntot, d, K, T, G = p.heads, p.n_tokens, p.d, p.n_centroids, p.n_stages, p.group_size
    HK = 2 * H
    log(f"aggressive setting: {HK} heads, {Ntot} tokens, T={T}, G={G}")
    X = torch.empty((2, H, Ntot, d), dtype=torch.bfloat16, device=dev)
    for i, t in enumerate(("K", "V")):
        X[i] = torch.cat(list(synthkv.gen_torch(p, t, dev, frames_per_call=p.chunk_frames)), dim=1)
    X = X.view(HK, Ntot, d)
    cfg = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype)
    dst = q.CompressedKV(cfg, HK, Ntot, p.chunk_tokens, dev)
    cache = q.CentroidCache(cfg, HK)
    enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
    out = torch.empty((HK, Ntot, d), dtype=torch.bfloat16, device=dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step():
        cache.reset()
        marks = [ev()]
        for c in range(p.n_chunks):
            b, e = p.chunk_range(c)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)
            marks.append(ev())
        q.decode(cfg, dst, 0, Ntot, out=out, stream=stream)
        marks.append(ev())
        return marks

    step()
    torch.cuda.synchronize()
    all_marks = [step() for _ in range(reps)]
    torch.cuda.synchronize()
    seg = [sum(m[i].elapsed_time(m[i + 1]) for m in all_marks) / reps for i in range(len(all_marks[0]) - 1)]
    ms = sum(seg)
    return {"workload": "aggressive setting: K and V of 24 heads x 128 as one 48-head tensor, 9,360 tokens in "
                        "2 chunks (cold, warm), 4 stages, 256 centroids, G=16, then the decode",
            "ms_per_step": round(ms, 4), "vectors_per_s": round(HK * Ntot / (ms * 1e-3), 1),
            "cold_chunk_ms": round(seg[0], 4), "warm_chunk_ms": round(seg[1], 4),
            "decode_us": round(seg[-1] * 1e3, 2), "reps": reps}


def run_stress(q, synthkv, torch, dev, stream, reps, attn_reps=0):
    p = synthkv.PRESETS[5]
    H, Ntot, d, K, T, G = p.heads, p.n_tokens, p.d, p.n_centroids, p.n_stages, p.group_size
    HK = 2 * H
    log(f"decode stress: generating and encoding {p.n_chunks} chunks of K+V ({Ntot} tokens, {HK} heads)")
    t0 = time.perf_counter()
    cfg = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype)
    dst = q.CompressedKV(cfg, HK, Ntot, p.chunk_tokens, dev)
    cache = q.CentroidCache(cfg, HK)
    enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
    gk = synthkv.gen_torch(p, "K", dev, frames_per_call=p.chunk_frames)
    gv = synthkv.gen_torch(p, "V", dev, frames_per_call=p.chunk_frames)
    for c, (xk, xv) in enumerate(zip(gk, gv)):
        enc.encode(torch.cat([xk, xv], dim=0), dst, c, cache=cache, stream=stream)
        if c % 50 == 0:
            torch.cuda.synchronize()
            log(f"  chunk {c}/{p.n_chunks}")
    torch.cuda.synchronize()
    del cache, enc
    out = torch.empty((HK, Ntot, d), dtype=torch.bfloat16, device=dev)
    total_b = decode_bytes(HK, Ntot, d, G, T, K, p.n_chunks)
    prep_s = time.perf_counter() - t0
    log(f"decode stress: {reps} timed decodes of the whole cache")
    for _ in range(2):
        q.decode(cfg, dst, 0, Ntot, out=out, stream=stream)
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        q.decode(cfg, dst, 0, Ntot, out=out, stream=stream)
        b.record(stream)
        times.append((a, b))
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in times) / reps
    gbs = total_b / (ms * 1e-3) / 1e9
    rec = {"workload": "K and V as one 24-head tensor, 128 dims, 700 frames of 30x52 (1,092,000 tokens, "
                       "234 chunks), 2 stages, 256 centroids, G=64; fused decode of the whole cache",
           "kv_decode_ms": round(ms, 4), "algorithmic_bytes": int(total_b), "gbs": round(gbs, 1),
           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "reps": reps, "setup_s": round(prep_s, 1)}
    attn = None
    if attn_reps > 0:
        attn = run_attention(q, torch, p, cfg, dst, out, stream, attn_reps)
    return rec, attn


def run_attention(q, torch, p, cfg, dst, out, stream, reps):
    """Attention of one chunk's queries (4,680 per head, 12 heads) over the whole
    long-horizon cache (1,092,000 keys), keys rotated by a rotary table, read
    straight from the compressed cache (qvg_attention), next to the unfused
    path: the rotated decode of K and decode of V to bf16, then PyTorch's
    scaled_dot_product_attention."""
    H, Ntot, d = p.heads, p.n_tokens, p.d
    Nq = p.chunk_tokens
    dev = out.device
    log(f"attention: {H} heads, {Nq} queries over {Ntot} compressed keys")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    qd = (torch.randn((H, Nq, d), generator=g, device=dev) * 0.1).to(torch.bfloat16)
    pos = torch.arange(Ntot, device=dev, dtype=torch.float32)[:, None]
    inv = torch.pow(10000.0, -torch.arange(d // 2, device=dev, dtype=torch.float32) / (d // 2))[None, :]
    ang = pos * inv
    rope = torch.stack((torch.cos(ang), torch.sin(ang)), dim=-1).contiguous()
    del pos, ang
    flops = 4.0 * H * Nq * Ntot * d

    def fused():
        return q.attention(cfg, dst, dst, qd, 0, Ntot, k_head0=0, v_head0=H, rope=rope, stream=stream)

    fused()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        o_f = fused()
        b.record(stream)
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b))
    ms = sorted(t)[len(t) // 2]
    tf = flops / (ms * 1e-3) / 1e12
    rec = {"workload": f"{H} heads, {Nq} queries (one chunk) over {Ntot} keys of the long-horizon cache, keys "
                       "rotated by a rotary table, K/V rebuilt in the kernel from the compressed cache",
           "fused_ms": round(ms, 3), "tflops": round(tf, 1), "reps": reps,
           "roofline": dict(kernel="attention", bound="mfma", achieved=round(tf, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                            unit="TFLOP/s", frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4), traffic=None,
                            avg_launch_ms=round(ms, 3), algorithmic_per_launch=flops,
                            timed="HIP events around each call (attention + split merge), on its stream")}
    # unfused: decode to bf16 (keys rotated), then scaled_dot_product_attention
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        import torch.nn.functional as F

        def unfused():
            q.decode(cfg, dst, 0, Ntot, out=out, stream=stream, rope=rope, rope_heads=H)
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                return F.scaled_dot_product_attention(qd[None], out[None, :H], out[None, H:])

        o_u = unfused()
        torch.cuda.synchronize()
        tu, td = [], []
        for _ in range(reps):
            a, m_, b = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record(stream)
            q.decode(cfg, dst, 0, Ntot, out=out, stream=stream, rope=rope, rope_heads=H)
            m_.record(stream)
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                o_u = F.scaled_dot_product_attention(qd[None], out[None, :H], out[None, H:])
            b.record(stream)
            torch.cuda.synchronize()
            tu.append(a.elapsed_time(b))
            td.append(a.elapsed_time(m_))
        rec.update(unfused_ms=round(sorted(tu)[len(tu) // 2], 3), unfused_decode_ms=round(sorted(td)[len(td) // 2], 3),
                   unfused_bf16_kv_bytes=int(2 * H * Ntot * d * 2),
                   max_abs_diff_vs_unfused=float((o_f - o_u[0].float()).abs().max()))
    except Exception as ex:   # no fused SDPA backend: report the fused path alone
        rec.update(unfused_ms=None, unfused_error=str(ex)[:200])
    del rope
    return rec


def run_stage_errors(q, synthkv, torch, dev, stream):
    """The aggressive setting's error per stage on the HIP path: the whole
    48-head tensor (K and V of 24 heads, 9,360 tokens in 2 chunks) encoded with
    T = 0..4 stages (T = 0 is single-shot round-to-nearest 2-bit with the same
    E4M3 group-16 scales), decoded in fp32; MSE over all elements in fp64, for
    K and V separately, and each stage's ratio MSE(t-1) / MSE(t)."""
    p = synthkv.PRESETS[4]
    H, Ntot, d, K, G = p.heads, p.n_tokens, p.d, p.n_centroids, p.group_size
    HK = 2 * H
    log(f"per-stage error: aggressive setting, T = 0..{p.n_stages}")
    X = torch.empty((2, H, Ntot, d), dtype=torch.bfloat16, device=dev)
    for i, t in enumerate(("K", "V")):
        X[i] = torch.cat(list(synthkv.gen_torch(p, t, dev, frames_per_call=p.chunk_frames)), dim=1)
    X = X.view(HK, Ntot, d)
    Xd = X.double()
    mse = {"K": [], "V": []}
    for T in range(0, p.n_stages + 1):
        cfg = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype)
        dst = q.CompressedKV(cfg, HK, Ntot, p.chunk_tokens, dev)
        cache = q.CentroidCache(cfg, HK) if T else None
        enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
        for c in range(p.n_chunks):
            b, e = p.chunk_range(c)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)
        y = q.decode(cfg, dst, 0, Ntot, out_dtype="f32", stream=stream)
        err = (y.double() - Xd).pow(2)
        mse["K"].append(float(err[:H].mean()))
        mse["V"].append(float(err[H:].mean()))
        del dst, cache, enc, y, err
    out = {}
    for t in ("K", "V"):
        m = mse[t]
        out[t] = {"mse": [float(f"{v:.6g}") for v in m],
                  "ratio_per_stage": [round(m[i - 1] / m[i], 3) for i in range(1, len(m))],
                  "total_vs_rtn": round(m[0] / m[-1], 2)}
    return {"workload": "aggressive setting: K and V of 24 heads x 128, 9,360 tokens in 2 chunks (cold, warm), "
                        "256 centroids, G=16, E4M3 scales; T = 0 is single-shot round-to-nearest 2-bit",
            "stages": list(range(0, p.n_stages + 1)), **out,
            "pages_context": "real-model KV: 5.83x, 1.39x, 1.15x for stages 1-3 (not this data)"}


def run_convergence(q, synthkv, torch, dev, stream, X, p, HK):
    """Rounds to convergence, cold vs warm, on the HIP path: the 13B layer's
    chunks encoded with the device-side stop (converge = 1: labels unchanged,
    exact; converge = 5: fewer than 0.1% of 4,680 tokens moved), at most 30
    rounds; per chunk the mean / max rounds over heads and stages, and the
    chunk time next to the fixed counts (10 cold, 3 warm)."""
    d, K, T, G = p.d, p.n_centroids, p.n_stages, p.group_size
    res = {}
    for conv in (1, 5):
        cfg = q.config(d, K, T, G, 30, 30, p.codec_seed("K"), p.dtype, conv)
        dst = q.CompressedKV(cfg, HK, p.n_tokens, p.chunk_tokens, dev)
        cache = q.CentroidCache(cfg, HK)
        enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
        log(f"convergence: converge={conv}, at most 30 rounds")
        chunks = []
        for c in range(p.n_chunks - 1):   # the full chunks
            b, e = p.chunk_range(c)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)
            e1.record(stream)
            r = enc.rounds(stream).float()
            torch.cuda.synchronize()
            chunks.append({"chunk": c, "start": "cold" if c == 0 else "warm",
                           "rounds_mean": round(float(r.mean()), 2), "rounds_max": int(r.max()),
                           "rounds_mean_K": round(float(r[:, :HK // 2].mean()), 2),
                           "rounds_mean_V": round(float(r[:, HK // 2:].mean()), 2),
                           "ms": round(e0.elapsed_time(e1), 3)})
        warm = [c["rounds_mean"] for c in chunks[1:]]
        res[f"converge_{conv}"] = {"chunks": chunks, "cold_rounds_mean": chunks[0]["rounds_mean"],
                                   "warm_rounds_mean": round(sum(warm) / len(warm), 2),
                                   "cold_over_warm": round(chunks[0]["rounds_mean"] / (sum(warm) / len(warm)), 2)}
    return res


def run_fp8_tables(q, synthkv, torch, dev, stream, X, p, HK, ref_out):
    """The bench step's encode and decode with the centroid tables stored in
    FP8 (E4M3 times a power of two per table): step time, decode bandwidth,
    reconstruction error next to bf16 tables, and the bytes."""
    d, K, T, G = p.d, p.n_centroids, p.n_stages, p.group_size
    cfg = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype, 0, "e4m3")
    dst = q.CompressedKV(cfg, HK, p.n_tokens, p.chunk_tokens, dev)
    cache = q.CentroidCache(cfg, HK)
    enc = q.Encoder(cfg, HK, p.chunk_tokens, dev)
    out = torch.empty_like(ref_out)
    log("FP8 centroid tables: encode + decode of the layer")

    def step():
        cache.reset()
        for c in range(p.n_chunks):
            b, e = p.chunk_range(c)
            enc.encode(X[:, b:e], dst, c, cache=cache, stream=stream)

    step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / 3
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    t = 0.0
    for _ in range(5):
        flush.sum()
        a = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        q.decode(cfg, dst, 0, p.n_tokens, out=out, stream=stream)
        b_.record(stream)
        torch.cuda.synchronize()
        t += a.elapsed_time(b_)
    dec_ms = t / 5
    del flush
    dec_b = HK * p.n_tokens * (d // 4 + d // G + T + 2 * d) + p.n_chunks * T * HK * (K * d + 16)
    H = HK // 2
    Xd = X.double()
    m8 = [float((out[s].double() - Xd[s]).pow(2).mean()) for s in (slice(0, H), slice(H, HK))]
    mb = [float((ref_out[s].double() - Xd[s]).pow(2).mean()) for s in (slice(0, H), slice(H, HK))]
    total = sum(q.qvg_cache_view_bytes(cfg, HK, p.n_tokens, p.chunk_tokens))
    cfg_n = q.config(d, K, T, G, p.iters_cold, p.iters_warm, p.codec_seed("K"), p.dtype)
    total_n = sum(q.qvg_cache_view_bytes(cfg_n, HK, p.n_tokens, p.chunk_tokens))
    raw = HK * p.n_tokens * d * 2
    return {"encode_ms_per_step": round(enc_ms, 4), "decode_us": round(dec_ms * 1e3, 2),
            "decode_algorithmic_bytes": int(dec_b), "decode_gbs": round(dec_b / (dec_ms * 1e-3) / 1e9, 1),
            "mse_K": float(f"{m8[0]:.6g}"), "mse_V": float(f"{m8[1]:.6g}"),
            "mse_K_bf16_tables": float(f"{mb[0]:.6g}"), "mse_V_bf16_tables": float(f"{mb[1]:.6g}"),
            "compressed_bytes": int(total), "compressed_bytes_bf16_tables": int(total_n),
            "ratio": round(raw / total, 3), "ratio_bf16_tables": round(raw / total_n, 3)}


def run_latency(q, synthkv, torch, dev, stream):
    """One chunk of one head's K and V (the single-head workload, 4,680 tokens,
    cold, 10 rounds, 2 stages): encode and decode latency."""
    p = synthkv.PRESETS[2]
    X = torch.cat([torch.from_numpy(synthkv.gen_numpy(p, t)) for t in ("K", "V")]).to(torch.bfloat16).to(dev)
    cfg = q.config(p.d, p.n_centroids, p.n_stages, p.group_size, p.iters_cold, p.iters_warm, p.codec_seed("K"),
                   p.dtype)
    dst = q.CompressedKV(cfg, 2, p.n_tokens, p.chunk_tokens, dev)
    enc = q.Encoder(cfg, 2, p.chunk_tokens, dev)
    out = torch.empty((2, p.n_tokens, p.d), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        enc.encode(X, dst, 0, stream=stream)
    torch.cuda.synchronize()
    te, td = [], []
    for _ in range(10):
        a, b_, c_ = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        enc.encode(X, dst, 0, stream=stream)
        b_.record(stream)
        q.decode(cfg, dst, 0, p.n_tokens, out=out, stream=stream)
        c_.record(stream)
        torch.cuda.synchronize()
        te.append(a.elapsed_time(b_))
        td.append(b_.elapsed_time(c_))
    te.sort()
    td.sort()
    return {"workload": "one head's K and V, one chunk of 4,680 tokens, cold (10 rounds), 2 stages",
            "encode_ms_median": round(te[5], 4), "decode_us_median": round(td[5] * 1e3, 2)}


def cpu_baseline(p, heads, gpu_ms_step, vec_step):
    """The oracle (NumPy, fp64) on the host cores, three legs, each the median of
    3 runs: a cold single-head chunk of K and V (the single-head workload:
    4,680 tokens, 10 rounds, 2 stages), a warm chunk of the 13B layer on
    `heads` key and `heads` value heads (3 rounds, from the previous chunk's
    centroids), and the decode of 10 chunks of the long-horizon cache on two
    heads.  Their per-vector times give the headline workload's step on the
    host (1 cold + 7 warm + 1 ragged chunk x 80 head-tensors + the full
    decode): a baseline, extrapolated and labeled so."""
    import platform

    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synthkv

    def ocfg(pr, t):
        return oracle.CodecConfig(d=pr.d, n_centroids=pr.n_centroids, n_stages=pr.n_stages,
                                  group_size=pr.group_size, iters_cold=pr.iters_cold, iters_warm=pr.iters_warm,
                                  seed=pr.codec_seed(t), dtype=pr.dtype)

    def median3(f):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    log("cpu baseline: oracle legs (median of 3 each)")
    p2 = synthkv.PRESETS[2]
    x2 = {t: synthkv.gen_numpy(p2, t) for t in ("K", "V")}
    cold_s = median3(lambda: [oracle.encode_chunk(x2[t], ocfg(p2, t)) for t in ("K", "V")])
    cold_vec = cold_s / (2 * p2.n_tokens)
    xs = {t: synthkv.gen_numpy(p, t, heads=heads, n_tokens=2 * p.chunk_tokens) for t in ("K", "V")}
    prev = {t: oracle.encode_chunk(xs[t][:, :p.chunk_tokens], ocfg(p, t)).cache for t in ("K", "V")}
    warm_s = median3(lambda: [oracle.encode_chunk(xs[t][:, p.chunk_tokens:], ocfg(p, t), cache=prev[t])
                              for t in ("K", "V")])
    warm_vec = warm_s / (2 * heads * p.chunk_tokens)
    p5 = synthkv.PRESETS[5]
    n10 = 10 * p5.chunk_tokens
    x5 = synthkv.gen_numpy(p5, "K", heads=2, n_tokens=n10)
    # the decode's time does not depend on how well k-means converged: one round
    oc5 = oracle.CodecConfig(**{**ocfg(p5, "K").__dict__, "iters_cold": 1})
    encs = [oracle.encode_chunk(x5[:, c * p5.chunk_tokens:(c + 1) * p5.chunk_tokens], oc5) for c in range(10)]
    dec_s = median3(lambda: [oracle.decode(e, p5.group_size, "bf16") for e in encs])
    dec_vec = dec_s / (2 * n10)
    rag = (p.n_tokens - (p.n_chunks - 1) * p.chunk_tokens) / p.chunk_tokens
    n_warm = p.n_chunks - 2
    hk = 2 * p.heads
    est = hk * p.chunk_tokens * (cold_vec + (n_warm + rag) * warm_vec) + hk * p.n_tokens * dec_vec
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas"})
    cpu_model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    dec_b_vec = (p5.d // 4 + p5.d // p5.group_size + p5.n_stages + 2 * p5.d
                 + p5.n_stages * p5.n_centroids * p5.d * 2 / p5.chunk_tokens)
    return {"value": round(vec_step / est, 1), "unit": "KV vectors/s", "cores": threads,
            "kind": "oracle",
            "sample": "three legs, median of 3 each: cold single-head chunk of K and V (4,680 tokens); warm "
                      f"13B-layer chunk on {heads} K + {heads} V heads; decode of 10 long-horizon chunks on 2 "
                      "heads; per-vector times extrapolated to one step of the headline workload",
            "legs": {"cold_chunk_KV_s": round(cold_s, 3), "cold_vectors_per_s": round(1 / cold_vec, 1),
                     "warm_chunk_s": round(warm_s, 3), "warm_vectors_per_s": round(1 / warm_vec, 1),
                     "decode_10_chunks_s": round(dec_s, 3), "decode_vectors_per_s": round(1 / dec_vec, 1),
                     "decode_gbs": round(dec_b_vec / dec_vec / 1e9, 3)},
            "est_step_s": round(est, 2), "gpu_speedup": round(est / (gpu_ms_step * 1e-3), 1),
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model, "blas": blas,
            "blas_threads": threads}


if __name__ == "__main__":
    main()
