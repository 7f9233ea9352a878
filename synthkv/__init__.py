"""Seeded synthetic key/value tensors with the statistics the Quant VideoGen pages
describe, plus the five workload presets used by the tests and the benchmark.

This module only produces *inputs*.  It holds none of the codec's arithmetic
(no clustering, no quantisation, no reconstruction): the CPU oracle under
``oracle/`` and the HIP library both consume what it makes, and neither is
imported here.

What the pages fix about the data (restated, not quoted):

* 163.com article, section 2 (video statistics): key magnitudes reach about
  1e2 and value magnitudes about 1e3, and which channel is an outlier changes
  from token to token.
* 163.com article, section 3, and gist.science (German) technical summary
  section 2A: tokens that are adjacent in space or in time have high cosine
  similarity in latent space.
* 163.com article, section 1: a 5 s 480p clip is about 38,000 latent tokens.

Recipe (per head, per tensor):

1. Spatial bases ``S_f`` for every frame: N(0, 1) on a ``[rows][cols][d]`` grid,
   blurred with a separable Gaussian over the two grid axes (sigma 1.5 tokens on
   the 8x8 grid, 3.0 on the 30x52 grid), then every channel of every frame is
   divided by its standard deviation.
2. Temporal AR(1): ``B_0 = S_0``, ``B_f = rho*B_{f-1} + sqrt(1-rho^2)*S_f`` with
   ``rho = 0.95``, so adjacent frames have cosine similarity of about 0.95.
3. Outliers: two fixed channels per head with fixed signs; the value there is
   replaced by ``sign * M * (1 + 0.1 z)``, ``M = 100`` for keys, ``1000`` for
   values.
4. With probability ``resample_p`` a token's two outlier channels are redrawn
   uniformly (distinct).
5. Additive N(0, 0.05^2) noise on every element.
6. Cast to fp32 or to bf16 (round to nearest even).

Tokens are ordered frame, then grid row, then grid column.  Keys (tau = 0) and
values (tau = 1) of preset ``c`` and head ``h`` draw from
``numpy.random.default_rng(SeedSequence([1000*c + tau, h]))``.

``gen_torch`` is the same recipe on a torch device with torch's own generator
(used where the host would be too slow, e.g. the 700-frame cache).  It does not
reproduce ``gen_numpy`` bit for bit; tests that need the oracle on such data
copy the sampled chunk back to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np

RHO = 0.95
NOISE_STD = 0.05
OUTLIER_SCALE = {"K": 100.0, "V": 1000.0}
N_OUTLIER = 2


@dataclasses.dataclass(frozen=True)
class Preset:
    """A workload: the tensor shapes, the generator knobs and the codec settings."""

    index: int
    name: str
    heads: int
    grid: Tuple[int, int]          # latent rows x cols per frame
    frames: int                    # latent frames generated
    n_tokens: int                  # tokens kept (frames*rows*cols, or fewer)
    d: int                         # head dimension
    dtype: str                     # "f32" or "bf16" (input and centroid storage)
    tensors: Tuple[str, ...]       # ("K",) or ("K", "V")
    sigma: float                   # spatial blur, in tokens
    resample_p: float              # per-token outlier-channel resampling
    n_centroids: int
    n_stages: int
    group_size: int
    iters_cold: int
    iters_warm: int
    chunk_frames: int = 3          # tokens per chunk = chunk_frames*rows*cols

    @property
    def frame_tokens(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def chunk_tokens(self) -> int:
        return min(self.chunk_frames * self.frame_tokens, self.n_tokens)

    @property
    def n_chunks(self) -> int:
        return -(-self.n_tokens // self.chunk_tokens)

    def chunk_range(self, c: int) -> Tuple[int, int]:
        b = c * self.chunk_tokens
        return b, min(b + self.chunk_tokens, self.n_tokens)

    def codec_seed(self, tensor: str) -> int:
        return 1000 * self.index + (0 if tensor == "K" else 1)


PRESETS = {
    1: Preset(1, "tiny sanity chunk, fp32, 1 head, 2 frames of 8x8, d=64",
              heads=1, grid=(8, 8), frames=2, n_tokens=128, d=64, dtype="f32",
              tensors=("K",), sigma=1.5, resample_p=0.0,
              n_centroids=16, n_stages=1, group_size=16, iters_cold=5, iters_warm=5,
              chunk_frames=2),
    2: Preset(2, "single-head K/V chunk, bf16, 3 frames of 30x52, d=128",
              heads=1, grid=(30, 52), frames=3, n_tokens=4680, d=128, dtype="bf16",
              tensors=("K", "V"), sigma=3.0, resample_p=0.01,
              n_centroids=256, n_stages=2, group_size=64, iters_cold=10, iters_warm=3),
    3: Preset(3, "13B-shaped layer, bf16, 40 heads x 128, 38,000 tokens",
              heads=40, grid=(30, 52), frames=25, n_tokens=38000, d=128, dtype="bf16",
              tensors=("K", "V"), sigma=3.0, resample_p=0.01,
              n_centroids=256, n_stages=2, group_size=64, iters_cold=10, iters_warm=3),
    4: Preset(4, "aggressive setting, bf16, 24 heads x 128, 6 frames (9,360 tokens)",
              heads=24, grid=(30, 52), frames=6, n_tokens=9360, d=128, dtype="bf16",
              tensors=("K", "V"), sigma=3.0, resample_p=0.01,
              n_centroids=256, n_stages=4, group_size=16, iters_cold=10, iters_warm=3),
    5: Preset(5, "long-horizon decode stress, bf16, 12 heads x 128, 700 frames",
              heads=12, grid=(30, 52), frames=700, n_tokens=1092000, d=128, dtype="bf16",
              tensors=("K", "V"), sigma=3.0, resample_p=0.01,
              n_centroids=256, n_stages=2, group_size=64, iters_cold=10, iters_warm=3),
}


def _gauss_taps(sigma: float) -> np.ndarray:
    r = int(4.0 * sigma + 0.5)
    x = np.arange(-r, r + 1, dtype=np.float64)
    w = np.exp(-0.5 * (x / sigma) ** 2)
    return w / w.sum()


def _round_bf16(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _head_numpy(p: Preset, tensor: str, h: int, n_tokens: int,
                frame_begin: int = 0) -> np.ndarray:
    """One head, tokens ``[frame_begin*frame_tokens, +n_tokens)``, float32 ``[N][d]``.

    Every draw is made frame by frame, so a shorter run is a prefix of a longer
    one and a window is a slice of the full tensor."""
    from scipy.ndimage import gaussian_filter

    tau = 0 if tensor == "K" else 1
    rng = np.random.default_rng(np.random.SeedSequence([1000 * p.index + tau, h]))
    d = p.d
    rows, cols = p.grid
    ft = p.frame_tokens
    ch = rng.choice(d, size=N_OUTLIER, replace=False)
    sign = rng.choice(np.array([-1.0, 1.0]), size=N_OUTLIER)
    M = OUTLIER_SCALE[tensor]
    f_end = frame_begin + -(-n_tokens // ft)
    B = None
    out = []
    for f in range(f_end):
        S = rng.standard_normal((rows, cols, d))
        z = rng.standard_normal((ft, N_OUTLIER))
        res = rng.random(ft) < p.resample_p
        c1 = rng.integers(0, d, size=ft)
        c2 = (c1 + 1 + rng.integers(0, d - 1, size=ft)) % d
        noise = rng.standard_normal((ft, d))
        S = gaussian_filter(S, sigma=(p.sigma, p.sigma, 0.0), mode="reflect", truncate=4.0)
        S /= S.reshape(-1, d).std(axis=0)
        B = S if B is None else RHO * B + math.sqrt(1.0 - RHO * RHO) * S
        if f < frame_begin:
            continue
        X = B.reshape(ft, d).copy()
        idx = np.arange(ft)
        X[idx, np.where(res, c1, ch[0])] = sign[0] * M * (1.0 + 0.1 * z[:, 0])
        X[idx, np.where(res, c2, ch[1])] = sign[1] * M * (1.0 + 0.1 * z[:, 1])
        out.append(X + NOISE_STD * noise)
    X = np.concatenate(out, axis=0)[:n_tokens].astype(np.float32)
    if p.dtype == "bf16":
        X = _round_bf16(X)
    return X


def gen_numpy(p: Preset, tensor: str, n_tokens: Optional[int] = None,
              heads: Optional[int] = None, frame_begin: int = 0) -> np.ndarray:
    """Host tensor ``[H][N][d]`` float32 (bf16-representable values for bf16 presets)."""
    n = p.n_tokens if n_tokens is None else n_tokens
    H = p.heads if heads is None else heads
    return np.stack([_head_numpy(p, tensor, h, n, frame_begin) for h in range(H)])


def gen_torch(p: Preset, tensor: str, device, n_tokens: Optional[int] = None,
              heads: Optional[int] = None, frames_per_call: int = 3, seed_offset: int = 0):
    """Same recipe on a torch device; yields ``[H][n][d]`` blocks of
    ``frames_per_call`` frames (the last block may be shorter), in the preset's dtype."""
    import torch
    import torch.nn.functional as F

    n = p.n_tokens if n_tokens is None else n_tokens
    H = p.heads if heads is None else heads
    tau = 0 if tensor == "K" else 1
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (1000 * p.index + tau) + seed_offset)
    d = p.d
    rows, cols = p.grid
    taps = torch.tensor(_gauss_taps(p.sigma), dtype=torch.float32, device=device)
    r = (taps.numel() - 1) // 2
    ch = torch.stack([torch.randperm(d, generator=g, device=device)[:N_OUTLIER] for _ in range(H)])
    sign = torch.randint(0, 2, (H, N_OUTLIER), generator=g, device=device).float() * 2 - 1
    M = OUTLIER_SCALE[tensor]
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32

    def blur(S):  # S [H*F][d][rows][cols]
        S = F.pad(S, (r, r, 0, 0), mode="reflect")
        S = F.conv2d(S.reshape(-1, 1, rows, cols + 2 * r), taps.view(1, 1, 1, -1))
        S = S.reshape(-1, d, rows, cols)
        S = F.pad(S, (0, 0, r, r), mode="reflect")
        S = F.conv2d(S.reshape(-1, 1, rows + 2 * r, cols), taps.view(1, 1, -1, 1))
        return S.reshape(-1, d, rows, cols)

    B = None
    done = 0
    n_frames = -(-n // p.frame_tokens)
    f = 0
    while f < n_frames:
        nf = min(frames_per_call, n_frames - f)
        S = torch.randn((H * nf, d, rows, cols), generator=g, device=device)
        S = blur(S)
        S = S / S.std(dim=(2, 3), keepdim=True)
        S = S.reshape(H, nf, d, rows * cols).permute(0, 1, 3, 2)  # [H][nf][tok][d]
        frames = []
        for i in range(nf):
            B = S[:, i] if B is None else RHO * B + math.sqrt(1 - RHO * RHO) * S[:, i]
            frames.append(B)
        X = torch.cat(frames, dim=1)  # [H][nf*ft][d]
        take = min(X.shape[1], n - done)
        X = X[:, :take].contiguous()
        z = torch.randn((H, take, N_OUTLIER), generator=g, device=device)
        res = torch.rand((H, take), generator=g, device=device) < p.resample_p
        c1 = torch.randint(0, d, (H, take), generator=g, device=device)
        c2 = (c1 + 1 + torch.randint(0, d - 1, (H, take), generator=g, device=device)) % d
        cha = torch.where(res, c1, ch[:, :1].expand(H, take))
        chb = torch.where(res, c2, ch[:, 1:2].expand(H, take))
        va = sign[:, :1] * M * (1 + 0.1 * z[..., 0])
        vb = sign[:, 1:2] * M * (1 + 0.1 * z[..., 1])
        X.scatter_(2, cha.unsqueeze(-1), va.unsqueeze(-1))
        X.scatter_(2, chb.unsqueeze(-1), vb.unsqueeze(-1))
        X += NOISE_STD * torch.randn(X.shape, generator=g, device=device)
        yield X.to(dt)
        done += take
        f += nf


def rope_axis_pairs(d: int) -> Tuple[int, int, int]:
    """How the d/2 rotation pairs of a head split over the three latent axes
    (frame, grid row, grid column): the rows and columns get 2*(d//6) channels
    each and the frames the rest (22/21/21 pairs at d = 128)."""
    hw = 2 * (d // 6)
    return (d - 2 * hw) // 2, hw // 2, hw // 2


def rope_table(p: Preset, tok_begin: int, tok_end: int, base: float = 10000.0) -> np.ndarray:
    """Per-token rotation table ``[tok_end - tok_begin][d/2][2]`` float32 of
    (cos, sin) for a 3-D rotary position scheme over the preset's latent grid.

    Token n sits at (frame, row, col) in the token order above.  Pair i of the
    axis group with g pairs turns by ``position * base**(-i / g)`` radians; the
    angle, cos and sin are taken in float64 and rounded to float32 once.  This
    is an input of the decode (the model's position encoding), not part of the
    codec."""
    n = np.arange(tok_begin, tok_end, dtype=np.int64)
    rows, cols = p.grid
    pos = (n // (rows * cols), (n // cols) % rows, n % cols)
    ang = []
    for a, g in enumerate(rope_axis_pairs(p.d)):
        inv = base ** (-np.arange(g, dtype=np.float64) / g)
        ang.append(pos[a].astype(np.float64)[:, None] * inv[None, :])
    ang = np.concatenate(ang, axis=1)
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
