"""Plain CPU reference of the Quant VideoGen (QVG) KV-cache codec.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the HIP library never calls it
and shares no code with it.

Every step follows the pages' description of the method, one head and one
chunk at a time, in float64 unless the format fixes the precision:

* Semantic-aware smoothing (163.com article, section 3; gist.science German
  summary, section 2A; Portuguese summary, section 2A): cluster the token
  vectors of a block with k-means, take each group's mean as its centroid,
  subtract it and quantise the residual.
* Progressive residual quantisation (163.com article, section 4; German
  summary, section 2B): R(0) = X; stage t applies the smoothing to R(t-1) and
  yields R(t), C(t) and the assignment pi(t); the final residual R(T) is
  quantised.  Reconstruction starts from the dequantised R(T) and adds back the
  stored centroids stage by stage.
* Streaming centroid cache (163.com article, section 5; German summary,
  section 2C): the previous chunk's centroids start the next chunk's k-means.
* Storage format (163.com article, section 5, implementation details, and
  section 6 for INT2; section 7 for group sizes 16/64 and 256 centroids held as
  uint8): 2-bit codes, FP8 E4M3 per-group scales, uint8 assignments.

Readings taken where the pages are silent (each is also used by the HIP path):

* k-means runs per head over the d-dim rows of one chunk; a cold start draws
  Forgy rows from a seeded SplitMix64 shuffle (``oracle.rng``); a fixed number
  of Lloyd iterations is run, then one final assignment; ties go to the lowest
  centroid index; an empty cluster keeps its previous centroid.
* Distances ``|c|^2 - 2<x, c>`` use operands rounded to bf16 ("parity" mode);
  the centroid update averages the unrounded rows: their exact sum rounded to
  float64, divided by the count in float64, rounded to float32.
* Centroids are stored in the input's precision (bf16 for bf16 tensors, fp32
  for fp32); the residual is taken against the stored centroids, in fp32.
* Quantiser: contiguous groups of G channels within a token row; scale
  s = E4M3(fp32(max|r| / 1.5)) saturating at 448; four levels (q - 1.5) * s,
  q = [r >= -s] + [r >= 0] + [r >= s]; four codes per byte, first channel in
  the low bits.
* Decode: y = (q - 1.5) * s, then y += C(t)[pi(t)] for t = T .. 1 in fp32,
  then round to the output type.
* Keys are cached before the rotary position embedding (163.com article,
  section 5, implementation details), so a decode may rotate them.  The pages
  do not fix the rotation's layout; pair p is channels (2p, 2p + 1), rotated
  by the caller's (cos, sin) for that token and pair, each product and sum
  rounded to fp32, before the one rounding to the output type.

"exact" mode drops the bf16 operand rounding and the float32 rounding of the
centroids; it exists for the textbook pins (SciPy's k-means) only.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

from .formats import bf16_round, e4m3_decode, e4m3_encode
from .rng import forgy_indices

F32 = np.float32


@dataclasses.dataclass(frozen=True)
class CodecConfig:
    d: int
    n_centroids: int
    n_stages: int
    group_size: int
    iters_cold: int
    iters_warm: int
    seed: int
    dtype: str = "bf16"        # "bf16" or "f32": input values and centroid storage
    converge: int = 0          # 0: fixed round counts; c >= 1: stop once a round moves fewer than c tokens
    centroid_format: str = "native"   # "native": stored in dtype; "e4m3": FP8 E4M3 times 2^e per table
    scale_mode: str = "e4m3"   # "e4m3": group scales saturate at 448; "two_level": 2^f per (chunk, head) x E4M3


# --------------------------------------------------------------------------
# k-means (semantic-aware smoothing)
# --------------------------------------------------------------------------

def _exact_distance(x: np.ndarray, c: np.ndarray) -> float:
    """|c|^2 - 2<x, c> rounded once from the exact value (every term is an
    exact float64 product of two bf16/fp32 numbers; math.fsum sums exactly)."""
    terms = list(c * c) + list(-2.0 * x * c)
    return math.fsum(terms)


def assign(R: np.ndarray, C: np.ndarray, mode: str = "parity") -> np.ndarray:
    """Index of the nearest centroid for every row of R (lowest index on ties).

    D[n, k] = |c_k|^2 - 2 <x_n, c_k>; the |x_n|^2 term is the same for every k
    and is left out.  Rows whose two best distances are within float64 noise
    are re-decided on exactly rounded distances."""
    if mode == "parity":
        xb, cb = bf16_round(R), bf16_round(C)
    else:
        xb, cb = np.asarray(R, np.float64), np.asarray(C, np.float64)
    cn = (cb * cb).sum(axis=1)
    D = cn[None, :] - 2.0 * (xb @ cb.T)
    best = D.min(axis=1)
    scale = (xb * xb).sum(axis=1) + cn.max()
    tol = 1e-12 * scale + 1e-300
    lab = np.argmin(D, axis=1)
    near = ((D <= (best + tol)[:, None]).sum(axis=1) > 1).nonzero()[0]
    for n in near:
        cand = np.nonzero(D[n] <= best[n] + tol[n])[0]
        ex = [_exact_distance(xb[n], cb[k]) for k in cand]
        m = min(ex)
        lab[n] = cand[ex.index(m)]       # cand is ascending: lowest index wins
    return lab


def exact_column_sums(rows: np.ndarray) -> np.ndarray:
    """Sum of each column, computed exactly and rounded once to float64
    (math.fsum is exactly rounded), so the result does not depend on order."""
    return np.array([math.fsum(rows[:, j]) for j in range(rows.shape[1])], dtype=np.float64)


def update(R: np.ndarray, lab: np.ndarray, C_prev: np.ndarray,
           mode: str = "parity") -> Tuple[np.ndarray, np.ndarray]:
    """New centroid = mean of the rows assigned to it; an empty cluster keeps
    its previous centroid.  The sum of the rows is exact (rounded once to
    float64), divided by the count in float64 and, in parity mode, rounded once
    more to float32.  Returns (centroids, counts)."""
    R = np.asarray(R, np.float64)
    K = C_prev.shape[0]
    C = np.array(C_prev, dtype=np.float64, copy=True)
    counts = np.bincount(lab, minlength=K)
    order = np.argsort(lab, kind="stable")
    starts = np.concatenate([[0], np.cumsum(counts)])
    for k in range(K):
        if counts[k] == 0:
            continue
        rows = R[order[starts[k]:starts[k + 1]]]
        mean = exact_column_sums(rows) / counts[k]
        C[k] = mean.astype(F32) if mode == "parity" else mean
    return C, counts


def lloyd(R: np.ndarray, C0: np.ndarray, iters: int, mode: str = "parity", converge: int = 0,
          labels_history: Optional[list] = None):
    """`iters` rounds of (assign, update) then one final assign.
    Returns (centroids, labels, sse_history) where sse_history[i] is the
    sum of squared distances after update i (float64, unrounded rows); its
    length is the number of updates run.

    converge = c >= 1 turns the round count into a maximum: the rounds stop
    at the first assignment (after the first round) that moves fewer than c
    tokens to another centroid than the round before, without running that
    round's update.  This is the plain reading of the pages' statement that
    k-means needs fewer rounds once it starts from the previous chunk's
    centroids (163.com article, section 5; German summary, section 2C):
    Lloyd's method is run until its labels settle.  With c = 1 the stop is exact: the same
    labels give the same centroids, so every later round would repeat them
    and the result equals that of any larger fixed count.  labels_history
    (a list) receives every round's assignment, the final one excluded."""
    C = np.array(C0, dtype=np.float64, copy=True)
    if mode == "parity":
        C = C.astype(F32).astype(np.float64)
    hist = []
    prev = None
    for _ in range(iters):
        lab = assign(R, C, mode)
        if labels_history is not None:
            labels_history.append(lab)
        if converge and prev is not None and int((lab != prev).sum()) < converge:
            break
        C, _ = update(R, lab, C, mode)
        hist.append(float(((np.asarray(R, np.float64) - C[lab]) ** 2).sum()))
        prev = lab
    lab = assign(R, C, mode)
    return C, lab, hist


# --------------------------------------------------------------------------
# centroid storage in FP8
# --------------------------------------------------------------------------
#
# A variant of the storage format: the pages count the centroids as a minor
# share of the compressed cache next to the 2-bit values (163.com article,
# section 6) and store the scales in FP8 E4M3 (section 5); storing the
# centroid tables in the same FP8 format halves their bytes.  Reading: one
# power-of-two factor 2^e per stored table (chunk, stage, head), the smallest
# that keeps the table's largest magnitude within E4M3's 448, and every value
# rounded to the nearest E4M3 value of v / 2^e (ties to even).  A power of two
# keeps the scaling exact, so every stored value is an E4M3 value times 2^e,
# which bf16 and fp32 hold exactly.

E4M3_TABLE_HEADER = 16   # bytes in front of each stored FP8 table: its exponent e (int32) and padding


def e4m3_table_exponent(C: np.ndarray) -> int:
    """Smallest integer e with max|C| <= 448 * 2^e (0 for an all-zero table)."""
    amax = float(np.max(np.abs(np.asarray(C, np.float64))))
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 9                  # a first guess, then exact comparisons
    while amax > math.ldexp(448.0, e):
        e += 1
    while amax <= math.ldexp(448.0, e - 1):
        e -= 1
    return e


def store_e4m3(C: np.ndarray):
    """(e, codes, values) of one centroid table stored in FP8: codes are the
    E4M3FN bytes of C / 2^e, values their decoded magnitudes times 2^e."""
    e = e4m3_table_exponent(C)
    codes = e4m3_encode(np.ldexp(np.asarray(C, np.float64), -e))
    return e, codes, np.ldexp(e4m3_decode(codes), e)


# --------------------------------------------------------------------------
# 2-bit group quantisation and its inverse
# --------------------------------------------------------------------------

def group_quant(R32: np.ndarray, G: int, f: int = 0):
    """Quantise rows of fp32 values in groups of G channels.

    f >= 0 is the second-level exponent of the two-level scale: the group's
    scale is stored as the E4M3FN code of fp32(a / 1.5) / 2^f and worth its
    value times 2^f (f = 0: the plain E4M3 scale).
    Returns (q [N][d] in {0..3}, packed [N][d/4] uint8, scale codes [N][d/G]
    uint8 E4M3FN)."""
    R32 = np.asarray(R32, dtype=F32)
    N, d = R32.shape
    g = R32.reshape(N, d // G, G)
    a = np.abs(g).max(axis=2)                         # float32
    s_code = e4m3_encode(np.ldexp((a / F32(1.5)).astype(np.float64), -f))   # fp32 division, exact 2^-f, E4M3
    s = np.ldexp(e4m3_decode(s_code), f).astype(F32)[:, :, None]
    q = (g >= -s).astype(np.uint8) + (g >= 0) + (g >= s)
    q = q.reshape(N, d).astype(np.uint8)
    packed = pack2(q)
    return q, packed, s_code


def pack2(q: np.ndarray) -> np.ndarray:
    """Four 2-bit codes per byte, the lowest channel in the lowest bits."""
    q = np.asarray(q, dtype=np.uint8)
    N, d = q.shape
    b = q.reshape(N, d // 4, 4)
    return (b[..., 0] | (b[..., 1] << 2) | (b[..., 2] << 4) | (b[..., 3] << 6)).astype(np.uint8)


def unpack2(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    N, nb = p.shape
    out = np.empty((N, nb, 4), dtype=np.uint8)
    for j in range(4):
        out[..., j] = (p >> (2 * j)) & 3
    return out.reshape(N, nb * 4)


def two_level_exponent(R32: np.ndarray) -> int:
    """Second-level exponent f of one chunk of one head: the smallest f >= 0
    with fp32(max|r| / 1.5) <= 448 * 2^f, so that no group's scale saturates.
    The pages store the group scales in E4M3, whose largest value (448) is
    below what value outliers near 1e3 need (163.com article, sections 2 and
    5); a power of two per chunk and head extends the range exactly."""
    amax15 = float(np.float32(np.abs(np.asarray(R32, F32)).max()) / F32(1.5))
    f = 0
    while amax15 > math.ldexp(448.0, f):
        f += 1
    return f


def dequant(packed: np.ndarray, s_code: np.ndarray, G: int, f: int = 0) -> np.ndarray:
    """(q - 1.5) * s in float32 (the product is exact); s = E4M3 value x 2^f."""
    q = unpack2(packed).astype(F32)
    N, d = q.shape
    s = np.ldexp(e4m3_decode(s_code), f).astype(F32)
    return ((q.reshape(N, d // G, G) - F32(1.5)) * s[:, :, None]).reshape(N, d)


# --------------------------------------------------------------------------
# Encode / decode of one chunk (all heads)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Encoded:
    codes: np.ndarray        # [H][N][d/4] uint8
    scales: np.ndarray       # [H][N][d/G] uint8 (E4M3FN)
    assign: np.ndarray       # [T][H][N] uint8
    centroids: np.ndarray    # [T][H][K][d] float32 (stored values)
    cache: np.ndarray        # [T][H][K][d] float32 (unrounded, for the next chunk)
    residuals: Optional[List[np.ndarray]] = None   # R(0..T), each [H][N][d]
    sse: Optional[List[List[List[float]]]] = None  # [t][h] -> per-iteration SSE
    rounds: Optional[np.ndarray] = None            # [T][H] Lloyd updates run
    cent_exp: Optional[np.ndarray] = None          # [T][H] table exponents (FP8 centroid storage)
    scale_exp: Optional[np.ndarray] = None         # [H] second-level scale exponents (two-level scales)


def _store(C: np.ndarray, dtype: str, fmt: str = "native") -> np.ndarray:
    if fmt == "e4m3":
        return store_e4m3(C)[2].astype(F32)
    return (bf16_round(C) if dtype == "bf16" else np.asarray(C, np.float64)).astype(F32)


def encode_chunk(X: np.ndarray, cfg: CodecConfig, cache: Optional[np.ndarray] = None,
                 init: Optional[np.ndarray] = None, mode: str = "parity",
                 keep_residuals: bool = False, iters: Optional[int] = None,
                 head_offset: int = 0) -> Encoded:
    """Encode one chunk X [H][N][d] (float32 array holding the input values).

    cache: [T][H][K][d] float32 centroids of the previous chunk (warm start,
    iters_warm rounds) or None (cold start: Forgy rows, iters_cold rounds).
    init: explicit starting centroids [T][H][K][d], used like a cache.
    iters: overrides the round count (tests).
    head_offset: global index of X's first head (it keys the cold-start draw)."""
    X = np.asarray(X, dtype=F32)
    H, N, d = X.shape
    K, T, G = cfg.n_centroids, cfg.n_stages, cfg.group_size
    start = init if init is not None else cache
    n_it = iters if iters is not None else (cfg.iters_warm if start is not None else cfg.iters_cold)
    codes = np.zeros((H, N, d // 4), np.uint8)
    scales = np.zeros((H, N, d // G), np.uint8)
    asg = np.zeros((T, H, N), np.uint8)
    cdt = F32 if mode == "parity" else np.float64
    cent = np.zeros((T, H, K, d), cdt)
    new_cache = np.zeros((T, H, K, d), cdt)
    residuals = [X.astype(np.float64)] if keep_residuals else None
    sse = [[None] * H for _ in range(T)]
    rounds = np.zeros((T, H), np.int32)
    fp8 = cfg.centroid_format == "e4m3"
    cexp = np.zeros((T, H), np.int32) if fp8 else None
    two = cfg.scale_mode == "two_level"
    sexp = np.zeros(H, np.int32) if two else None
    Rall = X.astype(np.float64)
    for h in range(H):
        R = Rall[h]
        for t in range(1, T + 1):
            if start is not None:
                C0 = np.asarray(start[t - 1, h], np.float64)
            else:
                C0 = R[forgy_indices(N, K, cfg.seed, head_offset + h, t)]
            C, lab, hist = lloyd(R, C0, n_it, mode, converge=cfg.converge)
            sse[t - 1][h] = hist
            rounds[t - 1, h] = len(hist)
            Cs = _store(C, cfg.dtype, cfg.centroid_format) if mode == "parity" else C
            if fp8:
                # the stage's labels are nearest under the centroids as stored
                cexp[t - 1, h] = e4m3_table_exponent(C)
                lab = assign(R, Cs.astype(np.float64), mode)
            asg[t - 1, h] = lab.astype(np.uint8)
            cent[t - 1, h] = Cs
            new_cache[t - 1, h] = C.astype(F32) if mode == "parity" else C
            R = R - Cs.astype(np.float64)[lab]
            if mode == "parity":
                R = R.astype(F32).astype(np.float64)
            if keep_residuals:
                if len(residuals) <= t:
                    residuals.append(np.zeros_like(Rall))
                residuals[t][h] = R
        f = two_level_exponent(R) if two else 0
        if two:
            sexp[h] = f
        _, packed, s_code = group_quant(R.astype(F32), G, f)
        codes[h] = packed
        scales[h] = s_code
    return Encoded(codes, scales, asg, cent, new_cache, residuals, sse, rounds, cexp, sexp)


def rope_rotate(y: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rotary position embedding of fp32 rows y [..., N, d] by table [N][d/2][2]
    of (cos, sin): channels (2p, 2p + 1) = (a, b) become (a cos - b sin,
    a sin + b cos).  numpy's float32 arithmetic rounds every product and every
    sum on its own, which is the rounding the reading above fixes."""
    y = np.asarray(y, dtype=F32)
    table = np.asarray(table, dtype=F32)
    a, b = y[..., 0::2], y[..., 1::2]
    c, s = table[..., 0], table[..., 1]
    out = np.empty_like(y)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def decode_chunk(codes: np.ndarray, scales: np.ndarray, asg: np.ndarray,
                 cent: np.ndarray, G: int, out: str = "f32",
                 rope: Optional[np.ndarray] = None, rope_heads: Optional[int] = None,
                 scale_exp: Optional[np.ndarray] = None) -> np.ndarray:
    """Rebuild [H][N][d] from one chunk's stored encoding.

    out="f32": fp32 sums in the order dequant + C(T) + ... + C(1);
    out="bf16": the same, rounded to bf16 (returned as float32 values);
    out="f64": the exact float64 sum (for error bounds).
    rope: [N][d/2][2] (cos, sin) that rotates heads [0, rope_heads) (all heads
    when rope_heads is None) after the fp32 sums and before the rounding to the
    output type (f32 and bf16 only).  scale_exp: [H] second-level exponents
    of two-level scales (None: plain E4M3 scales)."""
    H, N, _ = codes.shape
    T = asg.shape[0]
    nrot = 0 if rope is None else (H if rope_heads is None else rope_heads)
    ys = []
    for h in range(H):
        y = dequant(codes[h], scales[h], G, 0 if scale_exp is None else int(scale_exp[h]))
        if out == "f64":
            assert rope is None
            y = y.astype(np.float64)
            for t in range(T - 1, -1, -1):
                y = y + cent[t, h].astype(np.float64)[asg[t, h]]
        else:
            for t in range(T - 1, -1, -1):
                y = (y + cent[t, h][asg[t, h]]).astype(F32)
            if h < nrot:
                y = rope_rotate(y, rope)
            if out == "bf16":
                y = bf16_round(y).astype(F32)
        ys.append(y)
    return np.stack(ys)


def decode(enc: Encoded, G: int, out: str = "f32") -> np.ndarray:
    return decode_chunk(enc.codes, enc.scales, enc.assign, enc.centroids, G, out, scale_exp=enc.scale_exp)


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale Q K^T) V per head, in float64, and the natural log of each
    query's softmax denominator.  Q [H][Nq][d], K and V [H][Nk][d] -> (O
    [H][Nq][d], lse [H][Nq]).  The scores are shifted by their row maximum
    before exponentiation, which leaves the result unchanged."""
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S = scale * np.einsum("hqd,hkd->hqk", Q, K)
    m = S.max(axis=2, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(axis=2, keepdims=True)
    return np.einsum("hqk,hkd->hqd", E / den, V), (m + np.log(den))[..., 0]


def attention_tolerance(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Elementwise error allowed to an attention that rounds its softmax weights
    to bf16 before the weighted sum of V (each weight within 2^-8 of itself
    relative, the exponentials and fp32 sums within far less):
    2^-7 sum_j p_j |v_j| + 2^-20 max|v| per output element."""
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S = scale * np.einsum("hqd,hkd->hqk", Q, K)
    E = np.exp(S - S.max(axis=2, keepdims=True))
    P = E / E.sum(axis=2, keepdims=True)
    return 2.0 ** -7 * np.einsum("hqk,hkd->hqd", P, np.abs(V)) + 2.0 ** -20 * np.abs(V).max()


def rtn_reconstruct(X: np.ndarray, G: int) -> np.ndarray:
    """Round-to-nearest baseline: the same quantiser applied to X directly."""
    X = np.asarray(X, dtype=F32)
    out = []
    for h in range(X.shape[0]):
        _, packed, s_code = group_quant(X[h], G)
        out.append(dequant(packed, s_code, G))
    return np.stack(out)


def mse(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.mean((np.asarray(a, np.float64) - np.asarray(b, np.float64)) ** 2))


# --------------------------------------------------------------------------
# Byte accounting (closed forms)
# --------------------------------------------------------------------------

def kv_cache_bytes(layers: int, height: int, width: int, frames: int, hidden: int,
                   bytes_per_value: int) -> int:
    """Raw KV memory = 2 * L * (H*W*T) * d * bytes, with T the number of latent
    frames (163.com article, section 1)."""
    return 2 * layers * (height * width * frames) * hidden * bytes_per_value


def chunk_bytes(cfg: CodecConfig, heads: int, n_tokens: int) -> Dict[str, int]:
    """Bytes one encoded chunk occupies, by component."""
    d, K, T, G = cfg.d, cfg.n_centroids, cfg.n_stages, cfg.group_size
    bc = 2 if cfg.dtype == "bf16" else 4
    table = K * d + E4M3_TABLE_HEADER if cfg.centroid_format == "e4m3" else K * d * bc
    return {
        "codes": heads * n_tokens * d // 4,
        "scales": heads * n_tokens * d // G,
        "assign": T * heads * n_tokens,
        "centroids": T * heads * table,
    }


def compression_ratio(cfg: CodecConfig, heads: int, n_tokens: int,
                      include_centroids: bool = True, raw_bytes_per_value: int = 2) -> float:
    b = chunk_bytes(cfg, heads, n_tokens)
    total = b["codes"] + b["scales"] + b["assign"] + (b["centroids"] if include_centroids else 0)
    return heads * n_tokens * cfg.d * raw_bytes_per_value / total


def bits_per_value_ratio(code_bits: float, meta_bits_per_group: float, group: int,
                         raw_bits: float = 16.0) -> float:
    """Compression of a plain group quantiser: raw bits / (code + metadata bits)."""
    return raw_bits / (code_bits + meta_bits_per_group / group)
