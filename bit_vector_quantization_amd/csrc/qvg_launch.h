// Internal launch interface between the C ABI layer (qvg_api.cpp) and the
// gfx950 kernels (qvg_kernels.hip).  Every launcher enqueues on `stream` and
// returns the launch status; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qvg {

enum { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };   // DT_E4M3: stored centroid tables only

constexpr int MAX_PREV = 7;   // earlier stages a residual can be rebuilt from

// Rows of the padded centroid tables (bf16 operands and norms) per head.
inline int padded_k(int k) { return (k + 15) / 16 * 16; }

// The rows R(t-1) a stage works on, rebuilt on the fly from the chunk's input
// and the stored centroids and assignments of the P earlier stages:
//   R(0) = x,  R(p+1) = fp32(R(p) - cent[p][h][pi[p][h][n]])
// x: [H][N][D] of the tensor dtype, head stride x_hs elements; cent[p]:
// [H][K][D] of the tensor dtype; pi[p]: uint8, head stride pi_hs.
struct Src {
    const void *x;
    int64_t x_hs;
    const void *cent[MAX_PREV];
    const uint8_t *pi[MAX_PREV];
    int64_t pi_hs;
    int P;
    int K;
    // magnitude statistics of the earlier stages' stored tables,
    // [P][H][TSTAT_BLOCKS] partial pairs (see launch_store_centroids), or null
    const uint32_t *tstats;
};

// Cold start: indices [T][H][K] of the Forgy rows of every (stage, head).
hipError_t launch_forgy(int T, int H, int N, int K, uint64_t seed, int32_t *idx, hipStream_t s);

// Per-head value statistics (see launch_value_stats): VSTAT_BLOCKS partial
// pairs {smallest nonzero magnitude - 1, largest magnitude} per head.
constexpr int VSTAT_BLOCKS = 8;

// Starting centroids from fp32 `warm` [H][K][D] (when non-null) or from the rows
// idx[h][k] of R(t-1).  Writes C fp32 [H][K][D] and Cb bf16 [H][Kp][D] (padding
// rows zero), zeroes cnt0 and fill0 [H][Kp] (non-null) for the first
// histogram, and sets vstats_clear (non-null) to neutral value statistics.
hipError_t launch_init_centroids(int D, int dtype, int H, int K, const Src &src, const int32_t *idx,
                                 const float *warm, float *C, uint16_t *Cb, int32_t *cnt0, int32_t *fill0,
                                 uint32_t *vstats_clear, hipStream_t s);

// Convergence-driven rounds (off when threshold == 0).  Round `round` of a
// stage: its assign adds the labels it changed per head into changed[h]; its
// update stops head h (done[h] = 1, rounds[h] = round, ndone += 1) when
// round > 0 and changed[h] < threshold, and otherwise clears changed_next[h]
// for the next round's assign.  Every later launch of the stage skips heads
// with done[h] set.
struct ConvState {
    int32_t *changed = nullptr, *changed_next = nullptr, *done = nullptr, *rounds = nullptr, *ndone = nullptr;
    int threshold = 0;
    int round = 0;
};

// pi[h][n] = argmin_{k < K} |Cb[h][k]|^2 - 2 <bf16(R(t-1)[h][n]), Cb[h][k]>: bf16
// MFMA with fp32 accumulation ranks the centroids, the best two are re-decided
// exactly in fp64.  counts (non-null) [H][Kp] += tokens per centroid.  vstats
// (non-null; a bf16 tensor without earlier stages only): the input's value
// statistics are folded into partial 0 of each head (cleared beforehand).
// rout (non-null; a bf16 tensor whose operands take the specialised load)
// [H][N][D] bf16 receives bf16(fp32(R(t-1) - Cb[pi])), the operand that the
// next stage's assign would otherwise rebuild from x and the stored tables and
// assignments: R(t-1) is the operand itself when rsrc is null (src without
// earlier stages), else rebuilt in fp32 by rsrc (any number of stages; rout may
// be the buffer the operands come from, as each tile reads its own rows before
// it writes them).  skip
// (non-null) [H]: heads with skip[h] != 0 are left alone (and with *nskip ==
// H nothing is done).  changed (non-null) [H] += labels that differ from
// what pi held before.
hipError_t launch_assign(int D, int dtype, int H, int N, int K, const Src &src, const uint16_t *Cb, uint8_t *pi,
                         int64_t pi_hs, int32_t *counts, uint32_t *vstats, uint16_t *rout, const Src *rsrc,
                         const int32_t *skip, const int32_t *nskip, int32_t *changed, hipStream_t s);

// Histogram of an assignment (counts must be zero on entry).
hipError_t launch_count(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts,
                        hipStream_t s);

// Groups each head's tokens by centroid: offsets [H][Kp] (exclusive prefix of
// counts) and order [H][N]; fill [H][Kp] must be zero on entry.  The order of
// the tokens of one centroid is unspecified.
hipError_t launch_scatter(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, const int32_t *counts,
                          int32_t *fill, int32_t *offsets, int32_t *order, const int32_t *skip, hipStream_t s);

// Every centroid with tokens becomes the exactly summed mean of their rows of
// R(t-1) (rounded once to fp64, divided by the count, rounded to fp32); C and
// Cb are refreshed for those centroids.  zero_cnt / zero_fill (non-null)
// [H][Kp] are cleared for the next round.
hipError_t launch_update(int D, int dtype, int H, int N, int K, const Src &src, const int32_t *counts,
                         const int32_t *offsets, const int32_t *order, float *C, uint16_t *Cb, int32_t *zero_cnt,
                         int32_t *zero_fill, const ConvState &cv, hipStream_t s);

// The same update without a global sort (k_update_seg): each workgroup lists the
// tokens of a run of centroids in LDS from pi (uint8, head stride pi_hs, the
// assignment the counts were taken from).  For N <= SEG_MAX_N.  xstats
// (value_stats_words(H) words from launch_value_stats over the chunk's input,
// or null) lets whole runs of centroids skip the per-value exactness checks.
constexpr int SEG_MAX_N = 16384;
bool update_seg_fits(int N);
size_t value_stats_words(int H);
hipError_t launch_value_stats(int dtype, int H, const void *x, int64_t x_hs, int64_t count, uint32_t *stats,
                              hipStream_t s);
hipError_t launch_update_seg(int D, int dtype, int H, int N, int K, const Src &src, const uint8_t *pi,
                             int64_t pi_hs, const int32_t *counts, const uint32_t *xstats, float *C, uint16_t *Cb,
                             int32_t *zero_cnt, int32_t *zero_fill, const ConvState &cv, hipStream_t s);

// dst_slice [H][K][D] = C rounded to dtype; cache_slice [H][K][D] = C (if non-null);
// tstats (if non-null) receives TSTAT_BLOCKS partial pairs per head of the
// stored magnitudes: {smallest nonzero - 1 (0xFFFFFFFF: all zero), largest} of
// the bf16 (15-bit) or fp32 (31-bit) magnitude bits.  K D <= 8192 TSTAT_BLOCKS.
constexpr int TSTAT_BLOCKS = 4;
hipError_t launch_store_centroids(int D, int H, int K, const float *C, int dtype, void *dst_slice,
                                  float *cache_slice, uint32_t *tstats, hipStream_t s);

// FP8 storage of one stage's tables (see k_store_e4m3): dst [H] tables of
// table_bytes = 16 + K D bytes (exponent header, E4M3 codes); mirror [H][K][D]
// of the tensor dtype and Cb [H][Kp][D] bf16 receive the stored values; cache
// and tstats as for launch_store_centroids.
hipError_t launch_store_e4m3(int D, int dtype, int H, int K, const float *C, uint8_t *dst, int64_t table_bytes,
                             void *mirror, uint16_t *Cb, float *cache, uint32_t *tstats, hipStream_t s);

// r = R(t-1) - cent[pi] (cent non-null; cent [H][cent_rows][D] of the tensor
// dtype) or r = R(t-1); then 2-bit codes and E4M3 scales of r, head stride
// q_cap tokens.
// Two-level scales: amax_out (non-null, [H] zeroed beforehand) makes this
// launch only gather max|r| per head; amax_in (non-null) quantises with the
// second-level exponent it implies and writes it to exp_out [H].
hipError_t launch_quant(int D, int dtype, int H, int N, const Src &src, const void *cent, int cent_rows,
                        const uint8_t *pi, int64_t pi_hs, uint8_t *codes, uint8_t *scales, int64_t q_cap,
                        int G, uint32_t *amax_out, const uint32_t *amax_in, int8_t *exp_out, hipStream_t s);

// Fused dequantise + reconstruct of tokens [tok_begin, tok_begin + ntok), with an
// optional rotary position embedding of the first rope_heads heads.
struct DecodeArgs {
    const uint8_t *codes, *scales, *assign;
    const void *cent;
    int cent_dtype;   // DT_BF16, DT_F32, or DT_E4M3: tables of 16 + K D bytes
    int64_t cap;
    int chunk_tokens, H, K, T, G, D;
    int64_t tok_begin, ntok;
    // rotation table [ntok][D/2] of (cos, sin) fp32 pairs for heads < rope_heads,
    // or null
    const float *rope = nullptr;
    int rope_heads = 0;
    // second-level exponents of two-level scales, [n_chunks][H] of the view, or null
    const int8_t *scale_exp = nullptr;
    void *out;
    int out_dtype;
    int64_t out_hs;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Attention over the compressed cache (k_attention + k_attn_merge): one
// compressed tensor as the kernel reads it (bf16 tables, or FP8 tables of
// 16 + K D bytes), d = 128.
struct AttnSrc {
    const uint8_t *codes, *scales, *assign;
    const void *cent;
    const int8_t *scale_exp;   // [n_chunks][heads] two-level exponents, or null
    int64_t cap;
    int chunk_tokens, heads, K, G;
};
struct AttnArgs {
    AttnSrc k, v;
    int khead0, vhead0;   // attention head h reads K head khead0 + h and V head vhead0 + h
    int T, fp8;
    int64_t tok_begin, tok_end, keys_per_split;
    const float *rope;    // [tok_end - tok_begin][D/2] (cos, sin) for the keys, or null
    const uint16_t *q;    // bf16 [H][Nq][D], head stride q_hs
    int64_t q_hs;
    int H, Nq, splits;
    float scale_log2;     // the score scale times log2(e)
    float *part_o;        // [splits][H][Nq][D] fp32
    float *part_ml;       // [splits][H][Nq][2] fp32
};
hipError_t launch_attention(const AttnArgs &a, float *out, int64_t out_hs, float *lse, hipStream_t s);

// Events the next kernel launch records at its own start and end
// (hipExtLaunchKernelGGL); the library's profiler sets them around one launcher
// call, and the launch clears them.  Thread-local; null when profiling is off.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents &launch_events();

// Device address, on the current device, of the library's fixed scratch array
// of STATIC_SCRATCH_BYTES (looked up once per device, then reused).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t static_scratch(void **ptr);

// Fills n int32 with zero.
hipError_t launch_zero(int32_t *p, int64_t n, hipStream_t s);
// Fills n int32 with v.
hipError_t launch_fill(int32_t *p, int64_t n, int32_t v, hipStream_t s);

}  // namespace qvg
