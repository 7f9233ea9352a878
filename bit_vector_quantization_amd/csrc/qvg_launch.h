// Internal launch interface between the C ABI layer (qvg_api.cpp) and the
// gfx950 kernels (qvg_kernels.hip).  Every launcher enqueues on `stream` and
// returns the launch status; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qvg {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Rows of the padded centroid tables (bf16 operands and norms) per head.
inline int padded_k(int k) { return (k + 15) / 16 * 16; }

// Cold start: indices [H][K] of the Forgy rows of (seed, head, stage).
hipError_t launch_forgy(int H, int N, int K, uint64_t seed, int stage, int32_t *idx,
                        hipStream_t s);

// Starting centroids: from fp32 `warm` [H][K][D] (when non-null) or from the rows
// idx[h][k] of src (dtype src_dtype, head stride in elements).  Writes C fp32
// [H][K][D], Cb bf16 [H][Kp][D] (padding rows zero) and cnorm = |Cb|^2 fp64
// [H][Kp] (padding +inf).
hipError_t launch_init_centroids(int D, int H, int K, const void *src, int src_dtype,
                                 int64_t src_hs, const int32_t *idx, const float *warm, float *C,
                                 uint16_t *Cb, double *cnorm, hipStream_t s);

// pi[h][n] = argmin_k cnorm[k] - 2 <xb[h][n], Cb[h][k]>: bf16 MFMA with fp32
// accumulation ranks the centroids, the best two are re-decided exactly in fp64.
hipError_t launch_assign(int D, int H, int N, const uint16_t *xb, int64_t x_hs,
                         const uint16_t *Cb, const double *cnorm, int Kp, uint8_t *pi,
                         int64_t pi_hs, hipStream_t s);

// Counting sort of each head's tokens by centroid (stable): counts and exclusive
// offsets [H][Kp], order [H][N].
hipError_t launch_bucket(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts,
                         int32_t *offsets, int32_t *order, hipStream_t s);

// Mean of the unrounded rows of every non-empty centroid (fp64 sum in token
// order); refreshes C, Cb and cnorm of those centroids.
hipError_t launch_update(int D, int H, int N, int K, const void *src, int src_dtype, int64_t src_hs,
                         const int32_t *counts, const int32_t *offsets, const int32_t *order,
                         float *C, uint16_t *Cb, double *cnorm, hipStream_t s);

// dst_slice [H][K][D] = C rounded to dtype; cache_slice [H][K][D] = C (if non-null).
hipError_t launch_store_centroids(int D, int H, int K, const float *C, int dtype, void *dst_slice,
                                  float *cache_slice, hipStream_t s);

enum { RES_WRITE = 0, RES_QUANT = 1, QUANT_ONLY = 2 };

// r = src - cent[pi] (RES_*) or r = src (QUANT_ONLY); then either R fp32 + Rb bf16
// (RES_WRITE) or 2-bit codes + E4M3 scales (RES_QUANT / QUANT_ONLY).
//   cent: [H][cent_rows][D] of cent_dtype; codes/scales: head stride q_cap tokens.
hipError_t launch_residual(int D, int mode, const void *src, int src_dtype, int64_t src_hs, int H,
                           int N, const void *cent, int cent_dtype, int cent_rows,
                           const uint8_t *pi, int64_t pi_hs, float *R, uint16_t *Rb, int64_t r_hs,
                           uint8_t *codes, uint8_t *scales, int64_t q_cap, int G, hipStream_t s);

// Fused dequantise + reconstruct of tokens [tok_begin, tok_begin + ntok).
struct DecodeArgs {
    const uint8_t *codes, *scales, *assign;
    const void *cent;
    int cent_dtype;
    int64_t cap;
    int chunk_tokens, H, K, T, G, D;
    int64_t tok_begin, ntok;
    void *out;
    int out_dtype;
    int64_t out_hs;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// bf16 copy of an fp32 [H][N][D] tensor (round to nearest even), output contiguous.
hipError_t launch_cast_bf16(const float *x, int64_t x_hs, int H, int N, int D, uint16_t *out,
                            hipStream_t s);

}  // namespace qvg
