// gfx950 kernels of the Quant VideoGen KV-cache codec.
//
// Method: "Quant VideoGen: Auto-Regressive Long Video Generation via 2-Bit
// KV-Cache Quantization", as summarised by the 163.com article (sections 3-5, 7)
// and gist.science (German / Portuguese technical summaries, sections 2A-2C):
// k-means smoothing of each chunk's token rows, progressive residual stages,
// 2-bit group quantisation with FP8 E4M3 scales, and a fused dequantise +
// centroid reconstruction.
//
// Layout conventions: tensors are [H][N][D] (head, token, channel); bf16 values
// travel as raw uint16 bits.  All kernels are wave64.
//
// Floating-point contract: every product that feeds an add here is exact
// (bf16 x bf16 squares/products, 2 * x, (q - 1.5) * s), so FMA contraction
// cannot change a result; divisions are IEEE (correctly rounded).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qvg_launch.h"

namespace qvg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP FP8 E4M3FN of a non-negative value: round to nearest even, saturating at
// 448 (code 0x7E).  Below 2^-6 the grid is the subnormal one, 2^-9 apart.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
    if (!(v < 448.0f)) return 0x7Eu;
    if (v < 0.015625f) return (uint32_t)rintf(v * 512.0f);   // 0..8; 8 is 2^-6 = code 0x08
    uint32_t u = __float_as_uint(v);
    uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;     // exponent and 3 mantissa bits
    uint32_t code = r - (120u << 3);                           // rebias 127 -> 7
    return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = c >> 3, m = c & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Blocks are dispatched round-robin over the 8 XCDs; give each XCD one
// contiguous range of logical tiles so that neighbouring tiles share its L2.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t nblocks) {
    const uint32_t X = 8;
    uint32_t q = nblocks / X, r = nblocks % X;
    uint32_t xcd = bid % X, local = bid / X;
    return xcd * q + (xcd < r ? xcd : r) + local;
}

template <typename T>
__device__ __forceinline__ void load16(const T *p, float (&v)[16]);

template <>
__device__ __forceinline__ void load16<uint16_t>(const uint16_t *p, float (&v)[16]) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load16<float>(const float *p, float (&v)[16]) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 f = q[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

__device__ __forceinline__ void store16_bf16(uint16_t *p, const float (&v)[16]) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
    uint4 *q = reinterpret_cast<uint4 *>(p);
    q[0] = make_uint4(w[0], w[1], w[2], w[3]);
    q[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

__device__ __forceinline__ void store16_f32(float *p, const float (&v)[16]) {
    float4 *q = reinterpret_cast<float4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// ---------------------------------------------------------------------------
// cold start: Forgy rows from a keyed partial Fisher-Yates shuffle
// ---------------------------------------------------------------------------

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t &s) {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// One wave per head.  Step i of the shuffle swaps a[i] with a[j], j = i + r mod
// (N - i); only displaced positions are kept, in a small LDS table searched by
// the whole wave, so the cost does not depend on N.
constexpr int FORGY_TABLE = 256;   // at most one new displaced position per step, K <= 256 steps

__global__ __launch_bounds__(64) void k_forgy(int N, int K, uint64_t seed, int stage, int32_t *idx) {
    __shared__ int32_t keys[FORGY_TABLE];
    __shared__ int32_t vals[FORGY_TABLE];
    __shared__ int32_t sel[FORGY_TABLE];
    const int h = blockIdx.x, lane = threadIdx.x;
    uint64_t st = (seed * 65536ull + (uint64_t)h) * 64ull + (uint64_t)stage;
    const int steps = K < N ? K : N;
    int n_ent = 0;
    for (int i = 0; i < steps; ++i) {
        const uint64_t r = splitmix64(st);
        const int j = i + (int)(r % (uint64_t)(N - i));
        int vi_l = i, vj_l = j, ej_l = -1;
        bool fi = false, fj = false;
        for (int e = lane; e < n_ent; e += 64) {
            const int kk = keys[e];
            if (kk == i) { vi_l = vals[e]; fi = true; }
            if (kk == j) { vj_l = vals[e]; ej_l = e; fj = true; }
        }
        const uint64_t mi = __ballot(fi), mj = __ballot(fj);
        const int vi = mi ? __shfl(vi_l, __ffsll((long long)mi) - 1) : i;
        const int vj = mj ? __shfl(vj_l, __ffsll((long long)mj) - 1) : j;
        const int ej = mj ? __shfl(ej_l, __ffsll((long long)mj) - 1) : -1;
        __syncthreads();
        if (lane == 0) {
            sel[i] = vj;                      // position i is final after step i
            if (ej >= 0) vals[ej] = vi;       // a[j] = old a[i]
            else { keys[n_ent] = j; vals[n_ent] = vi; }
        }
        if (ej < 0) ++n_ent;
        __syncthreads();
    }
    // fewer tokens than centroids: entry k repeats entry k mod N
    int32_t *out = idx + (size_t)h * K;
    for (int k = lane; k < K; k += 64) out[k] = sel[k < steps ? k : k % N];
}

hipError_t launch_forgy(int H, int N, int K, uint64_t seed, int stage, int32_t *idx, hipStream_t s) {
    hipLaunchKernelGGL(k_forgy, dim3(H), dim3(64), 0, s, N, K, seed, stage, idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// starting centroids -> C (fp32), Cb (bf16 operand), cnorm = |Cb|^2 (fp64; exact for
// the value ranges met in practice, every square of a bf16 being exact)
// ---------------------------------------------------------------------------

template <int D, typename SrcT>
__device__ __forceinline__ void load_row_part(const SrcT *row, int lane, float (&v)[D / 64]);

template <>
__device__ __forceinline__ void load_row_part<128, uint16_t>(const uint16_t *row, int lane, float (&v)[2]) {
    uint32_t w = reinterpret_cast<const uint32_t *>(row)[lane];
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load_row_part<128, float>(const float *row, int lane, float (&v)[2]) {
    float2 f = reinterpret_cast<const float2 *>(row)[lane];
    v[0] = f.x;
    v[1] = f.y;
}
template <>
__device__ __forceinline__ void load_row_part<64, uint16_t>(const uint16_t *row, int lane, float (&v)[1]) {
    v[0] = bf16_to_f32(row[lane]);
}
template <>
__device__ __forceinline__ void load_row_part<64, float>(const float *row, int lane, float (&v)[1]) {
    v[0] = row[lane];
}

// Writes one centroid row (C, Cb, cnorm) from the lane's D/64 values.
template <int D>
__device__ __forceinline__ void write_centroid(int h, int k, int K, int Kp, int lane, const float (&v)[D / 64],
                                               float *C, uint16_t *Cb, double *cnorm) {
    constexpr int P = D / 64;
    double sq = 0.0;
    uint32_t b[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        b[i] = f32_to_bf16(v[i]);
        double bd = (double)bf16_to_f32(b[i]);
        sq += bd * bd;
    }
    float *c = C + ((size_t)h * K + k) * D + lane * P;
    uint16_t *cb = Cb + ((size_t)h * Kp + k) * D + lane * P;
    if constexpr (P == 2) {
        reinterpret_cast<float2 *>(c)[0] = make_float2(v[0], v[1]);
        reinterpret_cast<uint32_t *>(cb)[0] = b[0] | (b[1] << 16);
    } else {
        c[0] = v[0];
        cb[0] = (uint16_t)b[0];
    }
    sq = wave_sum(sq);
    if (lane == 0) cnorm[(size_t)h * Kp + k] = sq;
}

template <int D, typename SrcT>
__global__ __launch_bounds__(64) void k_init_centroids(int K, int Kp, const SrcT *src, int64_t src_hs,
                                                       const int32_t *idx, const float *warm, float *C,
                                                       uint16_t *Cb, double *cnorm) {
    constexpr int P = D / 64;
    const int k = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    if (k >= K) {  // padding rows: never chosen
        uint16_t *cb = Cb + ((size_t)h * Kp + k) * D + lane * P;
#pragma unroll
        for (int i = 0; i < P; ++i) cb[i] = 0;
        if (lane == 0) cnorm[(size_t)h * Kp + k] = __builtin_inf();
        return;
    }
    float v[P];
    if (warm) {
        const float *w = warm + ((size_t)h * K + k) * D;
        load_row_part<D, float>(w, lane, v);
    } else {
        const int n = idx[(size_t)h * K + k];
        load_row_part<D, SrcT>(src + (size_t)h * src_hs + (size_t)n * D, lane, v);
    }
    write_centroid<D>(h, k, K, Kp, lane, v, C, Cb, cnorm);
}

hipError_t launch_init_centroids(int D, int H, int K, const void *src, int src_dtype, int64_t src_hs,
                                 const int32_t *idx, const float *warm, float *C, uint16_t *Cb, double *cnorm,
                                 hipStream_t s) {
    const int Kp = padded_k(K);
    dim3 g(Kp, H), b(64);
#define QVG_INIT(DD, TT)                                                                                      \
    hipLaunchKernelGGL((k_init_centroids<DD, TT>), g, b, 0, s, K, Kp, (const TT *)src, src_hs, idx, warm, C, \
                       Cb, cnorm)
    if (D == 128) {
        if (src_dtype == DT_BF16) QVG_INIT(128, uint16_t); else QVG_INIT(128, float);
    } else {
        if (src_dtype == DT_BF16) QVG_INIT(64, uint16_t); else QVG_INIT(64, float);
    }
#undef QVG_INIT
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// assignment: distances on the matrix cores, exact decision between the two best
// ---------------------------------------------------------------------------
//
// D^T = Cb * Xb^T with v_mfma_f32_16x16x32_bf16: the A operand is a block of 16
// centroids, the B operand a block of 16 tokens, 32 channels per instruction.
// Lane l feeds row/column (l % 16) and channels 8*(l/16) .. +7 of the k-step for
// both operands, so the two sides pair the same channels whatever the order of
// the hardware's reduction.  The 16x16 result leaves centroid 4*(l/16)+r of
// token l%16 in accumulator r of lane l, so each lane keeps the two smallest
// fp32 distances of one token over its centroids and four lanes merge them.
//
// fp32 accumulation can misorder two centroids whose distances differ by a few
// fp32 ulps.  The final choice between the two best is therefore made on exact
// distances: every bf16 x bf16 product is exact in fp64 and the 128-term sums
// and |c|^2 are exact in fp64 for the value ranges met in practice, so the
// decision is that of the exactly computed |c|^2 - 2<x, c>, lowest index on ties.
//
// A workgroup is 4 waves x 64 tokens; the head's bf16 centroid table (swizzled
// 16-byte chunks) and its norms (fp32 and fp64) sit in LDS.

constexpr int ASSIGN_TB = 4;  // 16-token blocks per wave

__device__ __forceinline__ bool lex_less(float a, int ka, float b, int kb) {
    return a < b || (a == b && ka < kb);
}

template <int D>
__global__ __launch_bounds__(256) void k_assign(const uint16_t *__restrict__ xb, int64_t x_hs, int N,
                                                const uint16_t *__restrict__ Cb, const double *__restrict__ cnorm,
                                                int Kp, uint8_t *__restrict__ pi, int64_t pi_hs) {
    constexpr int KS = D / 32;   // k-steps
    constexpr int CH = D / 8;    // 16-byte chunks per row
    extern __shared__ uint4 lds[];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;

    const uint4 *csrc = reinterpret_cast<const uint4 *>(Cb + (size_t)h * Kp * D);
    for (int i = tid; i < Kp * CH; i += 256) {
        int row = i / CH, q = i - row * CH;
        lds[row * CH + (q ^ (row & (CH - 1)))] = csrc[i];
    }
    double *lcn64 = reinterpret_cast<double *>(lds + Kp * CH);
    float *lcn = reinterpret_cast<float *>(lcn64 + Kp);
    for (int i = tid; i < Kp; i += 256) {
        const double c = cnorm[(size_t)h * Kp + i];
        lcn64[i] = c;
        lcn[i] = (float)c;
    }

    const int tok0 = blockIdx.x * (64 * ASSIGN_TB) + wave * 64;
    const uint16_t *xh = xb + (size_t)h * x_hs;
    bf16x8_t bt[ASSIGN_TB][KS];
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        const int n = tok0 + 16 * b + r16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n < N) v = *reinterpret_cast<const uint4 *>(xh + (size_t)n * D + 32 * s + 8 * g);
            bt[b][s] = __builtin_bit_cast(bf16x8_t, v);
        }
    }
    __syncthreads();

    float v1[ASSIGN_TB], v2[ASSIGN_TB];
    int k1[ASSIGN_TB], k2[ASSIGN_TB];
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        v1[b] = v2[b] = __builtin_inff();
        k1[b] = k2[b] = 0;
    }

    const int ncb = Kp / 16;
    for (int cb = 0; cb < ncb; ++cb) {
        const int row = cb * 16 + r16;
        bf16x8_t a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            a[s] = __builtin_bit_cast(bf16x8_t, lds[row * CH + ((4 * s + g) ^ (row & (CH - 1)))]);
        const float4 cn = *reinterpret_cast<const float4 *>(lcn + cb * 16 + 4 * g);
        const float cnv[4] = {cn.x, cn.y, cn.z, cn.w};
#pragma unroll
        for (int b = 0; b < ASSIGN_TB; ++b) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bt[b][s], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // centroids reach a lane in increasing index order: strict < keeps the lower index
                const float d = cnv[r] - 2.0f * acc[r];
                const int k = cb * 16 + 4 * g + r;
                const bool lt1 = d < v1[b], lt2 = d < v2[b];
                v2[b] = lt1 ? v1[b] : (lt2 ? d : v2[b]);
                k2[b] = lt1 ? k1[b] : (lt2 ? k : k2[b]);
                v1[b] = lt1 ? d : v1[b];
                k1[b] = lt1 ? k : k1[b];
            }
        }
    }
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        // merge the four lanes' top-2 lists of each token
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float w1 = __shfl_xor(v1[b], o), w2 = __shfl_xor(v2[b], o);
            const int j1 = __shfl_xor(k1[b], o), j2 = __shfl_xor(k2[b], o);
            if (lex_less(w1, j1, v1[b], k1[b])) {
                if (!lex_less(v1[b], k1[b], w2, j2)) { v2[b] = w2; k2[b] = j2; }
                else { v2[b] = v1[b]; k2[b] = k1[b]; }
                v1[b] = w1;
                k1[b] = j1;
            } else if (lex_less(w1, j1, v2[b], k2[b])) {
                v2[b] = w1;
                k2[b] = j1;
            }
        }
        // exact distances of the two candidates: each lane sums its 32 channels
        const int c1 = k1[b], c2 = k2[b];
        double p1 = 0.0, p2 = 0.0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 xv = __builtin_bit_cast(uint4, bt[b][s]);
            const uint4 a1 = lds[c1 * CH + ((4 * s + g) ^ (c1 & (CH - 1)))];
            const uint4 a2 = lds[c2 * CH + ((4 * s + g) ^ (c2 & (CH - 1)))];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            const uint32_t aw[4] = {a1.x, a1.y, a1.z, a1.w};
            const uint32_t bw[4] = {a2.x, a2.y, a2.z, a2.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double xl = (double)__uint_as_float(xw[i] << 16), xh2 = (double)__uint_as_float(xw[i] & 0xFFFF0000u);
                p1 = fma(xl, (double)__uint_as_float(aw[i] << 16), p1);
                p1 = fma(xh2, (double)__uint_as_float(aw[i] & 0xFFFF0000u), p1);
                p2 = fma(xl, (double)__uint_as_float(bw[i] << 16), p2);
                p2 = fma(xh2, (double)__uint_as_float(bw[i] & 0xFFFF0000u), p2);
            }
        }
        p1 += __shfl_xor(p1, 16);
        p2 += __shfl_xor(p2, 16);
        p1 += __shfl_xor(p1, 32);
        p2 += __shfl_xor(p2, 32);
        const double e1 = lcn64[c1] - 2.0 * p1, e2 = lcn64[c2] - 2.0 * p2;
        const int best = (e2 < e1 || (e2 == e1 && c2 < c1)) ? c2 : c1;
        const int n = tok0 + 16 * b + r16;
        if (g == 0 && n < N) pi[(size_t)h * pi_hs + n] = (uint8_t)best;
    }
}

hipError_t launch_assign(int D, int H, int N, const uint16_t *xb, int64_t x_hs, const uint16_t *Cb,
                         const double *cnorm, int Kp, uint8_t *pi, int64_t pi_hs, hipStream_t s) {
    const size_t lds = (size_t)Kp * D * 2 + (size_t)Kp * 12;
    dim3 g((N + 64 * ASSIGN_TB - 1) / (64 * ASSIGN_TB), H), b(256);
    if (D == 128) {
        (void)hipFuncSetAttribute((const void *)k_assign<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k_assign<128>, g, b, lds, s, xb, x_hs, N, Cb, cnorm, Kp, pi, pi_hs);
    } else {
        (void)hipFuncSetAttribute((const void *)k_assign<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(k_assign<64>, g, b, lds, s, xb, x_hs, N, Cb, cnorm, Kp, pi, pi_hs);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// update, part 1: stable counting sort of each head's tokens by centroid
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_bucket(int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts,
                                                int32_t *offsets, int32_t *order) {
    __shared__ int32_t cnt[256];
    __shared__ int32_t off[256];
    __shared__ int32_t wsum[4];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t *p = pi + (size_t)h * pi_hs;
    cnt[tid] = 0;
    __syncthreads();
    for (int n = tid; n < N; n += 256) atomicAdd(&cnt[p[n]], 1);
    __syncthreads();
    const int v = cnt[tid];
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wsum[w];
    const int excl = x + add - v;
    off[tid] = excl;
    if (tid < Kp) {
        counts[(size_t)h * Kp + tid] = v;
        offsets[(size_t)h * Kp + tid] = excl;
    }
    __syncthreads();
    if (wave != 0) return;
    // one wave places the tokens in order, 64 at a time; equal keys in a batch
    // are ranked by lane (match on all 8 key bits)
    const uint64_t lt = (1ull << lane) - 1ull;
    int32_t *ord = order + (size_t)h * N;
    for (int base = 0; base < N; base += 64) {
        const int n = base + lane;
        const bool valid = n < N;
        const int k = valid ? p[n] : 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (k >> bit) & 1;
            const uint64_t bb = __ballot(valid && on);
            peers &= on ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt);
        int pos = 0;
        if (valid) pos = off[k] + rank;
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            ord[pos] = n;
            if (rank == 0) off[k] += __popcll(peers);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

hipError_t launch_bucket(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts, int32_t *offsets,
                         int32_t *order, hipStream_t s) {
    hipLaunchKernelGGL(k_bucket, dim3(H), dim3(256), 0, s, N, Kp, pi, pi_hs, counts, offsets, order);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// update, part 2: mean of each centroid's rows, fp64 in ascending token order
// ---------------------------------------------------------------------------

template <int D, typename SrcT>
__global__ __launch_bounds__(256) void k_update(int N, int K, int Kp, const SrcT *src, int64_t src_hs,
                                                const int32_t *counts, const int32_t *offsets,
                                                const int32_t *order, float *C, uint16_t *Cb, double *cnorm) {
    constexpr int P = D / 64;
    const int h = blockIdx.y, lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (k >= K) return;
    const int cnt = counts[(size_t)h * Kp + k];
    if (cnt == 0) return;  // empty cluster keeps its centroid
    const int32_t *ord = order + (size_t)h * N + offsets[(size_t)h * Kp + k];
    const SrcT *xh = src + (size_t)h * src_hs;
    double acc[P];
#pragma unroll
    for (int i = 0; i < P; ++i) acc[i] = -0.0;   // -0 + x == x for every x
    for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int m = cnt - i0 < 64 ? cnt - i0 : 64;
        const int my = lane < m ? ord[i0 + lane] : 0;
        int j = 0;
        for (; j + 8 <= m; j += 8) {
            float v[8][P];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int n = __shfl(my, j + u);
                load_row_part<D, SrcT>(xh + (size_t)n * D, lane, v[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int i = 0; i < P; ++i) acc[i] += (double)v[u][i];
        }
        for (; j < m; ++j) {
            float v[P];
            const int n = __shfl(my, j);
            load_row_part<D, SrcT>(xh + (size_t)n * D, lane, v);
#pragma unroll
            for (int i = 0; i < P; ++i) acc[i] += (double)v[i];
        }
    }
    float mean[P];
#pragma unroll
    for (int i = 0; i < P; ++i) mean[i] = (float)(acc[i] / (double)cnt);
    write_centroid<D>(h, k, K, Kp, lane, mean, C, Cb, cnorm);
}

hipError_t launch_update(int D, int H, int N, int K, const void *src, int src_dtype, int64_t src_hs,
                         const int32_t *counts, const int32_t *offsets, const int32_t *order, float *C,
                         uint16_t *Cb, double *cnorm, hipStream_t s) {
    const int Kp = padded_k(K);
    dim3 g((K + 3) / 4, H), b(256);
#define QVG_UPD(DD, TT)                                                                                     \
    hipLaunchKernelGGL((k_update<DD, TT>), g, b, 0, s, N, K, Kp, (const TT *)src, src_hs, counts, offsets, \
                       order, C, Cb, cnorm)
    if (D == 128) {
        if (src_dtype == DT_BF16) QVG_UPD(128, uint16_t); else QVG_UPD(128, float);
    } else {
        if (src_dtype == DT_BF16) QVG_UPD(64, uint16_t); else QVG_UPD(64, float);
    }
#undef QVG_UPD
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stored centroids and the streaming cache
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(64) void k_store_centroids(int K, const float *C, int dtype, void *dst, float *cache) {
    constexpr int P = D / 64;
    const int k = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
    const size_t off = ((size_t)h * K + k) * D + lane * P;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const float v = C[off + i];
        if (dtype == DT_BF16) reinterpret_cast<uint16_t *>(dst)[off + i] = (uint16_t)f32_to_bf16(v);
        else reinterpret_cast<float *>(dst)[off + i] = v;
        if (cache) cache[off + i] = v;
    }
}

hipError_t launch_store_centroids(int D, int H, int K, const float *C, int dtype, void *dst, float *cache,
                                  hipStream_t s) {
    dim3 g(K, H), b(64);
    if (D == 128) hipLaunchKernelGGL(k_store_centroids<128>, g, b, 0, s, K, C, dtype, dst, cache);
    else hipLaunchKernelGGL(k_store_centroids<64>, g, b, 0, s, K, C, dtype, dst, cache);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stage residual, optionally fused with the 2-bit group quantiser
// ---------------------------------------------------------------------------
//
// One thread owns 16 consecutive channels of one token; the G/16 threads of a
// group are adjacent lanes and combine their maxima with lane shuffles.

template <int D, int MODE, typename SrcT, typename CentT>
__global__ __launch_bounds__(256) void k_residual(const SrcT *src, int64_t src_hs, int N, const CentT *cent,
                                                  int cent_rows, const uint8_t *pi, int64_t pi_hs, float *R,
                                                  uint16_t *Rb, int64_t r_hs, uint8_t *codes, uint8_t *scales,
                                                  int64_t q_cap, int G) {
    constexpr int SL = D / 16;
    constexpr int TPB = 256 / SL;
    const int h = blockIdx.y;
    const int j = threadIdx.x % SL;
    const int n = blockIdx.x * TPB + threadIdx.x / SL;
    if (n >= N) return;   // whole groups leave together (SL divides 64)
    float r[16];
    load16<SrcT>(src + (size_t)h * src_hs + (size_t)n * D + 16 * j, r);
    if constexpr (MODE != QUANT_ONLY) {
        const int k = pi[(size_t)h * pi_hs + n];
        float c[16];
        load16<CentT>(cent + ((size_t)h * cent_rows + k) * D + 16 * j, c);
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = r[i] - c[i];
    }
    if constexpr (MODE == RES_WRITE) {
        const size_t off = (size_t)h * r_hs + (size_t)n * D + 16 * j;
        store16_f32(R + off, r);
        store16_bf16(Rb + off, r);
    } else {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(r[i]));
        const int lanes = G >> 4;
        for (int o = 1; o < lanes; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        const uint32_t sc = e4m3_encode_nonneg(a / 1.5f);
        const float s = e4m3_decode(sc);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t q = (uint32_t)(r[i] >= -s) + (uint32_t)(r[i] >= 0.f) + (uint32_t)(r[i] >= s);
            w |= q << (2 * i);
        }
        const size_t row = (size_t)h * q_cap + n;
        reinterpret_cast<uint32_t *>(codes + row * (D / 4))[j] = w;
        if ((j & (lanes - 1)) == 0) scales[row * (D / G) + (16 * j) / G] = (uint8_t)sc;
    }
}

hipError_t launch_residual(int D, int mode, const void *src, int src_dtype, int64_t src_hs, int H, int N,
                           const void *cent, int cent_dtype, int cent_rows, const uint8_t *pi, int64_t pi_hs,
                           float *R, uint16_t *Rb, int64_t r_hs, uint8_t *codes, uint8_t *scales, int64_t q_cap,
                           int G, hipStream_t s) {
    const int TPB = 256 / (D / 16);
    dim3 g((N + TPB - 1) / TPB, H), b(256);
#define QVG_RES(DD, MM, ST, CT)                                                                                \
    hipLaunchKernelGGL((k_residual<DD, MM, ST, CT>), g, b, 0, s, (const ST *)src, src_hs, N, (const CT *)cent, \
                       cent_rows, pi, pi_hs, R, Rb, r_hs, codes, scales, q_cap, G)
#define QVG_RES_C(DD, MM, ST)                                      \
    do {                                                           \
        if (cent_dtype == DT_BF16) QVG_RES(DD, MM, ST, uint16_t); \
        else QVG_RES(DD, MM, ST, float);                           \
    } while (0)
#define QVG_RES_S(DD, MM)                                          \
    do {                                                           \
        if (src_dtype == DT_BF16) QVG_RES_C(DD, MM, uint16_t);     \
        else QVG_RES_C(DD, MM, float);                             \
    } while (0)
#define QVG_RES_M(DD)                                              \
    do {                                                           \
        if (mode == RES_WRITE) QVG_RES_S(DD, RES_WRITE);           \
        else if (mode == RES_QUANT) QVG_RES_S(DD, RES_QUANT);      \
        else QVG_RES_S(DD, QUANT_ONLY);                            \
    } while (0)
    if (D == 128) QVG_RES_M(128); else QVG_RES_M(64);
#undef QVG_RES_M
#undef QVG_RES_S
#undef QVG_RES_C
#undef QVG_RES
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fused dequantise + reconstruct
// ---------------------------------------------------------------------------
//
// One thread owns 16 channels of one token: one 32-bit word of codes, one scale
// byte, T assignment bytes, T gathered 16-channel centroid slices (the chunk's
// tables stay in L2), and a 32- or 64-byte store.  Blocks walk (head, token)
// tiles, XCD-contiguous.

template <int D, typename CentT, typename OutT>
__global__ __launch_bounds__(256) void k_decode(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                const uint8_t *__restrict__ assign, const CentT *__restrict__ cent,
                                                int64_t cap, int chunk_tokens, int H, int K, int T, int G,
                                                int64_t tok_begin, int64_t ntok, OutT *__restrict__ out,
                                                int64_t out_hs, uint32_t blocks_per_head) {
    constexpr int SL = D / 16;
    constexpr int TPB = 256 / SL;
    const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int h = tile / blocks_per_head;
    const int64_t nl = (int64_t)(tile % blocks_per_head) * TPB + threadIdx.x / SL;
    const int j = threadIdx.x % SL;
    if (nl >= ntok) return;
    const int64_t n = tok_begin + nl;
    const int64_t c = n / chunk_tokens;
    const size_t row = (size_t)h * cap + n;
    const uint32_t w = reinterpret_cast<const uint32_t *>(codes + row * (D / 4))[j];
    const float s = e4m3_decode(scales[row * (D / G) + (16 * j) / G]);
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = ((float)((w >> (2 * i)) & 3u) - 1.5f) * s;
    for (int t = T - 1; t >= 0; --t) {
        int k = assign[((size_t)t * H + h) * cap + n];
        k = k < K ? k : K - 1;   // a corrupt byte cannot leave the chunk's table
        float cv[16];
        load16<CentT>(cent + ((((size_t)c * T + t) * H + h) * K + k) * D + 16 * j, cv);
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = y[i] + cv[i];
    }
    OutT *o = out + (size_t)h * out_hs + (size_t)nl * D + 16 * j;
    if constexpr (sizeof(OutT) == 2) store16_bf16(reinterpret_cast<uint16_t *>(o), y);
    else store16_f32(reinterpret_cast<float *>(o), y);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    const int TPB = 256 / (a.D / 16);
    const uint32_t bph = (uint32_t)((a.ntok + TPB - 1) / TPB);
    dim3 g(bph * a.H), b(256);
#define QVG_DEC(DD, CT, OT)                                                                                       \
    hipLaunchKernelGGL((k_decode<DD, CT, OT>), g, b, 0, s, a.codes, a.scales, a.assign, (const CT *)a.cent, a.cap, \
                       a.chunk_tokens, a.H, a.K, a.T, a.G, a.tok_begin, a.ntok, (OT *)a.out, a.out_hs, bph)
#define QVG_DEC_O(DD, CT)                                  \
    do {                                                   \
        if (a.out_dtype == DT_BF16) QVG_DEC(DD, CT, uint16_t); \
        else QVG_DEC(DD, CT, float);                       \
    } while (0)
#define QVG_DEC_C(DD)                                      \
    do {                                                   \
        if (a.cent_dtype == DT_BF16) QVG_DEC_O(DD, uint16_t); \
        else QVG_DEC_O(DD, float);                         \
    } while (0)
    if (a.D == 128) QVG_DEC_C(128); else QVG_DEC_C(64);
#undef QVG_DEC_C
#undef QVG_DEC_O
#undef QVG_DEC
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 -> bf16 operand copy
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_cast_bf16(const float *x, int64_t x_hs, int N, int D, uint16_t *out) {
    const int h = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index of 4 values
    const int64_t total4 = (int64_t)N * D / 4;
    if (i >= total4) return;
    const float4 v = reinterpret_cast<const float4 *>(x + (size_t)h * x_hs)[i];
    const uint32_t lo = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    const uint32_t hi = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
    reinterpret_cast<uint2 *>(out + (size_t)h * N * D)[i] = make_uint2(lo, hi);
}

hipError_t launch_cast_bf16(const float *x, int64_t x_hs, int H, int N, int D, uint16_t *out, hipStream_t s) {
    const int64_t total4 = (int64_t)N * D / 4;
    dim3 g((unsigned)((total4 + 255) / 256), H), b(256);
    hipLaunchKernelGGL(k_cast_bf16, g, b, 0, s, x, x_hs, N, D, out);
    return hipGetLastError();
}

}  // namespace qvg
