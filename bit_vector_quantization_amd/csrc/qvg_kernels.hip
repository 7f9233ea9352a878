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

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>


#include "qvg_launch.h"

namespace qvg {

// Every kernel launch: with the profiler's events set, the launch records them
// at the kernel's own start and end.
#define QVG_KERNEL(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                                    \
    do {                                                                                                      \
        LaunchEvents &le_ = launch_events();                                                                  \
        if (le_.start) {                                                                                      \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, le_.start, le_.stop, 0, __VA_ARGS__);   \
            le_.start = le_.stop = nullptr;                                                                   \
        } else {                                                                                              \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                              \
        }                                                                                                     \
    } while (0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (lo in bits 0-15), rounded to nearest even by
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

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

// Value of an E4M3FN code: its 4 exponent and 3 mantissa bits placed at fp32's
// bits 26..20 read as fp32 with bias 127 instead of 7, so one exact scaling by
// 2^120 gives the value; subnormal codes land on fp32 subnormals, which the
// scaling keeps exact (fp32 denormals are not flushed).  S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const float v = __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
    const float mag = (c & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : v;
    return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

// v plus its value in the lane that the DPP control CTRL selects (all lanes valid).
template <int CTRL>
__device__ __forceinline__ double dpp_add(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
    return v + __hiloint2double(hi, lo);
}

// Sum over aligned groups of L = 8 or 16 lanes, in every lane of the group, by
// DPP moves: lane swaps within quads (xor 1, xor 2), then the mirror within
// each half row (8 lanes) and, for 16, within the row.
template <int L>
__device__ __forceinline__ double group_sum(double v) {
    static_assert(L == 8 || L == 16, "groups of 8 or 16 lanes");
    v = dpp_add<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);   // row_half_mirror
    if constexpr (L == 16) v = dpp_add<0x140>(v);   // row_mirror
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

template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Channels [c0, c0 + 8) of row n of head h of R(P): the input minus the stored
// centroids of the P earlier stages, subtracted in stage order in fp32.
// (The stage loop is not unrolled: its pointers are read from the kernel
// arguments as needed instead of occupying registers for all MAX_PREV stages.)
template <int D, typename KVT>
__device__ __forceinline__ void src_row8(const Src &s, int h, int64_t n, int c0, float (&v)[8]) {
    load8<KVT>(static_cast<const KVT *>(s.x) + (size_t)h * s.x_hs + (size_t)n * D + c0, v);
#pragma unroll 1
    for (int p = 0; p < s.P; ++p) {
        const int k = s.pi[p][(size_t)h * s.pi_hs + n];
        float c[8];
        load8<KVT>(static_cast<const KVT *>(s.cent[p]) + ((size_t)h * s.K + k) * D + c0, c);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] - c[i];
    }
}

// The same 8 channels rounded to bf16 and packed for the matrix cores.
template <int D, typename KVT>
__device__ __forceinline__ uint4 src_row8_bf16(const Src &s, int h, int64_t n, int c0) {
    if constexpr (sizeof(KVT) == 2) {
        if (s.P == 0)   // the input itself is the operand
            return *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(s.x) + (size_t)h * s.x_hs +
                                                    (size_t)n * D + c0);
    }
    float v[8];
    src_row8<D, KVT>(s, h, n, c0, v);
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                      pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

#define QVG_DISPATCH_DT(D, dtype, ...)                          \
    do {                                                        \
        if (D == 128) {                                         \
            constexpr int DD = 128;                             \
            if (dtype == DT_BF16) { using KVT = uint16_t; __VA_ARGS__; } \
            else { using KVT = float; __VA_ARGS__; }           \
        } else {                                                \
            constexpr int DD = 64;                              \
            if (dtype == DT_BF16) { using KVT = uint16_t; __VA_ARGS__; } \
            else { using KVT = float; __VA_ARGS__; }           \
        }                                                       \
    } while (0)

// ---------------------------------------------------------------------------
// cold start: Forgy rows from a keyed partial Fisher-Yates shuffle
// ---------------------------------------------------------------------------

constexpr uint64_t SPLITMIX_GAMMA = 0x9E3779B97F4A7C15ull;

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output i of a stream keyed by
// `key` is the finaliser applied to key + (i + 1) * gamma.
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1) * SPLITMIX_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int FORGY_TABLE = 256;   // K <= 256 steps

// One workgroup per (head, stage).  Step i of the shuffle swaps a[i] with
// a[j_i], j_i = i + r_i mod (N - i), and position i is final after step i, so
// entry i is the value at position j_i once steps 0 .. i-1 are done.  The draws
// do not depend on the shuffle: all j_i are computed at once, and thread i
// finds its entry by undoing steps i-1 .. 0 on the position j_i (a swap of m
// and j_m maps m to j_m and j_m to m); the position it ends at is the value,
// since the shuffle starts from the identity.
__global__ __launch_bounds__(FORGY_TABLE) void k_forgy(int H, int N, int K, uint64_t seed, int32_t *idx) {
    __shared__ int32_t jv[FORGY_TABLE];
    __shared__ int32_t sel[FORGY_TABLE];
    const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    const uint64_t key = (seed * 65536ull + (uint64_t)h) * 64ull + (uint64_t)(t + 1);
    const int steps = K < N ? K : N;
    if (tid < steps) jv[tid] = tid + (int)(splitmix64_at(key, (uint64_t)tid) % (uint64_t)(N - tid));
    __syncthreads();
    if (tid < steps) {
        int p = jv[tid];
        for (int m = tid - 1; m >= 0; --m) {
            const int jm = jv[m];
            p = p == m ? jm : (p == jm ? m : p);
        }
        sel[tid] = p;
    }
    __syncthreads();
    // fewer tokens than centroids: entry k repeats entry k mod N
    int32_t *out = idx + ((size_t)t * H + h) * K;
    if (tid < K) out[tid] = sel[tid < steps ? tid : tid % N];
}

hipError_t launch_forgy(int T, int H, int N, int K, uint64_t seed, int32_t *idx, hipStream_t s) {
    QVG_KERNEL(k_forgy, dim3(H, T), dim3(FORGY_TABLE), 0, s, H, N, K, seed, idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// centroid rows: C (fp32) and Cb (bf16 operand)
// ---------------------------------------------------------------------------

// Starting centroids: D/8 threads per row (8 channels each), 256 threads per
// block, rows in (head, row) order over the padded tables.
template <int D, typename KVT>
__global__ __launch_bounds__(256) void k_init_centroids(int H, int K, int Kp, Src src, const int32_t *idx,
                                                        const float *warm, float *C, uint16_t *Cb, int32_t *cnt0,
                                                        int32_t *fill0, uint32_t *vstats_clear) {
    constexpr int TPR = D / 8;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rowg = g / TPR;
    if (rowg >= (int64_t)H * Kp) return;
    const int j = (int)(g - rowg * TPR);
    const int h = (int)(rowg / Kp), k = (int)(rowg - (int64_t)h * Kp);
    if (vstats_clear && k == 0 && j < 2 * VSTAT_BLOCKS)   // neutral value statistics
        vstats_clear[(size_t)h * 2 * VSTAT_BLOCKS + j] = (j & 1) ? 0u : 0xFFFFFFFFu;
    if (j == 0 && cnt0) {
        cnt0[(size_t)h * Kp + k] = 0;
        fill0[(size_t)h * Kp + k] = 0;
    }
    uint4 *cb = reinterpret_cast<uint4 *>(Cb + ((size_t)h * Kp + k) * D + j * 8);
    if (k >= K) {  // padding rows (the assign never chooses them)
        *cb = make_uint4(0, 0, 0, 0);
        return;
    }
    float v[8];
    if (warm) load8<float>(warm + ((size_t)h * K + k) * D + j * 8, v);
    else src_row8<D, KVT>(src, h, idx[(size_t)h * K + k], j * 8, v);
    uint32_t bb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) bb[i] = f32_to_bf16(v[i]);
    float4 *c = reinterpret_cast<float4 *>(C + ((size_t)h * K + k) * D + j * 8);
    c[0] = make_float4(v[0], v[1], v[2], v[3]);
    c[1] = make_float4(v[4], v[5], v[6], v[7]);
    *cb = make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16));
}

hipError_t launch_init_centroids(int D, int dtype, int H, int K, const Src &src, const int32_t *idx,
                                 const float *warm, float *C, uint16_t *Cb, int32_t *cnt0, int32_t *fill0,
                                 uint32_t *vstats_clear, hipStream_t s) {
    const int Kp = padded_k(K);
    const int64_t threads = (int64_t)H * Kp * (D / 8);
    if ((threads + 255) / 256 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    QVG_DISPATCH_DT(D, dtype,
                    QVG_KERNEL((k_init_centroids<DD, KVT>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                               H, K, Kp, src, idx, warm, C, Cb, cnt0, fill0, vstats_clear));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// assignment: distances on the matrix cores, exact decision of near ties
// ---------------------------------------------------------------------------
//
// v_mfma_f32_16x16x32_bf16 accumulates, per token and centroid,
//   acc = <x, c> - |c|^2 / 2 - (|x|^2 (1 + 2^-12) + 2^-100) / 2
//       = -(|x - c|^2 + 2^-12 |x|^2 + 2^-100) / 2,
// negative and largest for the nearest centroid.  The A operand is a block of
// 16 centroids, the B operand a block of 16 tokens, 32 channels per
// instruction: lane l feeds row/column l % 16 with channels 8 (l / 16) .. +7
// of the k-step on both sides, and the 16x16 result leaves centroid
// 4 (l / 16) + r of token l % 16 in accumulator r of lane l.  The constant
// terms enter as the instruction's C operand.
//
// Each lane keeps the two largest accumulators of its token as keys: the
// value with its low mantissa byte replaced by the centroid's number
// (v_perm_b32).  Among negative floats a larger low byte is a smaller value,
// so equal truncated values go to the lower number; v_med3_f32 keeps the two
// best, and the four lanes of a token merge their pairs into its three best.
//
// Exactness.  The bf16 products are exact in fp32; the instruction adds them
// and C with fp32 roundings along a shallow tree (an in-kernel probe shows the
// partial sums rounded to fp32).  With four chained instructions every
// accumulator is within 24 ulp (2^-18.4 relative) of
//   S = |C| + sum |x_i c_i|  <=  |x|^2 + |c|^2 (about),
// which keeps every value negative (the 2^-12 |x|^2 margin is far larger)
// and misorders two centroids only if they lie within
// 2^-17.4 (|x|^2 + max |c|^2) of each other; a key is within 2^-15 of its
// value.  (The 24 ulp assume every rounding directed, 1 ulp, at each of six
// levels of each instruction; round-to-nearest halves it.)  A candidate whose
// key is further below the best key k1 than
//   2^-17 (|x|^2 + max |c|^2) + 2^-14 (|k1| + |k|)
// cannot be the nearest; a token with no such second or third candidate keeps
// the fp32 winner.  The others are re-decided on fp64 distances of the two or
// three candidates, 16 lanes per token: every bf16 x bf16 product is exact in
// fp64 and the sums are exact for the value ranges met in practice, so the
// decision is that of |c|^2 - 2 <x, c>, lowest index on ties.  Every centroid
// that could be the nearest is a candidate unless four or more lie within
// the band, or three within one lane's quarter of the centroids (the lane
// keeps two); then a candidate within the band is chosen, whose distance is
// within the band of the nearest one's.
//
// A workgroup is 16 waves, each taking 32-token tiles; the bf16 tables of up
// to two heads (rows of D / 8 + 1 16-byte chunks, the last unused, so that the
// 16 rows of an operand read start on 16 different chunk positions: 68 KiB
// each at 256 x 128) and their norms sit in LDS: one workgroup per CU, four
// waves per SIMD.

constexpr int ASSIGN_TB = 2;              // 16-token blocks per wave
constexpr int TILE = 16 * ASSIGN_TB;      // tokens per wave
constexpr int ASSIGN_WAVES = 16;          // waves per workgroup
constexpr float PAD_HALF_NORM = -1e30f;   // padding rows: never the nearest

__device__ __forceinline__ float fmax_key(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, __FLT_MAX__); }
__device__ __forceinline__ float fmin_key(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, -__FLT_MAX__); }
// the largest of three keys in one instruction (the compiler would guard a
// chain of maxima with canonicalising moves; keys are never NaN)
__device__ __forceinline__ float fmax3_key(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// fp32(x - c) of eight bf16 pairs, rounded back to bf16.
__device__ __forceinline__ uint4 sub_bf16x8(uint4 x, uint4 c) {
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(__uint_as_float(xw[i] << 16) - __uint_as_float(cw[i] << 16),
                           __uint_as_float(xw[i] & 0xFFFF0000u) - __uint_as_float(cw[i] & 0xFFFF0000u));
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// The B operands of the TILE tokens from tok0 (zero past N): channels
// 32 s + 8 g .. +7 of R(P) for k-step s, rounded to bf16.  Rows past N read
// row N - 1 and are zeroed afterwards, so every load is issued unconditionally
// and the loads of a stage are in flight together.  ANYP: any number of
// earlier stages (else a bf16 tensor with at most one).
template <int D, typename KVT, bool ANYP>
__device__ __forceinline__ void assign_load(const Src &src, int h, int N, int tok0, bf16x8_t (&bt)[ASSIGN_TB][D / 32]) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    int n[ASSIGN_TB];   // tokens past N read row N - 1 again; their results are never stored
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) n[b] = min(tok0 + 16 * b + r16, N - 1);
    if constexpr (sizeof(KVT) == 2 && !ANYP) {
        {   // the input, or the input less one stored bf16 table
            uint4 xr[ASSIGN_TB][KS];
#pragma unroll
            for (int b = 0; b < ASSIGN_TB; ++b) {
                const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src.x) +
                                                                   (size_t)h * src.x_hs + (size_t)n[b] * D + 8 * g);
#pragma unroll
                for (int s = 0; s < KS; ++s) xr[b][s] = row[4 * s];
            }
            if (src.P == 1) {
                int k[ASSIGN_TB];
#pragma unroll
                for (int b = 0; b < ASSIGN_TB; ++b) k[b] = src.pi[0][(size_t)h * src.pi_hs + n[b]];
                // one token block at a time: the table rows come from L2, and
                // holding both blocks' rows at once would exceed the register budget
#pragma unroll
                for (int b = 0; b < ASSIGN_TB; ++b) {
                    const uint4 *row = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src.cent[0]) +
                                                                       ((size_t)h * src.K + k[b]) * D + 8 * g);
                    uint4 cr[KS];
#pragma unroll
                    for (int s = 0; s < KS; ++s) cr[s] = row[4 * s];
#pragma unroll
                    for (int s = 0; s < KS; ++s) xr[b][s] = sub_bf16x8(xr[b][s], cr[s]);
                }
            }
#pragma unroll
            for (int b = 0; b < ASSIGN_TB; ++b)
#pragma unroll
                for (int s = 0; s < KS; ++s) bt[b][s] = __builtin_bit_cast(bf16x8_t, xr[b][s]);
        }
        return;
    }
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        float v[KS][8];
        const KVT *xr = static_cast<const KVT *>(src.x) + (size_t)h * src.x_hs + (size_t)n[b] * D + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) load8<KVT>(xr + 32 * s, v[s]);
#pragma unroll 1
        for (int p = 0; p < src.P; ++p) {
            const int k = src.pi[p][(size_t)h * src.pi_hs + n[b]];
            const KVT *cr = static_cast<const KVT *>(src.cent[p]) + ((size_t)h * src.K + k) * D + 8 * g;
            float c[KS][8];
#pragma unroll
            for (int s = 0; s < KS; ++s) load8<KVT>(cr + 32 * s, c[s]);
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) v[s][i] = v[s][i] - c[s][i];
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 w = make_uint4(pack_bf16x2(v[s][0], v[s][1]), pack_bf16x2(v[s][2], v[s][3]),
                                       pack_bf16x2(v[s][4], v[s][5]), pack_bf16x2(v[s][6], v[s][7]));
            bt[b][s] = __builtin_bit_cast(bf16x8_t, w);
        }
    }
}

// One wave: the nearest centroid of the TILE tokens from tok0, whose operands are in bt.
// ROUT: the next stage's operand may be written (launches with the specialised operand load).
template <int D, typename KVT, bool ROUT>
__device__ __forceinline__ void assign_wave(const Src &src, int h, int N, int tok0, const bf16x8_t (&bt)[ASSIGN_TB][D / 32],
                                            const uint4 *lds, const double *lcn64, const float *lhcn, int32_t *list,
                                            uint8_t *labs, int Kp, uint8_t *pi, int64_t pi_hs, int32_t *counts,
                                            uint16_t *rout, const Src &rsrc, int32_t *changed) {
    constexpr int KS = D / 32;
    constexpr int CH = D / 8;
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    // |x|^2 of each token and its share hb of the C operand
    float hb[ASSIGN_TB];
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        float t = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 xv = __builtin_bit_cast(uint4, bt[b][s]);
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xv.x), __builtin_bit_cast(bf16x2_t, xv.x), t, false);
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xv.y), __builtin_bit_cast(bf16x2_t, xv.y), t, false);
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xv.z), __builtin_bit_cast(bf16x2_t, xv.z), t, false);
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xv.w), __builtin_bit_cast(bf16x2_t, xv.w), t, false);
        }
        t += __shfl_xor(t, 16);
        t += __shfl_xor(t, 32);
        hb[b] = -0.5f * fmaf(t, 1.0f + 0x1p-12f, 0x1p-100f);
        if (g == 0) list[16 * b + r16] = __float_as_int(t);   // |x|^2 waits in LDS (the list space)
    }
    // the two best keys of each (lane, token); the low byte holds 4 cb + r,
    // the lane's part 4 g of the centroid number is put in before the merge
    float q1[ASSIGN_TB], q2[ASSIGN_TB];
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) q1[b] = q2[b] = -__FLT_MAX__;
    const uint32_t sel = 0x07060500u;   // bytes 3..1 from the accumulator, byte 0 from the number
    const int ncb = Kp / 16;
    // row cb * 16 + r16 of the table, the lane's chunk 4 s + g of step s: rows
    // are CH + 1 chunks apart, so every address is a constant offset from one
    // base (and the 16 rows of a read fall on 16 different chunk positions)
    const uint4 *arow = lds + r16 * (CH + 1) + g;
    const float4 *cnp = reinterpret_cast<const float4 *>(lhcn + 4 * g);
    // accumulators of the centroid block at offset j blocks from the pointers
    auto dots = [&](int j, f32x4_t (&acc)[ASSIGN_TB]) {
        bf16x8_t a[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = __builtin_bit_cast(bf16x8_t, arow[j * 16 * (CH + 1) + 4 * s]);
        const float4 cn = cnp[j * 4];
#pragma unroll
        for (int b = 0; b < ASSIGN_TB; ++b)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a[0], bt[b][0], f32x4_t{cn.x + hb[b], cn.y + hb[b], cn.z + hb[b], cn.w + hb[b]}, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < KS; ++s)
#pragma unroll
            for (int b = 0; b < ASSIGN_TB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bt[b][s], acc[b], 0, 0, 0);
    };
    // fold the accumulators of centroid block cb into the two best keys, two
    // keys at a time: with q1 >= q2, the second largest of {q1, q2, ka, kb} is
    // max(q2, med3(q1, ka, kb))
    auto keys = [&](int cb, const f32x4_t (&acc)[ASSIGN_TB]) {
#pragma unroll
        for (int b = 0; b < ASSIGN_TB; ++b) {
            float key[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                key[r] = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(acc[b][r]), (uint32_t)(4 * cb + r), sel));
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                q2[b] = fmax_key(q2[b], __builtin_amdgcn_fmed3f(q1[b], key[r], key[r + 1]));
                q1[b] = fmax3_key(q1[b], key[r], key[r + 1]);
            }
        }
    };
    // Two-stage pipeline: the matrix cores work on block cb + 1 while the
    // vector ALUs fold block cb.
    f32x4_t accA[ASSIGN_TB], accB[ASSIGN_TB];
    // a wave in its block loop issues ahead of the SIMD's other waves (in the
    // merge, the near-tie pass or a tile's setup), so the matrix core stays fed
    __builtin_amdgcn_s_setprio(2);
    dots(0, accA);
    int cb = 0;
    for (; cb + 2 < ncb; cb += 2) {
        dots(1, accB);
        keys(cb, accA);
        dots(2, accA);
        keys(cb + 1, accB);
        arow += 32 * (CH + 1);
        cnp += 8;
    }
    if (cb + 1 < ncb) {
        dots(1, accB);
        keys(cb, accA);
        keys(cb + 1, accB);
    } else {
        keys(cb, accA);
    }
    __builtin_amdgcn_s_setprio(0);
    float xx[ASSIGN_TB];
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) xx[b] = __int_as_float(list[16 * b + r16]);
    __builtin_amdgcn_wave_barrier();
    // merge the four lanes of each token into its three best keys, settle the
    // clear cases, list the near ties
    int n_list = 0;
    int nchg = 0;   // labels this lane changed (counted when `changed` is set)
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        uint32_t u1 = __float_as_uint(q1[b]), u2 = __float_as_uint(q2[b]);
        u1 = (u1 & 0xFFFFFF03u) | ((u1 & 0xFCu) << 2) | (uint32_t)(4 * g);
        u2 = (u2 & 0xFFFFFF03u) | ((u2 & 0xFCu) << 2) | (uint32_t)(4 * g);
        float k1 = __uint_as_float(u1), k2 = __uint_as_float(u2), k3 = -__FLT_MAX__;
        // the three largest of two sorted triples a, w: the j-th largest of the
        // union is the maximum over i of min(a_i, w_(j-i)) with a_0 = w_0 = +inf
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float w1 = __shfl_xor(k1, o), w2 = __shfl_xor(k2, o), w3 = __shfl_xor(k3, o);
            k3 = fmax_key(fmax_key(k3, w3), fmax_key(fmin_key(k1, w2), fmin_key(k2, w1)));
            k2 = fmax_key(fmin_key(k1, w1), fmax_key(k2, w2));
            k1 = fmax_key(k1, w1);
        }
        const int c1 = (int)(__float_as_uint(k1) & 0xFFu), c2 = (int)(__float_as_uint(k2) & 0xFFu);
        const int c3 = (int)(__float_as_uint(k3) & 0xFFu);
        const float tol2 = 0x1p-17f * (xx[b] - 2.0f * fminf(lhcn[c1], lhcn[c2])) + 0x1p-14f * (fabsf(k1) + fabsf(k2));
        const float tol3 = 0x1p-17f * (xx[b] - 2.0f * fminf(lhcn[c1], lhcn[c3])) + 0x1p-14f * (fabsf(k1) + fabsf(k3));
        const bool third = (k1 - k3) <= tol3;   // c3 might be the nearest too
        const bool tie = third || (k1 - k2) <= tol2;
        const int n = tok0 + 16 * b + r16;
        const bool mine = g == 0 && n < N;
        if (mine && !tie) {
            uint8_t *pp = pi + (size_t)h * pi_hs + n;
            if (changed) nchg += (int)*pp != c1;
            *pp = (uint8_t)c1;
            if (counts) atomicAdd(&counts[(size_t)h * Kp + c1], 1);
            if (rout) labs[16 * b + r16] = (uint8_t)c1;
        }
        const uint64_t m = __ballot(mine && tie);
        if (mine && tie) {
            const int pos = n_list + __popcll(m & ((1ull << lane) - 1ull));
            list[pos] = ((16 * b + r16) << 24) | (c1 << 16) | (c2 << 8) | (third ? c3 : c2);
        }
        n_list += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    // near ties: 16 lanes per token, 8 channels each, fp64 distances of the two
    // (or three) candidates
    const int sub = lane & 15, grp = lane >> 4;
    for (int j0 = 0; j0 < n_list; j0 += 4) {
        const int j = j0 + grp;
        const int e = list[j < n_list ? j : 0];
        const int nl = (e >> 24) & 0xFF, c1 = (e >> 16) & 0xFF, c2 = (e >> 8) & 0xFF, c3 = e & 0xFF;
        const int n = tok0 + nl;
        const bool any3 = __ballot(j < n_list && c3 != c2) != 0;   // a third candidate in this batch
        double p1 = 0.0, p2 = 0.0, p3 = 0.0;   // <x, c1>, <x, c2>, <x, c3>
        if (j < n_list && sub < CH) {
            const uint4 xv = src_row8_bf16<D, KVT>(src, h, n, 8 * sub);
            const uint4 a1 = lds[c1 * (CH + 1) + sub];
            const uint4 a2 = lds[c2 * (CH + 1) + sub];
            const uint4 a3 = lds[c3 * (CH + 1) + sub];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
            const uint32_t aw[4] = {a1.x, a1.y, a1.z, a1.w};
            const uint32_t bw[4] = {a2.x, a2.y, a2.z, a2.w};
            const uint32_t cw[4] = {a3.x, a3.y, a3.z, a3.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double xl = (double)__uint_as_float(xw[i] << 16);
                const double xh = (double)__uint_as_float(xw[i] & 0xFFFF0000u);
                p1 = fma(xl, (double)__uint_as_float(aw[i] << 16), p1);
                p1 = fma(xh, (double)__uint_as_float(aw[i] & 0xFFFF0000u), p1);
                p2 = fma(xl, (double)__uint_as_float(bw[i] << 16), p2);
                p2 = fma(xh, (double)__uint_as_float(bw[i] & 0xFFFF0000u), p2);
                if (any3) {
                    p3 = fma(xl, (double)__uint_as_float(cw[i] << 16), p3);
                    p3 = fma(xh, (double)__uint_as_float(cw[i] & 0xFFFF0000u), p3);
                }
            }
        }
        p1 = group_sum<16>(p1);
        p2 = group_sum<16>(p2);
        if (any3) p3 = group_sum<16>(p3);
        if (j < n_list && sub == 0) {
            const double e1 = lcn64[c1] - 2.0 * p1, e2 = lcn64[c2] - 2.0 * p2;
            int best = (e2 < e1 || (e2 == e1 && c2 < c1)) ? c2 : c1;
            if (c3 != c2) {
                const double eb = best == c1 ? e1 : e2, e3 = lcn64[c3] - 2.0 * p3;
                if (e3 < eb || (e3 == eb && c3 < best)) best = c3;
            }
            uint8_t *pp = pi + (size_t)h * pi_hs + n;
            if (changed) nchg += (int)*pp != best;
            *pp = (uint8_t)best;
            if (counts) atomicAdd(&counts[(size_t)h * Kp + best], 1);
            if (rout) labs[nl] = (uint8_t)best;
        }
    }
    if (changed) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) nchg += __shfl_xor(nchg, o);
        if (lane == 0 && nchg) atomicAdd(&changed[h], nchg);
    }
    if (!ROUT || !rout) return;
    // the next stage's operand bf16(R(t)) = bf16(fp32(R(t-1) - c)), c the token's
    // stored row: from the operands when they are R(t-1) itself (the input of
    // stage 1), else from R(t-1) rebuilt in fp32 by rsrc
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int b = 0; b < ASSIGN_TB; ++b) {
        const int n = tok0 + 16 * b + r16;
        const int L = n < N ? (int)labs[16 * b + r16] : 0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 c = lds[L * (CH + 1) + 4 * s + g];
            uint4 r;
            if (rsrc.P == 0) {
                r = sub_bf16x8(__builtin_bit_cast(uint4, bt[b][s]), c);
            } else {
                float v[8];
                src_row8<D, KVT>(rsrc, h, min(n, N - 1), 32 * s + 8 * g, v);
                const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = v[2 * i] - __uint_as_float(cw[i] << 16);
                    v[2 * i + 1] = v[2 * i + 1] - __uint_as_float(cw[i] & 0xFFFF0000u);
                }
                r = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7]));
            }
            if (n < N) *reinterpret_cast<uint4 *>(rout + ((size_t)h * N + n) * D + 32 * s + 8 * g) = r;
        }
    }
}

// Persistent workgroups, one per CU: each owns a contiguous run of the
// (head, tile) units, XCD by XCD so that an XCD's L2 serves the tables of a run
// of heads.  The run is taken in windows of at most two heads whose tables are
// staged together in LDS (a run shorter than a head's tiles is one window), and
// the waves take the window's tiles from an LDS counter.
template <int D, typename KVT, bool ANYP>
__global__ __launch_bounds__(64 * ASSIGN_WAVES, 4) void k_assign(Src src, int H, int N, const uint16_t *__restrict__ Cb,
                                                                 int K, int Kp, uint8_t *__restrict__ pi,
                                                                 int64_t pi_hs, int32_t *__restrict__ counts,
                                                                 uint32_t *__restrict__ vstats,
                                                                 uint16_t *__restrict__ rout, Src rsrc,
                                                                 const int32_t *__restrict__ skip,
                                                                 const int32_t *__restrict__ nskip,
                                                                 int32_t *__restrict__ changed) {
    constexpr int CH = D / 8;
    constexpr int NT = 64 * ASSIGN_WAVES;
    constexpr int STAGE = (256 * CH + NT - 1) / NT;   // table chunks per thread at 256 centroids
    extern __shared__ uint4 lds[];                      // two table slots
    double *lcn64 = reinterpret_cast<double *>(lds + 2 * Kp * (CH + 1));
    float *lhcn = reinterpret_cast<float *>(lcn64 + 2 * Kp);
    int32_t *lists = reinterpret_cast<int32_t *>(lhcn + 2 * Kp);
    int32_t *next = lists + ASSIGN_WAVES * TILE;
    uint8_t *labs = reinterpret_cast<uint8_t *>(next + 4);   // [ASSIGN_WAVES][TILE] labels for rout
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (nskip && *nskip >= H) return;   // every head has stopped
    const int T = (N + TILE - 1) / TILE;   // tiles per head
    const int64_t U = (int64_t)H * T;
    const int64_t r = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t u1 = U * (r + 1) / gridDim.x;
    const int nch = Kp * CH;
    for (int64_t u = U * r / gridDim.x; u < u1;) {
        const int h0 = (int)(u / T);
        const int nh = (int)min((int64_t)2, (u1 - 1) / T - h0 + 1);   // heads in this window
        const int e = (int)min(u1, (int64_t)(h0 + nh) * T);
        // the thread index is re-read here so that the staging addresses are
        // formed per window instead of being held in registers across windows
        int t0 = tid;
        asm volatile("" : "+v"(t0));
        for (int sl = 0; sl < nh; ++sl) {
            if (skip && skip[h0 + sl]) continue;   // a stopped head's tiles are not taken
            const uint4 *csrc = reinterpret_cast<const uint4 *>(Cb + (size_t)(h0 + sl) * Kp * D);
            uint4 st[STAGE];
#pragma unroll
            for (int k = 0; k < STAGE; ++k) {   // unconditional loads: rows past the table read its last chunk
                const int i = t0 + NT * k;
                st[k] = csrc[i < nch ? i : nch - 1];
            }
            uint4 *slot = lds + sl * Kp * (CH + 1);
#pragma unroll
            for (int k = 0; k < STAGE; ++k) {
                const int i = t0 + NT * k;
                const int row = i / CH, q = i - row * CH;
                if (i < nch) slot[row * (CH + 1) + q] = st[k];
                // |c|^2 of the row: the CH lanes holding its chunks are neighbours;
                // every bf16 square is exact in fp64
                const uint32_t w[4] = {st[k].x, st[k].y, st[k].z, st[k].w};
                double sq = 0.0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const double lo = (double)__uint_as_float(w[j] << 16), hi = (double)__uint_as_float(w[j] & 0xFFFF0000u);
                    sq = fma(lo, lo, sq);
                    sq = fma(hi, hi, sq);
                }
                sq = group_sum<CH>(sq);
                if (q == 0 && i < nch) {
                    const bool real = row < K;   // padding rows are never chosen
                    lcn64[sl * Kp + row] = real ? sq : __builtin_inf();
                    lhcn[sl * Kp + row] = real ? -0.5f * (float)sq : PAD_HALF_NORM;
                }
            }
        }
        if (tid == 0) *next = (int)u;
        __syncthreads();
        for (;;) {
            int m = 0;
            if (lane == 0) m = atomicAdd(next, 1);
            m = __builtin_amdgcn_readfirstlane(m);
            if (m >= e) break;
            const int h = m / T, sl = h - h0;
            if (skip && skip[h]) continue;
            const int tok0 = (m - h * T) * TILE;
            bf16x8_t bt[ASSIGN_TB][D / 32];
            assign_load<D, KVT, ANYP>(src, h, N, tok0, bt);
            if constexpr (!ANYP) {
                if (vstats) {   // the input's value statistics, from the operands (bf16 input, first stage)
                    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
                    for (int b = 0; b < ASSIGN_TB; ++b)
#pragma unroll
                        for (int ks = 0; ks < D / 32; ++ks) {
                            const uint4 q = __builtin_bit_cast(uint4, bt[b][ks]);
                            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) {
                                const uint32_t lo = w[jj] & 0x7FFFu, hi = (w[jj] >> 16) & 0x7FFFu;
                                mx = max(mx, max(lo, hi));
                                mn = min(mn, min(lo - 1u, hi - 1u));   // zero wraps to the largest value
                            }
                        }
                    mn = (uint32_t)wave_min_i((int)(mn ^ 0x80000000u)) ^ 0x80000000u;   // unsigned minimum
                    mx = wave_max_u(mx);
                    if (lane == 0) {
                        atomicMin(&vstats[(size_t)h * 2 * VSTAT_BLOCKS], mn);
                        atomicMax(&vstats[(size_t)h * 2 * VSTAT_BLOCKS + 1], mx);
                    }
                }
            }
            assign_wave<D, KVT, !ANYP>(src, h, N, tok0, bt, lds + sl * Kp * (CH + 1), lcn64 + sl * Kp, lhcn + sl * Kp,
                                lists + wave * TILE, labs + wave * TILE, Kp, pi, pi_hs, counts, rout, rsrc, changed);
        }
        __syncthreads();   // the tables are replaced only once every wave is done with them
        u = e;
    }
}

static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

hipError_t launch_assign(int D, int dtype, int H, int N, int K, const Src &src, const uint16_t *Cb, uint8_t *pi,
                         int64_t pi_hs, int32_t *counts, uint32_t *vstats, uint16_t *rout, const Src *rsrc,
                         const int32_t *skip, const int32_t *nskip, int32_t *changed, hipStream_t s) {
    const int Kp = padded_k(K);
    const size_t lds = 2 * ((size_t)Kp * (D / 8 + 1) * 16 + (size_t)Kp * 12) + (ASSIGN_WAVES * TILE + 4) * sizeof(int32_t) +
                       ASSIGN_WAVES * TILE;
    // one resident workgroup per CU, at least a tile per wave
    const int64_t units = (int64_t)H * ((N + TILE - 1) / TILE);
    if (units >= (int64_t)1 << 31) return hipErrorInvalidValue;
    const int64_t nb = std::min<int64_t>((int64_t)device_cus(), (units + ASSIGN_WAVES - 1) / ASSIGN_WAVES);
    dim3 g((unsigned)std::max<int64_t>(nb, 1)), b(64 * ASSIGN_WAVES);
    // bf16 tensors with at most one earlier stage (every stage at T <= 2) take the
    // specialised operand load
    const bool anyp = !(dtype == DT_BF16 && src.P <= 1);
    if (rout && (anyp || (!rsrc && src.P != 0))) return hipErrorInvalidValue;
    const Src &rs = rsrc ? *rsrc : src;   // where rout's fp32 R(t-1) comes from
    QVG_DISPATCH_DT(D, dtype, {
        if (anyp || sizeof(KVT) != 2) {
            (void)hipFuncSetAttribute((const void *)k_assign<DD, KVT, true>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            QVG_KERNEL((k_assign<DD, KVT, true>), g, b, lds, s, src, H, N, Cb, K, Kp, pi, pi_hs, counts,
                       (uint32_t *)nullptr, (uint16_t *)nullptr, src, skip, nskip, changed);
        } else {
            using KB = uint16_t;   // (this branch is only taken for bf16)
            (void)hipFuncSetAttribute((const void *)k_assign<DD, KB, false>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            QVG_KERNEL((k_assign<DD, KB, false>), g, b, lds, s, src, H, N, Cb, K, Kp, pi, pi_hs, counts, vstats, rout,
                       rs, skip, nskip, changed);
        }
    });
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// update, part 1: group each head's tokens by centroid
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_count(int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts) {
    const int h = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n < N) atomicAdd(&counts[(size_t)h * Kp + pi[(size_t)h * pi_hs + n]], 1);
}

hipError_t launch_count(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, int32_t *counts, hipStream_t s) {
    QVG_KERNEL(k_count, dim3((N + 255) / 256, H), dim3(256), 0, s, N, Kp, pi, pi_hs, counts);
    return hipGetLastError();
}

// Each block recomputes the head's exclusive prefix of the counts (256 values)
// and places its tokens with one atomic per token.
__global__ __launch_bounds__(256) void k_scatter(int N, int Kp, const uint8_t *pi, int64_t pi_hs,
                                                 const int32_t *counts, int32_t *fill, int32_t *offsets,
                                                 int32_t *order, const int32_t *skip) {
    __shared__ int32_t off[256];
    __shared__ int32_t wsum[4];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (skip && skip[h]) return;   // a stopped head's counts are stale
    const int v = tid < Kp ? counts[(size_t)h * Kp + tid] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wsum[w];
    const int excl = x + add - v;
    off[tid] = excl;
    if (blockIdx.x == 0 && tid < Kp) offsets[(size_t)h * Kp + tid] = excl;
    __syncthreads();
    const int n = blockIdx.x * 256 + tid;
    if (n < N) {
        const int k = pi[(size_t)h * pi_hs + n];
        const int pos = atomicAdd(&fill[(size_t)h * Kp + k], 1);
        order[(size_t)h * N + off[k] + pos] = n;
    }
}

hipError_t launch_scatter(int H, int N, int Kp, const uint8_t *pi, int64_t pi_hs, const int32_t *counts,
                          int32_t *fill, int32_t *offsets, int32_t *order, const int32_t *skip, hipStream_t s) {
    QVG_KERNEL(k_scatter, dim3((N + 255) / 256, H), dim3(256), 0, s, N, Kp, pi, pi_hs, counts, fill,
                       offsets, order, skip);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// update, part 2: exact mean of each centroid's rows
// ---------------------------------------------------------------------------
//
// One wave per (centroid, head), four per block.  D/8 lanes cover a row, so a
// wave reads 512/D rows per load and keeps four such loads in flight.
//
// Fast pass: each lane sums its 8 channels in plain fp64 and their magnitudes
// in fp32.  Any order of n additions stays within n 2^-53 sum|v| of the exact
// sum (Higham, Accuracy and Stability of Numerical Algorithms, 2nd ed., 4.2),
// and rounding to fp64, dividing by the count and rounding to fp32 is monotone
// in the sum; so when both ends of the interval the bound allows give the same
// fp32 mean, that mean is the one of the exact sum.  A centroid where some
// channel fails the test is summed again with the error-free two-sum: each
// lane keeps (sum, error) pairs, exact for the value ranges met in practice,
// and the order the rows arrive in does not matter either.  The row slots are
// merged with lane shuffles; the exact total is rounded once to fp64, divided
// by the count and rounded to fp32.

__device__ __forceinline__ void two_sum(double &s, double &e, double x) {
    const double t = s + x;
    const double bp = t - s;
    e += (s - (t - bp)) + (x - bp);
    s = t;
}

// Rows n[u] of R(P), channels [c0, c0 + 8), for U rows at once (every n[u] a
// valid row; slots with !valid[u] come out zero).  Every load of a stage is
// issued for all rows, unconditionally, before any is used.
template <int D, typename KVT, int U>
__device__ __forceinline__ void src_rows8(const Src &s, int h, const int (&n)[U], const bool (&valid)[U], int c0,
                                          float (&v)[U][8]) {
#pragma unroll
    for (int u = 0; u < U; ++u) load8<KVT>(static_cast<const KVT *>(s.x) + (size_t)h * s.x_hs + (size_t)n[u] * D + c0, v[u]);
#pragma unroll 1
    for (int p = 0; p < s.P; ++p) {
        int k[U];
#pragma unroll
        for (int u = 0; u < U; ++u) k[u] = s.pi[p][(size_t)h * s.pi_hs + n[u]];
        const KVT *cp = static_cast<const KVT *>(s.cent[p]) + (size_t)h * s.K * D + c0;
        float c[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8<KVT>(cp + (size_t)k[u] * D, c[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) v[u][i] = v[u][i] - c[u][i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[u][i] = valid[u] ? v[u][i] : 0.f;
}

// Visits the cnt rows of R(P) listed in ord, 8 channels from c0 per lane, as
// f(v) with v[8] in fp32 (only the lanes whose row slot holds a row call f).
template <int D, typename KVT, typename F>
__device__ __forceinline__ void for_rows(const Src &src, int h, const int32_t *ord, int cnt, int slot, int c0, F f) {
    constexpr int RPI = 64 / (D / 8);   // rows per load
    constexpr int UNROLL = 4;
    const int lane = threadIdx.x & 63;
    for (int i0 = 0; i0 < cnt; i0 += 64) {
        const int m = cnt - i0 < 64 ? cnt - i0 : 64;
        const int mine = ord[i0 + (lane < m ? lane : m - 1)];
        for (int j0 = 0; j0 < m; j0 += RPI * UNROLL) {
            float v[UNROLL][8];
            int n[UNROLL];
            bool ok[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int j = j0 + u * RPI + slot;
                n[u] = __shfl(mine, j < 64 ? j : 63);
                ok[u] = j < m;
            }
            src_rows8<D, KVT, UNROLL>(src, h, n, ok, c0, v);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                if (ok[u]) f(v[u]);
        }
    }
}

// fp32(fp64(t) / n) for an fp64 t: the rounding of the mean.
__device__ __forceinline__ float mean_of(double t, int cnt) { return (float)(t / (double)cnt); }

// The convergence test at the start of an update launch (see ConvState): true
// when head h has stopped (now or in an earlier round) and the workgroup has
// nothing to do.  `first` marks the one workgroup of the head that records.
__device__ __forceinline__ bool conv_stop(const ConvState &cv, int h, bool first) {
    if (!cv.threshold) return false;
    if (cv.done[h]) return true;
    if (cv.round > 0 && cv.changed[h] < cv.threshold) {
        if (first) {
            cv.done[h] = 1;
            cv.rounds[h] = cv.round;
            atomicAdd(cv.ndone, 1);
        }
        return true;
    }
    if (first) cv.changed_next[h] = 0;
    return false;
}

template <int D, typename KVT>
__global__ __launch_bounds__(256) void k_update(Src src, int N, int K, int Kp, const int32_t *counts,
                                                const int32_t *offsets, const int32_t *order, float *C, uint16_t *Cb,
                                                int32_t *zero_cnt, int32_t *zero_fill, ConvState cv) {
    constexpr int LPR = D / 8;        // lanes per row
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + (threadIdx.x >> 6), h = blockIdx.y;
    if (conv_stop(cv, h, blockIdx.x == 0 && threadIdx.x == 0)) return;
    if (k >= K) return;
    if (lane == 0 && zero_cnt) {
        zero_cnt[(size_t)h * Kp + k] = 0;
        zero_fill[(size_t)h * Kp + k] = 0;
    }
    const int cnt = counts[(size_t)h * Kp + k];
    if (cnt == 0) return;   // empty cluster keeps its centroid
    const int32_t *ord = order + (size_t)h * N + offsets[(size_t)h * Kp + k];
    const int slot = lane / LPR, c0 = (lane % LPR) * 8;
    float mean[8];
    bool ok = true;
    {
        double hs[8];
        float ab[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { hs[i] = 0.0; ab[i] = 0.f; }
        for_rows<D, KVT>(src, h, ord, cnt, slot, c0, [&](const float (&v)[8]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hs[i] += (double)v[i];
                ab[i] += fabsf(v[i]);
            }
        });
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hs[i] += __shfl_xor(hs[i], o);
                ab[i] += __shfl_xor(ab[i], o);
            }
        }
        // sum|v| <= 1.07 ab (an fp32 sum of cnt <= 2^20 magnitudes); the bound
        // takes 2^-51 for 1.1 x 2^-53 with room for both roundings
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double b = (double)ab[i] * (double)cnt * 0x1p-51 + fabs(hs[i]) * 0x1p-50;
            const float lo = mean_of(hs[i] - b, cnt), hi = mean_of(hs[i] + b, cnt);
            ok = ok && (lo == hi) && cnt <= (1 << 20);
            mean[i] = lo;
        }
    }
    if (!__all(ok)) {   // a channel near a rounding boundary: sum the rows exactly
        double hs[8], es[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { hs[i] = 0.0; es[i] = 0.0; }
        for_rows<D, KVT>(src, h, ord, cnt, slot, c0, [&](const float (&v)[8]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) two_sum(hs[i], es[i], (double)v[i]);
        });
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double oh = __shfl_xor(hs[i], o), oe = __shfl_xor(es[i], o);
                two_sum(hs[i], es[i], oh);
                es[i] += oe;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mean[i] = mean_of(hs[i] + es[i], cnt);
    }
    if (slot == 0) {
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = f32_to_bf16(mean[i]);
        float4 *c = reinterpret_cast<float4 *>(C + ((size_t)h * K + k) * D + c0);
        c[0] = make_float4(mean[0], mean[1], mean[2], mean[3]);
        c[1] = make_float4(mean[4], mean[5], mean[6], mean[7]);
        *reinterpret_cast<uint4 *>(Cb + ((size_t)h * Kp + k) * D + c0) =
            make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
    }
}

hipError_t launch_update(int D, int dtype, int H, int N, int K, const Src &src, const int32_t *counts,
                         const int32_t *offsets, const int32_t *order, float *C, uint16_t *Cb, int32_t *zero_cnt,
                         int32_t *zero_fill, const ConvState &cv, hipStream_t s) {
    const int Kp = padded_k(K);
    QVG_DISPATCH_DT(D, dtype,
                    QVG_KERNEL((k_update<DD, KVT>), dim3((K + 3) / 4, H), dim3(256), 0, s, src, N, K, Kp,
                                       counts, offsets, order, C, Cb, zero_cnt, zero_fill, cv));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// update, segmented: exact means from a per-workgroup token list in LDS
// ---------------------------------------------------------------------------
//
// SEG_RUNS workgroups per head, each with a run of at most SEG_KR consecutive
// centroids that holds about N / SEG_RUNS tokens: centroid k has token share
// floor(P(k) SEG_RUNS / N), where P(k) = count(0) + ... + count(k - 1) is the
// place of its first token in label order, and run r starts at the first
// centroid of share r, moved where needed to keep every run within SEG_KR
// centroids.  A workgroup takes as long as its run has tokens, so equal token
// counts keep the workgroups equally busy (fixed runs of 32 centroids differ
// by up to 1.6x in tokens after a few k-means rounds).  The runs of a head are
// neighbours in xcd_tile order, so they share one XCD's L2 (the head's
// assignments and centroid tables).
//  1. The head's histogram (from the assign) gives the run and its centroids'
//     places in a token list in LDS; one pass over the head's assignments puts
//     every token of the run there, with its labels of the first two earlier
//     stages packed beside it.  No global sort.
//  2. The waves split the run's list evenly.  A wave reads one row per load
//     instruction (64 lanes x D/64 channels, row addresses in scalar
//     registers), rebuilds R(t-1), and sums in fp64 registers while the rows
//     belong to one centroid; when the centroid changes, the partial sums go
//     into that centroid's LDS accumulator.
//  3. Exactness.  If every value of a channel is a multiple of 2^e and every
//     partial sum stays below 2^(53+e) in magnitude, each partial sum is an
//     fp64 number, so each addition (in registers or LDS atomics, in any
//     order) is exact and the accumulator holds the exact sum; fp32(sum / n)
//     is then the exactly rounded mean.
//     Run certificate (no per-value work): fp32(a - b) of two multiples of
//     2^e is again one (when it rounds, its ulp exceeds 2^e) and is at most
//     (|a| + |b|)(1 + 2^-24) in magnitude.  So every value of R(t-1) of a head
//     is a multiple of the smallest ulp among the head's input values and
//     stored centroid tables, and at most the sum of their largest magnitudes
//     (times 1 + 2^-20).  The first assign or k_value_stats provides the
//     input's part, k_store_centroids the tables' (when it stores them).  When
//     (largest count of the run) x (that magnitude) < 2^(53+e), every centroid
//     of the run is certified.
//     Otherwise each centroid collects max|v| and the lowest set bit of its
//     values during the sums and is certified on its own; a centroid without
//     a certificate is summed again by one wave with the interval test and the
//     two-sum pass of k_update.

constexpr int SEG_KR = 32;          // centroids per accumulator window
constexpr int SEG_RUNS = 9;         // workgroups (runs) per head
constexpr int SEG_WAVES = 8;
constexpr int SEG_U = 12;           // rows in flight per wave
constexpr int SEG_EMPTY_E = 4096;   // lowest-bit exponent of a centroid with only zeros so far

// Smallest nonzero and largest magnitude bits (bf16: 15 bits, fp32: 31 bits) of
// each head's count values, as VSTAT_BLOCKS partial pairs per head:
// stats[h][b] = {smallest nonzero magnitude - 1 (0xFFFFFFFF: all zero), largest}.
template <typename KVT>
__global__ __launch_bounds__(256) void k_value_stats(const KVT *x, int64_t x_hs, int64_t count, uint32_t *stats) {
    constexpr int PER = 16 / sizeof(KVT);
    constexpr int STRIDE = 256 * VSTAT_BLOCKS;
    const int h = blockIdx.y;
    const uint4 *p = reinterpret_cast<const uint4 *>(x + (size_t)h * x_hs);
    const int64_t nv = count / PER;   // count is a multiple of PER
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    // four loads in flight; indices past the end read the last chunk again,
    // which leaves a minimum and a maximum unchanged
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += 4 * STRIDE) {
        uint4 q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = p[std::min<int64_t>(i + k * STRIDE, nv - 1)];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(KVT) == 2) {
                    const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
                    mx = max(mx, max(lo, hi));
                    mn = min(mn, min(lo - 1u, hi - 1u));   // zero wraps to the largest value
                } else {
                    const uint32_t a = w[j] & 0x7FFFFFFFu;
                    mx = max(mx, a);
                    mn = min(mn, a - 1u);
                }
            }
        }
    }
    __shared__ uint32_t red[2][4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = mn;
        red[1][threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *o = stats + ((size_t)h * VSTAT_BLOCKS + blockIdx.x) * 2;
        o[0] = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
        o[1] = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    }
}

hipError_t launch_value_stats(int dtype, int H, const void *x, int64_t x_hs, int64_t count, uint32_t *stats,
                              hipStream_t s) {
    const int esz = dtype == DT_BF16 ? 2 : 4;
    if ((count * esz) % 16 != 0 || (x_hs * esz) % 16 != 0) return hipErrorInvalidValue;
    if (dtype == DT_BF16)
        QVG_KERNEL(k_value_stats<uint16_t>, dim3(VSTAT_BLOCKS, H), dim3(256), 0, s,
                   static_cast<const uint16_t *>(x), x_hs, count, stats);
    else
        QVG_KERNEL(k_value_stats<float>, dim3(VSTAT_BLOCKS, H), dim3(256), 0, s, static_cast<const float *>(x),
                   x_hs, count, stats);
    return hipGetLastError();
}

// Exponent of the smallest ulp of the values whose smallest nonzero magnitude
// has bits mbits (bf16: 2^(E-134) at exponent field E, subnormals below that;
// fp32: 2^(E-150)).
template <typename KVT>
__device__ __forceinline__ int ulp_exp_of(uint32_t mbits) {
    if constexpr (sizeof(KVT) == 2) return (int)(mbits >> 7) - 134;
    else return (int)(mbits >> 23) - 150;
}

template <typename KVT>
__device__ __forceinline__ float magnitude_of(uint32_t mbits) {
    if constexpr (sizeof(KVT) == 2) return __uint_as_float(mbits << 16);
    else return __uint_as_float(mbits);
}

// D/64 consecutive channels of a row, as fp32.
template <typename KVT, int CPL>
__device__ __forceinline__ void load_part(const KVT *p, float (&v)[CPL]) {
    if constexpr (sizeof(KVT) == 2) {
        if constexpr (CPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            v[0] = __uint_as_float(w << 16);
            v[1] = __uint_as_float(w & 0xFFFF0000u);
        } else {
            v[0] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
        }
    } else {
        if constexpr (CPL == 2) {
            const float2 f = *reinterpret_cast<const float2 *>(p);
            v[0] = f.x;
            v[1] = f.y;
        } else {
            v[0] = *reinterpret_cast<const float *>(p);
        }
    }
}

// Exponent of the lowest set bit of a nonzero fp32 value (a lower bound for
// subnormals), SEG_EMPTY_E for zeros.
__device__ __forceinline__ int lowest_bit_exp(float v) {
    const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
    const int e = (int)(b >> 23) + (int)__builtin_ctz(b | 0x800000u) - 150;
    return b ? e : SEG_EMPTY_E;
}

// Rows list[j .. j + m) (1 <= m <= U) of R(P), this lane's channels; slots
// u >= m read row list[j] again and come out zero.  A list entry is
// token | label(stage 1) << 16 | label(stage 2) << 24; entries are the same in
// every lane (read into scalar registers).  A row is addressed as the head's
// base plus a 32-bit byte offset, which keeps the scalar registers per row in
// flight to one, and every load is issued unconditionally (a load under a
// branch is waited for inside it).
template <int D, typename KVT, int U>
__device__ __forceinline__ void seg_rows(const Src &s, int h, int N, const uint32_t *list, int j, int m,
                                         float (&v)[U][D / 64]) {
    constexpr int CPL = D / 64;
    constexpr uint32_t ROW = D * sizeof(KVT);
    const uint32_t c0 = (threadIdx.x & 63) * CPL * sizeof(KVT);
    uint32_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) e[u] = __builtin_amdgcn_readfirstlane(list[j + (u < m ? u : 0)]);
    const char *x = reinterpret_cast<const char *>(static_cast<const KVT *>(s.x) + (size_t)h * s.x_hs);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // a token index is below N by construction; the clamp keeps every row read in bounds
        const uint32_t n = min(e[u] & 0xFFFFu, (uint32_t)N - 1u);
        load_part<KVT, CPL>(reinterpret_cast<const KVT *>(x + (n * ROW + c0)), v[u]);
    }
#pragma unroll 1
    for (int p = 0; p < s.P; ++p) {
        const char *cp = reinterpret_cast<const char *>(static_cast<const KVT *>(s.cent[p]) + (size_t)h * s.K * D);
        uint32_t k[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            k[u] = p < 2 ? (e[u] >> (16 + 8 * p)) & 0xFFu
                         : (uint32_t)s.pi[p][(size_t)h * s.pi_hs + min(e[u] & 0xFFFFu, (uint32_t)N - 1u)];
        float c[U][CPL];
#pragma unroll
        for (int u = 0; u < U; ++u) load_part<KVT, CPL>(reinterpret_cast<const KVT *>(cp + (k[u] * ROW + c0)), c[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < CPL; ++i) v[u][i] = v[u][i] - c[u][i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < CPL; ++i) v[u][i] = u < m ? v[u][i] : 0.f;
}

template <int D>
constexpr size_t seg_lds_bytes(int N, int K) {
    return (size_t)SEG_KR * D * 8 + (size_t)(K + 3 * SEG_KR + 1 + 8 + SEG_WAVES + SEG_RUNS) * 4 + (size_t)N * 4;
}

// Phase 2 of k_update_seg for one wave: list entries [beg, end).  CERT: also
// collect each centroid's max|v| and lowest set bit.
template <int D, typename KVT, bool CERT>
__device__ __forceinline__ void seg_sums(const Src &src, int h, int N, const uint32_t *list, const int32_t *s_off,
                                         double *acc, int32_t *s_emin, uint32_t *s_amax, int beg, int end) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    int ci = 0;   // the offsets are monotone, so the guards below never bind
    while (ci < SEG_KR - 1 && s_off[ci + 1] <= beg) ++ci;
    ci = __builtin_amdgcn_readfirstlane(ci);
    int bound = __builtin_amdgcn_readfirstlane(s_off[ci + 1]);
    double sum[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) sum[c] = 0.0;
    int emin = SEG_EMPTY_E;
    uint32_t amax = 0u;
    auto flush = [&]() {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            atomicAdd(&acc[ci * D + lane * CPL + c], sum[c]);
            sum[c] = 0.0;
        }
        if constexpr (CERT) {
            const int e = wave_min_i(emin);
            const uint32_t a = wave_max_u(amax);
            if (lane == 0) {
                atomicMin(&s_emin[ci], e);
                atomicMax(&s_amax[ci], a);
            }
            emin = SEG_EMPTY_E;
            amax = 0u;
        }
    };
    for (int j = beg; j < end; j += SEG_U) {
        const int m = min(SEG_U, end - j);
        float v[SEG_U][CPL];
        seg_rows<D, KVT, SEG_U>(src, h, N, list, j, m, v);
#pragma unroll
        for (int u = 0; u < SEG_U; ++u) {
            if (u < m) {
                if (j + u >= bound) {
                    flush();
                    do {
                        ++ci;
                        bound = __builtin_amdgcn_readfirstlane(s_off[ci + 1]);
                    } while (j + u >= bound && ci < SEG_KR - 1);
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    sum[c] += (double)v[u][c];
                    if constexpr (CERT) {
                        emin = min(emin, lowest_bit_exp(v[u][c]));
                        amax = max(amax, __float_as_uint(v[u][c]) & 0x7FFFFFFFu);
                    }
                }
            }
        }
    }
    flush();
}

template <int D, typename KVT>
__global__ __launch_bounds__(64 * SEG_WAVES) void k_update_seg(Src src, int H, int N, int K, int Kp,
                                                               const uint8_t *__restrict__ pi, int64_t pi_hs,
                                                               const int32_t *__restrict__ counts,
                                                               const uint32_t *__restrict__ xstats, float *C,
                                                               uint16_t *Cb, int32_t *zero_cnt,
                                                               int32_t *zero_fill, ConvState cv) {
    constexpr int CPL = D / 64;
    constexpr int NT = 64 * SEG_WAVES;
    extern __shared__ double seg_lds[];
    double *acc = seg_lds;                                              // [SEG_KR][D]
    // [K + SEG_KR + 1]: s_off[k] is the list offset of centroid k's first token
    // (relative to the run), so centroid k has s_off[k + 1] - s_off[k] tokens;
    // while the list is built s_off[k + 1] serves as centroid k's fill cursor
    // and ends at its next centroid's offset
    int32_t *s_off = reinterpret_cast<int32_t *>(acc + SEG_KR * D);
    int32_t *s_emin = s_off + K + SEG_KR + 1;                           // [SEG_KR]
    uint32_t *s_amax = reinterpret_cast<uint32_t *>(s_emin + SEG_KR);  // [SEG_KR] bits of max|v|
    // table min, table max, max count, run certified, tokens before the run,
    // tokens of the run, centroids before the run, centroids of the run
    uint32_t *s_misc = s_amax + SEG_KR;
    int32_t *s_wsum = reinterpret_cast<int32_t *>(s_misc + 8);         // [SEG_WAVES] scan totals
    uint32_t *s_rc = reinterpret_cast<uint32_t *>(s_wsum + SEG_WAVES); // [SEG_RUNS] centroids per token share
    uint32_t *list = s_rc + SEG_RUNS;                                   // [N]

    const uint32_t rb = xcd_tile(blockIdx.x, gridDim.x);
    const int h = (int)(rb / SEG_RUNS), r = (int)(rb % SEG_RUNS);
    if (h >= H) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (conv_stop(cv, h, r == 0 && tid == 0)) return;

    // The reads that do not depend on the counts are issued first, so that the
    // label batch, the tables and the counts are in flight together.
    // Labels of the earlier stages ride along in the list entries; missing
    // stages read the current labels again and drop them.
    const uint8_t *lab = pi + (size_t)h * pi_hs;
    const uint8_t *l1 = src.P >= 1 ? src.pi[0] + (size_t)h * src.pi_hs : lab;
    const uint8_t *l2 = src.P >= 2 ? src.pi[1] + (size_t)h * src.pi_hs : lab;
    const uint32_t m1 = src.P >= 1 ? 0xFFu : 0u, m2 = src.P >= 2 ? 0xFFu : 0u;
    constexpr int B = 10;   // labels per thread and batch: one batch up to 5,120 tokens
    uint32_t lk[B], la[B], lb[B];
    auto label_batch = [&](int n0) {   // unconditional loads, all in flight together
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int n = min(n0 + i * NT + tid, N - 1);
            lk[i] = lab[n];
            la[i] = l1[n];
            lb[i] = l2[n];
        }
    };
    label_batch(0);
    const int cnt_k = counts[(size_t)h * Kp + min(tid, K - 1)];   // (thread k < K holds centroid k)
    // the input's value statistics, read now for the run certificate
    uint32_t xmn = 0xFFFFFFFFu, xmx = 0u;
    if (xstats) {
#pragma unroll
        for (int b = 0; b < VSTAT_BLOCKS; ++b) {
            xmn = min(xmn, xstats[((size_t)h * VSTAT_BLOCKS + b) * 2]);
            xmx = max(xmx, xstats[((size_t)h * VSTAT_BLOCKS + b) * 2 + 1]);
        }
    }
    // magnitudes of the earlier stages' stored tables (folded in when they were stored)
    uint32_t tmn = 0xFFFFFFFFu, tmx = 0u;
    const bool tables_known = src.P == 0 || src.tstats != nullptr;
    if (xstats && src.tstats) {
#pragma unroll 1
        for (int p = 0; p < src.P; ++p)
#pragma unroll
            for (int b = 0; b < TSTAT_BLOCKS; ++b) {
                const uint32_t *t = src.tstats + (((size_t)p * H + h) * TSTAT_BLOCKS + b) * 2;
                tmn = min(tmn, t[0]);
                tmx = max(tmx, t[1]);
            }
    }

    // the head's exclusive prefix P(k), from wave-wide scans of the counts
    const int ck = tid < K ? cnt_k : 0;
    int incl = ck;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    if (tid < 8) s_misc[tid] = tid == 0 ? tmn : tid == 1 ? tmx : 0u;
    if (tid < SEG_RUNS) s_rc[tid] = 0;
    for (int i = tid; i < SEG_KR * D; i += NT) acc[i] = 0.0;
    if (tid < SEG_KR) {
        s_emin[tid] = SEG_EMPTY_E;
        s_amax[tid] = 0u;
    }
    __syncthreads();
    int pk = incl - ck;   // P(tid); thread K holds P(K) = N
    for (int w = 0; w < wave; ++w) pk += s_wsum[w];
    // the token share floor(P(k) SEG_RUNS / N) of every centroid, counted per share
    if (tid < K) atomicAdd(&s_rc[(int)min((int64_t)SEG_RUNS - 1, (int64_t)pk * SEG_RUNS / N)], 1u);
    __syncthreads();
    // Run boundaries b_0 = 0 <= b_1 <= ... <= b_SEG_RUNS = K (the same in every
    // workgroup of the head): b_{q+1} is the first centroid of token share
    // q + 1, moved to keep every run within SEG_KR centroids (no more than
    // SEG_KR after b_q, and no fewer than the later runs need to hold the rest).
    int ka = 0, kb = 0;
    {
        int t = 0, b = 0;
        for (int q = 0; q < SEG_RUNS; ++q) {
            t += (int)s_rc[q];   // centroids whose share is at most q
            const int lo = K - SEG_KR * (SEG_RUNS - 1 - q);
            const int nb = q == SEG_RUNS - 1 ? K : max(b, min(b + SEG_KR, max(t, lo)));
            if (q == r) {
                ka = b;
                kb = nb;
            }
            b = nb;
        }
    }
    if (ka == kb) return;   // a cluster before this run holds its share of tokens
    if (tid == ka) s_misc[4] = (uint32_t)pk;   // tokens before the run
    if (tid == kb) s_misc[5] = (uint32_t)pk;   // tokens up to its end
    if (tid >= ka && tid < kb) {
        atomicMax(&s_misc[2], (uint32_t)ck);
        if (zero_cnt) zero_cnt[(size_t)h * Kp + tid] = 0;
        if (zero_fill) zero_fill[(size_t)h * Kp + tid] = 0;
    }
    __syncthreads();
    const int p0 = (int)s_misc[4], S = (int)s_misc[5] - p0;   // the run's tokens: [p0, p0 + S) in label order
    // fill cursors (s_off[k + 1] for centroid k) start at the offsets
    if (tid < K + SEG_KR) s_off[tid + 1] = tid < ka ? 0 : tid < kb ? pk - p0 : S;
    if (tid == 0) s_off[0] = 0;
    if (tid == 0) {   // the run certificate
        bool ok = xstats != nullptr && tables_known;
        if (ok) {
            uint32_t mn = s_misc[0], mx = s_misc[1];
            double mag = (double)magnitude_of<KVT>(mx);   // the tables' largest magnitudes, summed over stages
            if (src.P > 1) mag *= (double)src.P;          // (a bound: each table's maximum is at most mx)
            mag += (double)magnitude_of<KVT>(xmx);
            mn = min(mn, xmn);
            const int e = mn == 0xFFFFFFFFu ? 1000 : ulp_exp_of<KVT>(mn + 1u);
            const double reach = (double)s_misc[2] * mag * (1.0 + 0x1p-20);
            ok = reach < ldexp(1.0, min(53 + e, 1023));
        }
        s_misc[3] = ok ? 1u : 0u;
    }
    __syncthreads();

    // 1. the run's tokens, grouped by centroid
    for (int n0 = 0; n0 < N; n0 += NT * B) {
        if (n0 > 0) label_batch(n0);
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const uint32_t k = n0 + i * NT + tid < N ? lk[i] - (uint32_t)ka : 0xFFFFFFFFu;
            if (k < (uint32_t)(kb - ka)) {
                const int pos = atomicAdd(&s_off[ka + k + 1], 1);
                if (pos < S)   // always, with counts taken from these labels
                    list[pos] = (uint32_t)(n0 + i * NT + tid) | ((la[i] & m1) << 16) | ((lb[i] & m2) << 24);
            }
        }
    }
    __syncthreads();

    const bool run_exact = s_misc[3] != 0u;
    {
        // the run's centroids [ka, ka + nk) and their list offsets off[0 .. nk]
        const int w0 = ka, nk = kb - ka;
        const int32_t *off = s_off + w0;
        // 2. segmented sums: wave w takes entries [w per, (w + 1) per) of the window's list
        {
            const int W0 = off[0], W1 = off[nk];
            const int per = (W1 - W0 + SEG_WAVES - 1) / SEG_WAVES;
            const int beg = min(W1, W0 + wave * per), end = min(W1, beg + per);
            if (beg < end) {
                // the streaming sums issue ahead of the other workgroups of the CU
                // in their prologue, list build or means
                __builtin_amdgcn_s_setprio(1);
                if (run_exact) seg_sums<D, KVT, false>(src, h, N, list, off, acc, s_emin, s_amax, beg, end);
                else seg_sums<D, KVT, true>(src, h, N, list, off, acc, s_emin, s_amax, beg, end);
                __builtin_amdgcn_s_setprio(0);
            }
        }
        __syncthreads();

        // 3. means: one wave per centroid
        for (int i = wave; i < nk; i += SEG_WAVES) {
            const int cnt = off[i + 1] - off[i];
            if (cnt == 0) continue;   // an empty cluster keeps its centroid
            const int k = w0 + i;
            const double reach = (double)cnt * (double)__uint_as_float(s_amax[i]);
            const bool exact = run_exact || reach < ldexp(1.0, min(53 + s_emin[i], 1023));
            float mean[CPL];
            if (exact) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) mean[c] = mean_of(acc[i * D + lane * CPL + c], cnt);
            } else {
                const int a = off[i], b = off[i + 1];
                double hs[CPL];
                float ab[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) { hs[c] = 0.0; ab[c] = 0.f; }
                for (int j = a; j < b; j += 4) {
                    float v[4][CPL];
                    seg_rows<D, KVT, 4>(src, h, N, list, j, min(4, b - j), v);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int c = 0; c < CPL; ++c) {
                            hs[c] += (double)v[u][c];
                            ab[c] += fabsf(v[u][c]);
                        }
                }
                bool ok = cnt <= (1 << 20);
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const double bd = (double)ab[c] * (double)cnt * 0x1p-51 + fabs(hs[c]) * 0x1p-50;
                    const float lo = mean_of(hs[c] - bd, cnt), hi = mean_of(hs[c] + bd, cnt);
                    ok = ok && lo == hi;
                    mean[c] = lo;
                }
                if (!__all(ok)) {
                    double es[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) { hs[c] = 0.0; es[c] = 0.0; }
                    for (int j = a; j < b; j += 4) {
                        float v[4][CPL];
                        seg_rows<D, KVT, 4>(src, h, N, list, j, min(4, b - j), v);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
#pragma unroll
                            for (int c = 0; c < CPL; ++c) two_sum(hs[c], es[c], (double)v[u][c]);
                    }
#pragma unroll
                    for (int c = 0; c < CPL; ++c) mean[c] = mean_of(hs[c] + es[c], cnt);
                }
            }
            uint32_t bb[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) bb[c] = f32_to_bf16(mean[c]);
            float *cr = C + ((size_t)h * K + k) * D + lane * CPL;
            uint16_t *br = Cb + ((size_t)h * Kp + k) * D + lane * CPL;
            if constexpr (CPL == 2) {
                *reinterpret_cast<float2 *>(cr) = make_float2(mean[0], mean[1]);
                *reinterpret_cast<uint32_t *>(br) = bb[0] | (bb[1] << 16);
            } else {
                cr[0] = mean[0];
                br[0] = (uint16_t)bb[0];
            }
        }
    }
}

bool update_seg_fits(int N) { return N >= 1 && N <= SEG_MAX_N; }

size_t value_stats_words(int H) { return (size_t)H * VSTAT_BLOCKS * 2; }

hipError_t launch_update_seg(int D, int dtype, int H, int N, int K, const Src &src, const uint8_t *pi,
                             int64_t pi_hs, const int32_t *counts, const uint32_t *xstats, float *C, uint16_t *Cb,
                             int32_t *zero_cnt, int32_t *zero_fill, const ConvState &cv, hipStream_t s) {
    if (!update_seg_fits(N)) return hipErrorInvalidValue;
    const int Kp = padded_k(K);
    const int64_t nb = (int64_t)H * SEG_RUNS;
    // every run fits one window of SEG_KR centroids; thread k of a workgroup holds centroid k
    if (nb >= (int64_t)1 << 31 || K > SEG_KR * SEG_RUNS || K >= 64 * SEG_WAVES - SEG_KR) return hipErrorInvalidValue;
    QVG_DISPATCH_DT(D, dtype, {
        const size_t lds = seg_lds_bytes<DD>(N, K);
        (void)hipFuncSetAttribute((const void *)k_update_seg<DD, KVT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
        QVG_KERNEL((k_update_seg<DD, KVT>), dim3((unsigned)nb), dim3(64 * SEG_WAVES), lds, s, src, H, N, K, Kp, pi,
                   pi_hs, counts, xstats, C, Cb, zero_cnt, zero_fill, cv);
    });
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stored centroids and the streaming cache
// ---------------------------------------------------------------------------

// TSTAT_BLOCKS workgroups per head, each with up to 1024 eight-value chunks of
// the head's K D values (four per thread, all loads issued together).  With
// tstats, each workgroup also writes the smallest nonzero and largest magnitude
// (bits of the stored dtype, without sign) of its stored values: partial pair
// tstats[h][b] = {smallest - 1 (0xFFFFFFFF: all zero), largest}.
__global__ __launch_bounds__(256) void k_store_centroids(int64_t per_head8, const float *C, int dtype, void *dst,
                                                         float *cache, uint32_t *tstats) {
    constexpr int CPT = 4;
    const int h = blockIdx.y, b = blockIdx.x;
    const int64_t beg = (int64_t)h * per_head8 + (int64_t)b * 256 * CPT;
    const int64_t end = (int64_t)h * per_head8 + min(per_head8, (int64_t)(b + 1) * 256 * CPT);
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    if (beg < end) {
        float4 a[CPT], c[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {   // chunks past the end read the last one again
            const int64_t g = min(beg + i * 256 + threadIdx.x, end - 1);
            a[i] = reinterpret_cast<const float4 *>(C)[2 * g];
            c[i] = reinterpret_cast<const float4 *>(C)[2 * g + 1];
        }
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t g = beg + i * 256 + threadIdx.x;
            const bool in = g < end;
            if (dtype == DT_BF16) {
                const uint4 q = make_uint4(pack_bf16x2(a[i].x, a[i].y), pack_bf16x2(a[i].z, a[i].w),
                                           pack_bf16x2(c[i].x, c[i].y), pack_bf16x2(c[i].z, c[i].w));
                if (in) reinterpret_cast<uint4 *>(dst)[g] = q;
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
                    mx = max(mx, max(lo, hi));
                    mn = min(mn, min(lo - 1u, hi - 1u));   // zero wraps to the largest value
                }
            } else {
                if (in) {
                    reinterpret_cast<float4 *>(dst)[2 * g] = a[i];
                    reinterpret_cast<float4 *>(dst)[2 * g + 1] = c[i];
                }
                const float f[8] = {a[i].x, a[i].y, a[i].z, a[i].w, c[i].x, c[i].y, c[i].z, c[i].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t m = __float_as_uint(f[j]) & 0x7FFFFFFFu;
                    mx = max(mx, m);
                    mn = min(mn, m - 1u);
                }
            }
            if (cache && in) {
                reinterpret_cast<float4 *>(cache)[2 * g] = a[i];
                reinterpret_cast<float4 *>(cache)[2 * g + 1] = c[i];
            }
        }
    }
    if (!tstats) return;
    __shared__ uint32_t red[2][4];
    mn = (uint32_t)wave_min_i((int)(mn ^ 0x80000000u)) ^ 0x80000000u;   // unsigned minimum
    mx = wave_max_u(mx);
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = mn;
        red[1][threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *o = tstats + ((size_t)h * TSTAT_BLOCKS + b) * 2;
        o[0] = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
        o[1] = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    }
}

// FP8 storage: one workgroup per head.  The table's exponent e is the smallest
// with max|C| <= 448 * 2^e; every value is stored as the E4M3FN code of
// C / 2^e (nearest, ties to even; the sign kept unless the code is zero), and
// its decoded value (code value times 2^e, exact in bf16 and fp32) goes to the
// mirror table [K][D] of the tensor dtype and to the operand table Cb [Kp][D],
// so that the stage's final assignment and the later residuals use the
// centroids as stored.  The table in dst: a 16-byte header (e as int32, then
// zeros) and K D code bytes.  tstats as for k_store_centroids, from the mirror.
template <typename KVT>
__global__ __launch_bounds__(1024) void k_store_e4m3(int K, int D, int Kp, const float *C, uint8_t *dst,
                                                     int64_t tbytes, KVT *mirror, uint16_t *Cb, float *cache,
                                                     uint32_t *tstats) {
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nv = (int64_t)K * D;   // a multiple of 8
    const float *c = C + h * nv;
    __shared__ uint32_t red[2][16];
    uint32_t mx = 0u;
    for (int64_t i = (int64_t)tid * 4; i < nv; i += 4096) {
        const float4 v = *reinterpret_cast<const float4 *>(c + i);
        mx = max(max(mx, __float_as_uint(v.x) & 0x7FFFFFFFu), __float_as_uint(v.y) & 0x7FFFFFFFu);
        mx = max(max(mx, __float_as_uint(v.z) & 0x7FFFFFFFu), __float_as_uint(v.w) & 0x7FFFFFFFu);
    }
    mx = wave_max_u(mx);
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    mx = 0u;
    for (int w = 0; w < 16; ++w) mx = max(mx, red[0][w]);
    const float amax = __uint_as_float(mx);
    int e = 0;
    if (amax > 0.f) {
        int q;
        (void)frexpf(amax, &q);                      // amax = m 2^q, 0.5 <= m < 1
        e = q - 9;
        while (amax > ldexpf(448.f, e)) ++e;         // exact comparisons with 448 2^e
        while (amax <= ldexpf(448.f, e - 1)) --e;
    }
    uint8_t *tb = dst + h * tbytes;
    if (tid < 4) reinterpret_cast<int32_t *>(tb)[tid] = tid == 0 ? e : 0;
    uint8_t *codes = tb + 16;
    uint32_t mn = 0xFFFFFFFFu, tmx = 0u;
    for (int64_t i = (int64_t)tid * 8; i < nv; i += 8192) {
        const float4 a = *reinterpret_cast<const float4 *>(c + i), b = *reinterpret_cast<const float4 *>(c + i + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t cb[8];
        float dv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t code = e4m3_encode_nonneg(ldexpf(fabsf(v[j]), -e));
            if (code && (__float_as_uint(v[j]) >> 31)) code |= 0x80u;
            cb[j] = code;
            dv[j] = ldexpf(e4m3_decode(code), e);
        }
        *reinterpret_cast<uint2 *>(codes + i) = make_uint2(cb[0] | (cb[1] << 8) | (cb[2] << 16) | (cb[3] << 24),
                                                           cb[4] | (cb[5] << 8) | (cb[6] << 16) | (cb[7] << 24));
        const int64_t row = i / D, col = i - row * D;
        uint32_t bb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bb[j] = __float_as_uint(dv[j]) >> 16;   // exact: at most 4 significant bits
        *reinterpret_cast<uint4 *>(Cb + ((size_t)h * Kp + row) * D + col) =
            make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16));
        KVT *mr = mirror + h * nv + i;
        if constexpr (sizeof(KVT) == 2) {
            *reinterpret_cast<uint4 *>(mr) =
                make_uint4(bb[0] | (bb[1] << 16), bb[2] | (bb[3] << 16), bb[4] | (bb[5] << 16), bb[6] | (bb[7] << 16));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t m = bb[j] & 0x7FFFu;
                tmx = max(tmx, m);
                mn = min(mn, m - 1u);
            }
        } else {
            reinterpret_cast<float4 *>(mr)[0] = make_float4(dv[0], dv[1], dv[2], dv[3]);
            reinterpret_cast<float4 *>(mr)[1] = make_float4(dv[4], dv[5], dv[6], dv[7]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t m = __float_as_uint(dv[j]) & 0x7FFFFFFFu;
                tmx = max(tmx, m);
                mn = min(mn, m - 1u);
            }
        }
        if (cache) {
            reinterpret_cast<float4 *>(cache + h * nv + i)[0] = a;
            reinterpret_cast<float4 *>(cache + h * nv + i)[1] = b;
        }
    }
    if (!tstats) return;
    mn = (uint32_t)wave_min_i((int)(mn ^ 0x80000000u)) ^ 0x80000000u;   // unsigned minimum
    tmx = wave_max_u(tmx);
    __syncthreads();
    if (lane == 0) {
        red[0][wave] = mn;
        red[1][wave] = tmx;
    }
    __syncthreads();
    if (tid < TSTAT_BLOCKS) {   // the head's pair, repeated in every partial slot
        uint32_t a = 0xFFFFFFFFu, b = 0u;
        for (int w = 0; w < 16; ++w) {
            a = min(a, red[0][w]);
            b = max(b, red[1][w]);
        }
        tstats[((size_t)h * TSTAT_BLOCKS + tid) * 2] = a;
        tstats[((size_t)h * TSTAT_BLOCKS + tid) * 2 + 1] = b;
    }
}

hipError_t launch_store_e4m3(int D, int dtype, int H, int K, const float *C, uint8_t *dst, int64_t table_bytes,
                             void *mirror, uint16_t *Cb, float *cache, uint32_t *tstats, hipStream_t s) {
    if (table_bytes != (int64_t)K * D + 16 || H >= 65536) return hipErrorInvalidValue;
    if (dtype == DT_BF16)
        QVG_KERNEL(k_store_e4m3<uint16_t>, dim3(H), dim3(1024), 0, s, K, D, padded_k(K), C, dst, table_bytes,
                   static_cast<uint16_t *>(mirror), Cb, cache, tstats);
    else
        QVG_KERNEL(k_store_e4m3<float>, dim3(H), dim3(1024), 0, s, K, D, padded_k(K), C, dst, table_bytes,
                   static_cast<float *>(mirror), Cb, cache, tstats);
    return hipGetLastError();
}

hipError_t launch_store_centroids(int D, int H, int K, const float *C, int dtype, void *dst, float *cache,
                                  uint32_t *tstats, hipStream_t s) {
    const int64_t per_head8 = (int64_t)K * D / 8;   // D is a multiple of 8
    if (per_head8 > (int64_t)TSTAT_BLOCKS * 256 * 4 || H >= 65536) return hipErrorInvalidValue;
    QVG_KERNEL(k_store_centroids, dim3(TSTAT_BLOCKS, H), dim3(256), 0, s, per_head8, C, dtype, dst, cache, tstats);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// last stage's residual and the 2-bit group quantiser
// ---------------------------------------------------------------------------
//
// One thread owns 16 consecutive channels of one token; the G/16 threads of a
// group are adjacent lanes and combine their maxima with lane shuffles.

// PM: the number of earlier stages when it is 0 or 1, else 2 (any number).
// Two-level scales take two launches: with amax_out the kernel only folds the
// head's largest |r| (fp32 bits) into amax_out[h]; with amax_in it quantises
// with the second-level exponent f, the smallest f >= 0 with
// fp32(max|r| / 1.5) <= 448 * 2^f (scale code = E4M3 of fp32(a / 1.5) / 2^f,
// worth its value times 2^f), and writes f to exp_out[h].
// Tokens per thread of the quantiser: two for bf16 tensors whose residual
// comes from the input less at most one earlier stage (more bytes in flight
// per wave), one where fp32 rows or a rebuild over several stages would take
// the registers that the waves in flight need.
template <typename KVT, int PM>
constexpr int quant_tokens() { return sizeof(KVT) == 2 && PM <= 1 ? 2 : 1; }

template <int D, typename KVT, bool CENT, int PM>
__global__ __launch_bounds__(256) void k_quant(Src src, int N, const KVT *cent, int cent_rows, const uint8_t *pi,
                                               int64_t pi_hs, uint8_t *codes, uint8_t *scales, int64_t q_cap, int G,
                                               uint32_t *amax_out, const uint32_t *amax_in, int8_t *exp_out) {
    constexpr int SL = D / 16;
    constexpr int TPB = 256 / SL;
    constexpr int QU = quant_tokens<KVT, PM>();
    // one-dimensional grid: the blocks of one head on one XCD, in token order,
    // so that the head's centroid tables are fetched into that XCD's L2 once
    // (a grid too large for one dimension has one row of blocks per head)
    const uint32_t bph = (N + TPB * QU - 1) / (TPB * QU);   // blocks per head
    const uint32_t tile = gridDim.y > 1 ? blockIdx.y * bph + blockIdx.x : xcd_tile(blockIdx.x, gridDim.x);
    const int h = (int)(tile / bph);
    const int j = threadIdx.x % SL;
    const int n0 = (int)(tile % bph) * TPB * QU + threadIdx.x / SL;
    if (n0 >= N) return;   // whole groups leave together (SL divides 64)
    int n[QU];   // the thread's tokens; one past N reads token n0 again and stores nothing
#pragma unroll
    for (int u = 0; u < QU; ++u) n[u] = n0 + u * TPB < N ? n0 + u * TPB : n0;
    float r[QU][16];
    if constexpr (PM <= 1) {
        // every label first, then every row: two dependent reads in all
        int k1[QU], kt[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            k1[u] = PM == 1 ? (int)src.pi[0][(size_t)h * src.pi_hs + n[u]] : 0;
            kt[u] = CENT ? (int)pi[(size_t)h * pi_hs + n[u]] : 0;
        }
        float c1[QU][16], ct[QU][16];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            load16<KVT>(static_cast<const KVT *>(src.x) + (size_t)h * src.x_hs + (size_t)n[u] * D + 16 * j, r[u]);
            if constexpr (PM == 1)
                load16<KVT>(static_cast<const KVT *>(src.cent[0]) + ((size_t)h * src.K + k1[u]) * D + 16 * j, c1[u]);
            if constexpr (CENT) load16<KVT>(cent + ((size_t)h * cent_rows + kt[u]) * D + 16 * j, ct[u]);
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            if constexpr (PM == 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) r[u][i] = r[u][i] - c1[u][i];
            }
            if constexpr (CENT) {
#pragma unroll
                for (int i = 0; i < 16; ++i) r[u][i] = r[u][i] - ct[u][i];
            }
        }
    } else {
        float a[8], b[8];
        src_row8<D, KVT>(src, h, n[0], 16 * j, a);
        src_row8<D, KVT>(src, h, n[0], 16 * j + 8, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) { r[0][i] = a[i]; r[0][8 + i] = b[i]; }
        if constexpr (CENT) {
            const int k = pi[(size_t)h * pi_hs + n[0]];
            float c[16];
            load16<KVT>(cent + ((size_t)h * cent_rows + k) * D + 16 * j, c);
#pragma unroll
            for (int i = 0; i < 16; ++i) r[0][i] = r[0][i] - c[i];
        }
    }
    const int lanes = G >> 4;
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const bool mine = u == 0 || n0 + u * TPB < N;
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(r[u][i]));
        if (amax_out) {   // first launch of a two-level quantisation
            if (mine) atomicMax(&amax_out[h], __float_as_uint(a));
            continue;
        }
        for (int o = 1; o < lanes; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        int f = 0;
        if (amax_in) {
            const float a15 = __uint_as_float(amax_in[h]) / 1.5f;
            while (a15 > ldexpf(448.f, f)) ++f;
            if (u == 0 && n0 == 0 && j == 0) exp_out[h] = (int8_t)f;
        }
        const uint32_t sc = e4m3_encode_nonneg(ldexpf(a / 1.5f, -f));
        const float s = ldexpf(e4m3_decode(sc), f);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t q = (uint32_t)(r[u][i] >= -s) + (uint32_t)(r[u][i] >= 0.f) + (uint32_t)(r[u][i] >= s);
            w |= q << (2 * i);
        }
        if (!mine) continue;
        const size_t row = (size_t)h * q_cap + n[u];
        reinterpret_cast<uint32_t *>(codes + row * (D / 4))[j] = w;
        if ((j & (lanes - 1)) == 0) scales[row * (D / G) + (16 * j) / G] = (uint8_t)sc;
    }
}

hipError_t launch_quant(int D, int dtype, int H, int N, const Src &src, const void *cent, int cent_rows,
                        const uint8_t *pi, int64_t pi_hs, uint8_t *codes, uint8_t *scales, int64_t q_cap, int G,
                        uint32_t *amax_out, const uint32_t *amax_in, int8_t *exp_out, hipStream_t s) {
    const int TPB = 256 / (D / 16);
    // blocks of TPB x (tokens per thread) tokens, per head
    auto grid = [&](int qu) {
        const int64_t bph = (N + (int64_t)TPB * qu - 1) / ((int64_t)TPB * qu), nb = (int64_t)H * bph;
        const bool one_dim = nb * 256 < ((int64_t)1 << 32);
        return dim3(one_dim ? (uint32_t)nb : (uint32_t)bph, one_dim ? 1u : (uint32_t)H);
    };
    const dim3 b(256);
#define QVG_QUANT_LAUNCH(CE, PMV)                                                                                  \
    QVG_KERNEL((k_quant<DD, KVT, CE, PMV>), grid(quant_tokens<KVT, PMV>()), b, 0, s, src, N, (const KVT *)cent, cent_rows, \
               pi, pi_hs, codes, scales, q_cap, G, amax_out, amax_in, exp_out)
    QVG_DISPATCH_DT(D, dtype, {
        if (cent) {
            if (src.P == 0) QVG_QUANT_LAUNCH(true, 0);
            else if (src.P == 1) QVG_QUANT_LAUNCH(true, 1);
            else QVG_QUANT_LAUNCH(true, 2);
        } else {
            if (src.P == 0) QVG_QUANT_LAUNCH(false, 0);
            else QVG_QUANT_LAUNCH(false, 2);
        }
    });
#undef QVG_QUANT_LAUNCH
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fused dequantise + reconstruct
// ---------------------------------------------------------------------------
//
// Per (token, slice): two 16-bit words of codes, two scale bytes, T assignment
// bytes, T centroid rows (two 8-channel chunks each) and two streaming stores.

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A decode slice: lane j of a token's D/16 lanes owns channels [8j, 8j + 8) and
// [D/2 + 8j, D/2 + 8j + 8), so each store instruction of a token's lanes writes
// one contiguous half row (whole cache lines).

// y[i] = (q_i - 1.5) s for the 8 two-bit codes in the low 16 bits of w
// (channel i in bits 2i, 2i+1).  With s != 0 every term is exact, so one fma
// per channel gives the same value; a zero scale takes the expression as
// written, for its signed zeros.
__device__ __forceinline__ void dequant8(uint32_t w, float s, float *y) {
    if (s != 0.f) {
        const float m = -1.5f * s;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t b = (w >> (2 * g)) & 0x0303u;   // channels g and g + 4
            asm volatile("" : "+v"(b));             // keeps the byte extracts as v_cvt_f32_ubyte0/1
            y[g] = fmaf((float)(b & 0xFFu), s, m);
            y[g + 4] = fmaf((float)((b >> 8) & 0xFFu), s, m);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = ((float)((w >> (2 * i)) & 3u) - 1.5f) * s;
    }
}

// y[i] += c_i for 8 centroid values (bf16: one 16-byte chunk; fp32: two)
template <typename CentT>
__device__ __forceinline__ void add8(const uint4 *c, float *y) {
    if constexpr (sizeof(CentT) == 2) {
        const uint32_t b[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = y[2 * i] + __uint_as_float(b[i] << 16);
            y[2 * i + 1] = y[2 * i + 1] + __uint_as_float(b[i] & 0xFFFF0000u);
        }
    } else {
        const float f[8] = {__uint_as_float(c[0].x), __uint_as_float(c[0].y), __uint_as_float(c[0].z),
                            __uint_as_float(c[0].w), __uint_as_float(c[1].x), __uint_as_float(c[1].y),
                            __uint_as_float(c[1].z), __uint_as_float(c[1].w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = y[i] + f[i];
    }
}

// 8 outputs to p, bf16 or fp32, with streaming stores (the output is not read
// back here; keeping it out of L2 leaves room for the centroid tables)
template <typename OutT>
__device__ __forceinline__ void store8_out(OutT *p, const float *v) {
    if constexpr (sizeof(OutT) == 2) {
        const u32x4_t q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                           pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t *>(p));
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4_t q = {__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                               __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3])};
            __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t *>(p) + i);
        }
    }
}

// Rotary position embedding of 8 consecutive channels, four adjacent pairs:
// (a, b) -> (a cos - b sin, a sin + b cos) with cs = cos, sin, cos, sin, ... of
// the pairs' angles.  Each product and each sum is rounded to fp32 on its own
// (no fused multiply-add), so the result does not depend on the compiler.
__device__ __forceinline__ void rope8(const float *cs, float *y) {
#pragma clang fp contract(off)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = y[2 * p], b = y[2 * p + 1], c = cs[2 * p], sn = cs[2 * p + 1];
        y[2 * p] = a * c - b * sn;
        y[2 * p + 1] = a * sn + b * c;
    }
}

__device__ __forceinline__ void load8_f32(const float *p, float *v) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The per-token inputs of slice j: two 16-bit code words and two scales.
template <int D>
__device__ __forceinline__ void slice_inputs(const uint8_t *codes, const uint8_t *scales, size_t row, int G, int j,
                                             uint32_t &w0, uint32_t &w1, uint32_t &sc0, uint32_t &sc1) {
    const uint16_t *c16 = reinterpret_cast<const uint16_t *>(codes + row * (D / 4));
    w0 = c16[j];
    w1 = c16[D / 16 + j];
    sc0 = scales[row * (D / G) + (8 * j) / G];
    sc1 = scales[row * (D / G) + (D / 2 + 8 * j) / G];
}

// Dequantise slice j, add the stages' centroid chunks from fetch(t, half, uint4*)
// for t = T-1 .. 0, rotate by the token's cos/sin row rp when it is not null,
// and store the two half rows of rb.
template <int D, typename CentT, typename OutT, typename Fetch>
__device__ __forceinline__ void decode_slice(int T, uint32_t w0, uint32_t w1, uint32_t sc0, uint32_t sc1, float sx,
                                             int j, const float *rp, OutT *rb, Fetch fetch) {
    float y[16];
    dequant8(w0, e4m3_decode(sc0) * sx, y);
    dequant8(w1, e4m3_decode(sc1) * sx, y + 8);
    for (int t = T - 1; t >= 0; --t) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            uint4 c[sizeof(CentT) == 2 ? 1 : 2];
            fetch(t, hf, c);
            add8<CentT>(c, y + 8 * hf);
        }
    }
    if (rp) {
        float cs[8];
        load8_f32(rp + 8 * j, cs);
        rope8(cs, y);
        load8_f32(rp + D / 2 + 8 * j, cs);
        rope8(cs, y + 8);
    }
    store8_out<OutT>(rb + 8 * j, y);
    store8_out<OutT>(rb + D / 2 + 8 * j, y + 8);
}

// Tables in L2: one thread per (token, slice) for DEC_U tokens; blocks walk
// (head, token) tiles, XCD-contiguous.  For TT >= 0 the stage count is a
// compile-time constant and every load of the thread's tokens is in flight
// before the first is used; TT = -1 takes T at run time.
constexpr int DEC_U = 2;

template <int D, typename CentT, typename OutT, int TT, bool FP8>
__global__ __launch_bounds__(256) void k_decode(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                const uint8_t *__restrict__ assign, const void *__restrict__ cent_v,
                                                int64_t cap, int chunk_tokens, int H, int K, int T_rt, int G,
                                                int64_t tok_begin, int64_t ntok, const float *__restrict__ rope,
                                                int rope_heads, const int8_t *__restrict__ scale_exp,
                                                OutT *__restrict__ out, int64_t out_hs, uint32_t blocks_per_head) {
    constexpr int SL = D / 16;
    constexpr int TPB = 256 / SL;
    constexpr int TS = TT > 0 ? TT : 1;
    const int T = TT >= 0 ? TT : T_rt;
    const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int h = tile / blocks_per_head;
    const int64_t nl0 = (int64_t)(tile % blocks_per_head) * (TPB * DEC_U) + threadIdx.x / SL;
    const int j = threadIdx.x % SL;
    if (nl0 >= ntok) return;
    uint32_t w0[DEC_U], w1[DEC_U], sc0[DEC_U], sc1[DEC_U];
    int k[DEC_U][TS];
    int64_t n[DEC_U];
    bool ok[DEC_U];
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
        ok[u] = nl0 + u * TPB < ntok;
        n[u] = tok_begin + (ok[u] ? nl0 + u * TPB : nl0);
        slice_inputs<D>(codes, scales, (size_t)h * cap + n[u], G, j, w0[u], w1[u], sc0[u], sc1[u]);
        if constexpr (TT > 0) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const int kk = assign[((size_t)t * H + h) * cap + n[u]];
                k[u][t] = kk < K ? kk : K - 1;   // a corrupt byte cannot leave the chunk's table
            }
        }
    }
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
        if (!ok[u]) continue;
        const int64_t c = n[u] / chunk_tokens;
        OutT *rb = out + (size_t)h * out_hs + (size_t)(n[u] - tok_begin) * D;
        const float *rp = rope && h < rope_heads ? rope + (size_t)(n[u] - tok_begin) * D : nullptr;
        const float sx = scale_exp ? ldexpf(1.f, scale_exp[c * H + h]) : 1.f;
        decode_slice<D, CentT, OutT>(T, w0[u], w1[u], sc0[u], sc1[u], sx, j, rp, rb, [&](int t, int hf, uint4 *cv) {
            int kk;
            if constexpr (TT > 0) {
                kk = k[u][t];
            } else {
                kk = assign[((size_t)t * H + h) * cap + n[u]];
                kk = kk < K ? kk : K - 1;
            }
            if constexpr (FP8) {   // 8 codes, widened to bf16 exactly: code value x 2^e
                const uint8_t *tbl = static_cast<const uint8_t *>(cent_v) + (((size_t)c * T + t) * H + h) * (K * D + 16);
                const float sc = ldexpf(1.f, *reinterpret_cast<const int32_t *>(tbl));
                const uint2 v = *reinterpret_cast<const uint2 *>(tbl + 16 + (size_t)kk * D + hf * (D / 2) + 8 * j);
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = q < 2 ? v.x : v.y, sh = 16 * (q & 1);
                    o[q] = (__float_as_uint(e4m3_decode((w >> sh) & 0xFFu) * sc) >> 16) |
                           (__float_as_uint(e4m3_decode((w >> (sh + 8)) & 0xFFu) * sc) & 0xFFFF0000u);
                }
                cv[0] = make_uint4(o[0], o[1], o[2], o[3]);
            } else {
                const uint4 *src = reinterpret_cast<const uint4 *>(
                    static_cast<const CentT *>(cent_v) + ((((size_t)c * T + t) * H + h) * K + kk) * D + hf * (D / 2) + 8 * j);
                cv[0] = src[0];
                if constexpr (sizeof(CentT) == 4) cv[1] = src[1];
            }
        });
    }
}

// Tables in LDS: one workgroup per (chunk, head, half row) stages that half of
// the chunk's T centroid tables of the head (swizzled 16-byte chunks, 64 KiB at
// T = 2, K = 256, d = 128, so two workgroups share a CU) and streams the chunk's
// tokens in trips of DEC_TRIP.  Each trip's codes, scales and assignments are
// first brought into LDS by one wide load per thread (the half row's codes of a
// token in one 8- or 16-byte load, its scale bytes in one load, one assignment
// byte per stage), instead of the 2 + 1 + T loads of 1-2 bytes that every lane
// of a token would otherwise issue.  Lane jj of a token's D/16 lanes then owns
// 8 channels, so one store instruction writes 128 contiguous bytes per token.
constexpr int DEC_LDS_THREADS = 1024;
constexpr int DEC_TRIP = 512;   // tokens per trip
constexpr int DEC_PARTS = 2;    // workgroups per (chunk, head), each with its part of every row
constexpr size_t DEC_LDS_MAX = 160 * 1024 - 1024;   // LDS bytes one workgroup may take

// Rotated decodes give each XCD one contiguous run of (chunk, head) units in
// chunk-major order, of about equal token work: the rotated heads of a chunk
// then share one XCD, whose L2 fetches the chunk's rows of the rotation table
// once for all of them (with the units spread over the XCDs by head, every XCD
// fetched every chunk's rows).  start[x] .. start[x + 1] are XCD x's units.
struct DecRuns {
    int64_t start[9];
};

// LDS bytes of one trip's staged codes, scales and assignments.
constexpr size_t dec_meta_bytes(int D, int G, int T) {
    return (size_t)DEC_TRIP * (D / 4 / DEC_PARTS) + (size_t)DEC_TRIP * (D / DEC_PARTS >= G ? D / DEC_PARTS / G : 1) +
           (size_t)T * DEC_TRIP;
}

// One token's scale bytes of part hf: SPT bytes (1, 2 or 4) in one load.
template <int SPT>
__device__ __forceinline__ uint32_t load_scales(const uint8_t *p) {
    if constexpr (SPT == 4) return *reinterpret_cast<const uint32_t *>(p);
    else if constexpr (SPT == 2) return *reinterpret_cast<const uint16_t *>(p);
    else return *p;
}

// FP8: the stored tables are E4M3 codes behind a 16-byte exponent header (CentT
// is then the bf16 form they take in LDS, exactly).
template <int D, int G, typename CentT, typename OutT, int TT, bool ROPE, bool FP8>
__global__ __launch_bounds__(DEC_LDS_THREADS, 8) void k_decode_lds(const uint8_t *__restrict__ codes,
                                                                   const uint8_t *__restrict__ scales,
                                                                   const uint8_t *__restrict__ assign,
                                                                   const void *__restrict__ cent_v, int64_t cap,
                                                                   int chunk_tokens, int H, int K,
                                                                   int64_t tok_begin, int64_t tok_end,
                                                                   int64_t c_first, int64_t n_units, DecRuns runs,
                                                                   const float *__restrict__ rope, int rope_heads,
                                                                   const int8_t *__restrict__ scale_exp,
                                                                   OutT *__restrict__ out, int64_t out_hs) {
    constexpr int PARTS = DEC_PARTS;
    constexpr int DP = D / PARTS;                             // channels of a part
    constexpr int LPT = DP / 8;                               // lanes per token (8 channels each)
    constexpr int CHH = DP * (int)sizeof(CentT) / 16;         // 16-byte chunks per part of a row
    constexpr int CP8 = 8 * (int)sizeof(CentT) / 16;          // chunks per 8 channels (1 bf16, 2 fp32)
    constexpr int CB = DP / 4;                                // code bytes of a part of a token (8 or 16)
    constexpr int SPT = DP >= G ? DP / G : 1;                 // scale bytes of a part of a token
    constexpr int STEP = DEC_LDS_THREADS / LPT;               // tokens per pass
    static_assert(DEC_TRIP % STEP == 0 && 2 * DEC_TRIP <= DEC_LDS_THREADS, "trip layout");
    extern __shared__ uint4 tab[];
    uint8_t *mcodes = reinterpret_cast<uint8_t *>(tab + TT * K * CHH);   // [DEC_TRIP][CB]
    uint8_t *msc = mcodes + DEC_TRIP * CB;                                 // [DEC_TRIP][SPT]
    uint8_t *mlab = msc + DEC_TRIP * SPT;                                  // [TT][DEC_TRIP]
    // The PARTS workgroups of one (chunk, head) are 8 apart in dispatch order:
    // the same XCD, running together, so a code line fetched by one is still in
    // that XCD's L2 for the other.  Workgroups past the last (chunk, head) of a
    // grid padded to a multiple of 8 x PARTS have nothing to do.
    // Rotated decodes: XCD blockIdx % 8 takes its run of units in order, the
    // PARTS workgroups of a unit one after the other.
    const int hf = (int)((blockIdx.x / 8) % PARTS);
    int64_t uu;
    if constexpr (ROPE) {
        const int x = blockIdx.x % 8;
        uu = runs.start[x] + blockIdx.x / 8 / PARTS;
        if (uu >= runs.start[x + 1]) return;
    } else {
        uu = (int64_t)(blockIdx.x / 8 / PARTS) * 8 + blockIdx.x % 8;
        if (uu >= n_units) return;
    }
    const int h = (int)(uu % H);
    const int64_t c = c_first + uu / H;
    const int tid = threadIdx.x;
    for (int t = 0; t < TT; ++t) {
        if constexpr (FP8) {
            // 16 codes per load become two bf16 chunks: value = code value x 2^e
            const uint8_t *tbl = static_cast<const uint8_t *>(cent_v) + (((size_t)c * TT + t) * H + h) * (K * D + 16);
            const float sc = ldexpf(1.f, *reinterpret_cast<const int32_t *>(tbl));
            const uint4 *src = reinterpret_cast<const uint4 *>(tbl + 16);
            constexpr int SCH = DP / 16;   // 16-byte code chunks per part of a row
            for (int i = tid; i < K * SCH; i += DEC_LDS_THREADS) {
                const int row = i / SCH, q = i - row * SCH;
                const int r = t * K + row;
                const uint4 v = src[(size_t)row * (D / 16) + hf * SCH + q];
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                uint32_t o[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t b0 = (w[k / 2] >> (16 * (k & 1))) & 0xFFu, b1 = (w[k / 2] >> (16 * (k & 1) + 8)) & 0xFFu;
                    o[k] = (__float_as_uint(e4m3_decode(b0) * sc) >> 16) | (__float_as_uint(e4m3_decode(b1) * sc) & 0xFFFF0000u);
                }
                tab[r * CHH + ((2 * q) ^ (r & (CHH - 1)))] = make_uint4(o[0], o[1], o[2], o[3]);
                tab[r * CHH + ((2 * q + 1) ^ (r & (CHH - 1)))] = make_uint4(o[4], o[5], o[6], o[7]);
            }
        } else {
            const CentT *cent = static_cast<const CentT *>(cent_v);
            const uint4 *src = reinterpret_cast<const uint4 *>(cent + (((size_t)c * TT + t) * H + h) * K * D);
            for (int i = tid; i < K * CHH; i += DEC_LDS_THREADS) {
                const int row = i / CHH, q = i - row * CHH;
                const int r = t * K + row;
                tab[r * CHH + (q ^ (r & (CHH - 1)))] = src[(size_t)row * PARTS * CHH + hf * CHH + q];
            }
        }
    }
    const int64_t tb = max(tok_begin, c * chunk_tokens), te = min(tok_end, (c + 1) * chunk_tokens);
    const size_t hrow = (size_t)h * cap;
    const size_t a_stage = (size_t)H * cap;
    // second level of two-level scales: 2^f for this (chunk, head), else 1
    const float sx = scale_exp ? ldexpf(1.f, scale_exp[c * H + h]) : 1.f;
    const int jj = tid % LPT, slot = tid / LPT;
    const int c0 = hf * DP + 8 * jj;   // first channel of the lane
    const int sofs = DP >= G ? (8 * jj) / G : 0;   // the lane's scale byte among its token's SPT
    OutT *const oh = out + (size_t)h * out_hs + c0;
    const bool rot = ROPE && h < rope_heads;
    for (int64_t i0 = tb; i0 < te; i0 += DEC_TRIP) {
        const int nt = (int)min((int64_t)DEC_TRIP, te - i0);
        // this trip's inputs, one wide load per thread (tokens past the trip's
        // end read its last token again and are never used)
        const int ms = tid & (DEC_TRIP - 1);
        const int64_t n = i0 + min(ms, nt - 1);
        uint4 cv = make_uint4(0, 0, 0, 0);
        uint32_t sv = 0;
        uint32_t lv[(TT + 1) / 2];
        if (tid < DEC_TRIP) {
            const uint8_t *cp = codes + (hrow + n) * (D / 4) + hf * CB;
            if constexpr (CB == 16) {
                cv = *reinterpret_cast<const uint4 *>(cp);
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(cp);
                cv.x = v.x;
                cv.y = v.y;
            }
        } else {
            sv = load_scales<SPT>(scales + (hrow + n) * (D / G) + (DP >= G ? hf * SPT : (hf * DP) / G));
        }
#pragma unroll
        for (int m = 0; m < (TT + 1) / 2; ++m) {   // stage 2m + (tid >= DEC_TRIP)
            const int t = 2 * m + (tid >= DEC_TRIP ? 1 : 0);
            lv[m] = t < TT ? assign[t * a_stage + hrow + n] : 0u;
        }
        __syncthreads();   // the previous trip's readers are done
        if (tid < DEC_TRIP) {
            if constexpr (CB == 16) reinterpret_cast<uint4 *>(mcodes)[ms] = cv;
            else reinterpret_cast<uint2 *>(mcodes)[ms] = make_uint2(cv.x, cv.y);
        } else {
            if constexpr (SPT == 4) reinterpret_cast<uint32_t *>(msc)[ms] = sv;
            else if constexpr (SPT == 2) reinterpret_cast<uint16_t *>(msc)[ms] = (uint16_t)sv;
            else msc[ms] = (uint8_t)sv;
        }
#pragma unroll
        for (int m = 0; m < (TT + 1) / 2; ++m) {
            const int t = 2 * m + (tid >= DEC_TRIP ? 1 : 0);
            if (t < TT) mlab[t * DEC_TRIP + ms] = (uint8_t)lv[m];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < DEC_TRIP / STEP; ++u) {
            const int i = u * STEP + slot;
            if (i >= nt) break;
            const size_t orow = (size_t)(i0 + i - tok_begin) * D;
            // the rotation table has the output's token rows; pair p of a row is
            // the float pair (cos, sin) at channels 2p, 2p + 1.  Requested before
            // the rebuild, which hides its latency (with bf16 tables; fp32 tables
            // leave no registers for it)
            constexpr bool EARLY = sizeof(CentT) == 2;
            float cs[8];
            if (EARLY && rot) load8_f32(rope + orow + c0, cs);
            const uint32_t w = reinterpret_cast<const uint16_t *>(mcodes)[i * (CB / 2) + jj];
            float y[8];
            dequant8(w, e4m3_decode(msc[i * SPT + sofs]) * sx, y);
#pragma unroll
            for (int t = TT - 1; t >= 0; --t) {
                const int kk = mlab[t * DEC_TRIP + i];
                const int r = t * K + (kk < K ? kk : K - 1);   // a corrupt byte cannot leave the chunk's table
                uint4 cv8[CP8];
#pragma unroll
                for (int q = 0; q < CP8; ++q) cv8[q] = tab[r * CHH + ((CP8 * jj + q) ^ (r & (CHH - 1)))];
                add8<CentT>(cv8, y);
            }
            if (rot) {
                if (!EARLY) load8_f32(rope + orow + c0, cs);
                rope8(cs, y);
            }
            store8_out<OutT>(oh + orow, y);
        }
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    // tables in LDS: bf16 (FP8 tables are widened to bf16 there) or fp32
    const size_t tab_bytes = (size_t)a.T * a.K * (a.D / DEC_PARTS) * (a.cent_dtype == DT_F32 ? 4 : 2);
    const size_t lds = tab_bytes + dec_meta_bytes(a.D, a.G, a.T);
    // the staged loads need the scale bytes of a part aligned to their size
    const bool scales_aligned = (reinterpret_cast<uintptr_t>(a.scales) & 3u) == 0;
    if (a.T >= 1 && a.T <= 4 && lds <= DEC_LDS_MAX && scales_aligned) {
        const int64_t c0 = a.tok_begin / a.chunk_tokens, c1 = (a.tok_begin + a.ntok - 1) / a.chunk_tokens;
        const int64_t units = (c1 - c0 + 1) * a.H;   // (chunk, head) pairs
        int64_t nb = (units + 7) / 8 * 8 * DEC_PARTS;
        DecRuns runs{};
        if (a.rope) {
            // runs of equal token work: unit u = (chunk c0 + u / H, head u % H)
            // holds the chunk's tokens inside [tok_begin, tok_begin + ntok)
            const int64_t tb = a.tok_begin, te = a.tok_begin + a.ntok, ct = a.chunk_tokens;
            auto tokens_before = [&](int64_t u) {   // token work of units [0, u)
                const int64_t full = u / a.H, part = u % a.H;
                auto chunk_tokens = [&](int64_t c) {
                    return std::min(te, (c + 1) * ct) - std::max(tb, c * ct);
                };
                // every chunk between the first and the last is whole
                int64_t w = 0;
                if (full > 0) {
                    w += chunk_tokens(c0) * a.H;
                    if (full > 1) {
                        const int64_t cl = c0 + full - 1;   // the last whole chunk counted
                        w += (full - 2) * ct * a.H + chunk_tokens(cl) * a.H;
                    }
                }
                if (part > 0) w += chunk_tokens(c0 + full) * part;
                return w;
            };
            const int64_t total = tokens_before(units);
            int64_t most = 0;
            runs.start[0] = 0;
            for (int x = 1; x <= 8; ++x) {
                // the first unit whose work before it reaches x / 8 of the total
                int64_t lo = runs.start[x - 1], hi = units;
                const int64_t goal = total * x / 8;
                while (lo < hi) {
                    const int64_t mid = (lo + hi) / 2;
                    if (tokens_before(mid) >= goal) hi = mid;
                    else lo = mid + 1;
                }
                runs.start[x] = x == 8 ? units : lo;
                most = std::max(most, runs.start[x] - runs.start[x - 1]);
            }
            nb = 8 * most * DEC_PARTS;
        }
        if (nb < (int64_t)UINT32_MAX) {
            dim3 g((unsigned)nb), b(DEC_LDS_THREADS);
#define QVG_DECL_R(DD, GG, CT, OT, TT, RO)                                                                        \
    do {                                                                                                          \
        if (a.cent_dtype == DT_E4M3) {                                                                            \
            (void)hipFuncSetAttribute((const void *)k_decode_lds<DD, GG, uint16_t, OT, TT, RO, true>,             \
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                      \
            QVG_KERNEL((k_decode_lds<DD, GG, uint16_t, OT, TT, RO, true>), g, b, lds, s, a.codes, a.scales,       \
                       a.assign, a.cent, a.cap, a.chunk_tokens, a.H, a.K, a.tok_begin, a.tok_begin + a.ntok, c0,  \
                       units, runs, a.rope, a.rope_heads, a.scale_exp, (OT *)a.out, a.out_hs);                          \
        } else {                                                                                                  \
            (void)hipFuncSetAttribute((const void *)k_decode_lds<DD, GG, CT, OT, TT, RO, false>,                  \
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                      \
            QVG_KERNEL((k_decode_lds<DD, GG, CT, OT, TT, RO, false>), g, b, lds, s, a.codes, a.scales, a.assign,  \
                       a.cent, a.cap, a.chunk_tokens, a.H, a.K, a.tok_begin, a.tok_begin + a.ntok, c0, units,     \
                       runs, a.rope, a.rope_heads, a.scale_exp, (OT *)a.out, a.out_hs);                                 \
        }                                                                                                         \
    } while (0)
#define QVG_DECL(DD, GG, CT, OT, TT)                               \
    do {                                                           \
        if (a.rope) QVG_DECL_R(DD, GG, CT, OT, TT, true);          \
        else QVG_DECL_R(DD, GG, CT, OT, TT, false);                \
    } while (0)
#define QVG_DECL_T(DD, GG, CT, OT)                         \
    do {                                                   \
        switch (a.T) {                                     \
            case 1: QVG_DECL(DD, GG, CT, OT, 1); break;    \
            case 2: QVG_DECL(DD, GG, CT, OT, 2); break;    \
            case 3: QVG_DECL(DD, GG, CT, OT, 3); break;    \
            default: QVG_DECL(DD, GG, CT, OT, 4); break;   \
        }                                                  \
    } while (0)
#define QVG_DECL_O(DD, GG, CT)                             \
    do {                                                   \
        if (a.out_dtype == DT_BF16) QVG_DECL_T(DD, GG, CT, uint16_t); \
        else QVG_DECL_T(DD, GG, CT, float);                \
    } while (0)
#define QVG_DECL_C(DD, GG)                                 \
    do {                                                   \
        if (a.cent_dtype != DT_F32) QVG_DECL_O(DD, GG, uint16_t); \
        else QVG_DECL_O(DD, GG, float);                    \
    } while (0)
#define QVG_DECL_G(DD)                                     \
    do {                                                   \
        switch (a.G) {                                     \
            case 16: QVG_DECL_C(DD, 16); break;            \
            case 32: QVG_DECL_C(DD, 32); break;            \
            case 64: QVG_DECL_C(DD, 64); break;            \
            default: QVG_DECL_C(DD, 128); break;           \
        }                                                  \
    } while (0)
            if (a.D == 128) QVG_DECL_G(128); else QVG_DECL_G(64);
#undef QVG_DECL_G
#undef QVG_DECL_C
#undef QVG_DECL_O
#undef QVG_DECL_T
#undef QVG_DECL
#undef QVG_DECL_R
            return hipGetLastError();
        }
    }
    const int TPB = 256 / (a.D / 16) * DEC_U;
    const uint32_t bph = (uint32_t)((a.ntok + TPB - 1) / TPB);
    dim3 g(bph * a.H), b(256);
#define QVG_DEC(DD, CT, OT, TT)                                                                                   \
    do {                                                                                                          \
        if (a.cent_dtype == DT_E4M3)                                                                              \
            QVG_KERNEL((k_decode<DD, uint16_t, OT, TT, true>), g, b, 0, s, a.codes, a.scales, a.assign, a.cent,   \
                       a.cap, a.chunk_tokens, a.H, a.K, a.T, a.G, a.tok_begin, a.ntok, a.rope, a.rope_heads,     \
                       a.scale_exp, (OT *)a.out, a.out_hs, bph);                                                  \
        else                                                                                                      \
            QVG_KERNEL((k_decode<DD, CT, OT, TT, false>), g, b, 0, s, a.codes, a.scales, a.assign, a.cent,        \
                       a.cap, a.chunk_tokens, a.H, a.K, a.T, a.G, a.tok_begin, a.ntok, a.rope, a.rope_heads,     \
                       a.scale_exp, (OT *)a.out, a.out_hs, bph);                                                  \
    } while (0)
#define QVG_DEC_T(DD, CT, OT)                              \
    do {                                                   \
        switch (a.T) {                                     \
            case 0: QVG_DEC(DD, CT, OT, 0); break;         \
            case 1: QVG_DEC(DD, CT, OT, 1); break;         \
            case 2: QVG_DEC(DD, CT, OT, 2); break;         \
            case 3: QVG_DEC(DD, CT, OT, 3); break;         \
            case 4: QVG_DEC(DD, CT, OT, 4); break;         \
            default: QVG_DEC(DD, CT, OT, -1); break;       \
        }                                                  \
    } while (0)
#define QVG_DEC_O(DD, CT)                                  \
    do {                                                   \
        if (a.out_dtype == DT_BF16) QVG_DEC_T(DD, CT, uint16_t); \
        else QVG_DEC_T(DD, CT, float);                     \
    } while (0)
#define QVG_DEC_C(DD)                                      \
    do {                                                   \
        if (a.cent_dtype != DT_F32) QVG_DEC_O(DD, uint16_t); \
        else QVG_DEC_O(DD, float);                         \
    } while (0)
    if (a.D == 128) QVG_DEC_C(128); else QVG_DEC_C(64);
#undef QVG_DEC_C
#undef QVG_DEC_O
#undef QVG_DEC_T
#undef QVG_DEC
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attention over the compressed cache
// ---------------------------------------------------------------------------
//
// softmax(scale Q K^T) V with K and V rebuilt inside the kernel, tile by tile,
// from the compressed cache (codes, scales, assignments, centroid tables): no
// decoded K or V ever goes to memory.  A workgroup of 16 waves takes 256
// queries of one head (16 per wave, their bf16 rows held as MFMA operands) and
// a range of keys (a split), 64 keys per tile:
//   1. every thread rebuilds 8 channels of one key of K and of V with the
//      decode's arithmetic (dequantise, add the stages' centroid rows in
//      reverse order in fp32, rotate the key if a table is given, round to
//      bf16), so the tiles equal qvg_decode's output bit for bit; K goes to
//      LDS row by row, V transposed;
//   2. S^T = K Q^T on v_mfma_f32_16x16x32_bf16: lane l holds the scores of
//      query l % 16 against keys 16 b + 4 (l / 16) + r, so every lane owns one
//      query's softmax statistics (online, base 2, merged over 4 lanes);
//   3. O^T += V^T P^T on the same instruction with the softmax weights (bf16)
//      taken from the lane's own registers: the instruction's k order is
//      permuted to the keys the lane holds, and V^T is read in that order.
// Each split writes its unnormalised O and (max, sum); k_attn_merge combines
// the splits by their log-sum-exp.
constexpr int ATT_WAVES = 16;
constexpr int ATT_BQ = 16 * ATT_WAVES;   // queries per workgroup
constexpr int ATT_BK = 64;               // keys per step of the scores and the softmax
constexpr int ATT_TILE = 128;            // keys rebuilt into LDS between two barriers
constexpr int ATT_D = 128;
constexpr int ATT_KROW = ATT_D + 8;      // bf16 per K row in LDS (padded against bank conflicts)
constexpr int ATT_VROW = ATT_TILE + 8;   // bf16 per transposed V row
// bf16 per group of 8 transposed V rows (the 8 channels one thread rebuilds):
// 4 more than 8 rows, so that the 16 groups begin on 16 different banks and the
// rebuild's 2-byte stores, which write one row of each group at once, do not
// all fall on one bank
constexpr int ATT_VGRP = 8 * ATT_VROW + 4;
// K tile, V^T tile, and each wave's query operands (kept in LDS rather than in
// registers while the tiles are rebuilt)
constexpr size_t ATT_LDS = (size_t)2 * (ATT_TILE * ATT_KROW + (ATT_D / 8) * ATT_VGRP) + (size_t)ATT_WAVES * (ATT_D / 32) * 64 * 16;

// 8 channels [8 j, 8 j + 8) of key n of one head of a compressed tensor, in
// three steps so that the loads of K and V go out together: fetch1 issues the
// loads that need nothing (codes, scale, second-level exponent, labels, FP8
// table exponents), fetch2 the centroid rows the labels select, and build
// dequantises and adds the rows from stage T - 1 down to 0 in fp32.
template <int TT, bool FP8>
struct AttnRow {
    uint32_t w, sc;
    int sexp;
    int64_t c;
    int lab[TT];
    int texp[TT];
    uint4 cv[TT];   // bf16 row chunk, or (FP8) the 8 code bytes in .x, .y
};

// The chunk of key n of a tile whose first key lies in chunk c0 (chunk c0 + 1
// starts at c1): one division per tile instead of one per key, and none when
// the chunks are at least a tile long.
struct AttnChunks {
    int64_t c0, c1;
    bool short_chunks;
};

__device__ __forceinline__ AttnChunks attn_chunks(int64_t t0, int chunk_tokens) {
    AttnChunks k;
    k.c0 = t0 / chunk_tokens;
    k.c1 = (k.c0 + 1) * chunk_tokens;
    k.short_chunks = chunk_tokens < ATT_TILE;
    return k;
}

__device__ __forceinline__ int64_t attn_chunk_of(const AttnChunks &k, int64_t n, int chunk_tokens) {
    if (k.short_chunks) return n / chunk_tokens;
    return k.c0 + (n >= k.c1 ? 1 : 0);
}

template <int TT, bool FP8>
__device__ __forceinline__ void attn_fetch1(const AttnSrc &a, const AttnChunks &ck, int head, int64_t n, int j,
                                            AttnRow<TT, FP8> &r) {
    constexpr int D = ATT_D;
    const size_t row = (size_t)head * a.cap + n;
    const int gs = __builtin_ctz(a.G);   // the group size is a power of two
    r.w = reinterpret_cast<const uint16_t *>(a.codes)[row * (D / 8) + j];
    r.sc = a.scales[(row << (7 - gs)) + ((8 * j) >> gs)];   // row x D / G + 8 j / G, D = 128
    r.c = attn_chunk_of(ck, n, a.chunk_tokens);
    r.sexp = a.scale_exp ? a.scale_exp[r.c * a.heads + head] : 0;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        r.lab[t] = a.assign[((size_t)t * a.heads + head) * a.cap + n];
        if constexpr (FP8)
            r.texp[t] = *reinterpret_cast<const int32_t *>(static_cast<const uint8_t *>(a.cent) +
                                                           (((size_t)r.c * TT + t) * a.heads + head) * (a.K * D + 16));
    }
}

template <int TT, bool FP8>
__device__ __forceinline__ void attn_fetch2(const AttnSrc &a, int head, int j, AttnRow<TT, FP8> &r) {
    constexpr int D = ATT_D;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int k = r.lab[t] < a.K ? r.lab[t] : a.K - 1;
        if constexpr (FP8) {
            const uint8_t *tbl = static_cast<const uint8_t *>(a.cent) + (((size_t)r.c * TT + t) * a.heads + head) *
                                                                            (a.K * D + 16);
            const uint2 v = *reinterpret_cast<const uint2 *>(tbl + 16 + (size_t)k * D + 8 * j);
            r.cv[t] = make_uint4(v.x, v.y, 0u, 0u);
        } else {
            r.cv[t] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.cent) +
                                                       ((((size_t)r.c * TT + t) * a.heads + head) * a.K + k) * D + 8 * j);
        }
    }
}

template <int TT, bool FP8>
__device__ __forceinline__ void attn_build(const AttnSrc &a, const AttnRow<TT, FP8> &r, float *y) {
    const float sx = a.scale_exp ? ldexpf(1.f, r.sexp) : 1.f;
    dequant8(r.w, e4m3_decode(r.sc) * sx, y);
#pragma unroll
    for (int t = TT - 1; t >= 0; --t) {
        uint4 cv;
        if constexpr (FP8) {
            const float sf = ldexpf(1.f, r.texp[t]);
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t ww = q < 2 ? r.cv[t].x : r.cv[t].y, sh = 16 * (q & 1);
                o[q] = (__float_as_uint(e4m3_decode((ww >> sh) & 0xFFu) * sf) >> 16) |
                       (__float_as_uint(e4m3_decode((ww >> (sh + 8)) & 0xFFu) * sf) & 0xFFFF0000u);
            }
            cv = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            cv = r.cv[t];
        }
        add8<uint16_t>(&cv, y);
    }
}

template <int TT, bool FP8>
__global__ __launch_bounds__(64 * ATT_WAVES, 1) void k_attention(AttnArgs a) {
    constexpr int D = ATT_D;
    extern __shared__ uint16_t att_lds[];
    uint16_t *lk = att_lds;                              // [ATT_TILE][ATT_KROW]
    uint16_t *lvt = lk + ATT_TILE * ATT_KROW;              // [D / 8][ATT_VGRP]: row c at (c / 8) ATT_VGRP + (c % 8) ATT_VROW
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, split = blockIdx.z;
    const int64_t kb0 = a.tok_begin + (int64_t)split * a.keys_per_split;
    const int64_t kb1 = min(a.tok_end, kb0 + a.keys_per_split);
    const int g = lane >> 4, c16 = lane & 15;
    const int q0 = blockIdx.x * ATT_BQ + wave * 16;
    // this wave's queries as B operands of S^T = K Q^T: column c16, channels 32 s + 8 g .. + 7
    // lq[wave][s][lane]: the lane's 16 bytes of k-step s, read back per tile so
    // that they hold no registers while the tiles are rebuilt (a wave reads
    // only what it wrote)
    uint4 *lq = reinterpret_cast<uint4 *>(lvt + (D / 8) * ATT_VGRP) + (size_t)wave * (D / 32) * 64 + lane;
    {
        const int qr = min(q0 + c16, a.Nq - 1);
        const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (size_t)h * a.q_hs + (size_t)qr * D + 8 * g);
#pragma unroll
        for (int s = 0; s < D / 32; ++s) lq[s * 64] = qp[4 * s];
    }
    // O^T = V^T P^T: lane holds channels 16 b + 4 g + r of query c16
    f32x4_t o[D / 16];
#pragma unroll
    for (int b = 0; b < D / 16; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -__builtin_inff(), l = 0.f;   // the lane's query: running maximum (base 2) and sum
    const int j = tid & 15;  // the 8-channel slice this thread rebuilds
    for (int64_t t0 = kb0; t0 < kb1; t0 += ATT_TILE) {
        __syncthreads();   // the previous tile's readers are done
        const AttnChunks ckk = attn_chunks(t0, a.k.chunk_tokens), ckv = attn_chunks(t0, a.v.chunk_tokens);
#pragma unroll 1
        for (int kp = 0; kp < ATT_TILE; kp += 64) {
            const int kk = (tid >> 4) + kp;   // the key this thread rebuilds
            const int64_t n = t0 + kk;
            float yk[8], yv[8];
            if (n < kb1) {
                AttnRow<TT, FP8> rk, rv;
                attn_fetch1<TT, FP8>(a.k, ckk, a.khead0 + h, n, j, rk);
                attn_fetch1<TT, FP8>(a.v, ckv, a.vhead0 + h, n, j, rv);
                float cs[8];
                if (a.rope) load8_f32(a.rope + (size_t)(n - a.tok_begin) * D + 8 * j, cs);
                attn_fetch2<TT, FP8>(a.k, a.khead0 + h, j, rk);
                attn_fetch2<TT, FP8>(a.v, a.vhead0 + h, j, rv);
                attn_build<TT, FP8>(a.k, rk, yk);
                if (a.rope) rope8(cs, yk);
                attn_build<TT, FP8>(a.v, rv, yv);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) yk[i] = yv[i] = 0.f;
            }
            *reinterpret_cast<uint4 *>(lk + kk * ATT_KROW + 8 * j) =
                make_uint4(pack_bf16x2(yk[0], yk[1]), pack_bf16x2(yk[2], yk[3]), pack_bf16x2(yk[4], yk[5]),
                           pack_bf16x2(yk[6], yk[7]));
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t pv = pack_bf16x2(yv[i], yv[i + 1]);
                lvt[j * ATT_VGRP + i * ATT_VROW + kk] = (uint16_t)pv;
                lvt[j * ATT_VGRP + (i + 1) * ATT_VROW + kk] = (uint16_t)(pv >> 16);
            }
        }
        __syncthreads();
        // a wave whose 16 queries all lie past Nq (the last query block of a
        // head) helps rebuild the tiles but has nothing to multiply
        if (q0 >= a.Nq) continue;
        bf16x8_t qb[D / 32];
#pragma unroll
        for (int s = 0; s < D / 32; ++s) qb[s] = __builtin_bit_cast(bf16x8_t, lq[s * 64]);
#pragma unroll 1
        for (int k0 = 0; k0 < ATT_TILE; k0 += ATT_BK) {   // steps of ATT_BK keys of the tile
        // S^T = K Q^T for 4 blocks of 16 keys: sacc[kb][r] = score of key
        // k0 + 16 kb + 4 g + r for the lane's query c16
        f32x4_t sacc[ATT_BK / 16];
#pragma unroll
        for (int kb = 0; kb < ATT_BK / 16; ++kb) {
            sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const uint16_t *kr = lk + (k0 + 16 * kb + c16) * ATT_KROW + 8 * g;
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
                sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(kr + 32 * s)), qb[s], sacc[kb], 0,
                    0, 0);
        }
        // online softmax in base 2 for the lane's query; its 64 scores sit in
        // the 4 lanes c16, c16 + 16, c16 + 32, c16 + 48
        float mx = -__builtin_inff();
        if (t0 + k0 + ATT_BK <= kb1) {   // every key of the step is in range
#pragma unroll
            for (int kb = 0; kb < ATT_BK / 16; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sacc[kb][r] = sacc[kb][r] * a.scale_log2;
                    mx = fmaxf(mx, sacc[kb][r]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < ATT_BK / 16; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = t0 + k0 + 16 * kb + 4 * g + r < kb1;
                    const float v = valid ? sacc[kb][r] * a.scale_log2 : -__builtin_inff();
                    sacc[kb][r] = v;
                    mx = fmaxf(mx, v);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float corr = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < ATT_BK / 16; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pe = __builtin_amdgcn_exp2f(sacc[kb][r] - mn);
                sacc[kb][r] = pe;
                rs += pe;
            }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        l = l * corr + rs;
        // once the running maxima settle, corr is exactly 1 for every query of
        // the wave and the rescale would change nothing
        if (__builtin_amdgcn_ballot_w64(corr != 1.f)) {
#pragma unroll
            for (int b = 0; b < D / 16; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[b][r] *= corr;
        }
        // O^T += V^T P^T over 32-key steps.  The step's k index 8 g + i stands
        // for key 4 g + i (i < 4) or 16 + 4 g + i - 4 (i >= 4) of the step, the
        // keys this lane holds P of, so P^T comes straight from registers; V^T
        // reads the same keys from the transposed tile.
#pragma unroll
        for (int s = 0; s < ATT_BK / 32; ++s) {
            const uint4 pw = make_uint4(pack_bf16x2(sacc[2 * s][0], sacc[2 * s][1]),
                                        pack_bf16x2(sacc[2 * s][2], sacc[2 * s][3]),
                                        pack_bf16x2(sacc[2 * s + 1][0], sacc[2 * s + 1][1]),
                                        pack_bf16x2(sacc[2 * s + 1][2], sacc[2 * s + 1][3]));
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
            for (int b = 0; b < D / 16; ++b) {
                const int vrow = 16 * b + c16;
                const uint16_t *vr = lvt + (vrow >> 3) * ATT_VGRP + (vrow & 7) * ATT_VROW + k0 + 32 * s + 4 * g;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vr), hi = *reinterpret_cast<const uint2 *>(vr + 16);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
                o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[b], 0, 0, 0);
            }
        }
        }
    }
    // this split's unnormalised output and row statistics
    const int qi = q0 + c16;
    if (qi < a.Nq) {
        const size_t base = ((size_t)split * a.H + h) * a.Nq + qi;
#pragma unroll
        for (int b = 0; b < D / 16; ++b)
            *reinterpret_cast<float4 *>(a.part_o + base * D + 16 * b + 4 * g) = make_float4(o[b][0], o[b][1], o[b][2], o[b][3]);
        if (g == 0) {
            a.part_ml[base * 2] = m;
            a.part_ml[base * 2 + 1] = l;
        }
    }
}

// Combines the splits of every (head, query): O = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s and lse = (M + log2 sum_s 2^(m_s - M) l_s) ln 2.
__global__ __launch_bounds__(128) void k_attn_merge(const float *part_o, const float *part_ml, int splits, int H,
                                                    int Nq, float *out, int64_t out_hs, float *lse) {
    const int qi = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    float M = -__builtin_inff();
    for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[(((size_t)s * H + h) * Nq + qi) * 2]);
    float den = 0.f, num = 0.f;
    for (int s = 0; s < splits; ++s) {
        const size_t i = ((size_t)s * H + h) * Nq + qi;
        const float w = exp2f(part_ml[i * 2] - M);
        den += w * part_ml[i * 2 + 1];
        num += w * part_o[i * ATT_D + d];
    }
    out[(size_t)h * out_hs + (size_t)qi * ATT_D + d] = num / den;
    if (lse && d == 0) lse[(size_t)h * Nq + qi] = (M + log2f(den)) * 0.69314718055994530942f;
}

hipError_t launch_attention(const AttnArgs &a, float *out, int64_t out_hs, float *lse, hipStream_t s) {
    const dim3 g((unsigned)((a.Nq + ATT_BQ - 1) / ATT_BQ), (unsigned)a.H, (unsigned)a.splits), b(64 * ATT_WAVES);
#define QVG_ATT(TT, F8)                                                                                         \
    do {                                                                                                        \
        (void)hipFuncSetAttribute((const void *)k_attention<TT, F8>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                  (int)ATT_LDS);                                                                \
        QVG_KERNEL((k_attention<TT, F8>), g, b, ATT_LDS, s, a);                                                 \
    } while (0)
#define QVG_ATT_T(F8)                                                                                           \
    do {                                                                                                        \
        switch (a.T) {                                                                                          \
            case 1: QVG_ATT(1, F8); break;                                                                      \
            case 2: QVG_ATT(2, F8); break;                                                                      \
            case 3: QVG_ATT(3, F8); break;                                                                      \
            default: QVG_ATT(4, F8); break;                                                                     \
        }                                                                                                       \
    } while (0)
    if (a.fp8) QVG_ATT_T(true); else QVG_ATT_T(false);
#undef QVG_ATT_T
#undef QVG_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    QVG_KERNEL(k_attn_merge, dim3((unsigned)a.Nq, (unsigned)a.H), dim3(ATT_D), 0, s, a.part_o, a.part_ml, a.splits,
               a.H, a.Nq, out, out_hs, lse);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fixed device scratch of the entry point that allocates nothing
// ---------------------------------------------------------------------------

// One array per GPU, loaded with the code object and held until the process
// ends.  In host code `scratch` names only a host-side stand-in: kernels get
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void **ptr) {
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void *addr[MAX_DEVICES] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// zero fill
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_zero(int32_t *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
    QVG_KERNEL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_zero(int32_t *p, int64_t n, hipStream_t s) {
    QVG_KERNEL(k_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace qvg
