/*
 * qvg.h - C ABI of the Quant VideoGen (QVG) KV-cache codec for AMD MI355X (gfx950).
 *
 * The codec compresses the key or value cache of an autoregressive video
 * diffusion model chunk by chunk and rebuilds it for attention:
 *
 *   encode (per head, per chunk of a few latent frames):
 *     semantic-aware smoothing  = k-means over the chunk's d-dim token rows,
 *                                 subtract each row's centroid;
 *     progressive residual stages t = 1..T: R(0) = X, stage t clusters R(t-1)
 *                                 and yields R(t), centroids C(t), assignment pi(t);
 *     2-bit group quantisation of R(T) with FP8 E4M3 per-group scales.
 *   decode: dequantise R(T) and add back C(T)[pi(T)] + ... + C(1)[pi(1)] in one pass.
 *
 * Sources: "Quant VideoGen: Auto-Regressive Long Video Generation via 2-Bit
 * KV-Cache Quantization" as summarised by the 163.com article (sections 3-5 and 7),
 * and by gist.science (German and Portuguese technical summaries, sections 2A-2C).
 *
 * Conventions (all entry points):
 *  - Every function returns a qvg_status (int32_t).  Arguments are validated on
 *    the host before anything is launched; a rejected call launches nothing and
 *    leaves every buffer untouched.  A failed launch returns QVG_ERR_HIP.  A fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - Device pointers are caller-owned (allocated by the caller, e.g. through
 *    PyTorch) and must be 16-byte aligned; head strides are in elements and must
 *    keep every row 16-byte aligned.  The library allocates device memory only in
 *    qvg_centroid_cache_create and frees it in qvg_centroid_cache_destroy.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued
 *    asynchronously on it; the library never synchronises the device.  Calls that
 *    share a cache, a destination or a workspace must be ordered on one stream.
 *  - Input values must be finite.
 *  - Layouts are row-major; "[H][N][d]" means head-major, then token, then channel.
 *  - dtype codes: QVG_F32 = fp32, QVG_BF16 = bfloat16 (raw 16-bit storage).
 */
#ifndef QVG_H
#define QVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qvg_status;
enum {
    QVG_OK = 0,
    QVG_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or range        */
    QVG_ERR_UNSUPPORTED = -2, /* a configuration the kernels do not implement      */
    QVG_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes query */
    QVG_ERR_STATE = -4,       /* cache bound to another (config, heads)             */
    QVG_ERR_HIP = -5,         /* a HIP runtime call or launch failed                */
    QVG_ERR_OOM = -6          /* device allocation failed (cache creation)          */
};

enum { QVG_F32 = 0, QVG_BF16 = 1 };

/* How the per-group scales are formed (qvg_config.scale_mode). */
enum {
    QVG_SCALE_E4M3 = 0,     /* E4M3FN(max|r| / 1.5), saturating at 448                         */
    QVG_SCALE_TWO_LEVEL = 1 /* E4M3FN(max|r| / 1.5 / 2^f) worth its value * 2^f, with one f >= 0
                               per (chunk, head), the smallest that saturates no group          */
};

/* How the centroid tables are stored (qvg_config.centroid_format). */
enum {
    QVG_CENT_NATIVE = 0, /* in the tensor dtype (bf16 or fp32)                          */
    QVG_CENT_E4M3 = 1    /* FP8: per table a 16-byte header with an exponent e (int32,
                            then zeros) and K*d E4M3FN codes; value = code value * 2^e */
};

#define QVG_MAX_CENTROIDS 256 /* assignments are stored as uint8 (163.com, section 7) */
#define QVG_MAX_STAGES 8

/* Codec settings.  The pages fix 256 centroids with uint8 assignments and group
 * sizes 16 or 64 (163.com article, section 7); the rest are this library's
 * readings (cold start = Forgy rows from a SplitMix64-keyed shuffle; a number
 * of Lloyd rounds, then one final assignment).
 *   d            head dimension: 64 or 128
 *   n_centroids  K, 1..256
 *   n_stages     T, 0..8 (T = 0 quantises X directly: the round-to-nearest baseline)
 *   group_size   G in {16, 32, 64, 128}, dividing d (channels per scale)
 *   iters_cold   Lloyd rounds when the chunk starts from the seeded draw (>= 0)
 *   iters_warm   Lloyd rounds when it starts from cached/given centroids (>= 0)
 *   converge     0: exactly iters_cold / iters_warm rounds.  c >= 1: those are
 *                maxima, and a head's rounds of a stage stop at the first
 *                assignment after the first round that moves fewer than c of
 *                its tokens to another centroid, before that round's update
 *                (k-means run until its labels settle; the pages report fewer
 *                rounds when it starts from the cached centroids: 163.com
 *                article, section 5; gist.science summaries, section 2C).
 *                c = 1 stops at a fixed point, so the result equals that of any
 *                larger fixed count.  The decision is taken on the device per
 *                head, without a host synchronisation; qvg_encode_rounds
 *                reports the rounds run.
 *   seed         codec seed; the cold draw of (head h, stage t) is keyed by
 *                ((seed * 65536 + h) * 64 + t) mod 2^64
 *   dtype        QVG_BF16 or QVG_F32: the input X (and the stored centroids with
 *                QVG_CENT_NATIVE)
 *   centroid_format  QVG_CENT_NATIVE, or QVG_CENT_E4M3: every stored table
 *                (chunk, stage, head) in the FP8 format the pages use for the
 *                scales (163.com article, sections 5-7, where the centroids are
 *                a small share of the compressed bytes): e is the smallest
 *                exponent with max|C| <= 448 * 2^e, each value the E4M3FN code
 *                of C / 2^e (nearest, ties to even).  A stage's labels and the
 *                later residuals use the stored values; the streaming cache
 *                keeps the unrounded fp32 centroids.  Halves the table bytes.
 *   scale_mode   QVG_SCALE_E4M3, or QVG_SCALE_TWO_LEVEL: value residuals with
 *                outliers near 1e3 (163.com article, section 2) can exceed what an
 *                E4M3 scale holds (448 * 1.5 = 672); a second-level power of two
 *                per (chunk, head) in the view's scale_exp extends the range
 *                exactly.  It lowers the worst error of saturating groups; the
 *                larger step also applies to the rest of their group.  A chunk
 *                with no saturating group keeps f = 0 and the plain result.    */
typedef struct {
    int32_t d;
    int32_t n_centroids;
    int32_t n_stages;
    int32_t group_size;
    int32_t iters_cold;
    int32_t iters_warm;
    uint64_t seed;
    int32_t dtype;
    int32_t converge; /* >= 0 */
    int32_t centroid_format;
    int32_t scale_mode;
} qvg_config;

/* The compressed cache of one tensor (K or V) of one layer, caller-allocated.
 *   codes      [H][cap_tokens][d/4]       uint8, four 2-bit codes per byte, lowest channel in bits 0-1
 *   scales     [H][cap_tokens][d/G]       uint8, FP8 E4M3FN (OCP) per-group scales
 *   assign     [T][H][cap_tokens]         uint8 centroid index per token and stage
 *   centroids  [n_chunks][T][H] tables of K x d stored centroids: dtype values
 *              (QVG_CENT_NATIVE) or 16 + K*d bytes each (QVG_CENT_E4M3),
 *              n_chunks = ceil(cap_tokens / chunk_tokens)
 *   scale_exp  [n_chunks][H] int8 second-level scale exponents
 *              (QVG_SCALE_TWO_LEVEL; may be NULL otherwise)
 * Chunk c holds tokens [c * chunk_tokens, min((c + 1) * chunk_tokens, cap_tokens)).
 * Buffer sizes: qvg_cache_view_bytes.                                           */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    uint8_t *assign;
    void *centroids;
    int64_t cap_tokens;
    int32_t chunk_tokens;
    int32_t heads;
    int8_t *scale_exp;
} qvg_cache_view;

/* Streaming centroid cache (163.com article, section 5; gist.science summaries,
 * section 2C): the final fp32 centroids of every (stage, head) of the last
 * encoded chunk, used to start the next chunk's k-means.  Opaque. */
typedef struct qvg_centroid_cache qvg_centroid_cache;

/* Human-readable name of a status code (static string, never NULL). */
const char *qvg_status_string(qvg_status status);

/* Validates a configuration without touching the GPU: QVG_OK, QVG_ERR_INVALID_ARG
 * (out-of-range field) or QVG_ERR_UNSUPPORTED (valid but not implemented). */
qvg_status qvg_config_validate(const qvg_config *cfg);

/* Bytes one encoded chunk of `heads` x `n_tokens` occupies, by component, in
 * the storage format of the 163.com article (section 5, implementation details:
 * 2-bit codes with FP8 E4M3 per-group scales; section 7: uint8 assignments of
 * 256 centroids, group sizes 16 / 64; the stored centroids of every stage):
 * out[0] codes = H*N*d/4, out[1] scales = H*N*d/G, out[2] assignments = T*H*N,
 * out[3] centroids = T*H*K*d*sizeof(dtype) (QVG_CENT_E4M3: T*H*(16 + K*d)).
 * Host only. */
qvg_status qvg_chunk_bytes(const qvg_config *cfg, int32_t heads, int32_t n_tokens, uint64_t out[4]);

/* Sizes of the four buffers of a qvg_cache_view holding `cap_tokens` tokens per
 * head in chunks of `chunk_tokens`: out[0..3] = codes, scales, assign, centroids.
 * Host only. */
qvg_status qvg_cache_view_bytes(const qvg_config *cfg, int32_t heads, int64_t cap_tokens,
                                int32_t chunk_tokens, uint64_t out[4]);

/* Device workspace qvg_encode_chunk needs for `heads` x `n_tokens`.  Host only. */
qvg_status qvg_encode_workspace_bytes(const qvg_config *cfg, int32_t heads, int32_t n_tokens,
                                      uint64_t *bytes);

/* Creates a centroid cache for (cfg, heads) on the current device: one fp32
 * [T][H][K][d] buffer, marked empty.  QVG_ERR_OOM if the allocation fails. */
qvg_status qvg_centroid_cache_create(const qvg_config *cfg, int32_t heads, qvg_centroid_cache **out);

/* Marks the cache empty: the next encode through it starts cold. */
qvg_status qvg_centroid_cache_reset(qvg_centroid_cache *cache);

/* Frees the cache (NULL is accepted).  The caller must make sure no enqueued
 * work still uses it. */
qvg_status qvg_centroid_cache_destroy(qvg_centroid_cache *cache);

/* Device pointer to the cache's fp32 [T][H][K][d] centroids and whether they are
 * valid (1) or not (0).  For inspection and checkpointing. */
qvg_status qvg_centroid_cache_data(qvg_centroid_cache *cache, float **centroids, int32_t *valid);

/* Checkpointing of the streaming state: copies the cache's fp32 [T][H][K][d]
 * centroids to / from a caller-owned device buffer on `stream`.  Import marks the
 * cache valid (the next encode through it starts warm); export of an empty cache
 * is QVG_ERR_STATE. */
qvg_status qvg_centroid_cache_export(qvg_centroid_cache *cache, float *dst, void *stream);
qvg_status qvg_centroid_cache_import(qvg_centroid_cache *cache, const float *src, void *stream);

/* Encodes one chunk of one tensor and writes it into chunk `chunk_index` of `dst`
 * (163.com article, sections 3-5; gist.science German summary, sections 2A-2C).
 *   x               device [H][N][d] in cfg->dtype; head h starts at x + h * x_head_stride
 *                   elements, rows of d contiguous; x_head_stride >= N*d
 *   heads, n_tokens H = dst->heads, 1 <= N <= dst->chunk_tokens; a chunk shorter than
 *                   chunk_tokens must be the last one the view can hold
 *   init_centroids  NULL, or device fp32 [T][H][K][d] starting centroids used
 *                   like a warm cache (iters_warm rounds)
 *   cache           NULL (cold start, nothing recorded) or a cache created for
 *                   (cfg, heads): if it holds centroids they start the k-means
 *                   (iters_warm rounds), otherwise the seeded draw does
 *                   (iters_cold); afterwards it holds this chunk's final fp32
 *                   centroids.  init_centroids, when given, wins over the cache
 *                   for the start but the cache is still updated.
 *   workspace       device scratch of at least qvg_encode_workspace_bytes; its
 *                   contents on entry do not matter
 * Writes codes, scales, assignments of tokens [chunk_index*chunk_tokens, +N) and
 * the chunk's centroid block.  QVG_ERR_STATE if `cache` was created for another
 * (cfg, heads); QVG_ERR_WORKSPACE if workspace_bytes is too small. */
qvg_status qvg_encode_chunk(const qvg_config *cfg, const void *x, int64_t x_head_stride,
                            int32_t heads, int32_t n_tokens, const float *init_centroids,
                            qvg_centroid_cache *cache, const qvg_cache_view *dst,
                            int32_t chunk_index, void *workspace, uint64_t workspace_bytes,
                            void *stream);

/* Lloyd rounds (updates) that every (stage, head) ran in the last
 * qvg_encode_chunk call made with `workspace` (same cfg, heads, n_tokens), when
 * cfg->converge >= 1: device int32 [T][H], copied to rounds_out on `stream`
 * (163.com article, section 5: the cache's saving in k-means rounds).
 * QVG_ERR_STATE when cfg->converge == 0 or T == 0 (fixed counts). */
qvg_status qvg_encode_rounds(const qvg_config *cfg, int32_t heads, int32_t n_tokens, const void *workspace,
                             uint64_t workspace_bytes, int32_t *rounds_out, void *stream);

/* qvg_encode_chunk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same encode, bit for bit, with the workspace taken from a fixed device
 * array of QVG_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends.  The call allocates and frees nothing.
 *   Limit: qvg_encode_workspace_bytes(cfg, heads, n_tokens) must not exceed
 *   QVG_STATIC_SCRATCH_BYTES (at d = 128, K = 256, T = 2, bf16: up to 45 heads
 *   of a 4,680-token chunk); a larger call returns QVG_ERR_WORKSPACE and
 *   launches nothing.
 *   Every call on one GPU uses that GPU's one array, and its contents on entry
 *   do not matter: calls that overlap on one GPU (two streams, or two threads)
 *   race on it and must not be made.  The first call on a device looks the
 *   array's address up (QVG_ERR_HIP if that fails).
 * Other arguments, results and errors as qvg_encode_chunk. */
#define QVG_STATIC_SCRATCH_BYTES ((uint64_t)64 << 20)
qvg_status qvg_encode_chunk_static(const qvg_config *cfg, const void *x, int64_t x_head_stride,
                                   int32_t heads, int32_t n_tokens, const float *init_centroids,
                                   qvg_centroid_cache *cache, const qvg_cache_view *dst,
                                   int32_t chunk_index, void *stream);

/* Rebuilds tokens [tok_begin, tok_end) of every head from `src` in one fused pass
 * (163.com article, sections 4-5: reconstruction in reverse stage order; fused
 * dequantise-and-centroid kernel; gist.science summaries, section 2C):
 *   y = (q - 1.5) * scale, then y += C(t)[pi(t)] for t = T .. 1 in fp32,
 *   written as out_dtype (bf16 round-to-nearest-even, or fp32).
 *   out   device [H][tok_end - tok_begin][d]; head h at out + h * out_head_stride elements
 * Requires 0 <= tok_begin < tok_end <= src->cap_tokens; the tokens must have been
 * encoded. */
qvg_status qvg_decode(const qvg_config *cfg, const qvg_cache_view *src, int64_t tok_begin,
                      int64_t tok_end, void *out, int64_t out_head_stride, int32_t out_dtype,
                      void *stream);

/* qvg_decode with the rotary position embedding applied in the same pass.  Keys
 * are cached before the rotation because that distribution quantises better
 * (163.com article, section 5, implementation details), so a consumer of the
 * decoded keys must still rotate them; here that happens before the single
 * rounding to out_dtype.  The pages do not fix the rotation's layout: pair p of a
 * row is channels (2p, 2p + 1), and with (c, s) the cos and sin of the pair's
 * angle for that token,
 *   (a, b) -> (a*c - b*s, a*s + b*c), every product and sum rounded to fp32.
 *   rope        device fp32 [tok_end - tok_begin][d/2][2]: (cos, sin) of every pair
 *               of every decoded token, the same for all heads (any 1-D or
 *               per-axis 3-D position scheme); 16-byte aligned
 *   rope_heads  heads [0, rope_heads) are rotated (the keys of a K-then-V
 *               cache), the rest are decoded as by qvg_decode; 0 <= rope_heads <= H
 * Other arguments and errors as qvg_decode; a null or misaligned rope, or
 * rope_heads out of range, is QVG_ERR_INVALID_ARG. */
qvg_status qvg_decode_rope(const qvg_config *cfg, const qvg_cache_view *src, int64_t tok_begin,
                           int64_t tok_end, const float *rope, int32_t rope_heads, void *out,
                           int64_t out_head_stride, int32_t out_dtype, void *stream);

/* Attention that reads the compressed cache directly (163.com article, section 5:
 * the fused dequantisation kernel keeps the rebuilt keys and values out of
 * memory; gist.science summaries, section 2C): for attention head h and query i,
 *   O[h][i] = sum_j softmax_j(scale <q_i, k_j>) v_j,  lse[h][i] = ln sum_j exp(scale <q_i, k_j>),
 * over the keys j in [tok_begin, tok_end), with k_j and v_j the rows qvg_decode
 * (keys: qvg_decode_rope when `rope` is given) would write in bf16, rebuilt in
 * the kernel tile by tile and never stored.  Scores and sums in fp32 on the
 * matrix cores; the softmax weights enter the sum with V as bf16.
 *   k_src, k_head0   keys: attention head h reads head k_head0 + h of k_src
 *   v_src, v_head0   values: head v_head0 + h of v_src (one K-then-V cache of
 *                    2H heads: the same view, k_head0 = 0, v_head0 = H)
 *   rope             NULL, or fp32 [tok_end - tok_begin][d/2][2] (cos, sin) that
 *                    rotates the keys as qvg_decode_rope does; 16-byte aligned
 *   q                bf16 [heads][n_queries][d] (rotated by the caller), head
 *                    stride q_head_stride elements, 16-byte aligned
 *   scale            the score scale (> 0), e.g. 1 / sqrt(d)
 *   out              fp32 [heads][n_queries][d], head stride out_head_stride
 *   lse              NULL or fp32 [heads][n_queries]
 *   workspace        device scratch of qvg_attention_workspace_bytes(cfg, heads,
 *                    n_queries, tok_end - tok_begin) bytes (the key range is
 *                    split over workgroups; the splits merge by their lse)
 * Requires d = 128, a bf16 cache with 1-4 stages (QVG_ERR_UNSUPPORTED otherwise)
 * and both views holding the tokens; other conventions as qvg_decode. */
qvg_status qvg_attention_workspace_bytes(const qvg_config *cfg, int32_t heads, int32_t n_queries, int64_t n_keys,
                                         uint64_t *bytes);
qvg_status qvg_attention(const qvg_config *cfg, const qvg_cache_view *k_src, int32_t k_head0,
                         const qvg_cache_view *v_src, int32_t v_head0, int64_t tok_begin, int64_t tok_end,
                         const float *rope, const void *q, int64_t q_head_stride, int32_t heads, int32_t n_queries,
                         float scale, float *out, int64_t out_head_stride, float *lse, void *workspace,
                         uint64_t workspace_bytes, void *stream);

/* ---- stage-level entry points (same conventions), for parity checks and profiling ---- */

/* Workspace the stage-level k-means calls need for (heads, n_tokens, d, K). Host only. */
qvg_status qvg_stage_workspace_bytes(int32_t heads, int32_t n_tokens, int32_t d,
                                     int32_t n_centroids, uint64_t *bytes);

/* k-means assignment step (163.com article, section 3; German summary, section 2A):
 * pi[h][n] = argmin_k |c_k|^2 - 2 <x_n, c_k> with both operands rounded to bf16 and
 * the products accumulated in fp32 on the matrix cores; ties go to the lowest k.
 *   x          device [H][N][d] (x_dtype), head stride x_head_stride elements
 *   centroids  device fp32 [H][K][d]
 *   assign_out device uint8 [H][N], head stride assign_head_stride */
qvg_status qvg_kmeans_assign(const void *x, int32_t x_dtype, int64_t x_head_stride,
                             const float *centroids, int32_t heads, int32_t n_tokens, int32_t d,
                             int32_t n_centroids, uint8_t *assign_out, int64_t assign_head_stride,
                             void *workspace, uint64_t workspace_bytes, void *stream);

/* k-means update step (same sections): every centroid with at least one token
 * becomes the mean of its tokens' unrounded rows, defined exactly so that it does
 * not depend on the order of summation: the exact column sum, rounded once to
 * fp64, divided by the count in fp64, rounded to fp32.  A centroid with no token
 * keeps its value.
 *   centroids  device fp32 [H][K][d], read and overwritten
 *   counts_out NULL or device int32 [H][K] tokens per centroid */
qvg_status qvg_centroid_update(const void *x, int32_t x_dtype, int64_t x_head_stride,
                               const uint8_t *assign, int64_t assign_head_stride, int32_t heads,
                               int32_t n_tokens, int32_t d, int32_t n_centroids, float *centroids,
                               int32_t *counts_out, void *workspace, uint64_t workspace_bytes,
                               void *stream);

/* 2-bit group quantisation (163.com article, section 5): per token and group of G
 * channels, a = max|r|, scale = E4M3FN(a / 1.5) saturating at 448,
 * q = [r >= -s] + [r >= 0] + [r >= s], four codes per byte.
 *   r      device fp32 [H][N][d], head stride r_head_stride elements
 *   codes  device uint8 [H][N][d/4];  scales device uint8 [H][N][d/G] */
qvg_status qvg_group_quant(const float *r, int64_t r_head_stride, int32_t heads, int32_t n_tokens,
                           int32_t d, int32_t group_size, uint8_t *codes, uint8_t *scales,
                           void *stream);

/* Fused dequantise-and-reconstruct of one chunk's raw arrays (the kernel behind
 * qvg_decode; 163.com article, section 4: reconstruction from the final
 * quantised residual, adding back each stage's stored centroids in reverse;
 * section 5: the fused dequantisation kernel; storage format of sections 5 and 7):
 *   codes [H][N][d/4], scales [H][N][d/G], assign [T][H][N] uint8,
 *   centroids [T][H] tables in cfg's centroid format  ->  out [H][N][d] (out_dtype),
 *   contiguous.  QVG_ERR_UNSUPPORTED with two-level scales (use qvg_decode). */
qvg_status qvg_dequant_reconstruct(const qvg_config *cfg, int32_t heads, int32_t n_tokens,
                                   const uint8_t *codes, const uint8_t *scales,
                                   const uint8_t *assign, const void *centroids, void *out,
                                   int32_t out_dtype, void *stream);

/* ---- profiling aid: per-kernel timing with HIP events ---- */

/* One kernel's totals since profiling was enabled: launches, summed duration
 * (ms, between HIP events recorded on the launch stream around each launch),
 * and the launches' algorithmic work (FLOPs and HBM bytes the operation must
 * move, counted once). */
typedef struct {
    char name[32];
    int64_t launches;
    double total_ms;
    double flops;
    double bytes;
} qvg_kernel_stat;

/* on != 0: drop earlier records and bracket every following launch with two
 * events; on == 0: stop recording (records are kept for qvg_profile_read).
 * Process-wide; adds two event records per launch while on. */
qvg_status qvg_profile_enable(int32_t on);

/* Waits for the recorded events and writes up to max_entries per-kernel totals;
 * *n_entries receives the number of distinct kernels recorded. */
qvg_status qvg_profile_read(qvg_kernel_stat *out, int32_t max_entries, int32_t *n_entries);

#ifdef __cplusplus
}
#endif
#endif /* QVG_H */
