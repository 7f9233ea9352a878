// C ABI of the Quant VideoGen KV-cache codec: argument validation, workspace
// layout, the centroid cache object and the per-chunk stage loop.  Every step
// of the codec runs in the gfx950 kernels behind qvg_launch.h.
//
// The stage loop follows the pages' progressive residual quantisation
// (163.com article, section 4; gist.science German summary, section 2B): stage t
// clusters R(t-1), stores C(t) and pi(t) and forms R(t) = R(t-1) - C(t)[pi(t)];
// the last stage's residual goes straight into the 2-bit quantiser.  k-means
// starts from the streaming centroid cache when it holds the previous chunk's
// centroids (163.com article, section 5; German summary, section 2C).

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "qvg.h"
#include "qvg_launch.h"

struct qvg_centroid_cache {
    int32_t d, n_centroids, n_stages, heads;
    float *data;     // [T][H][K][d] fp32, device
    int32_t valid;   // host-side: set when an encode through this cache is enqueued
};

namespace qvg {
LaunchEvents &launch_events() {
    thread_local LaunchEvents ev;
    return ev;
}
}  // namespace qvg

namespace {

using namespace qvg;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
size_t dtype_size(int dt) { return dt == QVG_BF16 ? 2 : 4; }
// Bytes of one stored centroid table (one chunk, stage and head).
size_t table_bytes(const qvg_config &c) {
    const size_t kd = (size_t)c.n_centroids * c.d;
    return c.centroid_format == QVG_CENT_E4M3 ? kd + 16 : kd * dtype_size(c.dtype);
}

qvg_status check_config(const qvg_config *c) {
    if (!c) return QVG_ERR_INVALID_ARG;
    if (c->converge < 0) return QVG_ERR_INVALID_ARG;
    if (c->scale_mode != QVG_SCALE_E4M3 && c->scale_mode != QVG_SCALE_TWO_LEVEL) return QVG_ERR_INVALID_ARG;
    if (c->centroid_format != QVG_CENT_NATIVE && c->centroid_format != QVG_CENT_E4M3) return QVG_ERR_INVALID_ARG;
    if (c->d <= 0 || c->group_size <= 0) return QVG_ERR_INVALID_ARG;
    if (c->n_centroids < 1 || c->n_centroids > QVG_MAX_CENTROIDS) return QVG_ERR_INVALID_ARG;
    if (c->n_stages < 0 || c->n_stages > QVG_MAX_STAGES) return QVG_ERR_INVALID_ARG;
    if (c->iters_cold < 0 || c->iters_warm < 0) return QVG_ERR_INVALID_ARG;
    if (c->dtype != QVG_F32 && c->dtype != QVG_BF16) return QVG_ERR_INVALID_ARG;
    if (c->d % c->group_size != 0) return QVG_ERR_INVALID_ARG;
    if (c->d != 64 && c->d != 128) return QVG_ERR_UNSUPPORTED;
    const int g = c->group_size;
    if (g != 16 && g != 32 && g != 64 && g != 128) return QVG_ERR_UNSUPPORTED;
    return QVG_OK;
}

qvg_status hip_status(hipError_t e) { return e == hipSuccess ? QVG_OK : QVG_ERR_HIP; }

#define QVG_TRY(expr)                                  \
    do {                                               \
        qvg_status st_ = hip_status(expr);             \
        if (st_ != QVG_OK) return st_;                 \
    } while (0)

// ---- per-kernel timing with HIP events (qvg_profile_*) ----------------------

// While enabled, every kernel launch records two events at its own start and
// end (see LaunchEvents), kept with the launch's algorithmic FLOPs and HBM bytes.
struct ProfRecord {
    const char *name;
    hipEvent_t a, b;
    double flops, bytes;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// The launcher call inside a scope hands the pair of events to its kernel
// launch, which records them at the kernel's own start and end.
struct ProfScope {
    ProfRecord rec{};
    bool on = false;
    ProfScope(const char *name, double flops, double bytes) {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (!g_prof_on) return;
        rec.name = name;
        rec.a = prof_event();
        rec.b = prof_event();
        rec.flops = flops;
        rec.bytes = bytes;
        if (!rec.a || !rec.b) return;
        launch_events() = LaunchEvents{rec.a, rec.b};
        on = true;
    }
    ~ProfScope() {
        if (!on) return;
        LaunchEvents &le = launch_events();
        const bool launched = le.start == nullptr;   // the launch took the events
        le = LaunchEvents{};
        std::lock_guard<std::mutex> lk(g_prof_mu);
        if (launched) {
            g_prof.push_back(rec);
        } else {
            g_prof_pool.push_back(rec.a);
            g_prof_pool.push_back(rec.b);
        }
    }
};

#define QVG_LAUNCH(name, flops, bytes, expr)                   \
    do {                                                       \
        ProfScope prof_(name, (double)(flops), (double)(bytes));    \
        QVG_TRY(expr);                                         \
    } while (0)

// Convergence-driven rounds: changed[2][H], done[H], ndone, rounds[T][H] (int32).
size_t conv_words(int H, int T) { return (size_t)3 * H + 1 + (size_t)T * H; }

// Carves one workspace into the buffers of the encode stage loop.  The
// residuals R(t) are never stored: each kernel rebuilds them from the input
// and the earlier stages' stored centroids and assignments.
struct EncodeWorkspace {
    size_t C = 0, Cb = 0, cnt = 0, fill = 0, offsets = 0, order = 0, idx = 0, vstats = 0, tstats = 0, r1 = 0,
           conv = 0, mirror = 0, qmax = 0, total = 0;

    EncodeWorkspace(const qvg_config &c, int H, int N) {
        const size_t D = c.d, K = c.n_centroids, Kp = padded_k(c.n_centroids);
        const int T = c.n_stages;
        size_t off = 0;
        auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes, 256); return o; };
        qmax = take((size_t)H * 4);   // the quantiser's per-head maxima (two-level scales)
        if (T == 0) {
            total = off;
            return;
        }
        C = take((size_t)H * K * D * 4);
        Cb = take((size_t)H * Kp * D * 2);
        cnt = take((size_t)2 * H * Kp * 4);
        fill = take((size_t)2 * H * Kp * 4);
        offsets = take((size_t)H * Kp * 4);
        order = take((size_t)H * N * 4);
        idx = take((size_t)T * H * K * 4);
        vstats = take(value_stats_words(H) * 4);
        tstats = take((size_t)T * H * TSTAT_BLOCKS * 2 * 4);
        if (c.dtype == QVG_BF16 && T >= 2) r1 = take((size_t)H * N * D * 2);   // bf16(R(t)), the next stage's operand
        conv = take(conv_words(H, T) * 4);
        // FP8 tables: their values in the tensor dtype, which later residuals read
        if (c.centroid_format == QVG_CENT_E4M3) mirror = take((size_t)T * H * K * D * dtype_size(c.dtype));
        total = off;
    }
};

// Workspace of the stage-level k-means entry points.
struct StageWorkspace {
    size_t C = 0, Cb = 0, cnt = 0, fill = 0, offsets = 0, order = 0, vstats = 0, total = 0;
    StageWorkspace(int H, int N, int D, int K) {
        const size_t Kp = padded_k(K);
        size_t off = 0;
        auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes, 256); return o; };
        C = take((size_t)H * K * D * 4);
        Cb = take((size_t)H * Kp * D * 2);
        cnt = take((size_t)H * Kp * 4);
        fill = take((size_t)H * Kp * 4);
        offsets = take((size_t)H * Kp * 4);
        order = take((size_t)H * N * 4);
        vstats = take(value_stats_words(H) * 4);
        total = off;
    }
};

Src plain_src(const void *x, int64_t x_hs) {
    Src s{};
    s.x = x;
    s.x_hs = x_hs;
    s.P = 0;
    return s;
}

template <typename T>
T *at(void *base, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(base) + off); }

}  // namespace

extern "C" {

const char *qvg_status_string(qvg_status s) {
    switch (s) {
        case QVG_OK: return "QVG_OK";
        case QVG_ERR_INVALID_ARG: return "QVG_ERR_INVALID_ARG";
        case QVG_ERR_UNSUPPORTED: return "QVG_ERR_UNSUPPORTED";
        case QVG_ERR_WORKSPACE: return "QVG_ERR_WORKSPACE";
        case QVG_ERR_STATE: return "QVG_ERR_STATE";
        case QVG_ERR_HIP: return "QVG_ERR_HIP";
        case QVG_ERR_OOM: return "QVG_ERR_OOM";
        default: return "QVG_ERR_UNKNOWN";
    }
}

qvg_status qvg_config_validate(const qvg_config *cfg) { return check_config(cfg); }

qvg_status qvg_chunk_bytes(const qvg_config *cfg, int32_t heads, int32_t n_tokens, uint64_t out[4]) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_tokens < 1 || !out) return QVG_ERR_INVALID_ARG;
    const uint64_t H = heads, N = n_tokens, D = cfg->d;
    out[0] = H * N * D / 4;
    out[1] = H * N * D / cfg->group_size;
    out[2] = (uint64_t)cfg->n_stages * H * N;
    out[3] = (uint64_t)cfg->n_stages * H * table_bytes(*cfg);
    return QVG_OK;
}

qvg_status qvg_cache_view_bytes(const qvg_config *cfg, int32_t heads, int64_t cap_tokens, int32_t chunk_tokens,
                                uint64_t out[4]) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || cap_tokens < 1 || chunk_tokens < 1 || !out) return QVG_ERR_INVALID_ARG;
    const uint64_t H = heads, N = cap_tokens, D = cfg->d;
    const uint64_t chunks = (cap_tokens + chunk_tokens - 1) / chunk_tokens;
    out[0] = H * N * D / 4;
    out[1] = H * N * D / cfg->group_size;
    out[2] = (uint64_t)cfg->n_stages * H * N;
    out[3] = chunks * cfg->n_stages * H * table_bytes(*cfg);
    return QVG_OK;
}

qvg_status qvg_encode_workspace_bytes(const qvg_config *cfg, int32_t heads, int32_t n_tokens, uint64_t *bytes) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_tokens < 1 || !bytes) return QVG_ERR_INVALID_ARG;
    *bytes = EncodeWorkspace(*cfg, heads, n_tokens).total;
    return QVG_OK;
}

qvg_status qvg_stage_workspace_bytes(int32_t heads, int32_t n_tokens, int32_t d, int32_t n_centroids,
                                     uint64_t *bytes) {
    if (heads < 1 || n_tokens < 1 || n_centroids < 1 || n_centroids > QVG_MAX_CENTROIDS || !bytes)
        return QVG_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return QVG_ERR_UNSUPPORTED;
    *bytes = StageWorkspace(heads, n_tokens, d, n_centroids).total;
    return QVG_OK;
}

qvg_status qvg_centroid_cache_create(const qvg_config *cfg, int32_t heads, qvg_centroid_cache **out) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || !out) return QVG_ERR_INVALID_ARG;
    *out = nullptr;
    qvg_centroid_cache *c = new (std::nothrow) qvg_centroid_cache;
    if (!c) return QVG_ERR_OOM;
    c->d = cfg->d;
    c->n_centroids = cfg->n_centroids;
    c->n_stages = cfg->n_stages;
    c->heads = heads;
    c->data = nullptr;
    c->valid = 0;
    const size_t bytes = (size_t)cfg->n_stages * heads * cfg->n_centroids * cfg->d * sizeof(float);
    if (bytes && hipMalloc((void **)&c->data, bytes) != hipSuccess) {
        delete c;
        return QVG_ERR_OOM;
    }
    *out = c;
    return QVG_OK;
}

qvg_status qvg_centroid_cache_reset(qvg_centroid_cache *cache) {
    if (!cache) return QVG_ERR_INVALID_ARG;
    cache->valid = 0;
    return QVG_OK;
}

qvg_status qvg_centroid_cache_destroy(qvg_centroid_cache *cache) {
    if (!cache) return QVG_OK;
    qvg_status st = QVG_OK;
    if (cache->data && hipFree(cache->data) != hipSuccess) st = QVG_ERR_HIP;
    delete cache;
    return st;
}

qvg_status qvg_centroid_cache_data(qvg_centroid_cache *cache, float **centroids, int32_t *valid) {
    if (!cache || !centroids || !valid) return QVG_ERR_INVALID_ARG;
    *centroids = cache->data;
    *valid = cache->valid;
    return QVG_OK;
}

static size_t cache_bytes(const qvg_centroid_cache *c) {
    return (size_t)c->n_stages * c->heads * c->n_centroids * c->d * sizeof(float);
}

qvg_status qvg_centroid_cache_export(qvg_centroid_cache *cache, float *dst, void *stream) {
    if (!cache || !dst) return QVG_ERR_INVALID_ARG;
    if (!cache->valid) return QVG_ERR_STATE;
    const size_t bytes = cache_bytes(cache);
    if (bytes)
        QVG_TRY(hipMemcpyAsync(dst, cache->data, bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
    return QVG_OK;
}

qvg_status qvg_centroid_cache_import(qvg_centroid_cache *cache, const float *src, void *stream) {
    if (!cache || !src) return QVG_ERR_INVALID_ARG;
    const size_t bytes = cache_bytes(cache);
    if (bytes)
        QVG_TRY(hipMemcpyAsync(cache->data, src, bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
    cache->valid = 1;
    return QVG_OK;
}

static qvg_status encode_impl(const qvg_config *cfg, const void *x, int64_t x_head_stride, int32_t heads,
                              int32_t n_tokens, const float *init_centroids, qvg_centroid_cache *cache,
                              const qvg_cache_view *dst, int32_t chunk_index, void *workspace,
                              uint64_t workspace_bytes, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    const int H = heads, N = n_tokens, D = cfg->d, K = cfg->n_centroids, T = cfg->n_stages, G = cfg->group_size;
    const int Kp = padded_k(K);
    const size_t esz = dtype_size(cfg->dtype);
    if (H < 1 || N < 1 || !x || !aligned16(x)) return QVG_ERR_INVALID_ARG;
    if (x_head_stride < (int64_t)N * D || (x_head_stride * (int64_t)esz) % 16 != 0) return QVG_ERR_INVALID_ARG;
    if (!dst || dst->heads != H || dst->chunk_tokens < 1 || dst->cap_tokens < 1) return QVG_ERR_INVALID_ARG;
    if (chunk_index < 0 || N > dst->chunk_tokens) return QVG_ERR_INVALID_ARG;
    const int64_t tok0 = (int64_t)chunk_index * dst->chunk_tokens;
    if (tok0 + N > dst->cap_tokens) return QVG_ERR_INVALID_ARG;
    if (!dst->codes || !dst->scales || !aligned16(dst->codes)) return QVG_ERR_INVALID_ARG;
    const bool two = cfg->scale_mode == QVG_SCALE_TWO_LEVEL;
    if (two && !dst->scale_exp) return QVG_ERR_INVALID_ARG;
    if (T > 0 && (!dst->assign || !dst->centroids || !aligned16(dst->centroids))) return QVG_ERR_INVALID_ARG;
    if (init_centroids && !aligned16(init_centroids)) return QVG_ERR_INVALID_ARG;
    if (cache && (cache->heads != H || cache->d != D || cache->n_centroids != K || cache->n_stages != T))
        return QVG_ERR_STATE;
    const EncodeWorkspace ws(*cfg, H, N);
    if (!workspace || !aligned16(workspace)) return QVG_ERR_INVALID_ARG;
    if (workspace_bytes < ws.total) return QVG_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t cap = dst->cap_tokens;
    const double HND = (double)H * N * D;

    const Src src0 = plain_src(x, x_head_stride);
    // two-level scales: a first quantiser launch gathers each head's max|r|
    uint32_t *qmax = at<uint32_t>(workspace, ws.qmax);
    int8_t *sexp = two ? dst->scale_exp + (size_t)chunk_index * H : nullptr;
    auto quant = [&](const Src &qs, const void *cent, int cent_rows, const uint8_t *pi, double flops,
                     double bytes) -> qvg_status {
        if (two) {
            QVG_LAUNCH("zero", 0, H * 4.0, launch_zero(reinterpret_cast<int32_t *>(qmax), H, s));
            QVG_LAUNCH("quant_max", 0, bytes, launch_quant(D, cfg->dtype, H, N, qs, cent, cent_rows, pi, cap,
                                                           nullptr, nullptr, cap, G, qmax, nullptr, nullptr, s));
        }
        QVG_LAUNCH(T == 0 ? "group_quant" : "residual_quant", flops, bytes,
                   launch_quant(D, cfg->dtype, H, N, qs, cent, cent_rows, pi, cap, dst->codes + tok0 * (D / 4),
                                dst->scales + tok0 * (D / G), cap, G, nullptr, two ? qmax : nullptr, sexp, s));
        return QVG_OK;
    };
    if (T == 0) {
        st = quant(src0, nullptr, 0, nullptr, 0, HND * esz + HND / 4 + HND / G);
        if (st != QVG_OK) return st;
        if (cache) cache->valid = 1;
        return QVG_OK;
    }

    float *C = at<float>(workspace, ws.C);
    uint16_t *Cb = at<uint16_t>(workspace, ws.Cb);
    int32_t *cnt[2] = {at<int32_t>(workspace, ws.cnt), at<int32_t>(workspace, ws.cnt) + (size_t)H * Kp};
    int32_t *fill[2] = {at<int32_t>(workspace, ws.fill), at<int32_t>(workspace, ws.fill) + (size_t)H * Kp};
    int32_t *offsets = at<int32_t>(workspace, ws.offsets);
    int32_t *order = at<int32_t>(workspace, ws.order);
    int32_t *idx = at<int32_t>(workspace, ws.idx);
    uint32_t *vstats = at<uint32_t>(workspace, ws.vstats);
    uint32_t *tstats = at<uint32_t>(workspace, ws.tstats);   // [T][H][TSTAT_BLOCKS] stored-table magnitudes
    // bf16 tensors: the final assign of stage t < T leaves bf16(R(t)) [H][N][D],
    // which the assigns of stage t + 1 read in place of x less the earlier
    // stages' rows (one buffer, rewritten in place by each stage's final assign)
    uint16_t *r1 = cfg->dtype == QVG_BF16 && T >= 2 ? at<uint16_t>(workspace, ws.r1) : nullptr;
    Src r1src = plain_src(r1, (int64_t)N * D);
    const bool warm_cache = cache && cache->valid;
    const bool need_draw = !init_centroids && !warm_cache;
    // convergence-driven rounds (cfg->converge >= 1): per-head state in the workspace
    int32_t *conv = at<int32_t>(workspace, ws.conv);
    int32_t *chg[2] = {conv, conv + H};
    int32_t *done = conv + 2 * H, *ndone = conv + 3 * H, *rounds = conv + 3 * H + 1;
    const bool cvg = cfg->converge > 0;
    const bool fp8 = cfg->centroid_format == QVG_CENT_E4M3;
    if (need_draw) QVG_LAUNCH("forgy", 0, (double)T * H * K * 4, launch_forgy(T, H, N, K, cfg->seed, idx, s));

    // the exactness certificate of the update needs the input's value statistics:
    // the first assign gathers them for bf16 tensors, a pass of their own otherwise
    const bool seg = update_seg_fits(N);
    const bool stats_in_assign = seg && cfg->dtype == QVG_BF16;
    if (seg && !stats_in_assign)
        QVG_LAUNCH("value_stats", 0, HND * esz, launch_value_stats(cfg->dtype, H, x, x_head_stride, (int64_t)N * D,
                                                                   vstats, s));

    // R(t-1) is rebuilt from x and the stored centroids / assignments of stages 1..t-1
    Src src = src0;
    src.pi_hs = cap;
    src.K = K;
    src.tstats = tstats;
    const double table = (double)H * Kp * D * 2;
    for (int t = 1; t <= T; ++t) {
        uint8_t *pi = dst->assign + (size_t)(t - 1) * H * cap + tok0;
        const size_t slice = (size_t)(t - 1) * H * K * D;
        const float *warm = init_centroids ? init_centroids + slice : (warm_cache ? cache->data + slice : nullptr);
        const int iters = warm ? cfg->iters_warm : cfg->iters_cold;
        // algorithmic traffic: the input row plus one assignment byte per earlier stage
        const double row_bytes = HND * esz + (double)H * N * (t - 1);
        const double assign_flops = 2.0 * H * N * K * D;
        const bool use_r1 = r1 && t >= 2;
        const Src &asrc = use_r1 ? r1src : src;   // what the assigns read
        const double assign_bytes = (use_r1 ? HND * 2 : row_bytes) + H * N + table;
        QVG_LAUNCH("init_centroids", 0, (double)H * K * D * (esz + 4) + table,
                   launch_init_centroids(D, cfg->dtype, H, K, src, idx + (size_t)(t - 1) * H * K, warm, C, Cb,
                                         cnt[0], fill[0], t == 1 && stats_in_assign ? vstats : nullptr, s));
        if (cvg) {   // every head active, no changes counted yet, the round budget as the default count
            QVG_LAUNCH("zero", 0, (3.0 * H + 1) * 4, launch_zero(conv, 3 * (int64_t)H + 1, s));
            QVG_LAUNCH("fill", 0, H * 4.0, launch_fill(rounds + (size_t)(t - 1) * H, H, iters, s));
        }
        for (int it = 0; it < iters; ++it) {
            const int c = it & 1;
            ConvState cv;
            if (cvg) {
                cv.changed = chg[c];
                cv.changed_next = chg[c ^ 1];
                cv.done = done;
                cv.rounds = rounds + (size_t)(t - 1) * H;
                cv.ndone = ndone;
                cv.threshold = cfg->converge;
                cv.round = it;
            }
            QVG_LAUNCH("assign", assign_flops, assign_bytes,
                       launch_assign(D, cfg->dtype, H, N, K, asrc, Cb, pi, cap, cnt[c],
                                     t == 1 && it == 0 && stats_in_assign ? vstats : nullptr, nullptr, nullptr,
                                     cvg ? done : nullptr, cvg ? ndone : nullptr,
                                     cvg && it > 0 ? chg[c] : nullptr, s));
            if (seg) {
                QVG_LAUNCH("update", HND, row_bytes + H * N + (double)H * K * D * 4 + table,
                           launch_update_seg(D, cfg->dtype, H, N, K, src, pi, cap, cnt[c], vstats, C, Cb,
                                             cnt[c ^ 1], fill[c ^ 1], cv, s));
            } else {
                QVG_LAUNCH("scatter", 0, H * N * 5.0 + H * Kp * 8.0,
                           launch_scatter(H, N, Kp, pi, cap, cnt[c], fill[c], offsets, order, cvg ? done : nullptr,
                                          s));
                QVG_LAUNCH("update", HND, row_bytes + H * N * 4.0 + (double)H * K * D * 4 + table,
                           launch_update(D, cfg->dtype, H, N, K, src, cnt[c], offsets, order, C, Cb, cnt[c ^ 1],
                                         fill[c ^ 1], cv, s));
            }
        }
        // the stage's centroids as stored; with FP8 tables the store also puts
        // their values into the operand table, so the final assignment below is
        // nearest under the stored centroids in every format
        const size_t tbytes = table_bytes(*cfg);
        void *cslot = static_cast<char *>(dst->centroids) + ((size_t)chunk_index * T + (t - 1)) * H * tbytes;
        void *mslot = fp8 ? static_cast<void *>(at<char>(workspace, ws.mirror) + (size_t)(t - 1) * H * K * D * esz)
                          : nullptr;
        if (fp8) {
            QVG_LAUNCH("store_centroids", 0, (double)H * K * D * (4 + 1 + esz + 2 + (cache ? 4 : 0)),
                       launch_store_e4m3(D, cfg->dtype, H, K, C, static_cast<uint8_t *>(cslot), (int64_t)tbytes, mslot,
                                         Cb, cache ? cache->data + slice : nullptr,
                                         tstats + (size_t)(t - 1) * H * TSTAT_BLOCKS * 2, s));
        } else {
            QVG_LAUNCH("store_centroids", 0, (double)H * K * D * (4 + esz + (cache ? 4 : 0)),
                       launch_store_centroids(D, H, K, C, cfg->dtype, cslot, cache ? cache->data + slice : nullptr,
                                              tstats + (size_t)(t - 1) * H * TSTAT_BLOCKS * 2, s));
        }
        // the next stage's operand: from the input itself at t = 1, else from
        // R(t-1) rebuilt in fp32 out of x and the earlier stages' stored rows
        uint16_t *rout = r1 && t < T ? r1 : nullptr;
        QVG_LAUNCH("assign", assign_flops, assign_bytes + (rout ? HND * 2 : 0.0) + (rout && t > 1 ? row_bytes : 0.0),
                   launch_assign(D, cfg->dtype, H, N, K, asrc, Cb, pi, cap, nullptr, nullptr, rout,
                                 rout && t > 1 ? &src : nullptr, nullptr, nullptr, nullptr, s));
        if (t < T) {
            src.cent[t - 1] = fp8 ? mslot : cslot;
            src.pi[t - 1] = pi;
            src.P = t;
        } else {
            // the residual uses the stored centroids: the bf16 operand table for bf16
            // tensors (identical values), the fp32 table otherwise
            const void *cent = fp8 ? mslot : cfg->dtype == QVG_BF16 ? (const void *)Cb : (const void *)C;
            const int cent_rows = !fp8 && cfg->dtype == QVG_BF16 ? Kp : K;
            st = quant(src, cent, cent_rows, pi, HND * T,
                       row_bytes + H * N + (double)H * K * D * esz + HND / 4 + HND / G);
            if (st != QVG_OK) return st;
        }
    }
    if (cache) cache->valid = 1;
    return QVG_OK;
}

qvg_status qvg_encode_chunk(const qvg_config *cfg, const void *x, int64_t x_head_stride, int32_t heads,
                            int32_t n_tokens, const float *init_centroids, qvg_centroid_cache *cache,
                            const qvg_cache_view *dst, int32_t chunk_index, void *workspace,
                            uint64_t workspace_bytes, void *stream) {
    return encode_impl(cfg, x, x_head_stride, heads, n_tokens, init_centroids, cache, dst, chunk_index, workspace,
                       workspace_bytes, stream);
}

qvg_status qvg_encode_rounds(const qvg_config *cfg, int32_t heads, int32_t n_tokens, const void *workspace,
                             uint64_t workspace_bytes, int32_t *rounds_out, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_tokens < 1 || !workspace || !rounds_out) return QVG_ERR_INVALID_ARG;
    if (cfg->converge == 0 || cfg->n_stages == 0) return QVG_ERR_STATE;
    const EncodeWorkspace ws(*cfg, heads, n_tokens);
    if (workspace_bytes < ws.total) return QVG_ERR_WORKSPACE;
    const int32_t *rounds = at<int32_t>(const_cast<void *>(workspace), ws.conv) + 3 * (size_t)heads + 1;
    QVG_TRY(hipMemcpyAsync(rounds_out, rounds, (size_t)cfg->n_stages * heads * 4, hipMemcpyDeviceToDevice,
                           static_cast<hipStream_t>(stream)));
    return QVG_OK;
}

qvg_status qvg_encode_chunk_static(const qvg_config *cfg, const void *x, int64_t x_head_stride, int32_t heads,
                                   int32_t n_tokens, const float *init_centroids, qvg_centroid_cache *cache,
                                   const qvg_cache_view *dst, int32_t chunk_index, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_tokens < 1) return QVG_ERR_INVALID_ARG;
    if (EncodeWorkspace(*cfg, heads, n_tokens).total > STATIC_SCRATCH_BYTES) return QVG_ERR_WORKSPACE;
    void *ws = nullptr;
    QVG_TRY(static_scratch(&ws));
    return encode_impl(cfg, x, x_head_stride, heads, n_tokens, init_centroids, cache, dst, chunk_index, ws,
                       STATIC_SCRATCH_BYTES, stream);
}

static qvg_status decode_impl(const qvg_config *cfg, const qvg_cache_view *src, int64_t tok_begin,
                              int64_t tok_end, const float *rope, int32_t rope_heads, void *out,
                              int64_t out_head_stride, int32_t out_dtype, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (!src || src->heads < 1 || src->chunk_tokens < 1 || src->cap_tokens < 1) return QVG_ERR_INVALID_ARG;
    if (tok_begin < 0 || tok_end <= tok_begin || tok_end > src->cap_tokens) return QVG_ERR_INVALID_ARG;
    if (!src->codes || !src->scales || !aligned16(src->codes)) return QVG_ERR_INVALID_ARG;
    if (cfg->n_stages > 0 && (!src->assign || !src->centroids || !aligned16(src->centroids)))
        return QVG_ERR_INVALID_ARG;
    if (out_dtype != QVG_F32 && out_dtype != QVG_BF16) return QVG_ERR_INVALID_ARG;
    const int64_t ntok = tok_end - tok_begin;
    if (!out || !aligned16(out) || out_head_stride < ntok * cfg->d ||
        (out_head_stride * (int64_t)dtype_size(out_dtype)) % 16 != 0)
        return QVG_ERR_INVALID_ARG;
    if (ntok * (cfg->d / 16) / 256 + 1 > (int64_t)UINT32_MAX / src->heads) return QVG_ERR_UNSUPPORTED;
    DecodeArgs a;
    a.codes = src->codes;
    a.scales = src->scales;
    a.assign = src->assign;
    a.cent = src->centroids;
    a.cent_dtype = cfg->centroid_format == QVG_CENT_E4M3 ? DT_E4M3 : cfg->dtype;
    a.cap = src->cap_tokens;
    a.chunk_tokens = src->chunk_tokens;
    a.H = src->heads;
    a.K = cfg->n_centroids;
    a.T = cfg->n_stages;
    a.G = cfg->group_size;
    a.D = cfg->d;
    a.tok_begin = tok_begin;
    a.ntok = ntok;
    a.out = out;
    a.out_dtype = out_dtype;
    a.out_hs = out_head_stride;
    a.rope = rope;
    a.rope_heads = rope ? rope_heads : 0;
    if (cfg->scale_mode == QVG_SCALE_TWO_LEVEL) {
        if (!src->scale_exp) return QVG_ERR_INVALID_ARG;
        a.scale_exp = src->scale_exp;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t chunks = (tok_end - 1) / a.chunk_tokens - tok_begin / a.chunk_tokens + 1;
    double bytes = (double)a.H * ntok * (a.D / 4 + a.D / a.G + a.T + a.D * dtype_size(out_dtype)) +
                   (double)chunks * a.T * a.H * table_bytes(*cfg);
    double flops = (double)a.H * ntok * a.D * (a.T + 1);
    if (rope && rope_heads > 0) {
        bytes += (double)ntok * a.D * 4;             // the rotation table, read once
        flops += (double)rope_heads * ntok * a.D * 3;  // two products and one sum per output
        QVG_LAUNCH("decode_rope", flops, bytes, launch_decode(a, s));
    } else {
        QVG_LAUNCH("decode", flops, bytes, launch_decode(a, s));
    }
    return QVG_OK;
}

qvg_status qvg_decode(const qvg_config *cfg, const qvg_cache_view *src, int64_t tok_begin, int64_t tok_end,
                      void *out, int64_t out_head_stride, int32_t out_dtype, void *stream) {
    return decode_impl(cfg, src, tok_begin, tok_end, nullptr, 0, out, out_head_stride, out_dtype, stream);
}

qvg_status qvg_decode_rope(const qvg_config *cfg, const qvg_cache_view *src, int64_t tok_begin, int64_t tok_end,
                           const float *rope, int32_t rope_heads, void *out, int64_t out_head_stride,
                           int32_t out_dtype, void *stream) {
    if (!rope || !aligned16(rope) || !src || rope_heads < 0 || rope_heads > src->heads) return QVG_ERR_INVALID_ARG;
    return decode_impl(cfg, src, tok_begin, tok_end, rope, rope_heads, out, out_head_stride, out_dtype, stream);
}

// Splits of the key range of an attention call.  One attention workgroup runs
// per CU (256 on the chip) and the splits of a call are of equal length, so the
// workgroups run in rounds of 256 and a last round that is only partly full
// leaves CUs idle for a whole round.  Starting from enough workgroups to fill
// the chip twice over, up to four times that many splits are considered and
// the count whose workgroups fill their rounds best is taken (the fewest on a
// tie); at least 4 tiles of 64 keys per split, at most 64 splits.
static int attention_splits(int H, int Nq, int64_t Nk) {
    constexpr int64_t CUS = 256;
    const int64_t qblocks = (Nq + 255) / 256, w = qblocks * H;
    const int64_t most = std::max<int64_t>(1, std::min<int64_t>(64, Nk / 256));
    const int64_t sp0 = std::min<int64_t>(most, (2 * CUS + w - 1) / w);
    int64_t best = sp0;
    double best_fill = 0.0;
    for (int64_t sp = sp0; sp <= std::min<int64_t>(most, 4 * sp0); ++sp) {
        const int64_t wg = w * sp, rounds = (wg + CUS - 1) / CUS;
        const double fill = (double)wg / (double)(rounds * CUS);
        if (fill > best_fill + 1e-9) {
            best_fill = fill;
            best = sp;
        }
    }
    return (int)best;
}

qvg_status qvg_attention_workspace_bytes(const qvg_config *cfg, int32_t heads, int32_t n_queries, int64_t n_keys,
                                         uint64_t *bytes) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_queries < 1 || n_keys < 1 || !bytes) return QVG_ERR_INVALID_ARG;
    const int sp = attention_splits(heads, n_queries, n_keys);
    *bytes = round_up((size_t)sp * heads * n_queries * cfg->d * 4, 256) + (size_t)sp * heads * n_queries * 2 * 4;
    return QVG_OK;
}

static bool view_ok(const qvg_cache_view *v, int64_t tok_end) {
    return v && v->heads >= 1 && v->chunk_tokens >= 1 && tok_end <= v->cap_tokens && v->codes && v->scales &&
           v->assign && v->centroids && aligned16(v->codes) && aligned16(v->centroids);
}

qvg_status qvg_attention(const qvg_config *cfg, const qvg_cache_view *k_src, int32_t k_head0,
                         const qvg_cache_view *v_src, int32_t v_head0, int64_t tok_begin, int64_t tok_end,
                         const float *rope, const void *q, int64_t q_head_stride, int32_t heads, int32_t n_queries,
                         float scale, float *out, int64_t out_head_stride, float *lse, void *workspace,
                         uint64_t workspace_bytes, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (cfg->d != 128 || cfg->dtype != QVG_BF16 || cfg->n_stages < 1 || cfg->n_stages > 4) return QVG_ERR_UNSUPPORTED;
    if (heads < 1 || n_queries < 1 || tok_begin < 0 || tok_end <= tok_begin) return QVG_ERR_INVALID_ARG;
    if (!view_ok(k_src, tok_end) || !view_ok(v_src, tok_end)) return QVG_ERR_INVALID_ARG;
    if (k_head0 < 0 || v_head0 < 0 || k_head0 + heads > k_src->heads || v_head0 + heads > v_src->heads)
        return QVG_ERR_INVALID_ARG;
    if (!q || !aligned16(q) || q_head_stride < (int64_t)n_queries * cfg->d || (q_head_stride * 2) % 16 != 0)
        return QVG_ERR_INVALID_ARG;
    if (!out || out_head_stride < (int64_t)n_queries * cfg->d) return QVG_ERR_INVALID_ARG;
    if (rope && !aligned16(rope)) return QVG_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !(scale < 1e30f)) return QVG_ERR_INVALID_ARG;
    const int64_t nk = tok_end - tok_begin;
    uint64_t need = 0;
    st = qvg_attention_workspace_bytes(cfg, heads, n_queries, nk, &need);
    if (st != QVG_OK) return st;
    if (!workspace || !aligned16(workspace)) return QVG_ERR_INVALID_ARG;
    if (workspace_bytes < need) return QVG_ERR_WORKSPACE;
    if ((int64_t)(n_queries + 255) / 256 >= 65536 || heads >= 65536) return QVG_ERR_UNSUPPORTED;
    AttnArgs a{};
    auto src_of = [&](const qvg_cache_view *v) {
        AttnSrc r{};
        r.codes = v->codes;
        r.scales = v->scales;
        r.assign = v->assign;
        r.cent = v->centroids;
        r.cap = v->cap_tokens;
        r.chunk_tokens = v->chunk_tokens;
        r.heads = v->heads;
        r.K = cfg->n_centroids;
        r.G = cfg->group_size;
        r.scale_exp = cfg->scale_mode == QVG_SCALE_TWO_LEVEL ? v->scale_exp : nullptr;
        return r;
    };
    if (cfg->scale_mode == QVG_SCALE_TWO_LEVEL && (!k_src->scale_exp || !v_src->scale_exp)) return QVG_ERR_INVALID_ARG;
    a.k = src_of(k_src);
    a.v = src_of(v_src);
    a.khead0 = k_head0;
    a.vhead0 = v_head0;
    a.T = cfg->n_stages;
    a.fp8 = cfg->centroid_format == QVG_CENT_E4M3;
    a.splits = attention_splits(heads, n_queries, nk);
    a.tok_begin = tok_begin;
    a.tok_end = tok_end;
    a.keys_per_split = (nk + a.splits - 1) / a.splits;
    a.splits = (int)((nk + a.keys_per_split - 1) / a.keys_per_split);   // no empty split
    a.rope = rope;
    a.q = static_cast<const uint16_t *>(q);
    a.q_hs = q_head_stride;
    a.H = heads;
    a.Nq = n_queries;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_o = static_cast<float *>(workspace);
    a.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                          round_up((size_t)a.splits * heads * n_queries * cfg->d * 4, 256));
    const double flops = 4.0 * heads * n_queries * nk * cfg->d;
    const double bytes = (double)heads * nk * 2 * (cfg->d / 4 + cfg->d / cfg->group_size + cfg->n_stages) +
                         (double)heads * n_queries * cfg->d * (2 + 4);
    QVG_LAUNCH("attention", flops, bytes, launch_attention(a, out, out_head_stride, lse, static_cast<hipStream_t>(stream)));
    return QVG_OK;
}

qvg_status qvg_kmeans_assign(const void *x, int32_t x_dtype, int64_t x_head_stride, const float *centroids,
                             int32_t heads, int32_t n_tokens, int32_t d, int32_t n_centroids, uint8_t *assign_out,
                             int64_t assign_head_stride, void *workspace, uint64_t workspace_bytes, void *stream) {
    if (heads < 1 || n_tokens < 1 || n_centroids < 1 || n_centroids > QVG_MAX_CENTROIDS) return QVG_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return QVG_ERR_UNSUPPORTED;
    if (x_dtype != QVG_F32 && x_dtype != QVG_BF16) return QVG_ERR_INVALID_ARG;
    if (!x || !aligned16(x) || !centroids || !aligned16(centroids) || !assign_out) return QVG_ERR_INVALID_ARG;
    if (x_head_stride < (int64_t)n_tokens * d || (x_head_stride * (int64_t)dtype_size(x_dtype)) % 16 != 0)
        return QVG_ERR_INVALID_ARG;
    if (assign_head_stride < n_tokens) return QVG_ERR_INVALID_ARG;
    const StageWorkspace ws(heads, n_tokens, d, n_centroids);
    if (!workspace || !aligned16(workspace)) return QVG_ERR_INVALID_ARG;
    if (workspace_bytes < ws.total) return QVG_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Src src = plain_src(x, x_head_stride);
    float *C = at<float>(workspace, ws.C);
    uint16_t *Cb = at<uint16_t>(workspace, ws.Cb);
    const int Kp = padded_k(n_centroids);
    const double table = (double)heads * Kp * d * 2;
    QVG_LAUNCH("init_centroids", 0, (double)heads * n_centroids * d * 8 + table,
               launch_init_centroids(d, x_dtype, heads, n_centroids, src, nullptr, centroids, C, Cb, nullptr,
                                     nullptr, nullptr, s));
    QVG_LAUNCH("assign", 2.0 * heads * n_tokens * n_centroids * d,
               (double)heads * n_tokens * (d * dtype_size(x_dtype) + 1) + table,
               launch_assign(d, x_dtype, heads, n_tokens, n_centroids, src, Cb, assign_out, assign_head_stride, nullptr,
                             nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s));
    return QVG_OK;
}

qvg_status qvg_centroid_update(const void *x, int32_t x_dtype, int64_t x_head_stride, const uint8_t *assign,
                               int64_t assign_head_stride, int32_t heads, int32_t n_tokens, int32_t d,
                               int32_t n_centroids, float *centroids, int32_t *counts_out, void *workspace,
                               uint64_t workspace_bytes, void *stream) {
    if (heads < 1 || n_tokens < 1 || n_centroids < 1 || n_centroids > QVG_MAX_CENTROIDS) return QVG_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return QVG_ERR_UNSUPPORTED;
    if (x_dtype != QVG_F32 && x_dtype != QVG_BF16) return QVG_ERR_INVALID_ARG;
    if (!x || !aligned16(x) || !centroids || !aligned16(centroids) || !assign) return QVG_ERR_INVALID_ARG;
    if (x_head_stride < (int64_t)n_tokens * d || (x_head_stride * (int64_t)dtype_size(x_dtype)) % 16 != 0)
        return QVG_ERR_INVALID_ARG;
    if (assign_head_stride < n_tokens) return QVG_ERR_INVALID_ARG;
    const StageWorkspace ws(heads, n_tokens, d, n_centroids);
    if (!workspace || !aligned16(workspace)) return QVG_ERR_INVALID_ARG;
    if (workspace_bytes < ws.total) return QVG_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int Kp = padded_k(n_centroids);
    int32_t *cnt = at<int32_t>(workspace, ws.cnt);
    int32_t *fill = at<int32_t>(workspace, ws.fill);
    int32_t *offsets = at<int32_t>(workspace, ws.offsets);
    int32_t *order = at<int32_t>(workspace, ws.order);
    const double HND = (double)heads * n_tokens * d;
    QVG_LAUNCH("zero", 0, heads * Kp * 8.0, launch_zero(cnt, (int64_t)heads * Kp, s));
    QVG_LAUNCH("count", 0, (double)heads * n_tokens + heads * Kp * 4.0,
               launch_count(heads, n_tokens, Kp, assign, assign_head_stride, cnt, s));
    const double tables = (double)heads * n_centroids * d * 4 + (double)heads * Kp * d * 2;
    if (update_seg_fits(n_tokens)) {
        uint32_t *vstats = at<uint32_t>(workspace, ws.vstats);
        QVG_LAUNCH("value_stats", 0, HND * dtype_size(x_dtype),
                   launch_value_stats(x_dtype, heads, x, x_head_stride, (int64_t)n_tokens * d, vstats, s));
        QVG_LAUNCH("update", HND, HND * dtype_size(x_dtype) + (double)heads * n_tokens + tables,
                   launch_update_seg(d, x_dtype, heads, n_tokens, n_centroids, plain_src(x, x_head_stride), assign,
                                     assign_head_stride, cnt, vstats, centroids, at<uint16_t>(workspace, ws.Cb),
                                     nullptr, nullptr, ConvState{}, s));
    } else {
        QVG_LAUNCH("zero", 0, heads * Kp * 8.0, launch_zero(fill, (int64_t)heads * Kp, s));
        QVG_LAUNCH("scatter", 0, heads * n_tokens * 5.0 + heads * Kp * 8.0,
                   launch_scatter(heads, n_tokens, Kp, assign, assign_head_stride, cnt, fill, offsets, order, nullptr,
                                  s));
        QVG_LAUNCH("update", HND, HND * dtype_size(x_dtype) + heads * n_tokens * 4.0 + tables,
                   launch_update(d, x_dtype, heads, n_tokens, n_centroids, plain_src(x, x_head_stride), cnt, offsets,
                                 order, centroids, at<uint16_t>(workspace, ws.Cb),
                                 nullptr, nullptr, ConvState{}, s));
    }
    if (counts_out)
        QVG_TRY(hipMemcpy2DAsync(counts_out, (size_t)n_centroids * 4, cnt, (size_t)Kp * 4, (size_t)n_centroids * 4,
                                 heads, hipMemcpyDeviceToDevice, s));
    return QVG_OK;
}

qvg_status qvg_group_quant(const float *r, int64_t r_head_stride, int32_t heads, int32_t n_tokens, int32_t d,
                           int32_t group_size, uint8_t *codes, uint8_t *scales, void *stream) {
    if (heads < 1 || n_tokens < 1 || group_size < 1) return QVG_ERR_INVALID_ARG;
    if (d % group_size != 0) return QVG_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return QVG_ERR_UNSUPPORTED;
    if (group_size != 16 && group_size != 32 && group_size != 64 && group_size != 128) return QVG_ERR_UNSUPPORTED;
    if (!r || !aligned16(r) || !codes || !aligned16(codes) || !scales) return QVG_ERR_INVALID_ARG;
    if (r_head_stride < (int64_t)n_tokens * d || (r_head_stride * 4) % 16 != 0) return QVG_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const double HND = (double)heads * n_tokens * d;
    QVG_LAUNCH("group_quant", 0, HND * 4 + HND / 4 + HND / group_size,
               launch_quant(d, QVG_F32, heads, n_tokens, plain_src(r, r_head_stride), nullptr, 0, nullptr, 0, codes,
                            scales, n_tokens, group_size, nullptr, nullptr, nullptr, s));
    return QVG_OK;
}

qvg_status qvg_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) {
        for (auto &r : g_prof) {
            g_prof_pool.push_back(r.a);
            g_prof_pool.push_back(r.b);
        }
        g_prof.clear();
    }
    g_prof_on = on != 0;
    return QVG_OK;
}

qvg_status qvg_profile_read(qvg_kernel_stat *out, int32_t max_entries, int32_t *n_entries) {
    if (!n_entries || max_entries < 0 || (max_entries > 0 && !out)) return QVG_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    std::vector<qvg_kernel_stat> acc;
    for (const auto &r : g_prof) {
        if (hipEventSynchronize(r.b) != hipSuccess) return QVG_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return QVG_ERR_HIP;
        qvg_kernel_stat *e = nullptr;
        for (auto &x : acc)
            if (strncmp(x.name, r.name, sizeof x.name) == 0) e = &x;
        if (!e) {
            acc.emplace_back();
            e = &acc.back();
            memset(e, 0, sizeof *e);
            strncpy(e->name, r.name, sizeof e->name - 1);
        }
        e->launches += 1;
        e->total_ms += ms;
        e->flops += r.flops;
        e->bytes += r.bytes;
    }
    *n_entries = (int32_t)acc.size();
    for (int32_t i = 0; i < max_entries && i < (int32_t)acc.size(); ++i) out[i] = acc[i];
    return QVG_OK;
}

qvg_status qvg_dequant_reconstruct(const qvg_config *cfg, int32_t heads, int32_t n_tokens, const uint8_t *codes,
                                   const uint8_t *scales, const uint8_t *assign, const void *centroids, void *out,
                                   int32_t out_dtype, void *stream) {
    qvg_status st = check_config(cfg);
    if (st != QVG_OK) return st;
    if (heads < 1 || n_tokens < 1) return QVG_ERR_INVALID_ARG;
    if (cfg->scale_mode != QVG_SCALE_E4M3) return QVG_ERR_UNSUPPORTED;
    qvg_cache_view v;
    v.codes = const_cast<uint8_t *>(codes);
    v.scales = const_cast<uint8_t *>(scales);
    v.assign = const_cast<uint8_t *>(assign);
    v.centroids = const_cast<void *>(centroids);
    v.cap_tokens = n_tokens;
    v.chunk_tokens = n_tokens;
    v.heads = heads;
    v.scale_exp = nullptr;
    return qvg_decode(cfg, &v, 0, n_tokens, out, (int64_t)n_tokens * cfg->d, out_dtype, stream);
}

}  // extern "C"
