// C ABI of the rasterizer: context, argument checks, workspace and stage ordering.
//
// Stage order per frame (flowchart of the lesson "3D Gaussian Splatting from
// scratch": project -> assign to 16x16 tiles -> depth-sort per tile ->
// alpha-composite front to back):
//   gs_preprocess    preprocess kernel
//   gs_bin_and_sort  depth-first mode: radix sort of per-Gaussian depth keys,
//                    prefix sum of tile counts in depth order (its last kernel
//                    stores the pair count into host memory), pair listing in depth
//                    order, stable radix sort on the tile id, tile ranges (+ optional
//                    64-bit keys)
//                    key64 mode: prefix sum, 64-bit key listing in Gaussian order,
//                    radix sort over tile+depth bits, ranges
//   gs_composite     one workgroup per tile, heaviest tiles (longest lists) first
//   gs_backward      tile order by reverse-walk length (depth-first mode: prefix sum
//                    of tile counts in Gaussian order), per-tile reverse walk writing
//                    per-pair gradient records,
//                    per-Gaussian sums of those records + projection chain rule
#include <hip/hip_runtime.h>

#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "gs_internal.h"

using namespace gsr;

namespace {

// pair indices are uint32 throughout
constexpr int64_t kMaxPairs = 0xffffffffll;
// pair capacity per Gaussian up to which the depth-first square-rule listing takes a thread per
// rank (5 pairs per Gaussian at 10 k: 15.6 -> 7.1 us; 16 at 1 M: 38 -> 67 us, so not there)
constexpr int64_t kPairListPerRank = 8;

struct DeviceBuffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};

struct TimedSpan {
    int stage;
    hipEvent_t begin, end;
};

// Device memory of gs_render_noalloc: every intermediate buffer of a frame is carved from
// this array.  In host code `scratch` is only a stand-in for the symbol; the device address
// of each device's copy comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t kNoAllocBytes = GS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
unsigned char *g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_status[kMaxDevices] = {};
bool g_scratch_done[kMaxDevices] = {};

// Looks up (once per device, with that device current) the device address of `scratch`.
unsigned char *scratch_address(int device, hipError_t *status) {
    if (device < 0 || device >= kMaxDevices) {
        *status = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_done[device]) {
        void *ptr = nullptr;
        g_scratch_status[device] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (g_scratch_status[device] != hipSuccess) {
            (void)hipGetLastError();
            ptr = nullptr;
        }
        g_scratch_ptr[device] = static_cast<unsigned char *>(ptr);
        g_scratch_done[device] = true;
    }
    *status = g_scratch_status[device];
    return g_scratch_ptr[device];
}

}  // namespace

struct gs_context {
    int device = 0;
    int sort_mode = GS_SORT_DEPTH_FIRST;
    int emit_keys = 1;
    int profile = 0;
    int tile_test = GS_TILE_SQUARE;            // option
    int tile_test_used = GS_TILE_SQUARE;       // the rule of the last gs_preprocess
    int binning = GS_BINNING_AUTO;             // option (depth-first mode)
    int depth_order = GS_DEPTH_ORDER_BUCKETS;  // option (depth-first mode)
    int64_t max_dups = kMaxPairs;
    int64_t max_workspace = -1;
    size_t workspace = 0;
    char err[512] = {0};

    // per-Gaussian
    DeviceBuffer splat, depth, rect, tile_count, dkey[2], dval[2], dcount, offsets, scan_scratch, dsort_scratch,
        total, ellipse;
    // per-pair
    DeviceBuffer pkey32[2], pkey64[2], pval[2], keys_out, keys_unsorted, vals_unsorted, psort_scratch, part;
    // super-tile binning: the super list (ping-pong), its sort scratch and partition table,
    // per-(segment, tile) counts, per-tile totals
    DeviceBuffer skey[2], sval[2], ssort_scratch, seg_tiles, tile_total, pcount;
    bool packed_counts = false;                // the last gs_preprocess wrote pcount
    // bucketed depth order: the bound slots, the bucketed entries and the count tables
    DeviceBuffer drange, dentries, dbscratch;
    // the rectangles in rank order, written by the bucketed depth order (square rule)
    DeviceBuffer drect;
    const uint2 *ranked_rect = nullptr;        // this frame's, or null (the listings gather by Gaussian)
    bool depth_range = false;                  // the last gs_preprocess reduced its depths into drange
    // gs_cache_covariance: Sigma [6][cov_n] of the Gaussians with these quat / log_scale planes
    DeviceBuffer cov;
    const float *cov_quat = nullptr, *cov_log_scale = nullptr;
    int64_t cov_n = -1;
    // per-tile
    DeviceBuffer ranges, tile_order, tile_weight, tile_order_bwd, tile_cut;
    // gradients
    DeviceBuffer pair_base, pair_grad, scan_total, fix_list, fix_count;
    // 2D splat rasteriser
    DeviceBuffer s2_order, s2_rec, s2_trans, s2_partial;
    int64_t s2_n = -1;
    int32_t s2_height = 0, s2_width = 0;
    const float *s2_means = nullptr, *s2_depths = nullptr;

    unsigned long long *host_total = nullptr;   // pinned, host-coherent: [0] the pair count of each frame,
                                                // [1] fault bits raised by the exact-footprint listing,
                                                // [2] 1 when the bucketed depth order met a bucket too large
    unsigned long long *host_total_dev = nullptr;   // its device address (the scan stores the count there)

    // last gs_preprocess
    int64_t n = -1;
    int32_t sh_degree = -1;
    int32_t tiles_x = 0, tiles_y = 0;
    const float *g_mean = nullptr;             // Gaussian planes of the last gs_preprocess
    // last binning
    int64_t num_dups = 0;
    const uint32_t *rank_order = nullptr;      // depth-first: rank -> Gaussian (null: rank = index)
    const uint32_t *sorted_values = nullptr;   // last binning: sorted Gaussian indices
    const uint32_t *launch_order = nullptr;    // last binning: heaviest-first tile order (or null)
    const uint64_t *sorted_keys = nullptr;
    int64_t pair_capacity = 0;                 // entries the pair buffers hold
    int64_t super_capacity = 0;                // entries the super-list buffers hold
    // bucketed depth order: launch the larger-bucket kernel (set while the last bucketed frame
    // met a bucket too large for the per-bucket kernel; a frame that meets one without it
    // redoes its order with the radix sort)
    bool run_larger = true;

    std::vector<TimedSpan> spans;
    size_t spans_used = 0;

    // gs_render_noalloc: while set, ensure() carves buffers from this arena (the device's
    // `scratch`) instead of allocating
    unsigned char *arena = nullptr;
    size_t arena_size = 0, arena_used = 0;
};

namespace {

gs_status fail(gs_context *ctx, gs_status st, const char *fmt, ...) {
    if (ctx) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(ctx->err, sizeof(ctx->err), fmt, ap);
        va_end(ap);
    }
    return st;
}

#define GS_HIP(ctx, expr)                                                                        \
    do {                                                                                         \
        hipError_t e_ = (expr);                                                                  \
        if (e_ != hipSuccess)                                                                    \
            return fail((ctx), GS_ERR_DEVICE, "%s failed: %s", #expr, hipGetErrorString(e_));    \
    } while (0)

#define GS_TRY(expr)                      \
    do {                                  \
        gs_status s_ = (expr);            \
        if (s_ != GS_OK) return s_;       \
    } while (0)

gs_status check_launch(gs_context *ctx, const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return GS_OK;
}

// Makes the context's device current for the scope of one entry point.
struct DeviceScope {
    int prev = -1;
    hipError_t status = hipSuccess;
    explicit DeviceScope(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) status = hipSetDevice(dev);
    }
    ~DeviceScope() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

gs_status ensure(gs_context *ctx, DeviceBuffer &b, size_t bytes) {
    if (bytes <= b.bytes) return GS_OK;
    if (ctx->arena) {   // gs_render_noalloc: carve, never allocate
        const size_t off = (ctx->arena_used + 255) & ~(size_t)255;
        if (off > ctx->arena_size || bytes > ctx->arena_size - off)
            return fail(ctx, GS_ERR_CAPACITY,
                        "gs_render_noalloc: the frame needs more than the %zu-byte scratch (%zu in use, %zu more)",
                        ctx->arena_size, off, bytes);
        b.ptr = ctx->arena + off;
        b.bytes = bytes;
        ctx->arena_used = off + bytes;
        return GS_OK;
    }
    size_t want = bytes + bytes / 4;                 // grow with headroom
    want = (want + 255) & ~(size_t)255;
    const size_t after = ctx->workspace - b.bytes + want;
    if (ctx->max_workspace >= 0 && after > (size_t)ctx->max_workspace) {
        if (ctx->workspace - b.bytes + bytes > (size_t)ctx->max_workspace)
            return fail(ctx, GS_ERR_OUT_OF_MEMORY, "workspace limit %lld bytes exceeded (need %zu more)",
                        (long long)ctx->max_workspace, bytes - b.bytes);
        want = bytes;
    }
    if (b.ptr) {
        GS_HIP(ctx, hipFree(b.ptr));
        ctx->workspace -= b.bytes;
        b.ptr = nullptr;
        b.bytes = 0;
    }
    hipError_t e = hipMalloc(&b.ptr, want);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        b.ptr = nullptr;
        return fail(ctx, GS_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) failed: %s", want, hipGetErrorString(e));
    }
    b.bytes = want;
    ctx->workspace += want;
    return GS_OK;
}

template <typename T>
T *as(DeviceBuffer &b) {
    return reinterpret_cast<T *>(b.ptr);
}

// Profiling: HIP events around each stage, recorded on the caller's stream.
gs_status span_begin(gs_context *ctx, int stage, hipStream_t s) {
    if (!ctx->profile) return GS_OK;
    if (ctx->spans_used == ctx->spans.size()) {
        TimedSpan t{stage, nullptr, nullptr};
        GS_HIP(ctx, hipEventCreate(&t.begin));
        GS_HIP(ctx, hipEventCreate(&t.end));
        ctx->spans.push_back(t);
    }
    TimedSpan &t = ctx->spans[ctx->spans_used];
    t.stage = stage;
    GS_HIP(ctx, hipEventRecord(t.begin, s));
    return GS_OK;
}

gs_status span_end(gs_context *ctx, hipStream_t s) {
    if (!ctx->profile) return GS_OK;
    GS_HIP(ctx, hipEventRecord(ctx->spans[ctx->spans_used].end, s));
    ++ctx->spans_used;
    return GS_OK;
}

bool finite3(const float *v, int k) {
    for (int i = 0; i < k; ++i)
        if (!std::isfinite(v[i])) return false;
    return true;
}

int ceil_log2(int64_t v) {
    int b = 0;
    while (((int64_t)1 << b) < v) ++b;
    return b;
}

// Every device buffer of the context (destroy frees them; gs_render_noalloc swaps them out).
constexpr int kContextBuffers = 52;
void context_buffers(gs_context *ctx, DeviceBuffer *out[kContextBuffers]) {
    DeviceBuffer *all[kContextBuffers] = {
        &ctx->splat, &ctx->depth, &ctx->rect, &ctx->tile_count, &ctx->dkey[0], &ctx->dkey[1], &ctx->dval[0],
        &ctx->dval[1], &ctx->dcount, &ctx->offsets, &ctx->scan_scratch, &ctx->dsort_scratch, &ctx->total,
        &ctx->ellipse, &ctx->pkey32[0], &ctx->pkey32[1], &ctx->pkey64[0], &ctx->pkey64[1], &ctx->pval[0],
        &ctx->pval[1], &ctx->keys_out, &ctx->keys_unsorted, &ctx->vals_unsorted, &ctx->psort_scratch, &ctx->part,
        &ctx->ranges, &ctx->tile_order, &ctx->tile_weight, &ctx->tile_order_bwd, &ctx->tile_cut, &ctx->pair_base,
        &ctx->pair_grad, &ctx->scan_total, &ctx->fix_list, &ctx->fix_count, &ctx->s2_order, &ctx->s2_rec,
        &ctx->s2_trans, &ctx->s2_partial, &ctx->skey[0], &ctx->skey[1], &ctx->sval[0], &ctx->sval[1],
        &ctx->ssort_scratch, &ctx->seg_tiles, &ctx->tile_total, &ctx->pcount, &ctx->drange,
        &ctx->dentries, &ctx->dbscratch, &ctx->cov, &ctx->drect};
    for (int i = 0; i < kContextBuffers; ++i) out[i] = all[i];
}

gs_status check_projected(gs_context *ctx, const gs_projected *pr) {
    if (!pr) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "projected is NULL");
    if (ctx->n < 0 || pr->n != ctx->n || pr->splat != as<float>(ctx->splat) || pr->tiles_x != ctx->tiles_x ||
        pr->tiles_y != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "projected is not the last gs_preprocess output of this context");
    return GS_OK;
}

}  // namespace

extern "C" {

const char *gs_status_string(gs_status st) {
    switch (st) {
        case GS_OK: return "ok";
        case GS_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GS_ERR_OUT_OF_MEMORY: return "out of device memory";
        case GS_ERR_CAPACITY: return "pair capacity exceeded";
        case GS_ERR_DEVICE: return "HIP device error";
    }
    return "unknown status";
}

const char *gs_last_error(const gs_context *ctx) { return ctx ? ctx->err : ""; }

gs_status gs_check_arguments(const gs_gaussians *g, const gs_camera *cam, char *msg, size_t msg_len) {
    const char *why = nullptr;
    char buf[160];
    if (g) {
        if (g->n < 0 || g->n > 0x7fffffffll) {
            snprintf(buf, sizeof buf, "gaussian count %lld outside [0, 2^31)", (long long)g->n);
            why = buf;
        } else if (g->sh_degree < 0 || g->sh_degree > 3) {
            snprintf(buf, sizeof buf, "sh_degree %d outside [0, 3]", g->sh_degree);
            why = buf;
        } else if (g->n > 0 && (!g->mean || !g->quat || !g->log_scale || !g->opacity || !g->sh)) {
            why = "a Gaussian parameter pointer is NULL";
        }
    }
    if (!why && cam) {
        if (cam->width < 1 || cam->height < 1 || cam->width > 32768 || cam->height > 32768)
            why = "image size outside [1, 32768]";
        else if (!finite3(cam->R, 9) || !finite3(cam->t, 3) || !std::isfinite(cam->fx) ||
                 !std::isfinite(cam->fy) || !std::isfinite(cam->cx) || !std::isfinite(cam->cy) ||
                 !std::isfinite(cam->znear))
            why = "camera has a non-finite value";
        else if (!(cam->fx > 0.0f) || !(cam->fy > 0.0f))
            why = "focal lengths must be > 0";
        else if (!(cam->znear > 0.0f))
            why = "znear must be > 0";
    }
    if (!why) {
        if (msg && msg_len) msg[0] = 0;
        return GS_OK;
    }
    if (msg && msg_len) snprintf(msg, msg_len, "%s", why);
    return GS_ERR_INVALID_ARGUMENT;
}

gs_status gs_context_create(gs_context **out, int device) {
    if (!out) return GS_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) {
        (void)hipGetLastError();
        return GS_ERR_DEVICE;
    }
    gs_context *ctx = new gs_context();
    ctx->device = device;
    DeviceScope scope(device);
    if (scope.status != hipSuccess ||
        hipHostMalloc((void **)&ctx->host_total, 3 * sizeof(unsigned long long),
                      hipHostMallocCoherent | hipHostMallocMapped) != hipSuccess ||
        hipHostGetDevicePointer((void **)&ctx->host_total_dev, ctx->host_total, 0) != hipSuccess) {
        (void)hipGetLastError();
        delete ctx;
        return GS_ERR_DEVICE;
    }
    ctx->host_total[1] = ctx->host_total[2] = 0;
    hipError_t scratch_status;
    (void)scratch_address(device, &scratch_status);   // once per device; gs_render_noalloc reports failure
    *out = ctx;
    return GS_OK;
}

void gs_context_destroy(gs_context *ctx) {
    if (!ctx) return;
    DeviceScope scope(ctx->device);
    DeviceBuffer *all[kContextBuffers];
    context_buffers(ctx, all);
    for (DeviceBuffer *b : all)
        if (b->ptr) (void)hipFree(b->ptr);
    for (TimedSpan &t : ctx->spans) {
        (void)hipEventDestroy(t.begin);
        (void)hipEventDestroy(t.end);
    }
    if (ctx->host_total) (void)hipHostFree(ctx->host_total);
    delete ctx;
}

gs_status gs_context_set_option(gs_context *ctx, int option, int64_t value) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    switch (option) {
        case GS_OPT_SORT_MODE:
            if (value != GS_SORT_DEPTH_FIRST && value != GS_SORT_KEY64)
                return fail(ctx, GS_ERR_INVALID_ARGUMENT, "unknown sort mode %lld", (long long)value);
            ctx->sort_mode = (int)value;
            return GS_OK;
        case GS_OPT_EMIT_KEYS:
            if (value != 0 && value != 1) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "emit_keys must be 0 or 1");
            ctx->emit_keys = (int)value;
            return GS_OK;
        case GS_OPT_MAX_DUPS:
            if (value < 0 || value > kMaxPairs)
                return fail(ctx, GS_ERR_INVALID_ARGUMENT, "max_dups outside [0, 2^32-1]");
            ctx->max_dups = value;
            return GS_OK;
        case GS_OPT_MAX_WORKSPACE_BYTES:
            ctx->max_workspace = value < 0 ? -1 : value;
            return GS_OK;
        case GS_OPT_PROFILE:
            if (value != 0 && value != 1) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "profile must be 0 or 1");
            ctx->profile = (int)value;
            return GS_OK;
        case GS_OPT_TILE_TEST:
            if (value != GS_TILE_SQUARE && value != GS_TILE_ELLIPSE)
                return fail(ctx, GS_ERR_INVALID_ARGUMENT, "unknown tile test %lld", (long long)value);
            ctx->tile_test = (int)value;
            return GS_OK;
        case GS_OPT_BINNING:
            if (value != GS_BINNING_AUTO && value != GS_BINNING_SUPER_TILE && value != GS_BINNING_RADIX)
                return fail(ctx, GS_ERR_INVALID_ARGUMENT, "unknown binning %lld", (long long)value);
            ctx->binning = (int)value;
            return GS_OK;
        case GS_OPT_DEPTH_ORDER:
            if (value != GS_DEPTH_ORDER_BUCKETS && value != GS_DEPTH_ORDER_RADIX)
                return fail(ctx, GS_ERR_INVALID_ARGUMENT, "unknown depth order %lld", (long long)value);
            ctx->depth_order = (int)value;
            return GS_OK;
    }
    return fail(ctx, GS_ERR_INVALID_ARGUMENT, "unknown option %d", option);
}

gs_status gs_preprocess(gs_context *ctx, const gs_gaussians *g, const gs_camera *cam, gs_projected *out,
                        hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!g || !cam || !out) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL gaussians, camera or output");
    char why[160];
    if (gs_check_arguments(g, cam, why, sizeof why) != GS_OK) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");

    const int64_t n = g->n;
    const size_t nn = (size_t)(n > 0 ? n : 1);
    GS_TRY(ensure(ctx, ctx->splat, nn * GS_SPLAT_STRIDE * sizeof(float)));
    GS_TRY(ensure(ctx, ctx->depth, nn * sizeof(float)));
    GS_TRY(ensure(ctx, ctx->rect, nn * sizeof(uint2)));
    GS_TRY(ensure(ctx, ctx->tile_count, nn * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->dkey[0], nn * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->dval[0], nn * sizeof(uint32_t)));

    PreprocessParams p{};
    p.n = (int32_t)n;
    p.sh_coeffs = (g->sh_degree + 1) * (g->sh_degree + 1);
    p.mean = g->mean;
    p.quat = g->quat;
    p.log_scale = g->log_scale;
    p.opacity = g->opacity;
    p.sh = g->sh;
    memcpy(p.R, cam->R, sizeof p.R);
    memcpy(p.t, cam->t, sizeof p.t);
    p.fx = cam->fx;
    p.fy = cam->fy;
    p.cx = cam->cx;
    p.cy = cam->cy;
    p.znear = cam->znear;
    for (int i = 0; i < 3; ++i)   // camera centre C = -R^T t
        p.cam_pos[i] = (float)-((double)cam->R[i] * cam->t[0] + (double)cam->R[3 + i] * cam->t[1] +
                                (double)cam->R[6 + i] * cam->t[2]);
    p.tiles_x = (cam->width + GS_TILE - 1) / GS_TILE;
    p.tiles_y = (cam->height + GS_TILE - 1) / GS_TILE;
    p.splat = as<float>(ctx->splat);
    p.depth = as<float>(ctx->depth);
    p.rect = as<uint2>(ctx->rect);
    p.tile_count = as<uint32_t>(ctx->tile_count);
    p.depth_key = as<uint32_t>(ctx->dkey[0]);
    p.depth_index = as<uint32_t>(ctx->dval[0]);
    if (ctx->tile_test == GS_TILE_ELLIPSE) {
        GS_TRY(ensure(ctx, ctx->ellipse, nn * sizeof(EllipseRec)));
        p.ellipse = as<EllipseRec>(ctx->ellipse);
    }
    // super-tile binning gathers each ranked Gaussian's tile and super-tile counts in one word
    const int64_t super_tiles = (int64_t)((p.tiles_x + kSuperSide - 1) / kSuperSide) *
                                ((p.tiles_y + kSuperSide - 1) / kSuperSide);
    const bool want = ctx->binning == GS_BINNING_SUPER_TILE || (ctx->binning == GS_BINNING_AUTO && n >= kAutoSuperMin);
    const bool pack = ctx->sort_mode == GS_SORT_DEPTH_FIRST && want &&
                      (int64_t)p.tiles_x * p.tiles_y <= kMaxSuperBinningTiles && super_tiles <= kMaxSuper;
    if (pack) {
        GS_TRY(ensure(ctx, ctx->pcount, nn * sizeof(uint32_t)));
        p.packed_count = as<uint32_t>(ctx->pcount);
    }
    // the cached covariances, when they are these Gaussians' (never inside gs_render_noalloc)
    if (!ctx->arena && n > 0 && ctx->cov_n == n && ctx->cov_quat == g->quat && ctx->cov_log_scale == g->log_scale)
        p.cov = as<float>(ctx->cov);
    // the bucketed depth order takes its bounds from the depths of this projection; the slots
    // start empty (freshly carved or allocated), afterwards the order's last kernel empties them
    const bool depth_range = ctx->sort_mode == GS_SORT_DEPTH_FIRST && ctx->depth_order == GS_DEPTH_ORDER_BUCKETS;
    if (depth_range) {
        const void *before = ctx->drange.ptr;
        GS_TRY(ensure(ctx, ctx->drange, 2 * kDepthSlots * sizeof(uint32_t)));
        if (ctx->drange.ptr != before) {
            launch_depth_range_fill(as<uint32_t>(ctx->drange), stream);
            GS_TRY(check_launch(ctx, "depth bound slots"));
        }
        p.depth_range = as<uint32_t>(ctx->drange);
    }

    GS_TRY(span_begin(ctx, GS_STAGE_PREPROCESS, stream));
    launch_preprocess(p, stream);
    GS_TRY(check_launch(ctx, "preprocess"));
    GS_TRY(span_end(ctx, stream));

    ctx->n = n;
    ctx->packed_counts = pack;
    ctx->depth_range = depth_range;
    ctx->tile_test_used = ctx->tile_test;
    ctx->sh_degree = g->sh_degree;
    ctx->g_mean = g->mean;
    ctx->num_dups = -1;
    ctx->sorted_values = nullptr;
    ctx->tiles_x = p.tiles_x;
    ctx->tiles_y = p.tiles_y;
    out->n = n;
    out->tiles_x = p.tiles_x;
    out->tiles_y = p.tiles_y;
    out->splat = p.splat;
    out->depth = p.depth;
    out->rect = reinterpret_cast<const uint16_t *>(p.rect);
    out->tile_count = p.tile_count;
    return GS_OK;
}

// Enqueues the pair listing, the tile sort and the ranges for at most `cap` pairs.  The
// kernels read the actual pair count (the scan total) from device memory, so this can be
// enqueued before the host knows it.
static gs_status enqueue_pairs(gs_context *ctx, const gs_projected *pr, const uint32_t *order, int emit_keys,
                               int64_t cap, hipStream_t stream) {
    const int64_t tiles = (int64_t)ctx->tiles_x * ctx->tiles_y;
    const bool depth_first = ctx->sort_mode == GS_SORT_DEPTH_FIRST;
    const size_t mm = (size_t)cap;
    const int tile_bits = ceil_log2(tiles);
    unsigned long long *d_total = as<unsigned long long>(ctx->total);
    GS_TRY(ensure(ctx, ctx->pval[0], mm * 4));
    GS_TRY(ensure(ctx, ctx->pval[1], mm * 4));
    GS_TRY(ensure(ctx, ctx->psort_scratch, (size_t)sort_scratch_words(cap) * 4));
    GS_TRY(ensure(ctx, ctx->part, (size_t)duplicate_partition_words(cap) * 4));
    if (depth_first) {
        GS_TRY(ensure(ctx, ctx->pkey32[0], mm * 4));
        GS_TRY(ensure(ctx, ctx->pkey32[1], mm * 4));
        if (emit_keys) GS_TRY(ensure(ctx, ctx->keys_out, mm * 8));
    } else {
        GS_TRY(ensure(ctx, ctx->pkey64[0], mm * 8));
        GS_TRY(ensure(ctx, ctx->pkey64[1], mm * 8));
        if (emit_keys) {
            GS_TRY(ensure(ctx, ctx->keys_unsorted, mm * 8));
            GS_TRY(ensure(ctx, ctx->vals_unsorted, mm * 4));
        }
    }

    ctx->sorted_values = nullptr;
    ctx->sorted_keys = nullptr;
    ctx->launch_order = nullptr;
    if (ctx->n <= 0) {   // no pairs: every tile range is empty (otherwise the partition kernel clears them)
        GS_TRY(span_begin(ctx, GS_STAGE_RANGES, stream));
        launch_fill_u32(as<uint32_t>(ctx->ranges), 0u, tiles * 2, stream);
        GS_TRY(check_launch(ctx, "fill"));
        GS_TRY(span_end(ctx, stream));
        return GS_OK;
    }

    DuplicateParams d{};
    d.n_items = ctx->n;
    d.num_dups = d_total;
    d.capacity = cap;
    d.offsets = as<uint32_t>(ctx->offsets);
    d.order = order;
    d.rect = reinterpret_cast<const uint2 *>(pr->rect);
    d.rect_ranked = order ? ctx->ranked_rect : nullptr;
    d.depth = pr->depth;
    d.tiles_x = ctx->tiles_x;
    d.values = as<uint32_t>(ctx->pval[0]);
    d.clear = as<uint32_t>(ctx->ranges);
    d.clear_words = tiles * 2;
    if (ctx->tile_test_used == GS_TILE_ELLIPSE) {
        d.ellipse = as<EllipseRec>(ctx->ellipse);
        d.tile_count = pr->tile_count;
        d.fault = ctx->host_total_dev + 1;
    }
    RangesParams r{};
    r.num_dups = d_total;
    r.capacity = cap;
    r.ranges = as<uint32_t>(ctx->ranges);
    int buf = 0;
    if (depth_first) {
        // tile ids as 16-bit keys whenever they fit: 6 instead of 8 bytes per pair per pass
        const bool narrow = tiles <= 65536;
        if (narrow)
            d.tile_keys16 = as<uint16_t>(ctx->pkey32[0]);
        else
            d.tile_keys = as<uint32_t>(ctx->pkey32[0]);
        GS_TRY(span_begin(ctx, GS_STAGE_DUPLICATE, stream));
        // a thread per rank for short lists per Gaussian; the windowed listing balances long ones
        // (and walks the row spans of the exact-footprint rule); both list the same pairs
        if (!d.ellipse && cap <= kPairListPerRank * ctx->n)
            launch_pair_list(d, stream);
        else
            launch_duplicate(d, as<uint32_t>(ctx->part), stream);
        GS_TRY(check_launch(ctx, "duplicate"));
        GS_TRY(span_end(ctx, stream));
        GS_TRY(span_begin(ctx, GS_STAGE_TILE_SORT, stream));
        if (narrow)
            buf = radix_sort_pairs<uint16_t>(as<uint16_t>(ctx->pkey32[0]), as<uint32_t>(ctx->pval[0]),
                                             as<uint16_t>(ctx->pkey32[1]), as<uint32_t>(ctx->pval[1]), cap, d_total,
                                             0, tile_bits, as<uint32_t>(ctx->psort_scratch), stream);
        else
            buf = radix_sort_pairs<uint32_t>(as<uint32_t>(ctx->pkey32[0]), as<uint32_t>(ctx->pval[0]),
                                             as<uint32_t>(ctx->pkey32[1]), as<uint32_t>(ctx->pval[1]), cap, d_total,
                                             0, tile_bits, as<uint32_t>(ctx->psort_scratch), stream);
        GS_TRY(check_launch(ctx, "tile sort"));
        GS_TRY(span_end(ctx, stream));
        if (narrow)
            r.tile_keys16 = as<uint16_t>(ctx->pkey32[buf]);
        else
            r.tile_keys = as<uint32_t>(ctx->pkey32[buf]);
        if (emit_keys) {
            r.keys_out = as<uint64_t>(ctx->keys_out);
            r.values = as<uint32_t>(ctx->pval[buf]);
            r.depth = pr->depth;
            ctx->sorted_keys = r.keys_out;
        }
    } else {
        d.keys64 = as<uint64_t>(ctx->pkey64[0]);
        GS_TRY(span_begin(ctx, GS_STAGE_DUPLICATE, stream));
        launch_duplicate(d, as<uint32_t>(ctx->part), stream);
        GS_TRY(check_launch(ctx, "duplicate"));
        GS_TRY(span_end(ctx, stream));
        if (emit_keys) {   // the listing before sorting, kept for inspection
            GS_HIP(ctx, hipMemcpyAsync(ctx->keys_unsorted.ptr, d.keys64, mm * 8, hipMemcpyDeviceToDevice, stream));
            GS_HIP(ctx, hipMemcpyAsync(ctx->vals_unsorted.ptr, d.values, mm * 4, hipMemcpyDeviceToDevice, stream));
        }
        GS_TRY(span_begin(ctx, GS_STAGE_TILE_SORT, stream));
        buf = radix_sort_pairs<uint64_t>(as<uint64_t>(ctx->pkey64[0]), as<uint32_t>(ctx->pval[0]),
                                         as<uint64_t>(ctx->pkey64[1]), as<uint32_t>(ctx->pval[1]), cap, d_total, 0,
                                         32 + tile_bits, as<uint32_t>(ctx->psort_scratch), stream);
        GS_TRY(check_launch(ctx, "key sort"));
        GS_TRY(span_end(ctx, stream));
        r.keys64 = as<uint64_t>(ctx->pkey64[buf]);
        ctx->sorted_keys = r.keys64;
    }
    GS_TRY(span_begin(ctx, GS_STAGE_RANGES, stream));
    launch_ranges(r, stream);
    GS_TRY(check_launch(ctx, "ranges"));
    TileOrderParams o{};
    o.tiles = (int32_t)tiles;
    o.ranges = r.ranges;
    o.order = as<uint32_t>(ctx->tile_order);
    ctx->launch_order = launch_tile_order(o, stream) ? o.order : nullptr;
    GS_TRY(check_launch(ctx, "tile order"));
    GS_TRY(span_end(ctx, stream));
    ctx->sorted_values = as<uint32_t>(ctx->pval[buf]);
    return GS_OK;
}

// Rank -> Gaussian by (depth, index) into *order, and ctx->dcount = gather[rank -> Gaussian]
// (n > 1; otherwise the identity).  buckets: the bucketed order, whose overflow flag (device
// memory) comes back in *flag; else the four-pass radix sort of the depth bits.
static gs_status order_by_depth(gs_context *ctx, int64_t n, const uint32_t *gather, bool buckets,
                                const uint32_t **order, const unsigned long long **flag, hipStream_t stream,
                                const uint2 *rect = nullptr, bool packed = false) {
    const size_t nn = (size_t)(n > 0 ? n : 1);
    GS_TRY(ensure(ctx, ctx->dcount, nn * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->dval[1], nn * sizeof(uint32_t)));
    GS_TRY(span_begin(ctx, GS_STAGE_DEPTH_SORT, stream));
    if (buckets) {
        GS_TRY(ensure(ctx, ctx->dentries, nn * (rect ? 16 : 8)));   // with the rectangles: 16-byte entries
        GS_TRY(ensure(ctx, ctx->dbscratch, (size_t)depth_bucket_scratch_words(n) * sizeof(uint32_t)));
        DepthBucketParams b{};
        depth_bucket_layout(as<uint32_t>(ctx->dbscratch), n, b);
        b.keys = as<uint32_t>(ctx->dkey[0]);
        b.range = as<uint32_t>(ctx->drange);
        b.entries = as<uint64_t>(ctx->dentries);
        b.gather_src = gather;
        b.order = as<uint32_t>(ctx->dval[1]);
        b.gathered = as<uint32_t>(ctx->dcount);
        b.run_larger = ctx->run_larger ? 1 : 0;
        if (rect) {   // square rule: the counts follow from the rectangles, kept in rank order too
            GS_TRY(ensure(ctx, ctx->drect, nn * sizeof(uint2)));
            b.rect = rect;
            b.rect_out = as<uint2>(ctx->drect);
            b.packed_counts = packed ? 1 : 0;
            ctx->ranked_rect = b.rect_out;
        }
        launch_depth_bucket_sort(b, stream);
        GS_TRY(check_launch(ctx, "depth buckets"));
        *order = b.order;
        if (flag) *flag = b.flag;
    } else {
        // the last radix pass also gathers each ranked Gaussian's count
        GS_TRY(ensure(ctx, ctx->dkey[1], nn * sizeof(uint32_t)));
        GS_TRY(ensure(ctx, ctx->dsort_scratch, (size_t)sort_scratch_words(n) * 4));
        const int buf = radix_sort_pairs<uint32_t>(as<uint32_t>(ctx->dkey[0]), as<uint32_t>(ctx->dval[0]),
                                                   as<uint32_t>(ctx->dkey[1]), as<uint32_t>(ctx->dval[1]), n,
                                                   nullptr, 0, 32, as<uint32_t>(ctx->dsort_scratch), stream, gather,
                                                   as<uint32_t>(ctx->dcount));
        GS_TRY(check_launch(ctx, "depth sort"));
        *order = as<uint32_t>(ctx->dval[buf]);
        if (flag) *flag = nullptr;
    }
    return span_end(ctx, stream);
}

// Exclusive prefix of the per-rank counts into ctx->offsets (the super-list offsets when
// super_bin, the count word then holding both totals); the total also goes to host_total
// (device address of host-coherent memory, with host_total[2] = *flag first) when given.
static gs_status enqueue_scan(gs_context *ctx, const uint32_t *counts, int64_t n, bool super_bin,
                              unsigned long long *host_total, const unsigned long long *flag, hipStream_t stream) {
    unsigned long long *d_total = as<unsigned long long>(ctx->total);
    GS_TRY(span_begin(ctx, GS_STAGE_SCAN, stream));
    if (super_bin)
        launch_scan_pairs(counts, as<uint32_t>(ctx->offsets), n, d_total, as<unsigned long long>(ctx->scan_scratch),
                          stream, host_total, flag);
    else
        launch_scan(counts, nullptr, as<uint32_t>(ctx->offsets), n, d_total,
                    as<unsigned long long>(ctx->scan_scratch), stream, host_total, flag);
    GS_TRY(check_launch(ctx, "scan"));
    return span_end(ctx, stream);
}

// Depth-first binning through super-tiles (GS_BINNING_SUPER_TILE) for at most `cap` pairs and
// `scap` super-list entries: the super list, its sort by super-tile, the expansion into
// per-tile lists and the launch order.  The kernels read both counts from device memory
// (total[1] pairs, total[2] super-list entries), so this too can be enqueued before the host
// knows them.
static gs_status enqueue_super_pairs(gs_context *ctx, const gs_projected *pr, const uint32_t *order, int emit_keys,
                                     int64_t cap, int64_t scap, hipStream_t stream) {
    const int64_t tiles = (int64_t)ctx->tiles_x * ctx->tiles_y;
    const int32_t super_x = (ctx->tiles_x + kSuperSide - 1) / kSuperSide;
    const int32_t super_y = (ctx->tiles_y + kSuperSide - 1) / kSuperSide;
    const size_t mm = (size_t)cap, ss = (size_t)scap;
    const int64_t segs = super_segment_capacity(scap);
    unsigned long long *d_total = as<unsigned long long>(ctx->total);
    GS_TRY(ensure(ctx, ctx->pval[0], mm * 4));
    if (emit_keys) GS_TRY(ensure(ctx, ctx->keys_out, mm * 8));
    GS_TRY(ensure(ctx, ctx->skey[0], ss * 4));
    GS_TRY(ensure(ctx, ctx->skey[1], ss * 4));
    GS_TRY(ensure(ctx, ctx->sval[0], ss * 4));
    GS_TRY(ensure(ctx, ctx->sval[1], ss * 4));
    GS_TRY(ensure(ctx, ctx->ssort_scratch, (size_t)sort_scratch_words(scap) * 4));
    GS_TRY(ensure(ctx, ctx->seg_tiles, (size_t)segs * kWave * 4));
    const int64_t row_parts = (int64_t)ctx->tiles_y * super_x;
    const int64_t rows_at = (tiles + 1) & ~(int64_t)1;   // the row parts 8-byte aligned
    // tile totals, row parts, their offsets (up to kRowStride words apart)
    GS_TRY(ensure(ctx, ctx->tile_total, (size_t)(rows_at + row_parts + row_parts * kRowStride) * 4));
    ctx->sorted_values = nullptr;
    ctx->sorted_keys = nullptr;
    ctx->launch_order = nullptr;

    DuplicateParams d{};
    d.n_items = ctx->n;
    d.num_dups = d_total + 2;
    d.capacity = scap;
    d.offsets = as<uint32_t>(ctx->offsets);
    d.order = order;
    d.rect = reinterpret_cast<const uint2 *>(pr->rect);
    d.rect_ranked = order ? ctx->ranked_rect : nullptr;
    d.tiles_x = super_x;
    d.tile_keys = as<uint32_t>(ctx->skey[0]);
    d.values = as<uint32_t>(ctx->sval[0]);
    GS_TRY(span_begin(ctx, GS_STAGE_DUPLICATE, stream));
    launch_super_list(d, stream);
    GS_TRY(check_launch(ctx, "super-tile listing"));
    GS_TRY(span_end(ctx, stream));

    GS_TRY(span_begin(ctx, GS_STAGE_TILE_SORT, stream));
    // by the super-tile id, the key's low 8 bits (the local rectangle above them travels along)
    const int sbuf = radix_sort_pairs<uint32_t>(as<uint32_t>(ctx->skey[0]), as<uint32_t>(ctx->sval[0]),
                                                as<uint32_t>(ctx->skey[1]), as<uint32_t>(ctx->sval[1]), scap,
                                                d_total + 2, 0, kRadixBits, as<uint32_t>(ctx->ssort_scratch), stream);
    GS_TRY(check_launch(ctx, "super-tile sort"));
    SuperBinParams b{};
    b.tiles_x = ctx->tiles_x;
    b.tiles_y = ctx->tiles_y;
    b.super_x = super_x;
    b.super_y = super_y;
    b.super_totals = as<uint32_t>(ctx->ssort_scratch) + sort_totals_offset(scap);
    b.keys = as<uint32_t>(ctx->skey[sbuf]);
    b.gauss = as<uint32_t>(ctx->sval[sbuf]);
    b.ellipse = ctx->tile_test_used == GS_TILE_ELLIPSE ? as<EllipseRec>(ctx->ellipse) : nullptr;
    b.seg_tiles = as<uint32_t>(ctx->seg_tiles);
    b.seg_capacity = segs;
    b.tile_total = as<uint32_t>(ctx->tile_total);
    b.rows = b.tile_total + rows_at;
    b.row_start = b.rows + row_parts;
    b.ranges = as<uint32_t>(ctx->ranges);
    b.num_dups = d_total + 1;
    b.capacity = cap;
    b.values = as<uint32_t>(ctx->pval[0]);
    if (emit_keys) {
        b.depth = pr->depth;
        b.keys_out = as<uint64_t>(ctx->keys_out);
    }
    // the heaviest-first launch order comes from the place kernel's first workgroup
    b.order = tiles <= kMaxOrderedTiles ? as<uint32_t>(ctx->tile_order) : nullptr;
    launch_super_binning(b, stream);
    GS_TRY(check_launch(ctx, "super-tile expansion"));
    GS_TRY(span_end(ctx, stream));
    ctx->launch_order = b.order;
    ctx->sorted_values = b.values;
    ctx->sorted_keys = b.keys_out;
    return GS_OK;
}

// Binning of the last preprocess.  The pair count M is known on the host only after
// the prefix sum; rather than idling the GPU while the host waits for it, the pair
// kernels are enqueued first on buffers sized from earlier frames (capacity), and
// the host then checks M: if it exceeds the capacity (first frame, growth), the
// buffers grow and the pair kernels are enqueued again, so results are always exact.
static gs_status bin_and_sort(gs_context *ctx, const gs_projected *pr, int emit_keys, gs_binning *out,
                              hipStream_t stream) {
    const int64_t n = ctx->n;
    const int64_t tiles = (int64_t)ctx->tiles_x * ctx->tiles_y;
    const bool depth_first = ctx->sort_mode == GS_SORT_DEPTH_FIRST;
    const size_t nn = (size_t)(n > 0 ? n : 1);
    GS_TRY(ensure(ctx, ctx->offsets, nn * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->scan_scratch, (size_t)scan_scratch_words((int64_t)nn) * 8));
    GS_TRY(ensure(ctx, ctx->total, 3 * sizeof(unsigned long long)));
    GS_TRY(ensure(ctx, ctx->ranges, (size_t)tiles * 2 * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->tile_order, (size_t)tiles * sizeof(uint32_t)));

    // super-tile binning where it applies (depth-first mode; counts packed for the scan)
    const int64_t super_tiles = (int64_t)((ctx->tiles_x + kSuperSide - 1) / kSuperSide) *
                                ((ctx->tiles_y + kSuperSide - 1) / kSuperSide);
    const bool super_bin = depth_first && ctx->packed_counts && n >= 2 && tiles <= kMaxSuperBinningTiles &&
                           super_tiles <= kMaxSuper;   // the preprocess packed the counts for it
    const uint32_t *order = nullptr;
    int64_t M = 0, S = 0;
    int64_t depth_buckets = 0;   // buckets of the depth order that stood, 0: the radix sort
    bool speculated = false;
    ctx->ranked_rect = nullptr;
    if (n > 0) {
        const uint32_t *counts = pr->tile_count;   // tile counts in rank order
        // by buckets of depth when the preprocess left the depth bounds (a bucket too large
        // raises a flag that travels with the pair count; then the radix sort redoes it)
        const bool buckets = depth_first && ctx->depth_range && n >= 2;
        const uint32_t *gather = super_bin ? as<uint32_t>(ctx->pcount) : pr->tile_count;
        const unsigned long long *bucket_flag = nullptr;
        if (depth_first) {
            // square rule: the bucketed order writes the rectangles in rank order for the listing
            // (read as 16-byte vectors: a caller's rectangle plane that is not 16-byte aligned
            // takes the gathering path)
            const uint2 *rect = ctx->tile_test_used == GS_TILE_ELLIPSE || (reinterpret_cast<uintptr_t>(pr->rect) & 15)
                                    ? nullptr
                                    : reinterpret_cast<const uint2 *>(pr->rect);
            GS_TRY(order_by_depth(ctx, n, gather, buckets, &order, &bucket_flag, stream, rect, super_bin));
            counts = n > 1 ? as<uint32_t>(ctx->dcount) : pr->tile_count;
            if (buckets) depth_buckets = (int64_t)1 << depth_bucket_bits(n);
        }
        // the scan's last kernel stores the pair count straight into host-coherent memory (no copy
        // on the stream); a sentinel shows a count that never arrived
        constexpr unsigned long long kNoCount = ~0ull;
        *ctx->host_total = kNoCount;
        GS_TRY(enqueue_scan(ctx, counts, n, super_bin, ctx->host_total_dev, bucket_flag, stream));

        if (ctx->pair_capacity > 0 && (!super_bin || ctx->super_capacity > 0)) {
            if (super_bin)
                GS_TRY(enqueue_super_pairs(ctx, pr, order, emit_keys, ctx->pair_capacity, ctx->super_capacity,
                                           stream));
            else
                GS_TRY(enqueue_pairs(ctx, pr, order, emit_keys, ctx->pair_capacity, stream));
            speculated = true;
        }
        // The host polls the count itself: no event in the stream (an event record cost the
        // GPU ~5 us per frame at 10 k Gaussians).  After 200 ms without it, wait for the stream.
        unsigned long long published = __atomic_load_n(ctx->host_total, __ATOMIC_ACQUIRE);
        if (published == kNoCount) {
            const auto t0 = std::chrono::steady_clock::now();
            while ((published = __atomic_load_n(ctx->host_total, __ATOMIC_ACQUIRE)) == kNoCount &&
                   std::chrono::steady_clock::now() - t0 < std::chrono::milliseconds(200))
                __builtin_ia32_pause();
        }
        if (published == kNoCount) {   // not seen yet: wait for the whole stream, then it must be there
            GS_HIP(ctx, hipStreamSynchronize(stream));
            published = __atomic_load_n(ctx->host_total, __ATOMIC_ACQUIRE);
            if (published == kNoCount) return fail(ctx, GS_ERR_DEVICE, "the pair count did not reach the host");
        }
        if (super_bin) {
            M = (int64_t)(published & ((1ull << kPairShift) - 1));
            S = (int64_t)(published >> kPairShift);
        } else {
            M = (int64_t)published;
        }
        // the flag: low word, redo the order; high word, a larger bucket was met (the next
        // frame launches the larger-bucket kernel only if this one met such a bucket)
        const unsigned long long bflag = bucket_flag ? __atomic_load_n(ctx->host_total + 2, __ATOMIC_ACQUIRE) : 0ull;
        if (bucket_flag) ctx->run_larger = (bflag >> 32) != 0;
        if ((bflag & 0xffffffffull) != 0) {
            // a bucket too large to sort in LDS (or one for the larger-bucket kernel, which this
            // frame left out): order this frame by the radix sort, recount the offsets in that
            // order (the totals do not change) and list the pairs afresh
            GS_HIP(ctx, hipStreamSynchronize(stream));
            GS_TRY(order_by_depth(ctx, n, gather, false, &order, nullptr, stream));
            ctx->ranked_rect = nullptr;   // the listing gathers the rectangles by Gaussian again
            GS_TRY(enqueue_scan(ctx, counts, n, super_bin, nullptr, nullptr, stream));
            speculated = false;
            depth_buckets = 0;
        }
        // listings enqueued before this frame's count arrived have run (same stream)
        if (__atomic_load_n(ctx->host_total + 1, __ATOMIC_ACQUIRE) != 0) {
            __atomic_store_n(ctx->host_total + 1, 0ull, __ATOMIC_RELEASE);
            return fail(ctx, GS_ERR_DEVICE, "the exact-footprint pair listing of an earlier frame met a Gaussian "
                                            "whose row spans disagree with its tile count");
        }
        if (M > ctx->max_dups)
            return fail(ctx, GS_ERR_CAPACITY, "%lld (Gaussian, tile) pairs exceed the cap of %lld", (long long)M,
                        (long long)ctx->max_dups);
    }
    if (!speculated || M > ctx->pair_capacity || (super_bin && S > ctx->super_capacity)) {
        if (speculated) GS_HIP(ctx, hipStreamSynchronize(stream));   // buffers are about to move
        if (ctx->arena) {   // the fixed scratch: exactly the frame's pairs, no headroom
            ctx->pair_capacity = M > 1 ? M : 1;
            ctx->super_capacity = S > 1 ? S : 1;
        } else {
            const int64_t want = M + M / 4, swant = S + S / 4;
            ctx->pair_capacity = want > 4096 ? want : 4096;
            ctx->super_capacity = swant > 4096 ? swant : 4096;
        }
        if (super_bin)
            GS_TRY(enqueue_super_pairs(ctx, pr, order, emit_keys, ctx->pair_capacity, ctx->super_capacity, stream));
        else
            GS_TRY(enqueue_pairs(ctx, pr, order, emit_keys, ctx->pair_capacity, stream));
    }

    ctx->num_dups = M;
    ctx->rank_order = order;
    out->num_dups = M;
    out->tiles_x = ctx->tiles_x;
    out->tiles_y = ctx->tiles_y;
    out->tile_ranges = as<uint32_t>(ctx->ranges);
    out->values = ctx->sorted_values;
    out->keys = ctx->sorted_keys;
    const bool unsorted = M && !depth_first && emit_keys;
    out->keys_unsorted = unsorted ? as<uint64_t>(ctx->keys_unsorted) : nullptr;
    out->values_unsorted = unsorted ? as<uint32_t>(ctx->vals_unsorted) : nullptr;
    out->super_entries = super_bin ? S : 0;
    out->depth_buckets = depth_buckets;
    return GS_OK;
}

gs_status gs_cache_covariance(gs_context *ctx, const gs_gaussians *g, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (ctx->arena) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "gs_cache_covariance inside gs_render_noalloc");
    ctx->cov_n = -1;   // dropped unless rebuilt below
    ctx->cov_quat = ctx->cov_log_scale = nullptr;
    if (!g) return GS_OK;
    char why[160];
    if (gs_check_arguments(g, nullptr, why, sizeof why) != GS_OK) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    if (g->n > 0) {
        GS_TRY(ensure(ctx, ctx->cov, (size_t)g->n * 6 * sizeof(float)));
        launch_covariance(g->quat, g->log_scale, (int32_t)g->n, as<float>(ctx->cov), stream);
        GS_TRY(check_launch(ctx, "covariance cache"));
    }
    ctx->cov_n = g->n;
    ctx->cov_quat = g->quat;
    ctx->cov_log_scale = g->log_scale;
    return GS_OK;
}

gs_status gs_bin_and_sort(gs_context *ctx, const gs_projected *pr, const gs_camera *cam, gs_binning *out,
                          hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!out || !cam) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL camera or output");
    char why[160];
    if (gs_check_arguments(nullptr, cam, why, sizeof why) != GS_OK)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    GS_TRY(check_projected(ctx, pr));
    if ((cam->width + GS_TILE - 1) / GS_TILE != ctx->tiles_x || (cam->height + GS_TILE - 1) / GS_TILE != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "camera size differs from the one given to gs_preprocess");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    return bin_and_sort(ctx, pr, ctx->emit_keys, out, stream);
}

gs_status gs_composite_ex(gs_context *ctx, const gs_projected *pr, const gs_binning *bin, const gs_camera *cam,
                          const float bg[3], float *image, float *final_T, uint32_t *n_blend,
                          unsigned long long *blend_total, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!bin || !cam || !bg || !image) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL binning, camera, bg or image");
    char why[160];
    if (gs_check_arguments(nullptr, cam, why, sizeof why) != GS_OK)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    GS_TRY(check_projected(ctx, pr));
    if (bin->tile_ranges != as<uint32_t>(ctx->ranges) || bin->values != ctx->sorted_values ||
        bin->tiles_x != ctx->tiles_x || bin->tiles_y != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "binning is not the last gs_bin_and_sort output of this context");
    if ((cam->width + GS_TILE - 1) / GS_TILE != ctx->tiles_x || (cam->height + GS_TILE - 1) / GS_TILE != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "camera size differs from the one given to gs_preprocess");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    CompositeParams c{};
    c.width = cam->width;
    c.height = cam->height;
    c.tiles_x = ctx->tiles_x;
    c.tiles_y = ctx->tiles_y;
    c.splat = pr->splat;
    c.values = bin->values;
    c.ranges = bin->tile_ranges;
    for (int i = 0; i < 3; ++i) c.bg[i] = bg[i];
    c.image = image;
    c.final_T = final_T;
    c.n_blend = n_blend;
    c.blend_total = blend_total;
    c.tile_order = ctx->launch_order;
    GS_TRY(span_begin(ctx, GS_STAGE_COMPOSITE, stream));
    launch_composite(c, stream);
    GS_TRY(check_launch(ctx, "composite"));
    GS_TRY(span_end(ctx, stream));
    return GS_OK;
}

gs_status gs_composite(gs_context *ctx, const gs_projected *pr, const gs_binning *bin, const gs_camera *cam,
                       const float bg[3], float *image, hipStream_t stream) {
    return gs_composite_ex(ctx, pr, bin, cam, bg, image, nullptr, nullptr, nullptr, stream);
}

gs_status gs_render(gs_context *ctx, const gs_gaussians *g, const gs_camera *cam, const float bg[3], float *image,
                    hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!bg || !image) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL bg or image");
    gs_projected pr;
    GS_TRY(gs_preprocess(ctx, g, cam, &pr, stream));
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    gs_binning bin;
    GS_TRY(bin_and_sort(ctx, &pr, 0, &bin, stream));
    return gs_composite(ctx, &pr, &bin, cam, bg, image, stream);
}

gs_status gs_render_noalloc(gs_context *ctx, const gs_gaussians *g, const gs_camera *cam, const float bg[3],
                            float *image, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!g || !cam || !bg || !image) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL gaussians, camera, bg or image");
    char why[160];
    if (gs_check_arguments(g, cam, why, sizeof why) != GS_OK) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    if (ctx->arena) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "gs_render_noalloc is already running on this context");
    // what the Gaussians and the tiles need before any pair (per Gaussian: record 64, depth 4,
    // rect 8, count 4, packed count 4, two key/index pairs 16, bucket entry 16, gathered count 4,
    // rect in rank order 8, offsets 4; the bucket count tables; per tile: range 8, launch order
    // 4), checked before anything is enqueued; the pairs are checked once counted
    const int64_t tiles = (int64_t)((cam->width + GS_TILE - 1) / GS_TILE) * ((cam->height + GS_TILE - 1) / GS_TILE);
    const int64_t fixed = g->n * 132 + depth_bucket_scratch_words(g->n) * 4 + tiles * 12;
    if (fixed > (int64_t)(kNoAllocBytes / 2))
        return fail(ctx, GS_ERR_CAPACITY,
                    "gs_render_noalloc: %lld Gaussians and %lld tiles need %lld bytes, more than half of the "
                    "%zu-byte scratch", (long long)g->n, (long long)tiles, (long long)fixed, kNoAllocBytes);
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    hipError_t sst;
    unsigned char *base = scratch_address(ctx->device, &sst);
    if (!base) return fail(ctx, GS_ERR_DEVICE, "address of the scratch array: %s", hipGetErrorString(sst));

    // swap the context's own workspace out: every ensure() of this frame carves from the scratch
    DeviceBuffer *bufs[kContextBuffers];
    context_buffers(ctx, bufs);
    DeviceBuffer saved[kContextBuffers];
    for (int i = 0; i < kContextBuffers; ++i) {
        saved[i] = *bufs[i];
        *bufs[i] = DeviceBuffer{};
    }
    const int64_t saved_capacity = ctx->pair_capacity, saved_super = ctx->super_capacity;
    const int saved_profile = ctx->profile;
    ctx->pair_capacity = ctx->super_capacity = 0;   // size the pair buffers from the frame's own counts
    ctx->profile = 0;         // timing events would be allocated
    ctx->arena = base;
    ctx->arena_size = kNoAllocBytes;
    ctx->arena_used = 0;

    gs_projected pr;
    gs_binning bin;
    gs_status st = gs_preprocess(ctx, g, cam, &pr, stream);
    if (st == GS_OK) st = bin_and_sort(ctx, &pr, 0, &bin, stream);
    if (st == GS_OK) st = gs_composite(ctx, &pr, &bin, cam, bg, image, stream);

    for (int i = 0; i < kContextBuffers; ++i) *bufs[i] = saved[i];
    ctx->arena = nullptr;
    ctx->arena_size = ctx->arena_used = 0;
    ctx->pair_capacity = saved_capacity;
    ctx->super_capacity = saved_super;
    ctx->profile = saved_profile;
    // the frame's projection and binning lived in the scratch: none is left on the context
    ctx->n = -1;
    ctx->num_dups = -1;
    ctx->rank_order = ctx->sorted_values = ctx->launch_order = nullptr;
    ctx->sorted_keys = nullptr;
    ctx->g_mean = nullptr;
    return st;
}

gs_status gs_backward(gs_context *ctx, const gs_gaussians *g, const gs_camera *cam, const gs_projected *pr,
                      const gs_binning *bin, const float bg[3], const float *final_T, const uint32_t *n_blend,
                      const float *grad_image, const gs_gradients *grads, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (!g || !cam || !bin || !bg || !grads)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL gaussians, camera, binning, bg or gradients");
    char why[160];
    if (gs_check_arguments(g, cam, why, sizeof why) != GS_OK) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "%s", why);
    GS_TRY(check_projected(ctx, pr));
    if (g->n != ctx->n || g->sh_degree != ctx->sh_degree || g->mean != ctx->g_mean)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "gaussians are not the ones of the last gs_preprocess");
    if (ctx->num_dups < 0 || bin->tile_ranges != as<uint32_t>(ctx->ranges) || bin->values != ctx->sorted_values ||
        bin->num_dups != ctx->num_dups || bin->tiles_x != ctx->tiles_x || bin->tiles_y != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "binning is not the last gs_bin_and_sort output of this context");
    if ((cam->width + GS_TILE - 1) / GS_TILE != ctx->tiles_x || (cam->height + GS_TILE - 1) / GS_TILE != ctx->tiles_y)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "camera size differs from the one given to gs_preprocess");
    if (!final_T || !n_blend || !grad_image)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL final_T, n_blend or grad_image");
    const int64_t n = ctx->n;
    if (n > 0 && (!grads->mean || !grads->quat || !grads->log_scale || !grads->opacity || !grads->sh))
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "a parameter gradient pointer is NULL");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    if (n == 0) return GS_OK;

    const size_t nn = (size_t)n;
    const int64_t M = ctx->num_dups;
    GS_TRY(ensure(ctx, ctx->pair_grad, (size_t)(M > 0 ? M : 1) * kPairStride * sizeof(float)));
    GS_TRY(ensure(ctx, ctx->scan_total, sizeof(unsigned long long)));
    GS_TRY(ensure(ctx, ctx->fix_list, nn * kFixStride * sizeof(float)));
    GS_TRY(ensure(ctx, ctx->fix_count, (nn + 63) / 64 * sizeof(uint32_t)));
    // Gaussian g's records start at pair_base[g] = sum of tile_count over indices below g:
    // key64 mode listed the pairs in that order, depth-first mode needs its own prefix sum
    const int64_t tiles = (int64_t)ctx->tiles_x * ctx->tiles_y;
    GS_TRY(ensure(ctx, ctx->tile_weight, (size_t)tiles * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->tile_order_bwd, (size_t)tiles * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->tile_cut, (size_t)tiles * sizeof(unsigned long long)));
    const uint32_t *pair_base = as<uint32_t>(ctx->offsets);
    GS_TRY(span_begin(ctx, GS_STAGE_BACKWARD_SETUP, stream));
    if (ctx->rank_order) {
        GS_TRY(ensure(ctx, ctx->pair_base, nn * sizeof(uint32_t)));
        launch_scan(pr->tile_count, nullptr, as<uint32_t>(ctx->pair_base), n,
                    as<unsigned long long>(ctx->scan_total),
                    as<unsigned long long>(ctx->scan_scratch), stream);
        GS_TRY(check_launch(ctx, "pair offsets"));
        pair_base = as<uint32_t>(ctx->pair_base);
    }
    // heaviest-first launch order by each tile's reverse-walk length
    const uint32_t *bwd_order = nullptr;
    if (M > 0 && tiles <= kMaxOrderedTiles) {
        launch_backward_tile_weight(n_blend, bin->tile_ranges, cam->width, cam->height, ctx->tiles_x, ctx->tiles_y,
                                    as<uint32_t>(ctx->tile_weight), stream);
        TileOrderParams o{};
        o.tiles = (int32_t)tiles;
        o.weights = as<uint32_t>(ctx->tile_weight);
        o.order = as<uint32_t>(ctx->tile_order_bwd);
        if (launch_tile_order(o, stream)) bwd_order = o.order;
        GS_TRY(check_launch(ctx, "backward tile order"));
    }
    GS_TRY(span_end(ctx, stream));

    CompositeBackwardParams c{};
    c.width = cam->width;
    c.height = cam->height;
    c.tiles_x = ctx->tiles_x;
    c.tiles_y = ctx->tiles_y;
    c.splat = pr->splat;
    c.values = bin->values;
    c.ranges = bin->tile_ranges;
    c.rect = reinterpret_cast<const uint2 *>(pr->rect);
    c.pair_base = pair_base;
    c.final_T = final_T;
    c.n_blend = n_blend;
    c.grad_image = grad_image;
    for (int i = 0; i < 3; ++i) c.bg[i] = bg[i];
    c.pair_grad = as<float>(ctx->pair_grad);
    c.tile_order = bwd_order;
    c.cut = as<unsigned long long>(ctx->tile_cut);
    const EllipseRec *ell = ctx->tile_test_used == GS_TILE_ELLIPSE ? as<EllipseRec>(ctx->ellipse) : nullptr;
    c.ellipse = ell;
    GS_TRY(span_begin(ctx, GS_STAGE_BACKWARD_COMPOSITE, stream));
    if (M > 0) launch_composite_backward(c, stream);
    GS_TRY(check_launch(ctx, "composite backward"));
    GS_TRY(span_end(ctx, stream));

    GaussianBackwardParams q{};
    q.n = (int32_t)n;
    q.sh_coeffs = (g->sh_degree + 1) * (g->sh_degree + 1);
    q.mean = g->mean;
    q.quat = g->quat;
    q.log_scale = g->log_scale;
    q.sh = g->sh;
    memcpy(q.R, cam->R, sizeof q.R);
    memcpy(q.t, cam->t, sizeof q.t);
    q.fx = cam->fx;
    q.fy = cam->fy;
    for (int i = 0; i < 3; ++i)
        q.cam_pos[i] = (float)-((double)cam->R[i] * cam->t[0] + (double)cam->R[3 + i] * cam->t[1] +
                                (double)cam->R[6 + i] * cam->t[2]);
    q.tile_count = pr->tile_count;
    q.pair_base = pair_base;
    q.rect = reinterpret_cast<const uint2 *>(pr->rect);
    q.depth = pr->depth;
    q.cut = as<unsigned long long>(ctx->tile_cut);
    q.ellipse = ell;
    q.tiles_x = ctx->tiles_x;
    q.pair_grad = as<float>(ctx->pair_grad);
    q.fix_list = as<float>(ctx->fix_list);
    q.fix_count = as<uint32_t>(ctx->fix_count);
    q.g_mean = grads->mean;
    q.g_quat = grads->quat;
    q.g_log_scale = grads->log_scale;
    q.g_opacity = grads->opacity;
    q.g_sh = grads->sh;
    q.g_mean2d = grads->mean2d;
    q.g_conic = grads->conic;
    q.g_rgb = grads->rgb;
    GS_TRY(span_begin(ctx, GS_STAGE_BACKWARD_GAUSSIAN, stream));
    launch_gaussian_backward(q, stream);
    GS_TRY(check_launch(ctx, "gaussian backward"));
    GS_TRY(span_end(ctx, stream));
    return GS_OK;
}

static gs_status splat2d_check(gs_context *ctx, int64_t n, const float *means, const float *covs,
                               const float *colours, const float *opacities, const float *depths, int32_t height,
                               int32_t width) {
    if (n < 0 || n > 0x7fffffffll) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "splat count outside [0, 2^31)");
    if (height < 1 || width < 1 || height > 32768 || width > 32768)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "image size outside [1, 32768]");
    if (n > 0 && (!means || !covs || !colours || !opacities || !depths))
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "a splat array pointer is NULL");
    return GS_OK;
}

gs_status gs_scale_activation(gs_context *ctx, const float *log_scale, float *scale, int64_t n,
                              hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    if (n < 0) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "negative n");
    if (n > 0 && (!log_scale || !scale)) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL array");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    launch_scale_activation(log_scale, scale, n, stream);
    GS_TRY(check_launch(ctx, "scale activation"));
    return GS_OK;
}

gs_status gs_splat2d_forward(gs_context *ctx, int64_t n, const float *means, const float *covs,
                             const float *colours, const float *opacities, const float *depths, int32_t height,
                             int32_t width, const float bg[3], float *image, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    GS_TRY(splat2d_check(ctx, n, means, covs, colours, opacities, depths, height, width));
    if (!image) return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL image");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    const size_t nn = (size_t)(n > 0 ? n : 1);
    GS_TRY(ensure(ctx, ctx->s2_order, nn * sizeof(uint32_t)));
    GS_TRY(ensure(ctx, ctx->s2_rec, nn * 12 * sizeof(float)));
    GS_TRY(ensure(ctx, ctx->s2_trans, nn * (size_t)height * (size_t)width * sizeof(float)));
    Splat2DParams p{};
    p.n = (int32_t)n;
    p.height = height;
    p.width = width;
    p.means = means;
    p.covs = covs;
    p.colours = colours;
    p.opacities = opacities;
    p.depths = depths;
    for (int i = 0; i < 3; ++i) p.bg[i] = bg ? bg[i] : 0.0f;
    p.image = image;
    launch_splat2d_forward(p, as<uint32_t>(ctx->s2_order), as<float>(ctx->s2_rec), as<float>(ctx->s2_trans), stream);
    GS_TRY(check_launch(ctx, "splat2d forward"));
    ctx->s2_n = n;
    ctx->s2_height = height;
    ctx->s2_width = width;
    ctx->s2_means = means;
    ctx->s2_depths = depths;
    return GS_OK;
}

gs_status gs_splat2d_backward(gs_context *ctx, int64_t n, const float *means, const float *covs,
                              const float *colours, const float *opacities, const float *depths, int32_t height,
                              int32_t width, const float bg[3], const float *grad_image, float *grad_means,
                              float *grad_covs, float *grad_colours, float *grad_opacities, hipStream_t stream) {
    if (!ctx) return GS_ERR_INVALID_ARGUMENT;
    GS_TRY(splat2d_check(ctx, n, means, covs, colours, opacities, depths, height, width));
    if (n != ctx->s2_n || height != ctx->s2_height || width != ctx->s2_width || means != ctx->s2_means ||
        depths != ctx->s2_depths)
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "arguments differ from the last gs_splat2d_forward on this context");
    if (!grad_image || (n > 0 && (!grad_means || !grad_covs || !grad_colours || !grad_opacities)))
        return fail(ctx, GS_ERR_INVALID_ARGUMENT, "NULL gradient pointer");
    DeviceScope scope(ctx->device);
    if (scope.status != hipSuccess) return fail(ctx, GS_ERR_DEVICE, "hipSetDevice failed");
    if (n == 0) return GS_OK;
    const size_t tiles = (size_t)((width + GS_TILE - 1) / GS_TILE) * (size_t)((height + GS_TILE - 1) / GS_TILE);
    GS_TRY(ensure(ctx, ctx->s2_partial, (size_t)n * tiles * kPairGrad * sizeof(float)));
    Splat2DParams p{};
    p.n = (int32_t)n;
    p.height = height;
    p.width = width;
    p.means = means;
    p.covs = covs;
    p.colours = colours;
    p.opacities = opacities;
    p.depths = depths;
    for (int i = 0; i < 3; ++i) p.bg[i] = bg ? bg[i] : 0.0f;
    p.grad_image = grad_image;
    p.g_means = grad_means;
    p.g_covs = grad_covs;
    p.g_colours = grad_colours;
    p.g_opacities = grad_opacities;
    launch_splat2d_backward(p, as<float>(ctx->s2_rec), as<float>(ctx->s2_trans), as<float>(ctx->s2_partial), stream);
    GS_TRY(check_launch(ctx, "splat2d backward"));
    return GS_OK;
}

gs_status gs_profile_read(gs_context *ctx, gs_profile *out) {
    if (!ctx || !out) return GS_ERR_INVALID_ARGUMENT;
    DeviceScope scope(ctx->device);
    for (int i = 0; i < GS_STAGE_COUNT; ++i) {
        out->ms[i] = 0.0;
        out->launches[i] = 0;
    }
    for (size_t i = 0; i < ctx->spans_used; ++i) {
        TimedSpan &t = ctx->spans[i];
        GS_HIP(ctx, hipEventSynchronize(t.end));
        float ms = 0.0f;
        GS_HIP(ctx, hipEventElapsedTime(&ms, t.begin, t.end));
        out->ms[t.stage] += ms;
        out->launches[t.stage] += 1;
    }
    ctx->spans_used = 0;
    return GS_OK;
}

}  // extern "C"
