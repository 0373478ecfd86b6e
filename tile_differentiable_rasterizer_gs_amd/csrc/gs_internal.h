// Internal declarations of the HIP rasterizer library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gsrast.h"

namespace gsr {

constexpr int kTile = GS_TILE;
constexpr int kBlock = 256;      // threads per workgroup for every kernel (4 wave64)
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// exact-footprint tile rule (GS_TILE_ELLIPSE)
// ---------------------------------------------------------------------------
// Per Gaussian: e = (ymax, dyr, b/c, det/c), f = (c, u, v, valid) with [[a, b], [b, c]] the
// 2D covariance, ymax = 3 sqrt(c), dyr = 3b / sqrt(a); valid = 0 when a or c is not
// positive (then the whole square is kept).
struct EllipseRec {
    float4 e;
    float4 f;
};

__device__ __forceinline__ EllipseRec make_ellipse(float a, float b, float c, float det, float u, float v) {
#pragma clang fp contract(off)
    EllipseRec E;
    E.e = make_float4(3.0f * sqrtf(c), (3.0f * b) / sqrtf(a), b / c, det / c);
    E.f = make_float4(c, u, v, (c > 0.0f && E.e.x > 0.0f) ? 1.0f : 0.0f);
    return E;
}

// Kept tiles [*pa, *pb) of tile row ty of the square [x0, x1): those whose pixel-centre
// columns 16 tx .. 16 tx + 15 meet the x-extent of the 3-sigma ellipse over the row's
// pixel-centre band 16 ty .. 16 ty + 15.  The ellipse cut at height dy is centred at
// (b/c) dy with half-width sqrt((det/c)(9 - dy^2/c)); its right end peaks at dy = dyr,
// its left end at -dyr, each clamped to the band.  binary32 in this order, no
// contraction: the tile counts and keys are a function of the inputs alone.
__device__ __forceinline__ void row_span(const EllipseRec &E, uint32_t x0, uint32_t x1, uint32_t ty, uint32_t &pa,
                                         uint32_t &pb) {
#pragma clang fp contract(off)
    pa = pb = x0;
    if (E.f.w == 0.0f) {
        pb = x1;
        return;
    }
    const float ymax = E.e.x, dyr = E.e.y, bc = E.e.z, kc = E.e.w, c = E.f.x, u = E.f.y, v = E.f.z;
    const float p = (float)(16 * ty) - v;
    const float q = (float)(16 * ty + 15) - v;
    const float lo = fmaxf(p, -ymax), hi = fminf(q, ymax);
    if (!(lo <= hi)) return;
    const float dr = fminf(fmaxf(dyr, lo), hi);
    const float dl = fminf(fmaxf(-dyr, lo), hi);
    const float tr = fmaxf(9.0f - (dr * dr) / c, 0.0f);
    const float tl = fmaxf(9.0f - (dl * dl) / c, 0.0f);
    const float xr = bc * dr + sqrtf(kc * tr);
    const float xl = bc * dl - sqrtf(kc * tl);
    float fa = ceilf(((u + xl) - 15.0f) * 0.0625f);
    float fb = floorf((u + xr) * 0.0625f) + 1.0f;
    fa = fmaxf(fa, (float)x0);
    fb = fminf(fb, (float)x1);
    if (!(fa < fb)) return;
    pa = (uint32_t)fa;
    pb = (uint32_t)fb;
}

// Index of tile (tx, ty) among a Gaussian's kept tiles (row-major over the square).
__device__ __forceinline__ uint32_t kept_index(const EllipseRec &E, uint32_t x0, uint32_t x1, uint32_t y0,
                                               uint32_t tx, uint32_t ty) {
    uint32_t k = 0, a, b;
    for (uint32_t r = y0; r < ty; ++r) {
        row_span(E, x0, x1, r, a, b);
        k += b - a;
    }
    row_span(E, x0, x1, ty, a, b);
    return k + (tx - a);
}

// ---------------------------------------------------------------------------
// preprocess
// ---------------------------------------------------------------------------
// Scale activation: the binary64 exp of the log-scale, rounded to binary32 (the same
// value on any implementation whose binary64 exp rounds to the same binary32).
__device__ __forceinline__ float scale_activation(float log_scale) { return (float)exp((double)log_scale); }
void launch_scale_activation(const float *log_scale, float *scale, int64_t n, hipStream_t s);

struct PreprocessParams {
    int32_t n;
    int32_t sh_coeffs;           // K = (degree+1)^2
    const float *mean, *quat, *log_scale, *opacity, *sh;
    float R[9];
    float t[3];
    float fx, fy, cx, cy, znear;
    float cam_pos[3];            // camera centre in world space (colour direction)
    int32_t tiles_x, tiles_y;
    float *splat;                // [n][GS_SPLAT_STRIDE]
    float *depth;                // [n]
    uint2 *rect;                 // [n] {x0 | x1 << 16, y0 | y1 << 16}
    uint32_t *tile_count;        // [n]
    uint32_t *depth_key;         // [n] or null: visible ? bits(depth) : 0xffffffff
    uint32_t *depth_index;       // [n] or null: g
    EllipseRec *ellipse;         // [n] or null: exact-footprint rule (tile counts from the row spans)
};
void launch_preprocess(const PreprocessParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// exclusive prefix sum of uint32 values (optionally gathered in[gather[i]])
// ---------------------------------------------------------------------------
constexpr int kScanItems = 16;
constexpr int kScanTile = kBlock * kScanItems;   // 4096 values per workgroup
// number of uint64 scratch words launch_scan needs for n values
int64_t scan_scratch_words(int64_t n);
// out[i] = sum_{j<i} in[j]; *total = sum of all (device uint64).  n >= 1.
// host_total (optional): device address of host-coherent memory that also receives the sum.
void launch_scan(const uint32_t *in, const uint32_t *gather, uint32_t *out, int64_t n,
                 unsigned long long *total, unsigned long long *scratch, hipStream_t s,
                 unsigned long long *host_total = nullptr);

// ---------------------------------------------------------------------------
// stable LSD radix sort of (key, uint32 value) pairs
// ---------------------------------------------------------------------------
constexpr int kRadixBits = 8;
// uint32 scratch words radix_sort_pairs needs for n pairs
int64_t sort_scratch_words(int64_t n);
// Stable sort by key bits [begin_bit, end_bit), ping-ponging between (k0,v0) and (k1,v1);
// returns 0 if the result is in (k0,v0), 1 if in (k1,v1).  n bounds the element count
// (grid and scratch are sized from it); when n_dev is given the kernels sort
// min(n, *n_dev) elements, a count that only the device knows at launch.  If
// gathered_out is given, the last pass also writes gathered_out[i] = gather_src[value_i]
// for the sorted values.
template <typename K>
int radix_sort_pairs(K *k0, uint32_t *v0, K *k1, uint32_t *v1, int64_t n, const unsigned long long *n_dev,
                     int begin_bit, int end_bit, uint32_t *scratch, hipStream_t s,
                     const uint32_t *gather_src = nullptr, uint32_t *gathered_out = nullptr);

// ---------------------------------------------------------------------------
// pair listing, ranges
// ---------------------------------------------------------------------------
// Pair-list kernels read the pair count from device memory and handle
// min(count, capacity) entries; grids are sized from the capacity.
struct DuplicateParams {
    int64_t n_items;             // number of (ranked) Gaussians
    const unsigned long long *num_dups;   // device: total pairs (exclusive-scan total)
    int64_t capacity;            // entries the pair buffers hold
    const uint32_t *offsets;     // [n_items] exclusive prefix of tile counts (in rank order)
    const uint32_t *order;       // [n_items] rank -> Gaussian index, or null (rank = index)
    const uint2 *rect;
    const float *depth;
    int32_t tiles_x;
    uint64_t *keys64;            // key64 mode: (tile << 32) | bits(depth)
    uint32_t *tile_keys;         // depth-first mode: tile id ...
    uint16_t *tile_keys16;       // ... or as 16 bits (at most 65536 tiles); entry count multiple of 8 per block
    uint32_t *values;            // Gaussian index
    const EllipseRec *ellipse;   // null, or the exact-footprint rule: only the row spans are listed
    const uint32_t *tile_count;  // [n] (needed with ellipse)
    uint32_t *clear;             // zeroed by the partition kernel ([clear_words]; the tile ranges)
    int64_t clear_words;
};
// uint32 words of the partition table launch_duplicate needs
int64_t duplicate_partition_words(int64_t num_dups);
void launch_duplicate(const DuplicateParams &p, uint32_t *part, hipStream_t s);

struct RangesParams {
    const unsigned long long *num_dups;   // device
    int64_t capacity;
    const uint64_t *keys64;      // either keys64 (tile = key >> 32) ...
    const uint32_t *tile_keys;   // ... or tile ids ...
    const uint16_t *tile_keys16; // ... or 16-bit tile ids
    uint32_t *ranges;            // [tiles][2], zeroed beforehand
    // optional key emission (depth-first mode): keys_out[e] = tile << 32 | bits(depth[values[e]])
    const uint32_t *values;
    const float *depth;
    uint64_t *keys_out;
};
void launch_ranges(const RangesParams &p, hipStream_t s);
void launch_fill_u32(uint32_t *dst, uint32_t value, int64_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// compositing
// ---------------------------------------------------------------------------
// Exponent of one splat at one pixel, in the base-2 form the splat record stores:
// q = (A' dx + B' dy) dx + C' dy^2 + log2(o / GS_ALPHA_MAX), and
// alpha = min(GS_ALPHA_MAX, o G) = GS_ALPHA_MAX * min(1, 2^q), the min being the
// exp instruction's free output clamp (splat_alpha_scaled).  The forward and the
// backward compositing kernels both build q and the clamp from these helpers, so the
// backward recovers bit for bit the alpha the forward blended.
__device__ __forceinline__ float splat_row_term(float dy, float Cp, float log2_o) {
    return __builtin_fmaf(dy, Cp * dy, log2_o);   // C' dy^2 + log2 o
}
__device__ __forceinline__ float splat_exponent(float dx, float Ap, float bdy, float row_term) {
    return __builtin_fmaf(dx, __builtin_fmaf(Ap, dx, bdy), row_term);
}
// alpha / GS_ALPHA_MAX = min(1, 2^q) (v_exp_f32 with its clamp bit)
__device__ __forceinline__ float splat_alpha_scaled(float q) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(q), 0.0f, 1.0f);
}
// log2(o / GS_ALPHA_MAX) for o > 0, the row term's constant
__device__ __forceinline__ float splat_log2_scaled_opacity(float o) {
    return __log2f(o) + 0.0144995696951150766f;   // -log2(0.99)
}

struct CompositeParams {
    int32_t width, height, tiles_x, tiles_y;
    const float *splat;
    const uint32_t *values;
    const uint32_t *ranges;
    float bg[3];
    float *image;                // [H][W][3]
    float *final_T;              // optional [H][W]
    uint32_t *n_blend;           // optional [H][W]
    unsigned long long *blend_total;  // optional
    const uint32_t *tile_order;  // optional launch order: workgroup b composites tile_order[b]
};
void launch_composite(const CompositeParams &p, hipStream_t s);

// Heaviest-first tile order (bucket sort of per-tile weights: explicit `weights`, else
// the tile list lengths from `ranges`).  Returns false, launching nothing, when there
// are more than kMaxOrderedTiles tiles (callers then launch in tile order).
constexpr int32_t kMaxOrderedTiles = 1 << 16;
struct TileOrderParams {
    int32_t tiles;
    const uint32_t *ranges;
    const uint32_t *weights;
    uint32_t *order;
};
bool launch_tile_order(const TileOrderParams &p, hipStream_t s);
// weights[t] = min(largest n_blend over tile t's pixels, tile t's list length)
void launch_backward_tile_weight(const uint32_t *n_blend, const uint32_t *ranges, int32_t width, int32_t height,
                                 int32_t tiles_x, int32_t tiles_y, uint32_t *weights, hipStream_t s);

// ---------------------------------------------------------------------------
// gradients
// ---------------------------------------------------------------------------
// Per-pair gradient record: one (Gaussian, tile) pair's sums over the tile's pixels of
// the moments S1, dy S0, S2, dy S1, dy^2 S0 (d = alpha dL/dalpha; S0, S1, S2 = sums of d,
// d dx, d dx^2), which dL/d(u, v, A, B, C) are linear in with the Gaussian's conic, and of
// dL/d(opacity, r, g, b); 36 bytes.
constexpr int kPairGrad = 9;
constexpr int kPairStride = kPairGrad;

struct CompositeBackwardParams {
    int32_t width, height, tiles_x, tiles_y;
    const float *splat;
    const uint32_t *values, *ranges;
    const uint2 *rect;
    const uint32_t *pair_base;   // [n] record index of each Gaussian's first pair
    const float *final_T;        // [H][W] from the forward
    const uint32_t *n_blend;     // [H][W] from the forward
    const float *grad_image;     // [H][W][3]
    float bg[3];
    float *pair_grad;            // [pairs][kPairStride]: Gaussian g's pair k (row-major
                                 // over its rectangle) at pair_base[g] + k
    const uint32_t *tile_order;  // optional launch order: workgroup b walks tile_order[b]
    const EllipseRec *ellipse;   // null, or the exact-footprint rule (pair index from the row spans)
    unsigned long long *cut;     // [tiles] out: (depth bits << 32 | index) of the deepest entry
                                 // walked, 0 if none; records exist exactly for entries <= it
};
void launch_composite_backward(const CompositeBackwardParams &p, hipStream_t s);

struct GaussianBackwardParams {
    int32_t n;
    int32_t sh_coeffs;
    const float *mean, *quat, *log_scale, *sh;
    float R[9];
    float t[3];
    float fx, fy;
    float cam_pos[3];
    const uint32_t *tile_count, *pair_base;
    const uint2 *rect;           // tile rectangles (x0 | x1 << 16, y0 | y1 << 16)
    const float *depth;          // [n] camera-space z
    const unsigned long long *cut;   // [tiles] from the reverse walk
    const EllipseRec *ellipse;   // null, or the exact-footprint rule
    int32_t tiles_x;
    const float *pair_grad;
    float *g_mean, *g_quat, *g_log_scale, *g_opacity, *g_sh;
    float *g_mean2d, *g_conic, *g_rgb;   // optional screen-space gradients
};
void launch_gaussian_backward(const GaussianBackwardParams &p, hipStream_t s);

// ---------------------------------------------------------------------------
// the lesson's dense 2D splat rasteriser
// ---------------------------------------------------------------------------
struct Splat2DParams {
    int32_t n, height, width;
    const float *means, *covs, *colours, *opacities, *depths;   // [n][2], [n][2][2], [n][3], [n], [n]
    float bg[3];
    float *image;                // forward output [H][W][3]
    const float *grad_image;     // backward input [H][W][3]
    float *g_means, *g_covs, *g_colours, *g_opacities;
};
// order [n], rec [n][12], trans [n][H][W] (T before each splat in depth order)
void launch_splat2d_forward(const Splat2DParams &p, uint32_t *order, float *rec, float *trans, hipStream_t s);
// partial [n][tiles][9]
void launch_splat2d_backward(const Splat2DParams &p, const float *rec, const float *trans, float *partial,
                             hipStream_t s);

}  // namespace gsr
