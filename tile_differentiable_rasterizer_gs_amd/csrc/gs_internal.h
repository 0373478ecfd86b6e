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

// Depth key of a Gaussian without pairs (sorts after every depth).
constexpr uint32_t kNoPairsKey = 0xffffffffu;
// Slots of the visible depth range the preprocess leaves for the bucketed depth order:
// range[s] = min, range[kDepthSlots + s] = max of the depth bits reduced into slot s.
constexpr int kDepthSlots = 256;

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
    uint32_t *depth_key;         // [n] or null: visible ? bits(depth) : kNoPairsKey
    uint32_t *depth_index;       // [n] or null: g
    uint32_t *depth_range;       // [2][kDepthSlots] or null: atomic min / max of the visible depth bits
    EllipseRec *ellipse;         // [n] or null: exact-footprint rule (tile counts from the row spans)
    uint32_t *packed_count;      // [n] or null: pack_counts(tile count, rect), for super-tile binning
    const float *cov;            // [6][n] or null: cached 3D covariances (then quat and log_scale are not read)
};
void launch_preprocess(const PreprocessParams &p, hipStream_t s);
// cov[k][g], k = 0..5: upper triangle (xx, xy, xz, yy, yz, zz) of Gaussian g's 3D covariance,
// bit-identical to what the preprocess computes from quat and log_scale
void launch_covariance(const float *quat, const float *log_scale, int32_t n, float *cov, hipStream_t s);

// ---------------------------------------------------------------------------
// exclusive prefix sum of uint32 values (optionally gathered in[gather[i]])
// ---------------------------------------------------------------------------
constexpr int kScanItems = 8;
constexpr int kScanTile = kBlock * kScanItems;   // 2048 values per workgroup
// number of uint64 scratch words launch_scan needs for n values
int64_t scan_scratch_words(int64_t n);
// out[i] = sum_{j<i} in[j]; *total = sum of all (device uint64).  n >= 1.
// host_total (optional): device address of host-coherent memory that also receives the sum;
// with `flag` (device memory) host_total[2] first receives *flag, and the sum is stored
// with release order after it.
void launch_scan(const uint32_t *in, const uint32_t *gather, uint32_t *out, int64_t n,
                 unsigned long long *total, unsigned long long *scratch, hipStream_t s,
                 unsigned long long *host_total = nullptr, const unsigned long long *flag = nullptr);
// The same over packed counts (tile count | super count << kPackShift): out[i] = the super
// counts before i; total[0] = tiles | super-tiles << kPairShift (also to host_total),
// total[1] = the tile total, total[2] = the super-tile total.
void launch_scan_pairs(const uint32_t *packed, uint32_t *out, int64_t n, unsigned long long *total,
                       unsigned long long *scratch, hipStream_t s, unsigned long long *host_total,
                       const unsigned long long *flag = nullptr);

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
// Offset (in uint32 words) into the scratch of radix_sort_pairs(n) of the per-digit totals
// of the last pass: totals[d] = elements whose last-pass digit is d.
int64_t sort_totals_offset(int64_t n);

// ---------------------------------------------------------------------------
// depth order by buckets of depth (depth-first mode, GS_DEPTH_ORDER_BUCKETS)
// ---------------------------------------------------------------------------
constexpr int kBucketCap = 4096;          // largest bucket one workgroup sorts in LDS
constexpr int kMinBucketBits = 8, kMaxBucketBits = 13;
constexpr int64_t kBucketTarget = 512;    // Gaussians per bucket the bucket count aims at
constexpr int64_t kGroupKeys = 4096;      // Gaussians per counting group (at least)
constexpr int64_t kMaxCountWords = 1 << 21;   // bound on the (bucket, group) count table

struct DepthBucketParams {
    const uint32_t *keys;          // [n] bits(depth), kNoPairsKey for a Gaussian without pairs
    int64_t n;
    int32_t bucket_bits;           // B = 1 << bucket_bits buckets; bucket B: no pairs
    int32_t groups;                // G contiguous ranges of Gaussians
    uint32_t *range;               // [2][kDepthSlots] bound slots (reset by the last kernel)
    unsigned long long *flag;      // device: low word 1 when the order must be redone (a bucket
                                   // too large, or a larger bucket without run_larger), high
                                   // word 1 when a bucket too large for the per-bucket kernel
                                   // was met
    int32_t run_larger;            // launch the larger-bucket kernel (else such a bucket sets the
                                   // low word)
    uint32_t *big_count;           // device: buckets listed for the sub-bin kernel
    uint32_t *big_list;            // [B] their ids
    float *bounds;                 // [2] the frame's (zmin, B / (zmax - zmin)) for the sub-bins
    uint32_t *counts;              // [G][B + 1] from 64 groups on, else [B + 1][G]
    uint32_t *totals;              // [B + 1]
    uint32_t *starts;              // [B + 2]
    uint64_t *entries;             // [n] bits(depth) << 32 | index, grouped by bucket (with rect:
                                   // [n] 16-byte records: index, depth bits, rectangle)
    const uint32_t *gather_src;    // [n] per-Gaussian value to gather in rank order
    uint32_t *order;               // out [n]: rank -> Gaussian
    uint32_t *gathered;            // out [n]: gather_src[order[r]]
    const uint2 *rect;             // null, or [n] the square rule's tile rectangles: then the count
                                   // comes from the rectangle instead of gather_src (the tile count
                                   // (x1 - x0)(y1 - y0), packed with the super-tile count when
                                   // packed_counts), and rect_out[r] = rect[order[r]]
    uint2 *rect_out;
    int32_t packed_counts;
};
int depth_bucket_bits(int64_t n);
int depth_bucket_groups(int64_t n);
// uint32 words of scratch for n Gaussians, and the carving of p.flag, big_count, bounds,
// counts, totals, starts and big_list out of it (also sets p.n, p.bucket_bits, p.groups)
int64_t depth_bucket_scratch_words(int64_t n);
void depth_bucket_layout(uint32_t *scratch, int64_t n, DepthBucketParams &p);
void launch_depth_bucket_sort(const DepthBucketParams &p, hipStream_t s);
// sets the bound slots to the empty range (min = all ones, max = 0)
void launch_depth_range_fill(uint32_t *range, hipStream_t s);

// ---------------------------------------------------------------------------
// super-tile binning (depth-first mode, GS_BINNING_SUPER_TILE)
// ---------------------------------------------------------------------------
// Tiles are grouped 8 x 8 into super-tiles.  Each depth-ranked Gaussian is listed once per
// super-tile of its rectangle, that list is sorted stably by super-tile (one 8-bit radix
// pass), and each super-tile's list, cut into segments, is expanded into its 64 tiles.
constexpr int kSuperShift = 3;                     // 8 x 8 tiles per super-tile
constexpr int kSuperSide = 1 << kSuperShift;
constexpr int kMaxSuper = 1 << kRadixBits;         // super-tiles one 8-bit pass orders
constexpr int kMaxSuperBinningTiles = 1 << 16;     // tile counts fit the packed count below
constexpr int64_t kAutoSuperMin = 1 << 16;         // GS_BINNING_AUTO: super-tile binning from this many Gaussians
constexpr int kSegment = 64;                       // super-list entries per segment (one wave, one per lane)
// Words between consecutive row-part offsets in the wide place shape: every place wave reads
// the offsets of its super-tile's 8 tile rows, and spread over 8 cache lines those reads do
// not pile onto a few L2 channels (packed, the 5 M-Gaussian frame's place kernel took 7 %
// longer); below that shape they are packed (the 1 M frame's tile lists 2 us faster).
constexpr int kRowStride = 16;
constexpr int kPackShift = 17;                     // packed count: tile count | super count << 17
constexpr int kPairShift = 36;                     // scan of packed counts: tiles | super-tiles << 36

// Super-list key: the super-tile id (bits 0-7, what the list is sorted by) and the part of the
// Gaussian's tile rectangle inside that super-tile, relative to its first tile: columns
// [a, b) and rows [r0, r1), each bound in 4 bits.
__host__ __device__ inline uint32_t super_key(uint32_t sid, uint32_t a, uint32_t b, uint32_t r0, uint32_t r1) {
    return sid | (a << 8) | (b << 12) | (r0 << 16) | (r1 << 20);
}

// The super-tile rectangle of a tile rectangle {x0 | x1 << 16, y0 | y1 << 16} (empty stays empty).
__host__ __device__ inline uint2 super_rect(uint2 rc) {
    const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y0 = rc.y & 0xffffu, y1 = rc.y >> 16;
    if (x1 <= x0 || y1 <= y0) return make_uint2(0u, 0u);
    return make_uint2((x0 >> kSuperShift) | ((((x1 - 1) >> kSuperShift) + 1) << 16),
                      (y0 >> kSuperShift) | ((((y1 - 1) >> kSuperShift) + 1) << 16));
}
// A Gaussian's tile count and number of super-tiles in one word (tile count <= 65536).
__host__ __device__ inline uint32_t pack_counts(uint32_t tile_count, uint2 rc) {
    if (tile_count == 0) return 0u;
    const uint2 sr = super_rect(rc);
    return tile_count | (((sr.x >> 16) - (sr.x & 0xffffu)) * ((sr.y >> 16) - (sr.y & 0xffffu)) << kPackShift);
}

struct SuperBinParams {
    int32_t tiles_x, tiles_y, super_x, super_y;
    const uint32_t *super_totals;  // [kMaxSuper] entries of each super-tile in the sorted super list
    const uint32_t *keys;          // sorted super list: super_key of each entry
    const uint32_t *gauss;         // sorted super list: the Gaussian of each entry
    const EllipseRec *ellipse;     // null, or the exact-footprint rule (a row span per tile row)
    uint32_t *seg_tiles;           // [segment capacity][64] pairs per (segment, tile), then offsets
    int64_t seg_capacity;          // segments the grids cover
    uint32_t *tile_total;          // [tiles] pairs per tile
    uint32_t *rows;                // [tiles_y][super_x] pairs per (tile row, super-tile column): row parts
    uint32_t *row_start;           // [tiles_y][super_x] x row_stride: pairs before each row part in tile order
    int32_t row_stride;            // words between consecutive row_start entries (set by the launch)
    uint32_t *ranges;              // [tiles][2]
    const unsigned long long *num_dups;   // device: the frame's pair count
    int64_t capacity;              // entries `values` holds; with more pairs nothing is written
    uint32_t *values;              // out: Gaussian index per entry, by tile then depth
    const float *depth;            // key emission (optional): keys_out[e] = tile << 32 | bits(depth[g])
    uint64_t *keys_out;
    uint32_t *order;               // optional: the heaviest-first tile launch order, from tile_total
};
// Segments the grids need for a super list of `entries` entries.
int64_t super_segment_capacity(int64_t entries);
// Per-tile counts, ranges, then the values (and keys).
void launch_super_binning(const SuperBinParams &p, hipStream_t s);

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
    const uint2 *rect_ranked;    // null, or [n_items] each rank's rectangle (rect[order[i]], read in rank order)
    const float *depth;
    int32_t tiles_x;
    uint64_t *keys64;            // key64 mode: (tile << 32) | bits(depth)
    uint32_t *tile_keys;         // depth-first mode: tile id ...
    uint16_t *tile_keys16;       // ... or as 16 bits (at most 65536 tiles); entry count multiple of 8 per block
    uint32_t *values;            // Gaussian index
    const EllipseRec *ellipse;   // null, or the exact-footprint rule: only the row spans are listed
    unsigned long long *fault;   // with ellipse: host-coherent word, bit 0 set (system scope) when a
                                 // Gaussian's row spans do not add up to its tile count
    const uint32_t *tile_count;  // [n] (needed with ellipse)
    uint32_t *clear;             // zeroed by the partition kernel ([clear_words]; the tile ranges)
    int64_t clear_words;
};
// uint32 words of the partition table launch_duplicate needs
int64_t duplicate_partition_words(int64_t num_dups);
void launch_duplicate(const DuplicateParams &p, uint32_t *part, hipStream_t s);
// Depth-first listing under the square rule (tile_keys16 or tile_keys, values; no ellipse, no
// 64-bit keys), a thread per ranked Gaussian; also zeroes clear[0, clear_words).
void launch_pair_list(const DuplicateParams &p, hipStream_t s);
// The super list in rank order, a thread per ranked Gaussian: num_dups is the device's
// super-list total, offsets its prefix in rank order, tiles_x the super-tile width, and the
// super_key of each entry goes to tile_keys.
void launch_super_list(const DuplicateParams &p, hipStream_t s);

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
// The order is a counting sort by weight on a logarithmic scale: 2048 buckets of 1/64
// octave (the leading bit of the weight and the six below it), heaviest first.
constexpr int kOrderSubBits = 6;                              // bits below the leading one
constexpr int kOrderBuckets = 32 << kOrderSubBits;            // 2048
// Bucket of a weight: 2047 - (64 floor(log2 w) + the six bits after the leading one); weight 0
// goes last.
__device__ __forceinline__ uint32_t order_bucket(uint32_t w) {
    if (w == 0) return kOrderBuckets - 1;
    const uint32_t lead = 31u - (uint32_t)__clz(w);
    const uint32_t frac = ((w << (31u - lead)) >> (31 - kOrderSubBits)) & ((1u << kOrderSubBits) - 1u);
    return (uint32_t)(kOrderBuckets - 1) - ((lead << kOrderSubBits) + frac);
}
struct TileOrderParams {
    int32_t tiles;
    const uint32_t *ranges;
    const uint32_t *weights;
    uint32_t *order;
};
bool launch_tile_order(const TileOrderParams &p, hipStream_t s);

// The heaviest-first order by one workgroup of kThreads threads (a multiple of the wave, at most
// 1024, dividing kOrderBuckets): a counting sort over the order buckets in s_count
// [kOrderBuckets], with s_wave [kThreads / kWave] for the wave totals.  Order within a bucket
// depends on the LDS atomics' timing; it changes only when a tile runs.
__device__ __forceinline__ uint32_t order_weight(const TileOrderParams &p, int t) {
    return p.weights ? p.weights[t] : p.ranges[2 * t + 1] - p.ranges[2 * t];
}
template <int kThreads>
__device__ void order_tiles(const TileOrderParams &p, uint32_t *s_count, uint32_t *s_wave) {
    constexpr int kPer = kOrderBuckets / kThreads;        // buckets per thread in the scan
    constexpr int kKept = kThreads >= 1024 ? 8 : 4096 / kThreads;   // tiles whose bucket stays in registers
    static_assert(kPer * kThreads == kOrderBuckets && kThreads % kWave == 0, "order workgroup");
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int b = threadIdx.x; b < kOrderBuckets; b += kThreads) s_count[b] = 0;
    __syncthreads();
    uint32_t kept[kKept];
#pragma unroll
    for (int j = 0; j < kKept; ++j) {
        const int t = threadIdx.x + j * kThreads;
        kept[j] = t < p.tiles ? order_bucket(order_weight(p, t)) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kKept; ++j)
        if (threadIdx.x + j * kThreads < p.tiles) atomicAdd(&s_count[kept[j]], 1u);
    for (int t = threadIdx.x + kKept * kThreads; t < p.tiles; t += kThreads)
        atomicAdd(&s_count[order_bucket(order_weight(p, t))], 1u);
    __syncthreads();
    // exclusive prefix over the buckets: kPer consecutive buckets per thread, a scan per wave,
    // then the wave totals
    uint32_t c[kPer], sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        c[k] = s_count[threadIdx.x * kPer + k];
        sum += c[k];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t up = (uint32_t)__shfl_up((int)incl, off);
        if (lane >= off) incl += up;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    uint32_t base = incl - sum;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        s_count[threadIdx.x * kPer + k] = base;
        base += c[k];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kKept; ++j) {
        const int t = threadIdx.x + j * kThreads;
        if (t < p.tiles) p.order[atomicAdd(&s_count[kept[j]], 1u)] = (uint32_t)t;
    }
    for (int t = threadIdx.x + kKept * kThreads; t < p.tiles; t += kThreads)
        p.order[atomicAdd(&s_count[order_bucket(order_weight(p, t))], 1u)] = (uint32_t)t;
}
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
constexpr int kFixStride = 9;               // queue entry: Gaussian index, five moments, colour part of dL/dmean
constexpr float kChainKappa = 8.0f;         // a c / det above which the chain runs in binary64

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
    // Gaussians whose 2D covariance has a c / det above kChainKappa, queued by the binary32
    // chain rule for the binary64 geometric pass: wave w (Gaussians 64w .. 64w + 63) puts its
    // queued ones in fix_list[64w ..] ([n][kFixStride]: index, the five moments, the colour
    // part of dL/dmean) and their number in fix_count[w] ([ceil(n / 64)])
    float *fix_list;
    uint32_t *fix_count;
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
