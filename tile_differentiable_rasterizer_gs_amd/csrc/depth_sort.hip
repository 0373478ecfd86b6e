// Depth order of the Gaussians by buckets of depth (depth-first mode).
//
// Flowchart of the lesson "3D Gaussian Splatting from scratch", step "Depth-sort per
// tile": compositing needs every tile's Gaussians front to back.  The depth-first path
// orders all Gaussians once by (camera-space depth, index); the per-tile lists built in
// that order inherit it.  Here that order comes from one distribution pass and one sort in
// LDS per bucket, instead of four 8-bit radix passes of three kernels each:
//   bounds   the preprocess leaves the smallest and largest depth bits of the Gaussians
//            with pairs in kDepthSlots (min, max) slots, one atomic pair per wave
//   count    G groups, each a contiguous range of Gaussians, count how many fall into
//            each of B buckets: floor((z - zmin) * B / (zmax - zmin)), clamped to
//            [0, B - 1].  binary32 subtraction and product round monotonically, so the
//            bucket never decreases with the depth whatever the bounds (they only set the
//            balance).  Gaussians without pairs form bucket B.
//   column   per bucket: exclusive prefix of the group counts, and the bucket total.  From
//            kGroupMajorGroups groups on the table is group-major, so that count writes and
//            scatter reads a group's row whole, and a column workgroup takes 64 buckets, its
//            waves a quarter of the groups each, 64 neighbouring counts per row; with fewer
//            groups it is bucket-major, a workgroup per bucket (its fixed cost is lower)
//   scatter  each group puts its Gaussians at running per-bucket cursors in LDS: an entry
//            (bits(depth) << 32 | index) into the bucket's range, a Gaussian without
//            pairs straight into the output tail (their relative order is immaterial:
//            they have no pairs, and their gathered count is 0)
//   sort     one workgroup per bucket of at most kRankCap entries: a counting sort in LDS
//            into one sub-bin per thread (the fractional part of the same bucket
//            coordinate, monotone too), then each entry ranked among the few entries of its
//            sub-bin; it writes rank -> Gaussian and the gathered per-Gaussian count.
//            Larger buckets go to a list for
//   larger   per listed bucket (up to kBucketCap entries): the same with a 1024-thread
//            workgroup and 1024 sub-bins.  This kernel is launched only while the frames
//            before met such buckets (flag word 1); a frame that meets one without it is
//            redone like a frame with a bucket too large (below), and the next frame
//            launches it again
// Entries compare as 64-bit integers, i.e. by depth then index: the order the stable
// radix sort of the depth bits gives.  A bucket of more than kBucketCap entries (depths
// crowded into a sliver of the range) is written unsorted and raises a flag; the host
// reads it with the pair count and orders the frame with the radix sort instead.
#include <cfloat>

#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kGroupThreads = 1024;  // count and scatter workgroups
constexpr int kGroupBatch = 4;       // 16-byte key loads per thread in flight
constexpr int kXcds = 8;             // workgroups go round-robin to the eight XCDs
constexpr int kRankThreads = kBlock; // workgroups of the per-bucket kernel
constexpr int kRankCap = 8 * kRankThreads;   // largest bucket the per-bucket kernel sorts
constexpr int kBigThreads = 1024;    // workgroups of the larger-bucket kernel
constexpr int kGroupMajorGroups = 64;   // groups from which the count table is group-major
constexpr int64_t kSingleGroupKeys = 16384;   // up to this many Gaussians: one group, one launch
constexpr int kSubbinGroups = 128;   // workgroups that share the list of larger buckets (usually none)

struct Bounds {
    float zlo, scale;   // scale 0: every Gaussian with pairs in bucket 0
    int buckets;
};

__device__ inline uint32_t bucket_of(uint32_t key, const Bounds &b) {
#pragma clang fp contract(off)
    if (key == kNoPairsKey) return (uint32_t)b.buckets;
    if (b.scale == 0.0f) return 0u;
    const float t = (__uint_as_float(key) - b.zlo) * b.scale;
    if (!(t > 0.0f)) return 0u;
    return t < (float)b.buckets ? (uint32_t)t : (uint32_t)b.buckets - 1u;
}

// The frame's depth bounds from the slots (whole workgroup; a barrier inside).
__device__ inline Bounds load_bounds(const uint32_t *range, int buckets, uint32_t *s_lo, uint32_t *s_hi) {
    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    uint32_t lo = 0xffffffffu, hi = 0u;
    if (t < kDepthSlots) {
        lo = range[t];
        hi = range[kDepthSlots + t];
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
    }
    if (lane == 0 && w < kDepthSlots / kWave) {
        s_lo[w] = lo;
        s_hi[w] = hi;
    }
    __syncthreads();
    lo = s_lo[0];
    hi = s_hi[0];
#pragma unroll
    for (int i = 1; i < kDepthSlots / kWave; ++i) {
        lo = min(lo, s_lo[i]);
        hi = max(hi, s_hi[i]);
    }
    Bounds b;
    b.buckets = buckets;
    b.zlo = 0.0f;
    b.scale = 0.0f;
    if (lo < hi) {   // two distinct finite positive depths
        b.zlo = __uint_as_float(lo);
        const float span = __uint_as_float(hi) - b.zlo;
        const float sc = (float)buckets / span;
        if (span > 0.0f && sc <= FLT_MAX) b.scale = sc;
    }
    return b;
}

// Exclusive prefix over the workgroup of one value per thread (kThreads threads); *total
// gets the sum.  Barriers inside.
template <int kThreads>
__device__ inline uint32_t block_scan(uint32_t x, uint32_t *s_tmp /*[kThreads / kWave]*/, uint32_t *total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t inc = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)inc, d);
        if (lane >= d) inc += y;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        const uint32_t v = s_tmp[w];
        if (w < wave) before += v;
        all += v;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

// Group of this workgroup (XCD x takes the x-th contiguous block of groups, so that the runs
// consecutive groups write into one bucket meet in one L2) and its range of Gaussians
// (a multiple of 4 long, for 16-byte loads).  Returns false for a padding workgroup.
__device__ inline bool group_range(const DepthBucketParams &p, int *grp, int64_t *lo, int64_t *hi) {
    const int per_xcd = gridDim.x / kXcds;   // the grid is a multiple of kXcds
    *grp = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (*grp >= p.groups) return false;
    const int64_t chunk = ((p.n + p.groups - 1) / p.groups + 3) & ~(int64_t)3;
    *lo = min<int64_t>(p.n, (int64_t)*grp * chunk);
    *hi = min<int64_t>(p.n, *lo + chunk);
    return true;
}

// Visits every Gaussian of [lo, hi) once: f(index, key, rectangle), kGroupBatch 16-byte loads
// of four keys per thread issued together, and with kRect their four rectangles as two more
// 16-byte loads each (else the rectangle passed is empty).  pre() runs once in every thread
// after the first batch's loads are issued and before any f: the caller's set-up (bounds,
// cursors, barriers) overlaps those loads.
template <bool kRect = false, typename Pre, typename F>
__device__ inline void for_each_key(const uint32_t *keys, const uint2 *rect, int64_t lo, int64_t hi, Pre pre, F f) {
    const int64_t vlo = lo / 4, vhi = hi / 4;   // lo is a multiple of 4
    const uint4 *kv = reinterpret_cast<const uint4 *>(keys);
    const uint4 *rv = reinterpret_cast<const uint4 *>(rect);
    uint4 k[kGroupBatch], r[kGroupBatch][2];
    auto load = [&](int64_t j0) {
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const int64_t j = j0 + (int64_t)u * kGroupThreads;
            const int64_t jj = j < vhi ? j : j0;
            k[u] = kv[jj];
            if constexpr (kRect) {
                r[u][0] = rv[2 * jj];
                r[u][1] = rv[2 * jj + 1];
            } else {
                r[u][0] = r[u][1] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    int64_t j0 = vlo + threadIdx.x;
    if (j0 < vhi) load(j0);
    pre();
    for (bool first = true; j0 < vhi; j0 += (int64_t)kGroupThreads * kGroupBatch, first = false) {
        if (!first) load(j0);
#pragma unroll
        for (int u = 0; u < kGroupBatch; ++u) {
            const int64_t j = j0 + (int64_t)u * kGroupThreads;
            if (j < vhi) {
                f(4 * j, k[u].x, make_uint2(r[u][0].x, r[u][0].y));
                f(4 * j + 1, k[u].y, make_uint2(r[u][0].z, r[u][0].w));
                f(4 * j + 2, k[u].z, make_uint2(r[u][1].x, r[u][1].y));
                f(4 * j + 3, k[u].w, make_uint2(r[u][1].z, r[u][1].w));
            }
        }
    }
    for (int64_t i = max(lo, 4 * vhi) + threadIdx.x; i < hi; i += kGroupThreads)
        f(i, keys[i], kRect ? rect[i] : make_uint2(0u, 0u));
}

// The entries as 16-byte records (index, depth bits, rectangle) when p.rect is given.
__device__ inline uint4 *entries16(const DepthBucketParams &p) { return reinterpret_cast<uint4 *>(p.entries); }

// Where the count of (group, bucket b) lives in the table.
__device__ inline int64_t count_at(const DepthBucketParams &p, int nb, int grp, int b) {
    return p.groups >= kGroupMajorGroups ? (int64_t)grp * nb + b : (int64_t)b * p.groups + grp;
}

// count_at(group, b) = Gaussians of the group in bucket b (b = 0 .. B).  Group 0 also
// clears the overflow flag and the list of larger buckets.
__global__ __launch_bounds__(kGroupThreads) void bucket_count_kernel(DepthBucketParams p) {
    extern __shared__ uint32_t s_hist[];   // [B + 1]
    __shared__ uint32_t s_lo[kDepthSlots / kWave], s_hi[kDepthSlots / kWave];
    int grp;
    int64_t lo, hi;
    if (!group_range(p, &grp, &lo, &hi)) return;   // whole workgroup
    const int nb = (1 << p.bucket_bits) + 1;
    Bounds bd;
    for_each_key(
        p.keys, nullptr, lo, hi,
        [&]() {
            for (int i = threadIdx.x; i < nb; i += kGroupThreads) s_hist[i] = 0u;
            bd = load_bounds(p.range, 1 << p.bucket_bits, s_lo, s_hi);   // barrier inside
            if (grp == 0 && threadIdx.x == 0) {
                *p.flag = 0ull;
                *p.big_count = 0u;
            }
        },
        [&](int64_t, uint32_t key, uint2) { atomicAdd(&s_hist[bucket_of(key, bd)], 1u); });
    __syncthreads();
    for (int b = threadIdx.x; b < nb; b += kGroupThreads) p.counts[count_at(p, nb, grp, b)] = s_hist[b];
}

// Buckets [64 w, 64 w + 64) for workgroup w: each count becomes the exclusive prefix over the
// groups before it (in its bucket), and totals[b] the bucket's sum.  Lane l of each wave takes
// bucket 64 w + l; wave k takes the k-th sixteenth of the groups (at most 16, as G <= 256),
// whose counts it loads together, then stores their prefix plus the sums of the parts before.
constexpr int kColumnBuckets = kWave;
constexpr int kColumnThreads = 1024;
__global__ __launch_bounds__(kColumnThreads) void bucket_column_kernel(DepthBucketParams p) {
    constexpr int kQuarters = kColumnThreads / kWave;   // parts of the groups, one per wave
    constexpr int kPer = kBlock / kQuarters;             // groups per part at most (G <= kBlock)
    __shared__ uint32_t s_sum[kQuarters][kColumnBuckets];
    const int nb = (1 << p.bucket_bits) + 1;
    const int lane = threadIdx.x & (kWave - 1), q = threadIdx.x / kWave;
    const int b = blockIdx.x * kColumnBuckets + lane;
    const int g0 = p.groups * q / kQuarters, g1 = p.groups * (q + 1) / kQuarters;
    uint32_t *col = p.counts + b;
    uint32_t c[kPer];
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        c[k] = (b < nb && g0 + k < g1) ? col[(int64_t)(g0 + k) * nb] : 0u;
        sum += c[k];
    }
    s_sum[q][lane] = sum;
    __syncthreads();
    uint32_t run = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kQuarters; ++k) {
        const uint32_t v = s_sum[k][lane];
        run += k < q ? v : 0u;
        all += v;
    }
    if (b < nb) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            if (g0 + k < g1) col[(int64_t)(g0 + k) * nb] = run;
            run += c[k];
        }
        if (q == 0) p.totals[b] = all;
    }
}

static_assert(kColumnBuckets == kWave && kBlock % (kColumnThreads / kWave) == 0, "column kernel shapes");

// Bucket-major table (fewer than kGroupMajorGroups groups): one workgroup per bucket b (0 .. B),
// counts[b][*] -> exclusive prefix over groups; totals[b].
__global__ __launch_bounds__(kBlock) void bucket_column_small_kernel(DepthBucketParams p) {
    __shared__ uint32_t s_tmp[kBlock / kWave];
    uint32_t *row = p.counts + (int64_t)blockIdx.x * p.groups;
    const uint32_t v = (int)threadIdx.x < p.groups ? row[threadIdx.x] : 0u;   // groups <= kBlock
    uint32_t total;
    const uint32_t before = block_scan<kBlock>(v, s_tmp, &total);
    if ((int)threadIdx.x < p.groups) row[threadIdx.x] = before;
    if (threadIdx.x == 0) p.totals[blockIdx.x] = total;
}

// Each group places its Gaussians: bucket starts (exclusive prefix of the totals; group 0
// also stores them for the sort kernels) plus the group's prefix give the cursors.
template <bool kRect>
__global__ __launch_bounds__(kGroupThreads) void bucket_scatter_kernel(DepthBucketParams p) {
    extern __shared__ uint32_t s_cur[];   // [B + 1]
    __shared__ uint32_t s_lo[kDepthSlots / kWave], s_hi[kDepthSlots / kWave];
    __shared__ uint32_t s_tmp[kGroupThreads / kWave];
    int grp;
    int64_t lo, hi;
    if (!group_range(p, &grp, &lo, &hi)) return;   // whole workgroup
    const int nb = (1 << p.bucket_bits) + 1;
    Bounds bd;
    auto setup = [&]() {
        bd = load_bounds(p.range, 1 << p.bucket_bits, s_lo, s_hi);
        // thread t: buckets [b0, b1)
        const int per = (nb + kGroupThreads - 1) / kGroupThreads;
        const int b0 = min(nb, (int)threadIdx.x * per), b1 = min(nb, b0 + per);
        uint32_t sum = 0;
        for (int b = b0; b < b1; ++b) sum += p.totals[b];
        uint32_t all;
        uint32_t run = block_scan<kGroupThreads>(sum, s_tmp, &all);
        for (int b = b0; b < b1; ++b) {
            s_cur[b] = run + p.counts[count_at(p, nb, grp, b)];
            if (grp == 0) p.starts[b] = run;
            run += p.totals[b];
        }
        if (grp == 0 && threadIdx.x == 0) {
            p.starts[nb] = all;
            p.bounds[0] = bd.zlo;   // for the sub-bins of larger buckets
            p.bounds[1] = bd.scale;
        }
        __syncthreads();
    };
    for_each_key<kRect>(p.keys, p.rect, lo, hi, setup, [&](int64_t i, uint32_t key, uint2 rc) {
        const uint32_t b = bucket_of(key, bd);
        const uint32_t pos = atomicAdd(&s_cur[b], 1u);
        if ((int)b < nb - 1) {
            if constexpr (kRect) {   // the rectangle rides with the entry (read here in index order)
                entries16(p)[pos] = make_uint4((uint32_t)i, key, rc.x, rc.y);
            } else {
                p.entries[pos] = ((uint64_t)key << 32) | (uint32_t)i;
            }
        } else {
            p.order[pos] = (uint32_t)i;
            p.gathered[pos] = 0u;
            if (p.rect_out) p.rect_out[pos] = make_uint2(0u, 0u);
        }
    });
}

// At most kSingleGroupKeys Gaussians (one group): count, bucket starts and scatter in one
// workgroup and one launch instead of three (the count table is not needed).
template <bool kRect>
__global__ __launch_bounds__(kGroupThreads) void bucket_single_kernel(DepthBucketParams p) {
    extern __shared__ uint32_t s_cur[];   // [B + 1]: counts, then cursors
    __shared__ uint32_t s_lo[kDepthSlots / kWave], s_hi[kDepthSlots / kWave];
    __shared__ uint32_t s_tmp[kGroupThreads / kWave];
    const int nb = (1 << p.bucket_bits) + 1;
    Bounds bd;
    for_each_key(
        p.keys, nullptr, 0, p.n,
        [&]() {
            for (int i = threadIdx.x; i < nb; i += kGroupThreads) s_cur[i] = 0u;
            bd = load_bounds(p.range, 1 << p.bucket_bits, s_lo, s_hi);   // barrier inside
            if (threadIdx.x == 0) {
                *p.flag = 0ull;
                *p.big_count = 0u;
                p.bounds[0] = bd.zlo;   // for the sub-bins
                p.bounds[1] = bd.scale;
            }
        },
        [&](int64_t, uint32_t key, uint2) { atomicAdd(&s_cur[bucket_of(key, bd)], 1u); });
    __syncthreads();
    // thread t: buckets [b0, b1); their counts become the bucket starts (while the second
    // pass's first loads are in flight)
    auto starts = [&]() {
        const int per = (nb + kGroupThreads - 1) / kGroupThreads;
        const int b0 = min(nb, (int)threadIdx.x * per), b1 = min(nb, b0 + per);
        uint32_t sum = 0;
        for (int b = b0; b < b1; ++b) sum += s_cur[b];
        uint32_t all;
        uint32_t run = block_scan<kGroupThreads>(sum, s_tmp, &all);   // barriers inside
        for (int b = b0; b < b1; ++b) {
            const uint32_t c = s_cur[b];
            s_cur[b] = run;
            p.starts[b] = run;
            run += c;
        }
        if (threadIdx.x == 0) p.starts[nb] = all;
        __syncthreads();
    };
    for_each_key<kRect>(p.keys, p.rect, 0, p.n, starts, [&](int64_t i, uint32_t key, uint2 rc) {
        const uint32_t b = bucket_of(key, bd);
        const uint32_t pos = atomicAdd(&s_cur[b], 1u);
        if ((int)b < nb - 1) {
            if constexpr (kRect)
                entries16(p)[pos] = make_uint4((uint32_t)i, key, rc.x, rc.y);
            else
                p.entries[pos] = ((uint64_t)key << 32) | (uint32_t)i;
        } else {
            p.order[pos] = (uint32_t)i;
            p.gathered[pos] = 0u;
            if (p.rect_out) p.rect_out[pos] = make_uint2(0u, 0u);
        }
    });
}

// The frame's flag as two words (the host reads them as one 64-bit value): [0] the order must
// be redone by the radix sort, [1] a bucket too large for the per-bucket kernel was met.  Every
// writer stores 1, so concurrent plain stores agree.
__device__ inline uint32_t *flag_words(const DepthBucketParams &p) { return reinterpret_cast<uint32_t *>(p.flag); }

// What a sorted entry carries besides its Gaussian: the Gaussian's count, gathered right
// after the entry is read (so that a thread's reads are in flight together and overlap the
// sorting), or with kRect its rectangle, which the scatter stored in the entry itself (16
// bytes: index, depth bits, rectangle), from which the count follows (square rule) and which
// is written in rank order too (the pair listing then reads it coalesced instead of gathering
// it by Gaussian).
template <bool kRect>
struct Fetched {
    uint32_t cnt;
};
template <>
struct Fetched<true> {
    uint2 rc;
};
// Entry i of a bucket starting at `start` (i < size; else a padding entry 0, Gaussian 0's).
template <bool kRect>
__device__ inline uint64_t load_entry(const DepthBucketParams &p, uint32_t at, bool real, Fetched<kRect> &f) {
    if constexpr (kRect) {
        const uint4 q = real ? entries16(p)[at] : make_uint4(0u, 0u, 0u, 0u);
        f.rc = make_uint2(q.z, q.w);
        return ((uint64_t)q.y << 32) | q.x;
    } else {
        return real ? p.entries[at] : 0ull;
    }
}
template <bool kRect>
__device__ inline void fetch(const DepthBucketParams &p, uint64_t entry, Fetched<kRect> &f) {
    if constexpr (!kRect) f.cnt = p.gather_src[(uint32_t)entry];
}
// Writes a sorted entry: rank -> Gaussian, the Gaussian's count and (kRect) its rectangle.
template <bool kRect>
__device__ inline void emit(const DepthBucketParams &p, uint32_t at, uint64_t entry, const Fetched<kRect> &f) {
    p.order[at] = (uint32_t)entry;
    if constexpr (kRect) {
        const uint32_t area = ((f.rc.x >> 16) - (f.rc.x & 0xffffu)) * ((f.rc.y >> 16) - (f.rc.y & 0xffffu));
        p.gathered[at] = p.packed_counts ? pack_counts(area, f.rc) : area;
        p.rect_out[at] = f.rc;
    } else {
        p.gathered[at] = f.cnt;
    }
}

// Sub-bin of an entry of bucket b: the fractional part of the bucket coordinate
// t = (z - zmin) * scale (the same operations as bucket_of, so the same t) in kSub steps,
// clamped.  Monotone in the depth, like the bucket.
template <int kSub>
__device__ inline uint32_t sub_bin(uint64_t entry, uint32_t b, float zlo, float scale) {
#pragma clang fp contract(off)
    const float t = (__uint_as_float((uint32_t)(entry >> 32)) - zlo) * scale;
    const float f = (t - (float)b) * (float)kSub;
    if (!(f > 0.0f)) return 0u;
    return f < (float)kSub ? (uint32_t)f : (uint32_t)kSub - 1u;
}

// Sorts bucket b (`size` <= kE * kThreads entries from `start`) with the whole workgroup: a
// counting sort into kThreads sub-bins in LDS, then each entry ranked among the entries of
// its own sub-bin (about size / kThreads of them).  Barriers inside; the caller waits at a
// barrier before it reuses the LDS.
template <bool kRect, int kThreads, int kE>
__device__ inline void subbin_sort(const DepthBucketParams &p, uint32_t b, uint32_t start, uint32_t size,
                                   float zlo, float scale, uint64_t *s_ent, uint32_t *s_cnt, uint32_t *s_base,
                                   uint32_t *s_tmp) {
    uint64_t v[kE];
    uint32_t sub[kE], off[kE];
    Fetched<kRect> f[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const uint32_t i = threadIdx.x + e * kThreads;
        v[e] = load_entry<kRect>(p, start + i, i < size, f[e]);
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        fetch<kRect>(p, v[e], f[e]);   // a padding lane's entry is 0: Gaussian 0's, unused
        sub[e] = sub_bin<kThreads>(v[e], b, zlo, scale);
    }
    s_cnt[threadIdx.x] = 0u;   // one sub-bin per thread
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kE; ++e)
        if (threadIdx.x + e * kThreads < size) off[e] = atomicAdd(&s_cnt[sub[e]], 1u);
    __syncthreads();
    uint32_t total;
    const uint32_t c = s_cnt[threadIdx.x];
    s_base[threadIdx.x] = block_scan<kThreads>(c, s_tmp, &total);   // barriers inside
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kE; ++e)
        if (threadIdx.x + e * kThreads < size) s_ent[s_base[sub[e]] + off[e]] = v[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        if (threadIdx.x + e * kThreads < size) {
            const uint32_t lo = s_base[sub[e]], hi = lo + s_cnt[sub[e]];
            uint32_t r = 0;
            for (uint32_t q = lo; q < hi; ++q) r += (uint32_t)(s_ent[q] < v[e]);
            emit<kRect>(p, start + lo + r, v[e], f[e]);
        }
    }
}

// One workgroup per bucket of Gaussians with pairs: buckets of at most kRankCap entries are
// sorted here, larger ones listed for the larger-bucket kernel, and one of more than
// kBucketCap entries is written unsorted with the flag raised.  Workgroup 0 also empties the
// bound slots for the next preprocess (no later kernel reads them).
template <bool kRect>
__global__ __launch_bounds__(kRankThreads) void bucket_rank_kernel(DepthBucketParams p) {
    __shared__ uint64_t s_ent[kRankCap];
    __shared__ uint32_t s_cnt[kRankThreads], s_base[kRankThreads], s_tmp[kRankThreads / kWave];
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < kDepthSlots; i += kRankThreads) {
            p.range[i] = 0xffffffffu;
            p.range[kDepthSlots + i] = 0u;
        }
    }
    const uint32_t start = p.starts[blockIdx.x];
    const uint32_t size = p.starts[blockIdx.x + 1] - start;
    if (size == 0) return;
    if (size > (uint32_t)kRankCap) {
        if (threadIdx.x == 0) flag_words(p)[1] = 1u;   // a larger bucket was met
        if (size <= (uint32_t)kBucketCap && p.run_larger) {
            if (threadIdx.x == 0) p.big_list[atomicAdd(p.big_count, 1u)] = blockIdx.x;
            return;
        }
        // not sorted this frame (too large, or its kernel left out): the host redoes the
        // frame's order.  The entries are still written, unsorted, so that every rank names a
        // Gaussian with that Gaussian's own count for the kernels enqueued before the host
        // reads the flag (with stale ranks their listing walks would leave the rectangles).
        for (uint32_t i = threadIdx.x; i < size; i += kRankThreads) {
            Fetched<kRect> f;
            const uint64_t v = load_entry<kRect>(p, start + i, true, f);
            fetch<kRect>(p, v, f);
            emit<kRect>(p, start + i, v, f);
        }
        if (threadIdx.x == 0) flag_words(p)[0] = 1u;   // redo the frame's order
        return;
    }
    const float zlo = p.bounds[0], scale = p.bounds[1];
    if (size <= (uint32_t)kRankThreads)
        subbin_sort<kRect, kRankThreads, 1>(p, blockIdx.x, start, size, zlo, scale, s_ent, s_cnt, s_base, s_tmp);
    else if (size <= 2u * kRankThreads)
        subbin_sort<kRect, kRankThreads, 2>(p, blockIdx.x, start, size, zlo, scale, s_ent, s_cnt, s_base, s_tmp);
    else if (size <= 4u * kRankThreads)
        subbin_sort<kRect, kRankThreads, 4>(p, blockIdx.x, start, size, zlo, scale, s_ent, s_cnt, s_base, s_tmp);
    else
        subbin_sort<kRect, kRankThreads, 8>(p, blockIdx.x, start, size, zlo, scale, s_ent, s_cnt, s_base, s_tmp);
}

// The listed buckets (kRankCap < size <= kBucketCap), shared round-robin by the workgroups.
template <bool kRect>
__global__ __launch_bounds__(kBigThreads) void bucket_subbin_kernel(DepthBucketParams p) {
    __shared__ uint64_t s_ent[kBucketCap];
    __shared__ uint32_t s_cnt[kBigThreads], s_base[kBigThreads], s_tmp[kBigThreads / kWave];
    const uint32_t count = *p.big_count;
    const float zlo = p.bounds[0], scale = p.bounds[1];
    for (uint32_t li = blockIdx.x; li < count; li += gridDim.x) {
        const uint32_t b = p.big_list[li];
        const uint32_t start = p.starts[b];
        subbin_sort<kRect, kBigThreads, kBucketCap / kBigThreads>(p, b, start, p.starts[b + 1] - start, zlo, scale, s_ent,
                                                           s_cnt, s_base, s_tmp);
        __syncthreads();   // the next bucket reuses the LDS
    }
}

__global__ void fill_range_kernel(uint32_t *range) {
    for (int i = threadIdx.x; i < kDepthSlots; i += blockDim.x) {
        range[i] = 0xffffffffu;
        range[kDepthSlots + i] = 0u;
    }
}

}  // namespace

static_assert(kBucketCap % kBigThreads == 0 && kBucketCap >= kRankCap, "larger-bucket kernel shapes");
static_assert(kRankCap == 8 * kRankThreads, "per-bucket kernel shapes");

int depth_bucket_bits(int64_t n) {
    int bits = kMinBucketBits;
    while (bits < kMaxBucketBits && ((int64_t)1 << bits) * kBucketTarget < n) ++bits;
    return bits;
}

int depth_bucket_groups(int64_t n) {
    if (n <= kSingleGroupKeys) return 1;   // one workgroup does count, starts and scatter
    const int64_t buckets = ((int64_t)1 << depth_bucket_bits(n)) + 1;
    int64_t g = (n + kGroupKeys - 1) / kGroupKeys;
    const int64_t cap = kMaxCountWords / buckets;
    g = g < cap ? g : cap;
    g = g < kBlock ? g : kBlock;
    return (int)(g < 1 ? 1 : g);
}

int64_t depth_bucket_scratch_words(int64_t n) {
    const int64_t B = (int64_t)1 << depth_bucket_bits(n), nb = B + 1;
    // flag (u64), larger-bucket count (+ pad), bounds (2 floats), counts, totals, starts,
    // larger-bucket list
    return 2 + 2 + 2 + nb * depth_bucket_groups(n) + nb + (nb + 1) + B;
}

void depth_bucket_layout(uint32_t *scratch, int64_t n, DepthBucketParams &p) {
    p.n = n;
    p.bucket_bits = depth_bucket_bits(n);
    p.groups = depth_bucket_groups(n);
    const int64_t B = (int64_t)1 << p.bucket_bits, nb = B + 1;
    p.flag = reinterpret_cast<unsigned long long *>(scratch);   // scratch is 8-byte aligned
    p.big_count = scratch + 2;
    p.bounds = reinterpret_cast<float *>(scratch + 4);
    p.counts = scratch + 6;
    p.totals = p.counts + nb * p.groups;
    p.starts = p.totals + nb;
    p.big_list = p.starts + nb + 1;
}

void launch_depth_range_fill(uint32_t *range, hipStream_t s) { fill_range_kernel<<<1, kBlock, 0, s>>>(range); }

void launch_depth_bucket_sort(const DepthBucketParams &p, hipStream_t s) {
    if (p.n <= 0) return;
    const int buckets = 1 << p.bucket_bits;
    const unsigned grid = (unsigned)((p.groups + kXcds - 1) / kXcds * kXcds);
    const size_t lds = (size_t)(buckets + 1) * sizeof(uint32_t);
    if (p.groups == 1) {
        if (p.rect)
            bucket_single_kernel<true><<<1, kGroupThreads, lds, s>>>(p);
        else
            bucket_single_kernel<false><<<1, kGroupThreads, lds, s>>>(p);
    } else {
    bucket_count_kernel<<<grid, kGroupThreads, lds, s>>>(p);
    if (p.groups >= kGroupMajorGroups)
        bucket_column_kernel<<<(buckets + 1 + kColumnBuckets - 1) / kColumnBuckets, kColumnThreads, 0, s>>>(p);
    else
        bucket_column_small_kernel<<<buckets + 1, kBlock, 0, s>>>(p);
    if (p.rect)
        bucket_scatter_kernel<true><<<grid, kGroupThreads, lds, s>>>(p);
    else
        bucket_scatter_kernel<false><<<grid, kGroupThreads, lds, s>>>(p);
    }
    const unsigned larger = buckets < kSubbinGroups ? buckets : kSubbinGroups;
    if (p.rect) {
        bucket_rank_kernel<true><<<buckets, kRankThreads, 0, s>>>(p);
        if (p.run_larger) bucket_subbin_kernel<true><<<larger, kBigThreads, 0, s>>>(p);
    } else {
        bucket_rank_kernel<false><<<buckets, kRankThreads, 0, s>>>(p);
        if (p.run_larger) bucket_subbin_kernel<false><<<larger, kBigThreads, 0, s>>>(p);
    }
}

}  // namespace gsr
