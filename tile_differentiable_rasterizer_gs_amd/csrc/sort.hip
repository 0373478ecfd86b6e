// Pair listing, stable LSD radix sort and tile ranges.
//
// Flowchart of the lesson "3D Gaussian Splatting from scratch", steps "Assign to
// tiles (16x16 screen-space)" and "Depth-sort per tile": every (Gaussian, tile)
// pair is listed and the list is ordered by (tile, camera-space depth), equal
// depths by Gaussian index.  In the 64-bit mode the key of a pair is
// (tile_id << 32) | bits(depth); for depth > 0 the IEEE bit pattern orders like the
// value.  In the default mode the Gaussians are sorted by depth first, the pairs are
// listed in that order, and a stable sort on the tile id alone finishes the order.
//
// Radix sort: digits of at most 8 bits, least significant first (32-bit depth keys in
// 4 x 8, 13 tile bits in 7 + 6), three kernels per digit on a fixed grid of G
// workgroups, each owning one contiguous range of the input:
//   count   per-range digit counts, counts[d][range]
//   scan    one workgroup per digit: exclusive prefix over ranges, plus the digit total
//   scatter each range walks its tiles of 4096 pairs (1024 for inputs up to 4 M) in
//           order; a tile ranks its keys stably in LDS (a ballot per key bit finds the
//           lanes of a wave that share a digit) and writes them through LDS in
//           contiguous digit runs at running per-digit offsets.
// Ranges and tiles are processed in input order, so equal digits keep their
// order.  No workgroup waits on another (communication only across kernel
// boundaries): on MI355X the L2s of the eight XCDs are not coherent with each
// other, so polling another workgroup's results costs a fabric round trip.
// HBM traffic per pass and pair: read the key (count), read key+value and write
// key+value (scatter).
#include <type_traits>

#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kRadix = 1 << kRadixBits;
constexpr int kMaxSortGroups = 1024;             // workgroups per pass (4 per CU)
// pairs per thread and tile: 16 (4096-pair tiles) for long inputs, 4 (1024) for short
// ones so that enough workgroups exist to fill the GPU
constexpr int kItemsLarge = 16, kItemsSmall = 4;
constexpr int64_t kSmallSort = 1 << 22;

template <typename K>
__device__ inline uint32_t digit_of(K key, int shift, uint32_t mask) {
    return (uint32_t)(key >> shift) & mask;
}

__device__ inline uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroup exclusive scan over threadIdx.x of one uint32 per thread.
__device__ inline uint32_t block_exclusive_scan_u32(uint32_t x, uint32_t *s_tmp /*[4]*/) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t inc = x;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += y;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w)
        if (w < wave) before += s_tmp[w];
    __syncthreads();
    return before + inc - x;
}

// Range of the input owned by workgroup `group` (whole tiles of `tile` pairs).
__device__ inline void group_range(int64_t n, int64_t tile, int groups, int group, int64_t *lo, int64_t *hi) {
    const int64_t tiles = (n + tile - 1) / tile;
    const int64_t per = (tiles + groups - 1) / groups;
    *lo = min<int64_t>(n, (int64_t)group * per * tile);
    *hi = min<int64_t>(n, (int64_t)(group + 1) * per * tile);
}

// Lanes of this wave whose digit equals d (one ballot per digit bit); only lanes with
// `valid` take part.  kBits > 0: the digit width is a compile-time constant (unrolled).
template <int kBits>
__device__ inline uint64_t match_digit(uint32_t d, int bits, bool valid) {
    const uint64_t v = __ballot(valid);
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const int nb = kBits > 0 ? kBits : bits;
#pragma unroll
    for (int b = 0; b < (kBits > 0 ? kBits : 8); ++b) {
        if (kBits == 0 && b >= nb) break;
        const uint32_t neg = 0u - ((d >> b) & 1u);   // all ones where this lane's bit is set
        const uint64_t on = __ballot(neg != 0u);
        // keep the lanes whose bit equals this lane's: ~(on ^ neg), one 32-bit half at a time
        lo &= ~((uint32_t)on ^ neg);
        hi &= ~((uint32_t)(on >> 32) ^ neg);
    }
    return ((uint64_t)hi << 32) | lo;
}

// Element count of a pass: the host bound, or min(bound, *n_dev) when the count lives on the device.
__device__ inline int64_t live_count(int64_t n_cap, const unsigned long long *n_dev) {
    return n_dev ? min<int64_t>(n_cap, (int64_t)*n_dev) : n_cap;
}

// Digit counts of one range.  LDS atomics go to one of kCopies histograms per wave
// (chosen by lane), which keeps lanes that share a digit from serialising on one word.
template <typename K, int ITEMS>
__global__ __launch_bounds__(kBlock) void radix_count_kernel(const K *keys, int64_t n_cap,
                                                             const unsigned long long *n_dev, int shift, int bits,
                                                             uint32_t *counts /*[radix][groups]*/) {
    const int64_t n = live_count(n_cap, n_dev);
    constexpr int kCopies = 4 * (kBlock / kWave);
    constexpr int kStride = kRadix + 1;   // odd stride: copies of one digit sit in different banks
    __shared__ uint32_t s_count[kCopies * kStride];
    const uint32_t mask = (1u << bits) - 1;
    const int copy = (threadIdx.x / kWave) * 4 + (threadIdx.x & 3);
    for (int i = threadIdx.x; i < kCopies * kStride; i += kBlock) s_count[i] = 0;
    __syncthreads();
    int64_t lo, hi;
    group_range(n, (int64_t)kBlock * ITEMS, gridDim.x, blockIdx.x, &lo, &hi);
    // 16-byte loads of kV keys (lo is a multiple of the sort tile, so they are aligned), then the tail
    constexpr int kV = 16 / (int)sizeof(K);
    const int64_t nvec = (hi - lo) / kV;
    const uint4 *kvec = reinterpret_cast<const uint4 *>(keys + lo);
#pragma unroll 2
    for (int64_t j = threadIdx.x; j < nvec; j += kBlock) {
        const uint4 w = kvec[j];
        K k[kV];
        __builtin_memcpy(k, &w, sizeof w);
#pragma unroll
        for (int u = 0; u < kV; ++u) atomicAdd(&s_count[copy * kStride + digit_of(k[u], shift, mask)], 1u);
    }
    for (int64_t i = lo + nvec * kV + threadIdx.x; i < hi; i += kBlock)
        atomicAdd(&s_count[copy * kStride + digit_of(keys[i], shift, mask)], 1u);
    __syncthreads();
    if ((int)threadIdx.x <= (int)mask) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kCopies; ++w) c += s_count[w * kStride + threadIdx.x];
        counts[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = c;
    }
}

// One workgroup per digit d: counts[d][*] -> exclusive prefix over ranges; totals[d].
__global__ __launch_bounds__(kBlock) void radix_digit_scan_kernel(uint32_t *counts, int groups, uint32_t *totals) {
    __shared__ uint32_t s_tmp[kBlock / kWave];
    uint32_t *row = counts + (int64_t)blockIdx.x * groups;
    constexpr int kPer = kMaxSortGroups / kBlock;   // groups <= kMaxSortGroups
    static_assert(kPer == 4, "one 16-byte access per thread");
    // a thread's four counts as one 16-byte load and store when the row allows it (per-value
    // accesses would each spread over the wave's 1 KB span)
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0 && (int)threadIdx.x * kPer + kPer <= groups;
    uint32_t v[kPer];
    uint32_t sum = 0;
    if (vec) {
        const uint4 q = reinterpret_cast<const uint4 *>(row)[threadIdx.x];
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int g = threadIdx.x * kPer + k;
            v[k] = g < groups ? row[g] : 0u;
        }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) sum += v[k];
    uint32_t run = block_exclusive_scan_u32(sum, s_tmp);
    uint32_t out[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        out[k] = run;
        run += v[k];
    }
    if (vec) {
        reinterpret_cast<uint4 *>(row)[threadIdx.x] = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int g = threadIdx.x * kPer + k;
            if (g < groups) row[g] = out[k];
        }
    }
    if (threadIdx.x == kBlock - 1) totals[blockIdx.x] = run;
}

// gathered_out (optional): gathered_out[dst] = gather_src[value] for every moved pair.
// kBits > 0: the pass's digit width as a compile-time constant (else `bits`).
template <typename K, int ITEMS, int kBits>
__global__ __launch_bounds__(kBlock) void radix_scatter_kernel(const K *keys_in, const uint32_t *vals_in,
                                                               K *keys_out, uint32_t *vals_out, int64_t n_cap,
                                                               const unsigned long long *n_dev, int shift,
                                                               int bits, const uint32_t *counts,
                                                               const uint32_t *totals, const uint32_t *gather_src,
                                                               uint32_t *gathered_out) {
    const int64_t n = live_count(n_cap, n_dev);
    constexpr int kWaves = kBlock / kWave;
    constexpr int kSortItems = ITEMS;
    constexpr int kSortTile = kBlock * ITEMS;
    // keys narrower than 64 bits travel with their value as one 8-byte LDS entry
    constexpr bool kPacked = sizeof(K) <= 4;
    using Entry = typename std::conditional<kPacked, uint2, uint32_t>::type;
    __shared__ Entry s_pack[kPacked ? kSortTile : 1];
    __shared__ K s_keys[kPacked ? 1 : kSortTile];
    __shared__ uint32_t s_vals[kPacked ? 1 : kSortTile];
    __shared__ uint32_t s_wave_count[kWaves][kRadix];   // per-wave running counts, then wave prefixes
    __shared__ uint32_t s_next[kRadix];                 // next global position of each digit (this range)
    __shared__ uint32_t s_dst[kRadix];                  // s_next - the digit's start in the tile (>= 0)
    __shared__ uint32_t s_tmp[kWaves];

    const int radix = 1 << bits;
    const uint32_t mask = radix - 1;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    {
        // global start of (digit, range) = exclusive prefix of digit totals + prefix over ranges
        const uint32_t tot = (int)threadIdx.x < radix ? totals[threadIdx.x] : 0u;
        const uint32_t base = block_exclusive_scan_u32(tot, s_tmp);
        if ((int)threadIdx.x < radix) s_next[threadIdx.x] = base + counts[(int64_t)threadIdx.x * gridDim.x + blockIdx.x];
    }
    int64_t lo, hi;
    group_range(n, kSortTile, gridDim.x, blockIdx.x, &lo, &hi);
    for (int64_t tile = lo; tile < hi; tile += kSortTile) {
        for (int i = threadIdx.x; i < kWaves * kRadix; i += kBlock) (&s_wave_count[0][0])[i] = 0;
        __syncthreads();
        // wave w owns the contiguous segment [w*1024, (w+1)*1024) of the tile, in rounds of 64
        const int64_t seg = tile + (int64_t)wave * (kSortItems * kWave);
        K key[kSortItems];
        uint32_t val[kSortItems];
#pragma unroll
        for (int r = 0; r < kSortItems; ++r) {   // past the range: a repeat of the last pair, not ranked
            const int64_t i = min<int64_t>(seg + r * kWave + lane, hi - 1);
            key[r] = keys_in[i];
            val[r] = vals_in[i];
        }
        uint32_t rank[kSortItems];
#pragma unroll
        for (int r = 0; r < kSortItems; ++r) {
            const bool valid = seg + r * kWave + lane < hi;
            const uint32_t d = digit_of(key[r], shift, mask);
            const uint64_t peers = match_digit<kBits>(d, bits, valid);
            const uint32_t below = lanes_below(peers);
            const uint32_t prev = valid ? s_wave_count[wave][d] : 0u;
            rank[r] = prev + below;
            // every lane of a digit group writes the same new count
            if (valid) s_wave_count[wave][d] = prev + (uint32_t)__popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();
        // thread = digit: the tile's count of that digit, then each wave's first slot for it
        // (the digit's start in the tile plus the counts of the waves before)
        uint32_t tile_count = 0, before[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before[w] = tile_count;
            tile_count += s_wave_count[w][threadIdx.x];
        }
        const uint32_t local_start = block_exclusive_scan_u32(tile_count, s_tmp);   // barriers inside
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s_wave_count[w][threadIdx.x] = local_start + before[w];
        s_dst[threadIdx.x] = s_next[threadIdx.x] - local_start;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kSortItems; ++r) {
            if (seg + r * kWave + lane < hi) {
                const uint32_t d = digit_of(key[r], shift, mask);
                const uint32_t pos = s_wave_count[wave][d] + rank[r];
                if constexpr (kPacked) {
                    s_pack[pos] = make_uint2((uint32_t)key[r], val[r]);
                } else {
                    s_keys[pos] = key[r];
                    s_vals[pos] = val[r];
                }
            }
        }
        __syncthreads();
        const int count = (int)min<int64_t>(kSortTile, hi - tile);
        for (int q = threadIdx.x; q < count; q += kBlock) {
            K k;
            uint32_t v;
            if constexpr (kPacked) {
                const uint2 e = s_pack[q];
                k = (K)e.x;
                v = e.y;
            } else {
                k = s_keys[q];
                v = s_vals[q];
            }
            const int64_t dst = (int64_t)s_dst[digit_of(k, shift, mask)] + q;
            keys_out[dst] = k;
            vals_out[dst] = v;
            if (gathered_out) gathered_out[dst] = gather_src[v];
        }
        __syncthreads();
        s_next[threadIdx.x] += tile_count;   // every thread owns one digit slot
    }
}

// ---------------------------------------------------------------------------
// pair listing: entry e of the list belongs to the ranked Gaussian i with
// offsets[i] <= e < offsets[i+1]; its tiles run row-major over the rectangle.
// ---------------------------------------------------------------------------
// Entries per thread: 8 (2048 per workgroup), or 16 for long lists, where each workgroup's
// fixed cost (locating and staging its ranks) is then spread over twice the entries.
constexpr int kDupItems = 8, kDupItemsLong = 16;   // multiples of 8 (16-byte stores of 16-bit keys)
constexpr int64_t kLongListing = 1 << 26;           // pair capacity from which the long blocks are used
constexpr int kDupTileMin = kBlock * kDupItems;
// ranks a workgroup stages in LDS (more, i.e. fewer than two pairs per rank on average,
// are searched in global memory); half the 2049 a 2048-entry block can meet, for a
// smaller LDS footprint: at 1 M Gaussians no block meets more than ~450
constexpr int kDupWindow = 1025;

// part[b] = rank whose pairs contain entry b * tile; part[blocks] = rank of the last entry.
// Also zeroes clear[0, clear_words) (the tile ranges, so that tiles without pairs read as empty).
__global__ __launch_bounds__(kBlock) void partition_kernel(const uint32_t *offsets, int64_t n_items,
                                                           const unsigned long long *num_dev, int64_t cap,
                                                           int64_t tile, uint32_t *part, uint32_t *clear,
                                                           int64_t clear_words) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t w = i; w < clear_words; w += (int64_t)gridDim.x * kBlock) clear[w] = 0u;
    if (i >= n_items) return;
    const int64_t num = live_count(cap, num_dev);
    const int64_t start = offsets[i];
    const int64_t end = min<int64_t>(i + 1 < n_items ? (int64_t)offsets[i + 1] : (int64_t)*num_dev, num);
    for (int64_t b = (start + tile - 1) / tile; b * tile < end; ++b) part[b] = (uint32_t)i;
    if (start < end && end == num) part[(num + tile - 1) / tile] = (uint32_t)i;
}

__device__ inline int64_t last_le_global(const uint32_t *offsets, int64_t lo, int64_t hi, uint32_t e) {
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (offsets[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Workgroup b lists entries [b*kTile, (b+1)*kTile).  The ranks whose pairs meet that
// span are staged in LDS (up to kDupWindow of them; else they are searched in global
// memory), and each rank marks the threads whose first entry it holds; each thread then
// takes kItems consecutive entries and walks the rectangles row-major.
// kDepth: the 64-bit keys carry the depth bits (staged only then).
template <bool kDepth, int kItems>
__global__ __launch_bounds__(kBlock) void duplicate_kernel(DuplicateParams p, const uint32_t *part) {
    static_assert(kItems % 8 == 0, "listing stores whole 16-byte vectors");
    constexpr int kTile = kBlock * kItems;
    __shared__ uint32_t s_off[kDupWindow];
    __shared__ uint32_t s_g[kDupWindow];
    __shared__ uint2 s_rect[kDupWindow];
    __shared__ uint32_t s_depth[kDepth ? kDupWindow : 1];
    __shared__ uint16_t s_rank[kBlock];   // rank (in the window) holding each thread's first entry
    const int64_t num_dups = live_count(p.capacity, p.num_dups);
    const int64_t first = (int64_t)blockIdx.x * kTile;
    if (first >= num_dups) return;
    const int64_t lo = part[blockIdx.x];
    const int64_t hi = part[blockIdx.x + 1];   // rank of entry (b+1)*kTile, or of the last entry
    const int64_t window = hi - lo + 1;
    const bool staged = window <= kDupWindow;
    if (staged) {
        for (int64_t k = threadIdx.x; k < window; k += kBlock) {
            const int64_t i = lo + k;
            const uint32_t g = p.order ? p.order[i] : (uint32_t)i;
            s_off[k] = p.offsets[i];
            s_g[k] = g;
            s_rect[k] = p.rect_ranked ? p.rect_ranked[i] : p.rect[g];
            if (kDepth) s_depth[k] = __float_as_uint(p.depth[g]);
        }
        __syncthreads();
        // rank k holds entries [s_off[k], s_off[k+1]); thread t starts at first + kItems*t
        for (int64_t k = threadIdx.x; k < window; k += kBlock) {
            const int64_t a = (int64_t)s_off[k] - first;
            const int64_t b = k + 1 < window ? (int64_t)s_off[k + 1] - first : (int64_t)kTile;
            const int64_t t0 = a <= 0 ? 0 : (a + kItems - 1) / kItems;
            const int64_t t1 = min<int64_t>(kBlock, b <= 0 ? 0 : (b + kItems - 1) / kItems);
            for (int64_t t = t0; t < t1; ++t) s_rank[t] = (uint16_t)k;
        }
    }
    __syncthreads();
    const int64_t e0 = first + (int64_t)threadIdx.x * kItems;
    if (e0 >= num_dups) return;
    const int n_here = (int)min<int64_t>(kItems, num_dups - e0);

    // rank holding e0
    int64_t i;
    if (staged) {
        i = s_rank[threadIdx.x];
    } else {
        i = last_le_global(p.offsets, lo, hi, (uint32_t)e0) - lo;
    }
    auto load_rank = [&](int64_t k, uint32_t &g, uint32_t &off, uint2 &rc, uint32_t &db) {
        if (staged) {
            g = s_g[k];
            off = s_off[k];
            rc = s_rect[k];
            db = kDepth ? s_depth[k] : 0u;
        } else {
            const int64_t r = lo + k;
            g = p.order ? p.order[r] : (uint32_t)r;
            off = p.offsets[r];
            rc = p.rect_ranked ? p.rect_ranked[r] : p.rect[g];
            db = kDepth ? __float_as_uint(p.depth[g]) : 0u;
        }
    };
    // The rank after rank i that holds entry e_next: the last one whose offset is <= e_next
    // (ranks without pairs share the offset of the next rank with pairs).  Usually i + 1;
    // past a run of ranks without pairs, a bisection over the window.
    const int64_t last = hi - lo;
    auto rank_offset = [&](int64_t k) -> uint32_t { return staged ? s_off[k] : p.offsets[lo + k]; };
    auto next_rank = [&](int64_t i, uint32_t e_next) -> int64_t {
        ++i;
        if (i >= last || rank_offset(i + 1) > e_next) return i;
        int64_t a = i + 1, b = last;
        while (a < b) {
            const int64_t mid = a + (b - a + 1) / 2;
            if (rank_offset(mid) <= e_next) a = mid; else b = mid - 1;
        }
        return a;
    };
    uint32_t g, off, dbits;
    uint2 rc;
    load_rank(i, g, off, rc, dbits);
    uint32_t tiles[kItems], gs[kItems], dbs[kItems];
    if (p.ellipse) {
        // exact footprint: the kept tiles of each row form one span; walk the spans.  The
        // spans of a rank add up to its tile count (the preprocess summed the same spans),
        // so no walk leaves its rectangle or the staged ranks; should one ever try, the
        // thread repeats its last pair, raises the fault bit and stops walking.
        EllipseRec E = p.ellipse[g];
        uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y1 = rc.y >> 16;
        uint32_t ty = rc.y & 0xffffu, sa, sb;
        uint32_t j = (uint32_t)e0 - off;
        bool broken = false;
        row_span(E, x0, x1, ty, sa, sb);
        while (j >= sb - sa) {
            if (ty + 1 >= y1) {
                broken = true;
                j = 0;
                sa = x0;
                sb = x0 + 1;
                break;
            }
            j -= sb - sa;
            row_span(E, x0, x1, ++ty, sa, sb);
        }
        uint32_t tx = sa + j;
        for (int k = 0; k < n_here; ++k) {
            tiles[k] = ty * (uint32_t)p.tiles_x + tx;
            gs[k] = g;
            dbs[k] = dbits;
            if (++tx == sb && k + 1 < n_here && !broken) {
                do {   // next row with a span, else the next rank with pairs
                    if (++ty == y1) {
                        if (i >= last) {
                            broken = true;
                            break;
                        }
                        i = next_rank(i, (uint32_t)e0 + k + 1);
                        load_rank(i, g, off, rc, dbits);
                        E = p.ellipse[g];
                        x0 = rc.x & 0xffffu;
                        x1 = rc.x >> 16;
                        y1 = rc.y >> 16;
                        ty = rc.y & 0xffffu;
                    }
                    row_span(E, x0, x1, ty, sa, sb);
                } while (sa == sb);
                tx = sa;
            }
            if (broken) {   // repeat the last pair
                ty = tiles[k] / (uint32_t)p.tiles_x;
                tx = tiles[k] - ty * (uint32_t)p.tiles_x;
            }
        }
        if (broken) __hip_atomic_fetch_or(p.fault, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
    uint32_t x0 = rc.x & 0xffffu, w = (rc.x >> 16) - x0, y0 = rc.y & 0xffffu, h = (rc.y >> 16) - y0;
    uint32_t j = (uint32_t)e0 - off;
    uint32_t row = j / w, col = j - row * w;
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
        if (k < n_here) {
            tiles[k] = (y0 + row) * (uint32_t)p.tiles_x + x0 + col;
            gs[k] = g;
            dbs[k] = dbits;
            if (++col == w) {
                col = 0;
                if (++row == h && k + 1 < n_here) {
                    // next rank with pairs (ranks without pairs own no entries): usually the
                    // next one, its rectangle loaded anyway
                    load_rank(++i, g, off, rc, dbits);
                    if (((rc.x >> 16) - (rc.x & 0xffffu)) * ((rc.y >> 16) - (rc.y & 0xffffu)) == 0) {
                        i = next_rank(i - 1, (uint32_t)e0 + k + 1);
                        load_rank(i, g, off, rc, dbits);
                    }
                    x0 = rc.x & 0xffffu;
                    w = (rc.x >> 16) - x0;
                    y0 = rc.y & 0xffffu;
                    h = (rc.y >> 16) - y0;
                    row = 0;
                }
            }
        }
    }
    }
    if (n_here == kItems) {
        uint4 *vo = reinterpret_cast<uint4 *>(p.values + e0);
#pragma unroll
        for (int q = 0; q < kItems / 4; ++q)
            vo[q] = make_uint4(gs[4 * q], gs[4 * q + 1], gs[4 * q + 2], gs[4 * q + 3]);
        if (p.tile_keys) {
            uint4 *to = reinterpret_cast<uint4 *>(p.tile_keys + e0);
#pragma unroll
            for (int q = 0; q < kItems / 4; ++q)
                to[q] = make_uint4(tiles[4 * q], tiles[4 * q + 1], tiles[4 * q + 2], tiles[4 * q + 3]);
        }
        if (p.tile_keys16) {   // eight 16-bit tile ids = one 16-byte store
            uint4 *to = reinterpret_cast<uint4 *>(p.tile_keys16 + e0);
#pragma unroll
            for (int q = 0; q < kItems / 8; ++q) {
                const uint32_t *t = tiles + 8 * q;
                to[q] = make_uint4(t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16));
            }
        }
        if (p.keys64) {
#pragma unroll
            for (int k = 0; k < kItems; ++k) p.keys64[e0 + k] = ((uint64_t)tiles[k] << 32) | dbs[k];
        }
    } else {
        for (int k = 0; k < n_here; ++k) {
            p.values[e0 + k] = gs[k];
            if (p.tile_keys) p.tile_keys[e0 + k] = tiles[k];
            if (p.tile_keys16) p.tile_keys16[e0 + k] = (uint16_t)tiles[k];
            if (p.keys64) p.keys64[e0 + k] = ((uint64_t)tiles[k] << 32) | dbs[k];
        }
    }
}

// ranges from sorted tiles: 4 consecutive entries per thread
constexpr int kRangeItems = 4;

enum RangeKeys { kTileKeys32 = 0, kKeys64 = 1, kTileKeys16 = 2 };

template <int kKind>
__device__ __forceinline__ uint32_t tile_of_entry(const RangesParams &p, int64_t e) {
    if constexpr (kKind == kKeys64) return (uint32_t)(p.keys64[e] >> 32);
    else if constexpr (kKind == kTileKeys16) return p.tile_keys16[e];
    else return p.tile_keys[e];
}

// Depth-first listing under the square rule, a thread per ranked Gaussian: its pairs, row-major
// over its tile rectangle, at its offset from the prefix sum (as many as the distance to the
// next rank's offset); a rank of more than kPairListSolo pairs is written by its whole wave,
// one pair per lane.  Needs no partition table or staged rank window.  Pairs past the buffer's
// capacity are not written (a launch on buffers sized for an earlier frame, which the host
// then repeats).  Also zeroes clear[0, clear_words) (the tile ranges, so that tiles without
// pairs read as empty).
constexpr uint32_t kPairListSolo = 16;

template <bool kKey16>
__device__ inline void pair_entry(const DuplicateParams &p, int64_t k, uint32_t j, uint32_t g, uint2 rc) {
    const uint32_t x0 = rc.x & 0xffffu, w = (rc.x >> 16) - x0, y0 = rc.y & 0xffffu;
    const uint32_t row = j / w, tile = (y0 + row) * (uint32_t)p.tiles_x + x0 + (j - row * w);
    if constexpr (kKey16)
        p.tile_keys16[k] = (uint16_t)tile;
    else
        p.tile_keys[k] = tile;
    p.values[k] = g;
}

template <bool kKey16>
__global__ __launch_bounds__(kBlock) void pair_list_kernel(DuplicateParams p) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t w = i; w < p.clear_words; w += (int64_t)gridDim.x * kBlock) p.clear[w] = 0u;
    int64_t k0 = 0, stop = 0;
    uint32_t g = 0;
    uint2 rc = make_uint2(0u, 0u);
    if (i < p.n_items) {
        stop = min<int64_t>(p.capacity, i + 1 < p.n_items ? (int64_t)p.offsets[i + 1] : (int64_t)*p.num_dups);
        k0 = p.offsets[i];
        if (k0 < stop) {
            g = p.order ? p.order[i] : (uint32_t)i;
            rc = p.rect_ranked ? p.rect_ranked[i] : p.rect[g];
        }
    }
    const bool solo = stop - k0 > (int64_t)kPairListSolo;
    if (!solo)
        for (int64_t k = k0; k < stop; ++k) pair_entry<kKey16>(p, k, (uint32_t)(k - k0), g, rc);
    // the wave writes each large rank's pairs together
    const uint32_t lane = threadIdx.x & (kWave - 1);
    for (uint64_t m = __ballot(solo); m; m &= m - 1) {
        const int l = __builtin_ctzll(m);
        const int64_t a = ((int64_t)__builtin_amdgcn_readlane((int)(k0 >> 32), l) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)k0, l);
        const int64_t b = ((int64_t)__builtin_amdgcn_readlane((int)(stop >> 32), l) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)stop, l);
        const uint32_t gl = (uint32_t)__builtin_amdgcn_readlane((int)g, l);
        const uint2 rl = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)rc.x, l),
                                    (uint32_t)__builtin_amdgcn_readlane((int)rc.y, l));
        for (int64_t k = a + lane; k < b; k += kWave) pair_entry<kKey16>(p, k, (uint32_t)(k - a), gl, rl);
    }
}

template <int kKind>
__global__ __launch_bounds__(kBlock) void ranges_kernel(RangesParams p) {
    const int64_t num_dups = live_count(p.capacity, p.num_dups);
    const int64_t e0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kRangeItems;
    if (e0 >= num_dups) return;
    uint32_t t[kRangeItems + 1];
    const int cnt = (int)min<int64_t>(kRangeItems, num_dups - e0);
#pragma unroll
    for (int k = 0; k <= kRangeItems; ++k) {
        const int64_t e = e0 + k;
        t[k] = 0xffffffffu;
        if (k <= cnt && e < num_dups) t[k] = tile_of_entry<kKind>(p, e);
    }
    const uint32_t prev = e0 == 0 ? 0xffffffffu : tile_of_entry<kKind>(p, e0 - 1);
#pragma unroll
    for (int k = 0; k < kRangeItems; ++k) {
        if (k >= cnt) break;
        const int64_t e = e0 + k;
        const uint32_t before = k == 0 ? prev : t[k - 1];
        if (before != t[k]) p.ranges[2 * (int64_t)t[k]] = (uint32_t)e;
        if (t[k + 1] != t[k]) p.ranges[2 * (int64_t)t[k] + 1] = (uint32_t)(e + 1);
        if (p.keys_out) p.keys_out[e] = ((uint64_t)t[k] << 32) | __float_as_uint(p.depth[p.values[e]]);
    }
}

__global__ __launch_bounds__(kBlock) void fill_u32_kernel(uint32_t *dst, uint32_t value, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) dst[i] = value;
}


inline int64_t sort_tile(int64_t n) { return (int64_t)kBlock * (n <= kSmallSort ? kItemsSmall : kItemsLarge); }

inline int sort_groups(int64_t n) {
    const int64_t tiles = (n + sort_tile(n) - 1) / sort_tile(n);
    return (int)(tiles < 1 ? 1 : (tiles > kMaxSortGroups ? kMaxSortGroups : tiles));
}

template <typename K, int ITEMS>
void launch_pass(K *ki, uint32_t *vi, K *ko, uint32_t *vo, int64_t n, const unsigned long long *n_dev, int shift,
                 int bits, int groups, uint32_t *counts, uint32_t *totals, const uint32_t *gather_src,
                 uint32_t *gathered_out, hipStream_t s) {
    radix_count_kernel<K, ITEMS><<<groups, kBlock, 0, s>>>(ki, n, n_dev, shift, bits, counts);
    radix_digit_scan_kernel<<<1 << bits, kBlock, 0, s>>>(counts, groups, totals);
    switch (bits) {   // the digit widths the passes use (8-bit digits, 13 tile bits -> 7 + 6)
        case 8:
            radix_scatter_kernel<K, ITEMS, 8><<<groups, kBlock, 0, s>>>(ki, vi, ko, vo, n, n_dev, shift, bits, counts,
                                                                        totals, gather_src, gathered_out);
            break;
        case 7:
            radix_scatter_kernel<K, ITEMS, 7><<<groups, kBlock, 0, s>>>(ki, vi, ko, vo, n, n_dev, shift, bits, counts,
                                                                        totals, gather_src, gathered_out);
            break;
        case 6:
            radix_scatter_kernel<K, ITEMS, 6><<<groups, kBlock, 0, s>>>(ki, vi, ko, vo, n, n_dev, shift, bits, counts,
                                                                        totals, gather_src, gathered_out);
            break;
        default:
            radix_scatter_kernel<K, ITEMS, 0><<<groups, kBlock, 0, s>>>(ki, vi, ko, vo, n, n_dev, shift, bits, counts,
                                                                        totals, gather_src, gathered_out);
            break;
    }
}

}  // namespace

int64_t sort_scratch_words(int64_t n) { return (int64_t)kRadix * sort_groups(n) + kRadix; }
int64_t sort_totals_offset(int64_t n) { return (int64_t)kRadix * sort_groups(n); }

template <typename K>
int radix_sort_pairs(K *k0, uint32_t *v0, K *k1, uint32_t *v1, int64_t n, const unsigned long long *n_dev,
                     int begin_bit, int end_bit, uint32_t *scratch, hipStream_t s, const uint32_t *gather_src,
                     uint32_t *gathered_out) {
    if ((n <= 1 && !n_dev) || n <= 0 || end_bit <= begin_bit) return 0;
    const int groups = sort_groups(n);
    uint32_t *counts = scratch;
    uint32_t *totals = counts + (int64_t)kRadix * groups;
    // the fewest 8-bit-or-narrower passes, with the bits spread evenly (13 -> 7 + 6):
    // narrower digits give longer contiguous write runs per tile
    const int total_bits = end_bit - begin_bit;
    const int passes = (total_bits + kRadixBits - 1) / kRadixBits;
    int cur = 0, shift = begin_bit;
    for (int p = 0; p < passes; ++p) {
        const int bits = (total_bits - (shift - begin_bit) + (passes - p) - 1) / (passes - p);
        K *ki = cur ? k1 : k0;
        uint32_t *vi = cur ? v1 : v0;
        K *ko = cur ? k0 : k1;
        uint32_t *vo = cur ? v0 : v1;
        const bool last = p == passes - 1;
        if (n <= kSmallSort)
            launch_pass<K, kItemsSmall>(ki, vi, ko, vo, n, n_dev, shift, bits, groups, counts, totals,
                                        last ? gather_src : nullptr, last ? gathered_out : nullptr, s);
        else
            launch_pass<K, kItemsLarge>(ki, vi, ko, vo, n, n_dev, shift, bits, groups, counts, totals,
                                        last ? gather_src : nullptr, last ? gathered_out : nullptr, s);
        shift += bits;
        cur ^= 1;
    }
    return cur;
}

template int radix_sort_pairs<uint32_t>(uint32_t *, uint32_t *, uint32_t *, uint32_t *, int64_t,
                                        const unsigned long long *, int, int, uint32_t *, hipStream_t,
                                        const uint32_t *, uint32_t *);
template int radix_sort_pairs<uint64_t>(uint64_t *, uint32_t *, uint64_t *, uint32_t *, int64_t,
                                        const unsigned long long *, int, int, uint32_t *, hipStream_t,
                                        const uint32_t *, uint32_t *);
template int radix_sort_pairs<uint16_t>(uint16_t *, uint32_t *, uint16_t *, uint32_t *, int64_t,
                                        const unsigned long long *, int, int, uint32_t *, hipStream_t,
                                        const uint32_t *, uint32_t *);

int64_t duplicate_partition_words(int64_t num_dups) { return (num_dups + kDupTileMin - 1) / kDupTileMin + 1; }

void launch_duplicate(const DuplicateParams &p, uint32_t *part, hipStream_t s) {
    if (p.capacity <= 0 || p.n_items <= 0) return;
    const bool long_list = p.capacity >= kLongListing;
    const int64_t tile = (int64_t)kBlock * (long_list ? kDupItemsLong : kDupItems);
    partition_kernel<<<(unsigned)((p.n_items + kBlock - 1) / kBlock), kBlock, 0, s>>>(
        p.offsets, p.n_items, p.num_dups, p.capacity, tile, part, p.clear, p.clear_words);
    const unsigned nb = (unsigned)((p.capacity + tile - 1) / tile);
    if (p.keys64) {
        if (long_list)
            duplicate_kernel<true, kDupItemsLong><<<nb, kBlock, 0, s>>>(p, part);
        else
            duplicate_kernel<true, kDupItems><<<nb, kBlock, 0, s>>>(p, part);
    } else {
        if (long_list)
            duplicate_kernel<false, kDupItemsLong><<<nb, kBlock, 0, s>>>(p, part);
        else
            duplicate_kernel<false, kDupItems><<<nb, kBlock, 0, s>>>(p, part);
    }
}

void launch_pair_list(const DuplicateParams &p, hipStream_t s) {
    if (p.capacity <= 0 || p.n_items <= 0) return;
    const unsigned grid = (unsigned)((p.n_items + kBlock - 1) / kBlock);
    if (p.tile_keys16)
        pair_list_kernel<true><<<grid, kBlock, 0, s>>>(p);
    else
        pair_list_kernel<false><<<grid, kBlock, 0, s>>>(p);
}

void launch_ranges(const RangesParams &p, hipStream_t s) {
    if (p.capacity <= 0) return;
    const int64_t threads = (p.capacity + kRangeItems - 1) / kRangeItems;
    const unsigned grid = (unsigned)((threads + kBlock - 1) / kBlock);
    if (p.keys64)
        ranges_kernel<kKeys64><<<grid, kBlock, 0, s>>>(p);
    else if (p.tile_keys16)
        ranges_kernel<kTileKeys16><<<grid, kBlock, 0, s>>>(p);
    else
        ranges_kernel<kTileKeys32><<<grid, kBlock, 0, s>>>(p);
}

void launch_fill_u32(uint32_t *dst, uint32_t value, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    fill_u32_kernel<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(dst, value, n);
}

}  // namespace gsr
