// Pair listing, stable LSD radix sort and tile ranges.
//
// Flowchart of the lesson "3D Gaussian Splatting from scratch", steps "Assign to
// tiles (16x16 screen-space)" and "Depth-sort per tile": every (Gaussian, tile)
// pair is listed and the list is ordered by (tile, camera-space depth), equal
// depths by Gaussian index.  The key of a pair is (tile_id << 32) | bits(depth);
// for depth > 0 the IEEE bit pattern orders like the value.
//
// Radix sort, one pass per 8-bit digit, three kernels per pass:
//   histogram  per-workgroup digit counts (LDS atomics), digit-major layout
//   scan       exclusive prefix of the counts = global start of (digit, workgroup)
//   scatter    stable rank of every pair inside its workgroup, staged in LDS so the
//              global writes run in contiguous digit segments
// Stable ranking inside a wave64 uses a ballot per key bit to find the lanes that
// share a digit (the leader adds the group size to the wave's LDS counter);
// workgroup order is wave-major, so the pass preserves input order on ties.
// HBM traffic per pass and pair: read key+value twice (histogram + scatter),
// write once.
#include "gs_internal.h"

namespace gsr {
namespace {

template <typename K>
__device__ inline uint32_t digit_of(K key, int shift, uint32_t mask) {
    return (uint32_t)(key >> shift) & mask;
}

template <typename K>
__global__ __launch_bounds__(kBlock) void radix_histogram_kernel(const K *keys, int64_t n, int shift, int bits,
                                                                 uint32_t *hist, int64_t nblocks) {
    __shared__ uint32_t counts[kBlock / kWave][1 << kRadixBits];
    const int radix = 1 << bits;
    const uint32_t mask = radix - 1;
    const int wave = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < (kBlock / kWave) * (1 << kRadixBits); i += kBlock) (&counts[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll 4
    for (int k = 0; k < kSortItems; ++k) {
        const int64_t i = base + (int64_t)k * kBlock + threadIdx.x;
        if (i < n) atomicAdd(&counts[wave][digit_of(keys[i], shift, mask)], 1u);
    }
    __syncthreads();
    if ((int)threadIdx.x < radix) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) c += counts[w][threadIdx.x];
        hist[(int64_t)threadIdx.x * nblocks + blockIdx.x] = c;
    }
}

__device__ inline uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <typename K>
__global__ __launch_bounds__(kBlock) void radix_scatter_kernel(const K *keys_in, const uint32_t *vals_in,
                                                               K *keys_out, uint32_t *vals_out, int64_t n,
                                                               int shift, int bits, const uint32_t *offsets,
                                                               int64_t nblocks) {
    constexpr int kWaves = kBlock / kWave;
    constexpr int kRadix = 1 << kRadixBits;
    __shared__ K s_keys[kSortTile];
    __shared__ uint32_t s_vals[kSortTile];
    __shared__ uint32_t s_wave_count[kWaves][kRadix];   // per-wave running counts, then wave prefixes
    __shared__ uint32_t s_local_start[kRadix];          // start of each digit inside the workgroup
    __shared__ uint32_t s_global_start[kRadix];         // global start of (digit, this workgroup)
    __shared__ uint32_t s_wave_tot[kWaves];

    const int radix = 1 << bits;
    const uint32_t mask = radix - 1;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kWaves * kRadix; i += kBlock) (&s_wave_count[0][0])[i] = 0;
    if ((int)threadIdx.x < radix) s_global_start[threadIdx.x] = offsets[(int64_t)threadIdx.x * nblocks + blockIdx.x];
    __syncthreads();

    // wave w owns the contiguous segment [w*1024, (w+1)*1024) of the tile, in rounds of 64
    const int64_t seg = (int64_t)blockIdx.x * kSortTile + (int64_t)wave * (kSortItems * kWave);
    K key[kSortItems];
    uint32_t val[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const int64_t i = seg + r * kWave + lane;
        key[r] = i < n ? keys_in[i] : (K)0;
        val[r] = i < n ? vals_in[i] : 0u;
    }
    uint32_t rank[kSortItems];
#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        const bool valid = seg + r * kWave + lane < n;
        const uint32_t d = digit_of(key[r], shift, mask);
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < bits; ++b) {
            const bool bit = (d >> b) & 1u;
            const uint64_t on = __ballot(bit);
            peers &= bit ? on : ~on;
        }
        const uint32_t below = lanes_below(peers);
        const uint32_t prev = valid ? s_wave_count[wave][d] : 0u;
        rank[r] = prev + below;
        if (valid && below == 0) s_wave_count[wave][d] = prev + (uint32_t)__popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // per digit: exclusive prefix over waves, then over digits (workgroup-local start)
    uint32_t digit_total = 0;
    if ((int)threadIdx.x < kRadix) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_wave_count[w][threadIdx.x];
            s_wave_count[w][threadIdx.x] = digit_total;
            digit_total += c;
        }
    }
    {
        // workgroup exclusive scan of digit_total over threadIdx.x (= digit)
        uint32_t inc = digit_total;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t y = __shfl_up(inc, d, kWave);
            if (lane >= d) inc += y;
        }
        if (lane == kWave - 1) s_wave_tot[wave] = inc;
        __syncthreads();
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += s_wave_tot[w];
        if ((int)threadIdx.x < kRadix) s_local_start[threadIdx.x] = before + inc - digit_total;
    }
    __syncthreads();

#pragma unroll
    for (int r = 0; r < kSortItems; ++r) {
        if (seg + r * kWave + lane < n) {
            const uint32_t d = digit_of(key[r], shift, mask);
            const uint32_t pos = s_local_start[d] + s_wave_count[wave][d] + rank[r];
            s_keys[pos] = key[r];
            s_vals[pos] = val[r];
        }
    }
    __syncthreads();

    const int64_t tile_base = (int64_t)blockIdx.x * kSortTile;
    const int count = (int)min<int64_t>(kSortTile, n - tile_base);
    for (int p = threadIdx.x; p < count; p += kBlock) {
        const K k = s_keys[p];
        const uint32_t d = digit_of(k, shift, mask);
        const int64_t dst = (int64_t)s_global_start[d] + (p - (int64_t)s_local_start[d]);
        keys_out[dst] = k;
        vals_out[dst] = s_vals[p];
    }
}

// ---------------------------------------------------------------------------
// pair listing: entry e of the list belongs to the ranked Gaussian i with
// offsets[i] <= e < offsets[i+1]; its tiles run row-major over the rectangle.
// ---------------------------------------------------------------------------
constexpr int kDupItems = 8;
constexpr int kDupTile = kBlock * kDupItems;

__device__ inline int64_t last_le(const uint32_t *offsets, int64_t lo, int64_t hi, uint32_t e) {
    // largest i in [lo, hi] with offsets[i] <= e  (offsets non-decreasing, offsets[lo] <= e)
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (offsets[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kBlock) void duplicate_kernel(DuplicateParams p) {
    __shared__ int64_t s_window[2];
    const int64_t first = (int64_t)blockIdx.x * kDupTile;
    const int64_t last = min<int64_t>(first + kDupTile, p.num_dups) - 1;
    if (threadIdx.x == 0) s_window[0] = last_le(p.offsets, 0, p.n_items - 1, (uint32_t)first);
    if (threadIdx.x == 1) s_window[1] = last_le(p.offsets, 0, p.n_items - 1, (uint32_t)last);
    __syncthreads();
    const int64_t lo = s_window[0], hi = s_window[1];
#pragma unroll
    for (int k = 0; k < kDupItems; ++k) {
        const int64_t e = first + (int64_t)k * kBlock + threadIdx.x;
        if (e > last) break;
        const int64_t i = last_le(p.offsets, lo, hi, (uint32_t)e);
        const uint32_t g = p.order ? p.order[i] : (uint32_t)i;
        const uint32_t j = (uint32_t)e - p.offsets[i];
        const uint2 rc = p.rect[g];
        const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y0 = rc.y & 0xffffu;
        const uint32_t w = x1 - x0;
        const uint32_t row = j / w;
        const uint32_t tile = (y0 + row) * (uint32_t)p.tiles_x + x0 + (j - row * w);
        if (p.keys64) p.keys64[e] = ((uint64_t)tile << 32) | __float_as_uint(p.depth[g]);
        if (p.tile_keys) p.tile_keys[e] = tile;
        p.values[e] = g;
    }
}

__global__ __launch_bounds__(kBlock) void ranges_kernel(RangesParams p) {
    const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (e >= p.num_dups) return;
    auto tile_at = [&](int64_t i) -> uint32_t {
        return p.keys64 ? (uint32_t)(p.keys64[i] >> 32) : p.tile_keys[i];
    };
    const uint32_t t = tile_at(e);
    if (e == 0 || tile_at(e - 1) != t) p.ranges[2 * (int64_t)t] = (uint32_t)e;
    if (e == p.num_dups - 1 || tile_at(e + 1) != t) p.ranges[2 * (int64_t)t + 1] = (uint32_t)(e + 1);
    if (p.keys_out) p.keys_out[e] = ((uint64_t)t << 32) | __float_as_uint(p.depth[p.values[e]]);
}

__global__ __launch_bounds__(kBlock) void fill_u32_kernel(uint32_t *dst, uint32_t value, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) dst[i] = value;
}

inline int64_t sort_blocks(int64_t n) { return (n + kSortTile - 1) / kSortTile; }

}  // namespace

int64_t sort_scratch_words(int64_t n) {
    const int64_t hist = (int64_t)(1 << kRadixBits) * sort_blocks(n);
    return (hist + 1) / 2 + scan_scratch_words(hist) + 1;
}

template <typename K>
int radix_sort_pairs(K *k0, uint32_t *v0, K *k1, uint32_t *v1, int64_t n, int begin_bit, int end_bit,
                     unsigned long long *scratch, hipStream_t s) {
    if (n <= 1 || end_bit <= begin_bit) return 0;
    const int64_t nb = sort_blocks(n);
    uint32_t *hist = reinterpret_cast<uint32_t *>(scratch);
    const int64_t hist_words64 = ((int64_t)(1 << kRadixBits) * nb + 1) / 2;
    unsigned long long *scan_scratch = scratch + hist_words64 + 1;
    unsigned long long *scan_total = scratch + hist_words64;
    int cur = 0;
    for (int bit = begin_bit; bit < end_bit; bit += kRadixBits) {
        const int bits = min(kRadixBits, end_bit - bit);
        K *ki = cur ? k1 : k0;
        uint32_t *vi = cur ? v1 : v0;
        K *ko = cur ? k0 : k1;
        uint32_t *vo = cur ? v0 : v1;
        radix_histogram_kernel<K><<<(unsigned)nb, kBlock, 0, s>>>(ki, n, bit, bits, hist, nb);
        launch_scan(hist, nullptr, hist, (int64_t)(1 << bits) * nb, scan_total, scan_scratch, s);
        radix_scatter_kernel<K><<<(unsigned)nb, kBlock, 0, s>>>(ki, vi, ko, vo, n, bit, bits, hist, nb);
        cur ^= 1;
    }
    return cur;
}

template int radix_sort_pairs<uint32_t>(uint32_t *, uint32_t *, uint32_t *, uint32_t *, int64_t, int, int,
                                        unsigned long long *, hipStream_t);
template int radix_sort_pairs<uint64_t>(uint64_t *, uint32_t *, uint64_t *, uint32_t *, int64_t, int, int,
                                        unsigned long long *, hipStream_t);

void launch_duplicate(const DuplicateParams &p, hipStream_t s) {
    if (p.num_dups <= 0) return;
    const int64_t nb = (p.num_dups + kDupTile - 1) / kDupTile;
    duplicate_kernel<<<(unsigned)nb, kBlock, 0, s>>>(p);
}

void launch_ranges(const RangesParams &p, hipStream_t s) {
    if (p.num_dups <= 0) return;
    ranges_kernel<<<(unsigned)((p.num_dups + kBlock - 1) / kBlock), kBlock, 0, s>>>(p);
}

void launch_fill_u32(uint32_t *dst, uint32_t value, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    fill_u32_kernel<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(dst, value, n);
}

}  // namespace gsr
