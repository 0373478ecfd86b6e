// Exclusive prefix sum over uint32 values, reduce-then-scan.
//
// Used for the per-Gaussian tile counts (the offsets where each Gaussian's pairs
// start, and their total) and for the radix-sort digit histograms.  Each
// workgroup owns 2048 consecutive values (8 per thread, blocked), so a level
// reads its input once to reduce and once to scan: 8 B of HBM traffic per value
// plus the 4 B write.  Partial sums are uint64 so totals above 2^32 are reported
// exactly (the caller rejects them).
//
// Within a workgroup: per-thread serial sum -> wave64 inclusive scan with
// cross-lane shuffles -> four wave totals combined through LDS.
#include "gs_internal.h"

namespace gsr {
namespace {

// Summand of one packed count (tile count | super count << kPackShift): the two fields apart,
// tiles | super-tiles << kPairShift, so that one uint64 sum carries both totals.
__device__ inline unsigned long long scan_summand(uint32_t v) {
    return (unsigned long long)(v & ((1u << kPackShift) - 1u)) | ((unsigned long long)(v >> kPackShift) << kPairShift);
}

template <typename T>
__device__ inline T wave_inclusive_scan(T x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        T y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    return x;
}

// Exclusive scan of one value per thread across the workgroup; returns the
// workgroup total in *total (all threads).
template <typename T>
__device__ inline T block_exclusive_scan(T x, T *total) {
    __shared__ T wave_sums[kBlock / kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    T inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) wave_sums[wave] = inc;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) {
        T s = wave_sums[w];
        if (w < wave) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

// kPair: the inputs are packed counts (tile count | super count << kPackShift), summed as
// two fields of one uint64 (tiles | super-tiles << kPairShift; neither field overflows: the
// tile total is below 2^32 by the callers' cap, the super total below 2^28).
template <typename TIn, bool kPair>
__device__ inline void load_items(const TIn *in, const uint32_t *gather, int64_t n, int64_t base,
                                  unsigned long long v[kScanItems]) {
    const int64_t first = base + (int64_t)threadIdx.x * kScanItems;
    if constexpr (sizeof(TIn) == 4) {
        // a thread's eight values as two 16-byte loads (blocks start at multiples of 2048
        // values, so they are aligned when the array is): per-value loads would each touch a
        // wave's whole 2 KB span for 256 useful bytes
        static_assert(kScanItems == 8, "two 16-byte loads per thread");
        if (!gather && first + kScanItems <= n && (reinterpret_cast<uintptr_t>(in) & 15) == 0) {
            const uint4 *q = reinterpret_cast<const uint4 *>(in + first);
            const uint4 a = q[0], b = q[1];
            const uint32_t w[kScanItems] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < kScanItems; ++k)
                v[k] = kPair ? scan_summand(w[k]) : (unsigned long long)w[k];
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
        const int64_t i = first + k;
        v[k] = 0;
        if (i < n) v[k] = gather ? (unsigned long long)in[gather[i]] : (unsigned long long)in[i];
        if (kPair) v[k] = scan_summand((uint32_t)v[k]);
    }
}

template <typename TIn, bool kPair>
__global__ __launch_bounds__(kBlock) void scan_reduce_kernel(const TIn *in, const uint32_t *gather,
                                                             int64_t n, unsigned long long *partials) {
    unsigned long long v[kScanItems];
    load_items<TIn, kPair>(in, gather, n, (int64_t)blockIdx.x * kScanTile, v);
    unsigned long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) s += v[k];
    unsigned long long total;
    block_exclusive_scan(s, &total);
    if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

// out[i] = the block's offset + exclusive scan within the block.  The offset is
// prefix[block] (scanned block totals), or, with block_sums, the sum of the block
// totals before this block, added up here (few blocks: it saves a kernel).  When
// `total` is non-null the last block writes the grand total there, and also to
// `host_total` (host-coherent memory, a system-scope store) when that is non-null; with
// `flag`, host_total[2] = *flag is stored first and the total after it with release order,
// so a host that sees the total also sees the flag.
// kPair: packed inputs (load_items); out[i] is the super-tile part of the prefix.
// kDecode: the total is packed; total[1] and total[2] also get its two fields.
template <typename TIn, typename TOut, bool kPair, bool kDecode>
__global__ __launch_bounds__(kBlock) void scan_downsweep_kernel(const TIn *in, const uint32_t *gather,
                                                                int64_t n, const unsigned long long *prefix,
                                                                const unsigned long long *block_sums, TOut *out,
                                                                unsigned long long *total,
                                                                unsigned long long *host_total,
                                                                const unsigned long long *flag) {
    // the block's own values first: their loads are in flight while the offset is summed
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    unsigned long long v[kScanItems];
    load_items<TIn, kPair>(in, gather, n, base, v);
    unsigned long long offset = 0;
    if (prefix) {
        offset = prefix[blockIdx.x];
    } else if (block_sums) {
        unsigned long long before = 0;
        for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kBlock) before += block_sums[j];
        block_exclusive_scan(before, &offset);
    }
    unsigned long long s = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) s += v[k];
    unsigned long long block_total;
    unsigned long long run = block_exclusive_scan(s, &block_total) + offset;
    const int64_t first = base + (int64_t)threadIdx.x * kScanItems;
    if (sizeof(TOut) == 4 && first + kScanItems <= n && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        // two 16-byte stores, for the reason the loads are two
        uint32_t w[kScanItems];
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            w[k] = kPair ? (uint32_t)(run >> kPairShift) : (uint32_t)run;
            run += v[k];
        }
        uint4 *q = reinterpret_cast<uint4 *>(out + first);
        q[0] = make_uint4(w[0], w[1], w[2], w[3]);
        q[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            const int64_t i = first + k;
            if (i < n) out[i] = kPair ? (TOut)(run >> kPairShift) : (TOut)run;
            run += v[k];
        }
    }
    if (total && threadIdx.x == 0 && blockIdx.x == gridDim.x - 1) {
        const unsigned long long all = offset + block_total;
        *total = all;
        if (kDecode) {
            total[1] = all & ((1ull << kPairShift) - 1);
            total[2] = all >> kPairShift;
        }
        if (host_total && flag) {
            __hip_atomic_store(host_total + 2, *flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(host_total, all, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        } else if (host_total) {
            __hip_atomic_store(host_total, all, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

inline int64_t blocks_for(int64_t n) { return (n + kScanTile - 1) / kScanTile; }

// Up to this many blocks (2 M values) the downsweep sums the partials itself.
constexpr int64_t kDirectBlocks = 1024;

// Scans `in` (n values) into `out`; partials for the next level live in scratch.
template <typename TIn, typename TOut, bool kPair, bool kDecode>
void scan_level(const TIn *in, const uint32_t *gather, TOut *out, int64_t n, unsigned long long *total,
                unsigned long long *host_total, const unsigned long long *flag, unsigned long long *scratch,
                hipStream_t s) {
    const int64_t nb = blocks_for(n);
    if (nb == 1) {
        scan_downsweep_kernel<TIn, TOut, kPair, kDecode><<<1, kBlock, 0, s>>>(in, gather, n, nullptr, nullptr, out,
                                                                              total, host_total, flag);
        return;
    }
    unsigned long long *partials = scratch;
    scan_reduce_kernel<TIn, kPair><<<(unsigned)nb, kBlock, 0, s>>>(in, gather, n, partials);
    if (nb <= kDirectBlocks) {   // each block adds up the partials before it
        scan_downsweep_kernel<TIn, TOut, kPair, kDecode><<<(unsigned)nb, kBlock, 0, s>>>(
            in, gather, n, nullptr, partials, out, total, host_total, flag);
        return;
    }
    // exclusive scan of the partials (already in the packed form), in place (reads before
    // writes within each block); that level writes the total
    scan_level<unsigned long long, unsigned long long, false, kDecode>(partials, nullptr, partials, nb, total,
                                                                      host_total, flag, scratch + nb, s);
    scan_downsweep_kernel<TIn, TOut, kPair, false><<<(unsigned)nb, kBlock, 0, s>>>(in, gather, n, partials, nullptr,
                                                                                  out, nullptr, nullptr, nullptr);
}

}  // namespace

int64_t scan_scratch_words(int64_t n) {
    int64_t words = 0;
    for (int64_t nb = blocks_for(n); nb > 1; nb = blocks_for(nb)) words += nb;
    return words + 1;
}

void launch_scan(const uint32_t *in, const uint32_t *gather, uint32_t *out, int64_t n,
                 unsigned long long *total, unsigned long long *scratch, hipStream_t s,
                 unsigned long long *host_total, const unsigned long long *flag) {
    scan_level<uint32_t, uint32_t, false, false>(in, gather, out, n, total, host_total, flag, scratch, s);
}

void launch_scan_pairs(const uint32_t *packed, uint32_t *out, int64_t n, unsigned long long *total,
                       unsigned long long *scratch, hipStream_t s, unsigned long long *host_total,
                       const unsigned long long *flag) {
    scan_level<uint32_t, uint32_t, true, true>(packed, nullptr, out, n, total, host_total, flag, scratch, s);
}

}  // namespace gsr
