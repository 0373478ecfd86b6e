// Heaviest-first launch order for the per-tile compositing kernels.
//
// A compositing workgroup's run time grows with the work of its tile, and the tiles
// near the centre of a view carry several times the mean.  Launched in tile order,
// the heavy tiles start late and the frame ends with a few of them running on an
// otherwise idle chip.  Launching them first (longest-processing-time-first) evens
// the finish.  The order is a counting sort by weight on a logarithmic scale, 2048
// buckets of 1/64 octave (the leading bit of the weight and the six below it), so no
// pass for the largest weight is needed; order within a bucket is arbitrary, which
// only changes when a tile runs, never what it computes.
#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderSubBits = 6;                              // bits below the leading one
constexpr int kOrderBuckets = 32 << kOrderSubBits;            // 2048
constexpr int kOrderPer = kOrderBuckets / kOrderThreads;      // buckets per thread in the scan
constexpr int kOrderKept = 8;   // tiles per thread whose bucket stays in registers (8192 tiles)

__device__ __forceinline__ uint32_t tile_weight(const TileOrderParams &p, int t) {
    return p.weights ? p.weights[t] : p.ranges[2 * t + 1] - p.ranges[2 * t];
}

// Bucket of a weight, heaviest first: 2047 - (64 * floor(log2 w) + the six bits after
// the leading one); weight 0 goes last.
__device__ __forceinline__ uint32_t order_bucket(uint32_t w) {
    if (w == 0) return kOrderBuckets - 1;
    const uint32_t lead = 31u - (uint32_t)__clz(w);
    const uint32_t frac = ((w << (31u - lead)) >> (31 - kOrderSubBits)) & ((1u << kOrderSubBits) - 1u);
    return (uint32_t)(kOrderBuckets - 1) - ((lead << kOrderSubBits) + frac);
}

__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(TileOrderParams p) {
    __shared__ uint32_t s_count[kOrderBuckets];
    __shared__ uint32_t s_wave[kOrderThreads / kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int b = threadIdx.x; b < kOrderBuckets; b += kOrderThreads) s_count[b] = 0;
    __syncthreads();
    // each thread keeps the buckets of its first kOrderKept tiles (and recomputes the rest)
    uint32_t kept[kOrderKept];
#pragma unroll
    for (int j = 0; j < kOrderKept; ++j) {
        const int t = threadIdx.x + j * kOrderThreads;
        kept[j] = t < p.tiles ? order_bucket(tile_weight(p, t)) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kOrderKept; ++j)
        if (threadIdx.x + j * kOrderThreads < p.tiles) atomicAdd(&s_count[kept[j]], 1u);
    for (int t = threadIdx.x + kOrderKept * kOrderThreads; t < p.tiles; t += kOrderThreads)
        atomicAdd(&s_count[order_bucket(tile_weight(p, t))], 1u);
    __syncthreads();
    // exclusive prefix over the buckets: kOrderPer consecutive buckets per thread, a scan per
    // wave, then the wave totals
    uint32_t c[kOrderPer], sum = 0;
#pragma unroll
    for (int k = 0; k < kOrderPer; ++k) {
        c[k] = s_count[threadIdx.x * kOrderPer + k];
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
    for (int k = 0; k < kOrderPer; ++k) {
        s_count[threadIdx.x * kOrderPer + k] = base;
        base += c[k];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kOrderKept; ++j) {
        const int t = threadIdx.x + j * kOrderThreads;
        if (t < p.tiles) p.order[atomicAdd(&s_count[kept[j]], 1u)] = (uint32_t)t;
    }
    for (int t = threadIdx.x + kOrderKept * kOrderThreads; t < p.tiles; t += kOrderThreads)
        p.order[atomicAdd(&s_count[order_bucket(tile_weight(p, t))], 1u)] = (uint32_t)t;
}

// Backward work of a tile: the entries up to the deepest one any of its pixels blended.
__global__ __launch_bounds__(kWave) void backward_tile_weight_kernel(const uint32_t *__restrict__ n_blend,
                                                                      const uint32_t *__restrict__ ranges,
                                                                      int32_t width, int32_t height,
                                                                      int32_t tiles_x, uint32_t *weights) {
    const int tile = blockIdx.x;
    const int tx = tile % tiles_x, ty = tile / tiles_x;
    const int lane = threadIdx.x;
    const int iy = ty * kTile + (lane >> 2);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ix = tx * kTile + 4 * i + (lane & 3);
        if (ix < width && iy < height) m = max(m, n_blend[(size_t)iy * width + ix]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) weights[tile] = min(m, ranges[2 * tile + 1] - ranges[2 * tile]);
}

}  // namespace

bool launch_tile_order(const TileOrderParams &p, hipStream_t s) {
    if (p.tiles <= 0 || p.tiles > kMaxOrderedTiles) return false;
    tile_order_kernel<<<1, kOrderThreads, 0, s>>>(p);
    return true;
}

void launch_backward_tile_weight(const uint32_t *n_blend, const uint32_t *ranges, int32_t width, int32_t height,
                                 int32_t tiles_x, int32_t tiles_y, uint32_t *weights, hipStream_t s) {
    const unsigned tiles = (unsigned)(tiles_x * tiles_y);
    if (tiles == 0) return;
    backward_tile_weight_kernel<<<tiles, kWave, 0, s>>>(n_blend, ranges, width, height, tiles_x, weights);
}

}  // namespace gsr
