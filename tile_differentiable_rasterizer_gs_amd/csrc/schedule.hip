// Heaviest-first launch order for the per-tile compositing kernels.
//
// A compositing workgroup's run time grows with the work of its tile, and the tiles
// near the centre of a view carry several times the mean.  Launched in tile order,
// the heavy tiles start late and the frame ends with a few of them running on an
// otherwise idle chip.  Launching them first (longest-processing-time-first) evens
// the finish.  The order is a bucket sort by weight, coarsened to 256 buckets
// between 0 and the largest weight; order within a bucket is arbitrary, which only
// changes when a tile runs, never what it computes.
#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 256;

__device__ __forceinline__ uint32_t tile_weight(const TileOrderParams &p, int t) {
    return p.weights ? p.weights[t] : p.ranges[2 * t + 1] - p.ranges[2 * t];
}

__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(TileOrderParams p) {
    __shared__ uint32_t s_max;
    __shared__ uint32_t s_count[kOrderBuckets];
    __shared__ uint32_t s_wave[kOrderBuckets / kWave];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (threadIdx.x == 0) s_max = 0;
    for (int b = threadIdx.x; b < kOrderBuckets; b += kOrderThreads) s_count[b] = 0;
    __syncthreads();
    uint32_t m = 0;
    for (int t = threadIdx.x; t < p.tiles; t += kOrderThreads) m = max(m, tile_weight(p, t));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) atomicMax(&s_max, m);
    __syncthreads();
    const uint64_t wmax = (uint64_t)s_max + 1;
    // bucket 0 holds the heaviest tiles
    auto bucket = [&](uint32_t w) {
        return (uint32_t)(kOrderBuckets - 1) - (uint32_t)(((uint64_t)w * kOrderBuckets) / wmax);
    };
    for (int t = threadIdx.x; t < p.tiles; t += kOrderThreads) atomicAdd(&s_count[bucket(tile_weight(p, t))], 1u);
    __syncthreads();
    // exclusive prefix over the 256 buckets: a scan per wave, then the wave totals
    uint32_t c = 0, incl = 0;
    if (threadIdx.x < kOrderBuckets) {
        c = s_count[threadIdx.x];
        incl = c;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t up = (uint32_t)__shfl_up((int)incl, off);
            if (lane >= off) incl += up;
        }
        if (lane == kWave - 1) s_wave[wave] = incl;
    }
    __syncthreads();
    if (threadIdx.x < kOrderBuckets) {
        uint32_t base = 0;
        for (int w = 0; w < wave; ++w) base += s_wave[w];
        s_count[threadIdx.x] = base + incl - c;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < p.tiles; t += kOrderThreads)
        p.order[atomicAdd(&s_count[bucket(tile_weight(p, t))], 1u)] = (uint32_t)t;
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
