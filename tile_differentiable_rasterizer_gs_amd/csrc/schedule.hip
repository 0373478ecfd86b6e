// Heaviest-first launch order for the per-tile compositing kernels.
//
// A compositing workgroup's run time grows with the work of its tile, and the tiles
// near the centre of a view carry several times the mean.  Launched in tile order,
// the heavy tiles start late and the frame ends with a few of them running on an
// otherwise idle chip.  Launching them first (longest-processing-time-first) evens
// the finish.  The order is a counting sort by weight on a logarithmic scale, 2048
// buckets of 1/64 octave (the leading bit of the weight and the six below it), so no
// pass for the largest weight is needed; order within a bucket is arbitrary, which
// only changes when a tile runs, never what it computes.  The counting sort itself
// (order_tiles) also runs as one workgroup of the super-tile place kernel.
#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void tile_order_kernel(TileOrderParams p) {
    __shared__ uint32_t s_count[kOrderBuckets];
    __shared__ uint32_t s_wave[kOrderThreads / kWave];
    order_tiles<kOrderThreads>(p, s_count, s_wave);
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
