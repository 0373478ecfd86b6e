// Front-to-back alpha compositing, one 256-thread workgroup (four wave64) per 16x16 tile.
//
// Lesson "3D Gaussian Splatting from scratch", section "La règle de composition
// alpha": C = sum_i alpha_i T_i c_i with T_i = prod_{j<i} (1 - alpha_j) and
// alpha_i = o_i exp(-d^T Sigma'^-1 d / 2); section "Étape 2" clamps alpha to at
// most 0.99 and samples pixel (row i, column j) at (x = j, y = i).
//
// Each thread owns one pixel.  The tile's depth-sorted list is walked in batches
// of 256 splats: every thread gathers one splat record into LDS, then all threads
// read the batch back as wave-wide broadcasts.  A pixel stops after the blend that
// brings T below GS_T_EPS; a wave whose 64 pixels have all stopped skips the rest
// of the batch, and the workgroup leaves the list once a barrier count shows no
// live pixel.  Pure VALU work (one v_exp_f32 per pair): no dense contraction, so no
// MFMA.
#include "gs_internal.h"

namespace gsr {
namespace {

template <bool kAux>
__global__ __launch_bounds__(kBlock) void composite_kernel(CompositeParams p) {
    // batch of splats in LDS; conic pre-scaled so that alpha = o * exp2(A dx^2 + B dx dy + C dy^2)
    __shared__ float s_u[kBlock], s_v[kBlock], s_A[kBlock], s_B[kBlock], s_C[kBlock], s_o[kBlock];
    __shared__ float s_r[kBlock], s_g[kBlock], s_b[kBlock];

    const int tile = blockIdx.x;
    const int tile_x = tile % p.tiles_x, tile_y = tile / p.tiles_x;
    const int px = tile_x * kTile + (threadIdx.x & (kTile - 1));
    const int py = tile_y * kTile + (threadIdx.x / kTile);
    const bool inside = px < p.width && py < p.height;
    const float fx = (float)px, fy = (float)py;

    const uint32_t start = p.ranges[2 * tile], end = p.ranges[2 * tile + 1];
    float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
    uint32_t blended = 0;
    bool done = !inside;
    constexpr float kLog2e = 1.4426950408889634f;

    for (uint32_t base = start; base < end; base += kBlock) {
        const uint32_t idx = base + threadIdx.x;
        if (idx < end) {
            const uint32_t gi = p.values[idx];
            const float4 *rec = reinterpret_cast<const float4 *>(p.splat) + (size_t)gi * 3;
            const float4 a = rec[0], b = rec[1], c = rec[2];
            s_u[threadIdx.x] = a.x;
            s_v[threadIdx.x] = a.y;
            s_A[threadIdx.x] = -0.5f * kLog2e * a.z;
            s_B[threadIdx.x] = -kLog2e * a.w;
            s_C[threadIdx.x] = -0.5f * kLog2e * b.x;
            s_o[threadIdx.x] = b.y;
            s_r[threadIdx.x] = b.z;
            s_g[threadIdx.x] = b.w;
            s_b[threadIdx.x] = c.x;
        }
        __syncthreads();
        const int count = (int)min<uint32_t>(kBlock, end - base);
        for (int j = 0; j < count; ++j) {
            if (__all(done)) break;
            const float dx = fx - s_u[j], dy = fy - s_v[j];
            const float q = s_A[j] * dx * dx + s_B[j] * dx * dy + s_C[j] * dy * dy;
            const float alpha = fminf(GS_ALPHA_MAX, s_o[j] * __builtin_amdgcn_exp2f(q));
            if (!done) {
                const float w = T * alpha;
                cr += w * s_r[j];
                cg += w * s_g[j];
                cb += w * s_b[j];
                T -= w;
                if (kAux) ++blended;
                done = T < GS_T_EPS;
            }
        }
        if (__syncthreads_count(!done) == 0) break;
    }

    if (inside) {
        const size_t pix = (size_t)py * p.width + px;
        p.image[pix * 3 + 0] = cr + T * p.bg[0];
        p.image[pix * 3 + 1] = cg + T * p.bg[1];
        p.image[pix * 3 + 2] = cb + T * p.bg[2];
        if (kAux) {
            if (p.final_T) p.final_T[pix] = T;
            if (p.n_blend) p.n_blend[pix] = blended;
        }
    }
    if (kAux && p.blend_total) {
        __shared__ unsigned long long s_sum;
        if (threadIdx.x == 0) s_sum = 0;
        __syncthreads();
        atomicAdd(&s_sum, (unsigned long long)blended);
        __syncthreads();
        if (threadIdx.x == 0 && s_sum) atomicAdd(p.blend_total, s_sum);
    }
}

}  // namespace

void launch_composite(const CompositeParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)(p.tiles_x * p.tiles_y);
    if (tiles == 0) return;
    if (p.final_T || p.n_blend || p.blend_total)
        composite_kernel<true><<<tiles, kBlock, 0, s>>>(p);
    else
        composite_kernel<false><<<tiles, kBlock, 0, s>>>(p);
}

}  // namespace gsr
