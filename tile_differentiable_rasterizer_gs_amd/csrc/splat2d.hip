// The lesson's dense 2D splat rasteriser and its gradient.
//
// Lesson "3D Gaussian Splatting from scratch", sections "Étape 1: Un gaussien 2D" and
// "Étape 2: Rasteriser à éclaboussure en 2D": every splat is evaluated at every pixel
// (x = column, y = row), alpha = clamp(o exp(-d^T cov^-1 d / 2), 0, 0.99), splats are
// taken in ascending order of a per-splat depth scalar and composited front to back
// with the running transmittance, nothing stops early; "Étape 3"-"Étape 4" train such
// splats by gradient descent, so the rasteriser is differentiated in the means,
// covariances, colours and opacities (the depth only orders).
//
// Kernels:
//   splat2d_rank_kernel      rank of each splat in (depth, index) order (a total order
//                            on the depth bits, so the ranks are a permutation even for
//                            NaN depths); quadratic in n, meant for the lesson's sizes
//   splat2d_prepare_kernel   per splat, in rank order: mean, cov^-1 (general 2x2),
//                            colour, opacity
//   splat2d_forward_kernel   one 256-thread workgroup per 16x16 pixel tile; splats
//                            streamed through LDS in chunks; stores T before every
//                            splat (the backward's exact transmittance)
//   splat2d_backward_kernel  same tiling, splats walked back to front with the colour
//                            behind; per (splat, tile) the nine sums are reduced over the
//                            wave and the four waves and written to a fixed slot
//   splat2d_reduce_kernel    per splat: sum over tiles in tile order, then
//                            dL/dcov = -P^T M P^T with P = cov^-1 and M = sum dL/dq d d^T
// No floating-point atomics: gradients are bitwise reproducible.
#include "gs_internal.h"
#include "wave_reduce.h"

namespace gsr {
namespace {

constexpr int kS2Threads = 256;
constexpr int kS2Waves = kS2Threads / kWave;
constexpr int kS2Chunk = 512;      // splats per LDS chunk
constexpr int kS2Batch = 32;       // splats per reduction batch in the backward

// Per-splat record in rank order: mx, my, P00, P01 + P10, P11, opacity, r, g, b, P01, P10, index.
constexpr int kS2Rec = 12;

__device__ __forceinline__ uint32_t total_order_key(float d) {
    const uint32_t u = __float_as_uint(d);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kBlock) void splat2d_rank_kernel(const float *__restrict__ depths, int32_t n,
                                                              uint32_t *__restrict__ order) {
    __shared__ uint32_t s_key[kBlock];
    const int i = blockIdx.x * kBlock + threadIdx.x;
    const uint32_t mine = i < n ? total_order_key(depths[i]) : 0u;
    uint32_t rank = 0;
    for (int base = 0; base < n; base += kBlock) {
        __syncthreads();
        const int j = base + threadIdx.x;
        s_key[threadIdx.x] = j < n ? total_order_key(depths[j]) : 0xffffffffu;
        __syncthreads();
        const int m = min(kBlock, n - base);
        for (int k = 0; k < m; ++k) {
            const uint32_t other = s_key[k];
            rank += (other < mine) || (other == mine && base + k < i);
        }
    }
    if (i < n) order[rank] = (uint32_t)i;
}

__global__ __launch_bounds__(kBlock) void splat2d_prepare_kernel(Splat2DParams p, const uint32_t *__restrict__ order,
                                                                 float *__restrict__ rec) {
    const int r = blockIdx.x * kBlock + threadIdx.x;
    if (r >= p.n) return;
    const uint32_t g = order[r];
    const float a = p.covs[4 * g], b = p.covs[4 * g + 1], c = p.covs[4 * g + 2], d = p.covs[4 * g + 3];
    const float idet = 1.0f / (a * d - b * c);
    const float P00 = d * idet, P01 = -b * idet, P10 = -c * idet, P11 = a * idet;
    float *o = rec + (size_t)r * kS2Rec;
    o[0] = p.means[2 * g];
    o[1] = p.means[2 * g + 1];
    o[2] = P00;
    o[3] = P01 + P10;
    o[4] = P11;
    o[5] = p.opacities[g];
    o[6] = p.colours[3 * g];
    o[7] = p.colours[3 * g + 1];
    o[8] = p.colours[3 * g + 2];
    o[9] = P01;
    o[10] = P10;
    o[11] = __uint_as_float(g);
}

// alpha of one splat at one pixel; G = exp(-q/2), raw = o G
__device__ __forceinline__ float splat2d_alpha(const float *s, float x, float y, float &dx, float &dy, float &G,
                                               float &raw) {
    dx = x - s[0];
    dy = y - s[1];
    const float q = (s[2] * dx + s[3] * dy) * dx + s[4] * dy * dy;
    G = expf(-0.5f * q);
    raw = s[5] * G;
    return fminf(fmaxf(raw, 0.0f), 0.99f);
}

__device__ __forceinline__ void load_chunk(float *s_rec, const float *__restrict__ rec, int first, int count) {
    for (int k = threadIdx.x; k < count * kS2Rec; k += kS2Threads) s_rec[k] = rec[(size_t)first * kS2Rec + k];
}

__global__ __launch_bounds__(kS2Threads) void splat2d_forward_kernel(Splat2DParams p, const float *__restrict__ rec,
                                                                     float *__restrict__ trans) {
    __shared__ float s_rec[kS2Chunk * kS2Rec];
    const int tiles_x = (p.width + kTile - 1) / kTile;
    const int ix = (blockIdx.x % tiles_x) * kTile + (threadIdx.x & 15);
    const int iy = (blockIdx.x / tiles_x) * kTile + (threadIdx.x >> 4);
    const bool inside = ix < p.width && iy < p.height;
    const size_t pix = (size_t)iy * p.width + ix;
    const size_t npix = (size_t)p.width * p.height;
    const float x = (float)ix, y = (float)iy;
    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    for (int first = 0; first < p.n; first += kS2Chunk) {
        const int count = min(kS2Chunk, p.n - first);
        __syncthreads();
        load_chunk(s_rec, rec, first, count);
        __syncthreads();
        for (int k = 0; k < count; ++k) {
            const float *s = s_rec + k * kS2Rec;
            float dx, dy, G, raw;
            const float a = splat2d_alpha(s, x, y, dx, dy, G, raw);
            if (inside) trans[(size_t)(first + k) * npix + pix] = T;
            const float w = T * a;
            C0 = __builtin_fmaf(w, s[6], C0);
            C1 = __builtin_fmaf(w, s[7], C1);
            C2 = __builtin_fmaf(w, s[8], C2);
            T *= 1.0f - a;
        }
    }
    if (inside) {
        p.image[pix * 3 + 0] = C0 + T * p.bg[0];
        p.image[pix * 3 + 1] = C1 + T * p.bg[1];
        p.image[pix * 3 + 2] = C2 + T * p.bg[2];
    }
}

// Nine sums per (splat, tile): colour r, g, b; opacity; mean x, y; M00, M01, M11.
__global__ __launch_bounds__(kS2Threads) void splat2d_backward_kernel(Splat2DParams p, const float *__restrict__ rec,
                                                                      const float *__restrict__ trans,
                                                                      float *__restrict__ partial) {
    __shared__ float s_rec[kS2Chunk * kS2Rec];
    __shared__ float s_red[kS2Waves][kS2Batch][kPairGrad];
    const int tiles_x = (p.width + kTile - 1) / kTile;
    const int tiles = tiles_x * ((p.height + kTile - 1) / kTile);
    const int tile = blockIdx.x;
    const int ix = (tile % tiles_x) * kTile + (threadIdx.x & 15);
    const int iy = (tile / tiles_x) * kTile + (threadIdx.x >> 4);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const bool inside = ix < p.width && iy < p.height;
    const size_t pix = (size_t)iy * p.width + ix;
    const size_t npix = (size_t)p.width * p.height;
    const float x = (float)ix, y = (float)iy;
    float g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    if (inside) {
        g0 = p.grad_image[pix * 3 + 0];
        g1 = p.grad_image[pix * 3 + 1];
        g2 = p.grad_image[pix * 3 + 2];
    }
    float B0 = 0.0f, B1 = 0.0f, B2 = 0.0f;   // colour behind the current splat
    float bg_term = 0.0f;                     // T_final (bg . dL/dC), set at the last splat
    const int chunks = (p.n + kS2Chunk - 1) / kS2Chunk;
    for (int ci = chunks - 1; ci >= 0; --ci) {
        const int first = ci * kS2Chunk;
        const int count = min(kS2Chunk, p.n - first);
        __syncthreads();
        load_chunk(s_rec, rec, first, count);
        __syncthreads();
        for (int hi = count; hi > 0; hi -= kS2Batch) {
            const int lo = max(0, hi - kS2Batch);
            for (int k = hi - 1; k >= lo; --k) {
                const float *s = s_rec + k * kS2Rec;
                const int r = first + k;
                float dx, dy, G, raw;
                const float a = splat2d_alpha(s, x, y, dx, dy, G, raw);
                const float Ti = inside ? trans[(size_t)r * npix + pix] : 0.0f;
                if (r == p.n - 1) {
                    const float Tf = Ti * (1.0f - a);
                    bg_term = Tf * (p.bg[0] * g0 + p.bg[1] * g1 + p.bg[2] * g2);
                }
                const float cb0 = s[6] - B0, cb1 = s[7] - B1, cb2 = s[8] - B2;
                float d_a = Ti * (cb0 * g0 + cb1 * g1 + cb2 * g2) - bg_term / (1.0f - a);
                const bool smooth = raw >= 0.0f && raw <= 0.99f;
                d_a = smooth && inside ? d_a : 0.0f;
                const float w = inside ? a * Ti : 0.0f;
                B0 = __builtin_fmaf(a, cb0, B0);
                B1 = __builtin_fmaf(a, cb1, B1);
                B2 = __builtin_fmaf(a, cb2, B2);
                const float dq = -0.5f * raw * d_a;   // dL/dq
                // dq/dmean = -(P + P^T) d
                const float sx = s[2] * dx + 0.5f * s[3] * dy, sy = 0.5f * s[3] * dx + s[4] * dy;
                float v[kPairGrad];
                v[0] = w * g0;
                v[1] = w * g1;
                v[2] = w * g2;
                v[3] = G * d_a;
                v[4] = -2.0f * dq * sx;
                v[5] = -2.0f * dq * sy;
                v[6] = dq * dx * dx;
                v[7] = dq * dx * dy;
                v[8] = dq * dy * dy;
                float packed, last;
                reduce9(v, lane, packed, last);
                const float mine = gather9(packed, last, lane);
                if (lane < kPairGrad) s_red[wave][k - lo][lane] = mine;
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < (hi - lo) * kPairGrad; idx += kS2Threads) {
                const int k = idx / kPairGrad, c = idx - k * kPairGrad;
                const float sum = (s_red[0][k][c] + s_red[1][k][c]) + (s_red[2][k][c] + s_red[3][k][c]);
                partial[((size_t)(first + lo + k) * tiles + tile) * kPairGrad + c] = sum;
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kBlock) void splat2d_reduce_kernel(Splat2DParams p, const float *__restrict__ rec,
                                                                const float *__restrict__ partial, int tiles) {
    const int r = blockIdx.x * kBlock + threadIdx.x;
    if (r >= p.n) return;
    float acc[kPairGrad];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) acc[c] = 0.0f;
    for (int t = 0; t < tiles; ++t)
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) acc[c] += partial[((size_t)r * tiles + t) * kPairGrad + c];
    const float *s = rec + (size_t)r * kS2Rec;
    const uint32_t g = __float_as_uint(s[11]);
    p.g_colours[3 * g] = acc[0];
    p.g_colours[3 * g + 1] = acc[1];
    p.g_colours[3 * g + 2] = acc[2];
    p.g_opacities[g] = acc[3];
    p.g_means[2 * g] = acc[4];
    p.g_means[2 * g + 1] = acc[5];
    // dL/dcov = -P^T M P^T, M = [[M00, M01], [M01, M11]], P = [[P00, P01], [P10, P11]]
    const float P00 = s[2], P01 = s[9], P10 = s[10], P11 = s[4];
    const float M00 = acc[6], M01 = acc[7], M11 = acc[8];
    // X = P^T M: rows of P^T are (P00, P10), (P01, P11)
    const float X00 = P00 * M00 + P10 * M01, X01 = P00 * M01 + P10 * M11;
    const float X10 = P01 * M00 + P11 * M01, X11 = P01 * M01 + P11 * M11;
    // Y = X P^T
    p.g_covs[4 * g + 0] = -(X00 * P00 + X01 * P01);
    p.g_covs[4 * g + 1] = -(X00 * P10 + X01 * P11);
    p.g_covs[4 * g + 2] = -(X10 * P00 + X11 * P01);
    p.g_covs[4 * g + 3] = -(X10 * P10 + X11 * P11);
}

}  // namespace

void launch_splat2d_forward(const Splat2DParams &p, uint32_t *order, float *rec, float *trans, hipStream_t s) {
    if (p.n <= 0) {
        // no splat: the image is the background (the forward kernel with n = 0)
    } else {
        const unsigned g = (unsigned)((p.n + kBlock - 1) / kBlock);
        splat2d_rank_kernel<<<g, kBlock, 0, s>>>(p.depths, p.n, order);
        splat2d_prepare_kernel<<<g, kBlock, 0, s>>>(p, order, rec);
    }
    const unsigned tiles = (unsigned)(((p.width + kTile - 1) / kTile) * ((p.height + kTile - 1) / kTile));
    splat2d_forward_kernel<<<tiles, kS2Threads, 0, s>>>(p, rec, trans);
}

void launch_splat2d_backward(const Splat2DParams &p, const float *rec, const float *trans, float *partial,
                             hipStream_t s) {
    if (p.n <= 0) return;
    const int tiles = ((p.width + kTile - 1) / kTile) * ((p.height + kTile - 1) / kTile);
    splat2d_backward_kernel<<<(unsigned)tiles, kS2Threads, 0, s>>>(p, rec, trans, partial);
    splat2d_reduce_kernel<<<(unsigned)((p.n + kBlock - 1) / kBlock), kBlock, 0, s>>>(p, rec, partial, tiles);
}

}  // namespace gsr
