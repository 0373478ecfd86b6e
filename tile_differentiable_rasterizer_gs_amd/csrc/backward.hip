// Gradients of the rendered image with respect to the Gaussian parameters.
//
// Lesson "3D Gaussian Splatting from scratch", section "Pourquoi est-ce
// différenciable": projection, tile assignment, alpha compositing and SH
// evaluation are differentiable in (mu, q, s, opacity, SH coefficients).  The
// tile rectangles, the per-tile order and each pixel's stopping point are integer
// decisions of the forward pass and are held fixed.
//
// Three stages, all deterministic (no floating-point atomics):
//
// 1. composite_backward_kernel: one 256-thread workgroup per 16x16 tile, one pixel
//    per thread.  The tile's list is walked back to front from the largest blended
//    count of its pixels.  A pixel recovers T_i = T_{i+1} / (1 - alpha_i) from the
//    forward's final transmittance, recomputing alpha_i exactly as the forward did,
//    and accumulates the colour behind entry i, B_{i-1} = alpha_i c_i + (1 - alpha_i) B_i:
//      dL/dc_i     = alpha_i T_i dL/dC
//      dL/dalpha_i = T_i (c_i - B_i) . dL/dC - T_final (bg . dL/dC) / (1 - alpha_i)
//    and, where alpha_i = o G is below the 0.99 clamp, with G = exp(-Q/2),
//    Q = A dx^2 + 2 B dx dy + C dy^2:
//      dL/do = G dL/dalpha,  dL/dQ = -alpha dL/dalpha / 2,
//      dL/du = -2 (A dx + B dy) dL/dQ,  dL/dv = -2 (B dx + C dy) dL/dQ,
//      dL/d(A, B, C) = (dx^2, 2 dx dy, dy^2) dL/dQ.
//    The nine per-pixel values of each entry are summed over the wave (DPP row
//    shifts, then the four row totals) and over the four waves in a fixed order, and
//    written as one record at the pair's position in the listing (Gaussian-major),
//    so each Gaussian's records are contiguous.  Entries past the last one any pixel
//    of the tile blended get a zero record, so every record is written each call.
// 2. pair_reduce_*: sum of each Gaussian's records (one thread per Gaussian for short
//    lists, one workgroup per Gaussian for long ones) -> screen-space gradients.
// 3. project_backward_kernel: chain rule through the projection (conic <- 2D
//    covariance <- J W Sigma W^T J^T <- R(q) diag(exp(log s)), mean2d <- t) and the
//    SH colour (sections "L'étape de projection", "Étape 5", "Étape 6"), in fp32.
#include "gs_internal.h"

namespace gsr {
namespace {

// ---------------------------------------------------------------------------
// listing position of each Gaussian's first pair
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void pair_base_kernel(const uint32_t *__restrict__ order,
                                                           const uint32_t *__restrict__ offsets, int64_t n,
                                                           uint32_t *__restrict__ pair_base) {
    const int64_t r = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (r < n) pair_base[order[r]] = offsets[r];
}

// ---------------------------------------------------------------------------
// compositing backward
// ---------------------------------------------------------------------------
constexpr int kBwdThreads = 256;   // one pixel per thread, 4 waves of 16x4 pixels
constexpr int kBwdWaves = kBwdThreads / kWave;
constexpr int kBwdBatch = 64;      // entries staged per LDS batch

template <int kCtrl>
__device__ __forceinline__ float dpp_shifted(float v) {
    // row_shr: lane i reads lane i - n of its 16-lane row, 0 where that leaves the row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}

// Sum over the 64 lanes of a wave, returned uniformly (fixed association order).
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_shifted<0x111>(v);
    v += dpp_shifted<0x112>(v);
    v += dpp_shifted<0x114>(v);
    v += dpp_shifted<0x118>(v);   // lane 15 of each row now holds the row's sum
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return (r0 + r1) + (r2 + r3);
}

__global__ __launch_bounds__(kBwdThreads) void composite_backward_kernel(CompositeBackwardParams p) {
    // staged entries: u, v, A', B' | C', log2 o, 1/o, zero-opacity flag | A, B, C, r | g, b
    __shared__ float4 s_fwd[kBwdBatch], s_fwd2[kBwdBatch], s_conic[kBwdBatch];
    __shared__ float2 s_col[kBwdBatch];
    __shared__ uint32_t s_pos[kBwdBatch];
    __shared__ float s_red[kBwdWaves][kBwdBatch][kPairGrad];
    __shared__ uint32_t s_wave_max[kBwdWaves];

    const int tile = blockIdx.x;
    const int tile_x = tile % p.tiles_x, tile_y = tile / p.tiles_x;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int ix = tile_x * kTile + (threadIdx.x & 15);
    const int iy = tile_y * kTile + (threadIdx.x >> 4);
    const bool inside = ix < p.width && iy < p.height;
    const float x = (float)ix, y = (float)iy;

    float T = 0.0f, gC0 = 0.0f, gC1 = 0.0f, gC2 = 0.0f, bg_term = 0.0f;
    uint32_t n_mine = 0;
    if (inside) {
        const size_t pix = (size_t)iy * p.width + ix;
        T = p.final_T[pix];
        n_mine = p.n_blend[pix];
        gC0 = p.grad_image[pix * 3 + 0];
        gC1 = p.grad_image[pix * 3 + 1];
        gC2 = p.grad_image[pix * 3 + 2];
        bg_term = T * (p.bg[0] * gC0 + p.bg[1] * gC1 + p.bg[2] * gC2);
    }
    const uint32_t start = p.ranges[2 * tile], end = p.ranges[2 * tile + 1];
    // entries a pixel never reached need no work: start from the tile's largest count
    uint32_t m = n_mine;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) s_wave_max[wave] = m;
    __syncthreads();
    uint32_t n_max = 0;
#pragma unroll
    for (int w = 0; w < kBwdWaves; ++w) n_max = max(n_max, s_wave_max[w]);
    n_max = min(n_max, end - start);

    const uint32_t ty = (uint32_t)tile_y, tx = (uint32_t)tile_x;
    // entries no pixel of the tile reached contribute nothing: their records are zero
    for (uint32_t e = start + n_max + threadIdx.x; e < end; e += kBwdThreads) {
        const uint32_t g = p.values[e];
        const uint2 rc = p.rect[g];
        const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y0 = rc.y & 0xffffu;
        float *rec = p.pair_grad + (size_t)(p.pair_base[g] + (ty - y0) * (x1 - x0) + (tx - x0)) * kPairGrad;
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) rec[c] = 0.0f;
    }

    float B0 = 0.0f, B1 = 0.0f, B2 = 0.0f;   // colour behind the current entry
    for (int hi = (int)n_max; hi > 0; hi -= kBwdBatch) {
        const int lo = hi > kBwdBatch ? hi - kBwdBatch : 0;
        const int cnt = hi - lo;
        __syncthreads();   // the previous batch's staged entries and sums are consumed
        if ((int)threadIdx.x < cnt) {
            const uint32_t e = start + (uint32_t)(lo + threadIdx.x);
            const uint32_t g = p.values[e];
            const float4 *rec = reinterpret_cast<const float4 *>(p.splat) + (size_t)g * 4;
            const float4 r0 = rec[0], r1 = rec[1], r2 = rec[2], r3 = rec[3];
            const float o = r0.z;
            const bool zero_o = !(o > 0.0f);
            s_fwd[threadIdx.x] = make_float4(r0.x, r0.y, r0.w, r1.x);
            s_fwd2[threadIdx.x] = make_float4(r1.y, zero_o ? 0.0f : __log2f(o), zero_o ? 0.0f : 1.0f / o,
                                              zero_o ? 1.0f : 0.0f);
            s_conic[threadIdx.x] = make_float4(r2.z, r2.w, r3.x, r1.z);
            s_col[threadIdx.x] = make_float2(r1.w, r2.x);
            const uint2 rc = p.rect[g];
            const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y0 = rc.y & 0xffffu;
            s_pos[threadIdx.x] = p.pair_base[g] + (ty - y0) * (x1 - x0) + (tx - x0);
        }
        __syncthreads();
        for (int k = cnt - 1; k >= 0; --k) {
            const float4 f = s_fwd[k], f2 = s_fwd2[k], cn = s_conic[k];
            const float2 cl = s_col[k];
            const bool zero_o = f2.w != 0.0f;
            const float dx = x - f.x, dy = y - f.y;
            const float q = splat_exponent(dx, f.z, f.w * dy, splat_row_term(dy, f2.x, f2.y));
            const float raw = __builtin_amdgcn_exp2f(q);   // o G, or G when o == 0
            const float alpha = zero_o ? 0.0f : fminf(GS_ALPHA_MAX, raw);
            const bool active = (uint32_t)(lo + k) < n_mine;
            const float rinv = __builtin_amdgcn_rcpf(1.0f - alpha);
            const float Ti = T * rinv;
            const float c0 = cn.w, c1 = cl.x, c2 = cl.y;
            float d_alpha = Ti * ((c0 - B0) * gC0 + (c1 - B1) * gC1 + (c2 - B2) * gC2) - bg_term * rinv;
            const float wgt = alpha * Ti;
            const bool smooth = zero_o || raw < GS_ALPHA_MAX;   // below the clamp
            d_alpha = active ? d_alpha : 0.0f;
            const float G = zero_o ? raw : raw * f2.z;
            const float d_o = smooth ? G * d_alpha : 0.0f;
            const float dQ = smooth ? -0.5f * alpha * d_alpha : 0.0f;
            float v[kPairGrad];
            v[0] = -2.0f * dQ * (cn.x * dx + cn.y * dy);   // u
            v[1] = -2.0f * dQ * (cn.y * dx + cn.z * dy);   // v
            v[2] = dQ * dx * dx;                            // A
            v[3] = 2.0f * dQ * dx * dy;                     // B
            v[4] = dQ * dy * dy;                            // C
            v[5] = d_o;
            const float wa = active ? wgt : 0.0f;
            v[6] = wa * gC0;
            v[7] = wa * gC1;
            v[8] = wa * gC2;
            if (active) {
                B0 = __builtin_fmaf(alpha, c0 - B0, B0);
                B1 = __builtin_fmaf(alpha, c1 - B1, B1);
                B2 = __builtin_fmaf(alpha, c2 - B2, B2);
                T = Ti;
            }
#pragma unroll
            for (int c = 0; c < kPairGrad; ++c) {
                const float s = wave_sum(v[c]);
                if (lane == 0) s_red[wave][k][c] = s;
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < cnt * kPairGrad; idx += kBwdThreads) {
            const int k = idx / kPairGrad, c = idx - k * kPairGrad;
            const float s = (s_red[0][k][c] + s_red[1][k][c]) + (s_red[2][k][c] + s_red[3][k][c]);
            p.pair_grad[(size_t)s_pos[k] * kPairGrad + c] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// per-Gaussian sums of the pair records
// ---------------------------------------------------------------------------
constexpr uint32_t kShortList = 32;   // pairs summed by one thread; longer lists get a workgroup

__global__ __launch_bounds__(kBlock) void pair_reduce_short_kernel(PairReduceParams p) {
    const int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (g >= p.n) return;
    const uint32_t count = p.tile_count[g];
    if (count > kShortList) {
        p.big_list[atomicAdd(p.big_count, 1u)] = (uint32_t)g;
        return;
    }
    float acc[kPairGrad];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) acc[c] = 0.0f;
    const float *rec = p.pair_grad + (size_t)(count ? p.pair_base[g] : 0) * kPairGrad;
    for (uint32_t i = 0; i < count; ++i)
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) acc[c] += rec[(size_t)i * kPairGrad + c];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) p.screen[c * p.n + g] = acc[c];
}

__global__ __launch_bounds__(kBlock) void pair_reduce_long_kernel(PairReduceParams p) {
    __shared__ float s_part[kBlock / kWave][kPairGrad];
    const uint32_t total = *p.big_count;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    for (uint32_t b = blockIdx.x; b < total; b += gridDim.x) {
        const uint32_t g = p.big_list[b];
        const uint32_t count = p.tile_count[g];
        const float *rec = p.pair_grad + (size_t)p.pair_base[g] * kPairGrad;
        float acc[kPairGrad];
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) acc[c] = 0.0f;
        for (uint32_t i = threadIdx.x; i < count; i += kBlock)
#pragma unroll
            for (int c = 0; c < kPairGrad; ++c) acc[c] += rec[(size_t)i * kPairGrad + c];
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) {
            const float s = wave_sum(acc[c]);
            if (lane == 0) s_part[wave][c] = s;
        }
        __syncthreads();
        if (threadIdx.x < kPairGrad) {
            const int c = threadIdx.x;
            p.screen[c * p.n + g] = (s_part[0][c] + s_part[1][c]) + (s_part[2][c] + s_part[3][c]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// projection and colour backward
// ---------------------------------------------------------------------------
// d/d(x, y, z) of the SH basis polynomials of the forward pass (degree <= 3), contracted
// with per-coefficient weights wk: returns sum_k wk grad Y_k.
template <int K>
__device__ inline void sh_basis_vjp(float x, float y, float z, const float *wk, float g[3]) {
    g[0] = g[1] = g[2] = 0.0f;
    if constexpr (K > 1) {
        constexpr float k1 = 0.48860251190291992f;
        g[1] -= k1 * wk[1];
        g[2] += k1 * wk[2];
        g[0] -= k1 * wk[3];
    }
    if constexpr (K > 4) {
        constexpr float kxy = 1.0925484305920792f, k20 = 0.31539156525252005f, k22 = 0.54627421529603959f;
        g[0] += kxy * (y * wk[4] + z * wk[7]) - 2.0f * k20 * x * wk[6] + 2.0f * k22 * x * wk[8];
        g[1] += kxy * (x * wk[4] + z * wk[5]) - 2.0f * k20 * y * wk[6] - 2.0f * k22 * y * wk[8];
        g[2] += kxy * (y * wk[5] + x * wk[7]) + 4.0f * k20 * z * wk[6];
    }
    if constexpr (K > 9) {
        constexpr float k33 = 0.59004358992664352f, k32 = 2.8906114426405538f, k31 = 0.45704579946446572f;
        constexpr float k30 = 0.37317633259011540f, k32b = 1.4453057213202769f;
        const float xx = x * x, yy = y * y, zz = z * z;
        // Y9 = -k33 y (3xx - yy)
        g[0] += -6.0f * k33 * x * y * wk[9];
        g[1] += -3.0f * k33 * (xx - yy) * wk[9];
        // Y10 = k32 x y z
        g[0] += k32 * y * z * wk[10];
        g[1] += k32 * x * z * wk[10];
        g[2] += k32 * x * y * wk[10];
        // Y11 = -k31 y (4zz - xx - yy)
        g[0] += 2.0f * k31 * x * y * wk[11];
        g[1] += -k31 * (4.0f * zz - xx - 3.0f * yy) * wk[11];
        g[2] += -8.0f * k31 * y * z * wk[11];
        // Y12 = k30 z (2zz - 3xx - 3yy)
        g[0] += -6.0f * k30 * x * z * wk[12];
        g[1] += -6.0f * k30 * y * z * wk[12];
        g[2] += 3.0f * k30 * (2.0f * zz - xx - yy) * wk[12];
        // Y13 = -k31 x (4zz - xx - yy)
        g[0] += -k31 * (4.0f * zz - 3.0f * xx - yy) * wk[13];
        g[1] += 2.0f * k31 * x * y * wk[13];
        g[2] += -8.0f * k31 * x * z * wk[13];
        // Y14 = k32b z (xx - yy)
        g[0] += 2.0f * k32b * x * z * wk[14];
        g[1] += -2.0f * k32b * y * z * wk[14];
        g[2] += k32b * (xx - yy) * wk[14];
        // Y15 = -k33 x (xx - 3yy)
        g[0] += -3.0f * k33 * (xx - yy) * wk[15];
        g[1] += 6.0f * k33 * x * y * wk[15];
    }
}

template <int K>
__device__ inline void sh_basis_values(float x, float y, float z, float Y[K]) {
    Y[0] = 0.28209479177387814f;
    if constexpr (K > 1) {
        Y[1] = -0.48860251190291992f * y;
        Y[2] = 0.48860251190291992f * z;
        Y[3] = -0.48860251190291992f * x;
    }
    if constexpr (K > 4) {
        const float xx = x * x, yy = y * y, zz = z * z;
        Y[4] = 1.0925484305920792f * (x * y);
        Y[5] = 1.0925484305920792f * (y * z);
        Y[6] = 0.31539156525252005f * (2.0f * zz - xx - yy);
        Y[7] = 1.0925484305920792f * (x * z);
        Y[8] = 0.54627421529603959f * (xx - yy);
        if constexpr (K > 9) {
            Y[9] = -0.59004358992664352f * y * (3.0f * xx - yy);
            Y[10] = 2.8906114426405538f * (x * y) * z;
            Y[11] = -0.45704579946446572f * y * (4.0f * zz - xx - yy);
            Y[12] = 0.37317633259011540f * z * (2.0f * zz - 3.0f * xx - 3.0f * yy);
            Y[13] = -0.45704579946446572f * x * (4.0f * zz - xx - yy);
            Y[14] = 1.4453057213202769f * z * (xx - yy);
            Y[15] = -0.59004358992664352f * x * (xx - 3.0f * yy);
        }
    }
}

template <int K>
__global__ __launch_bounds__(kBlock) void project_backward_kernel(ProjectBackwardParams p) {
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= p.n) return;
    const int n = p.n;
    if (p.tile_count[g] == 0) {   // in no tile list: the image does not depend on it
        for (int i = 0; i < 3; ++i) p.g_mean[i * n + g] = 0.0f;
        for (int i = 0; i < 4; ++i) p.g_quat[i * n + g] = 0.0f;
        for (int i = 0; i < 3; ++i) p.g_log_scale[i * n + g] = 0.0f;
        p.g_opacity[g] = 0.0f;
        for (int i = 0; i < 3 * K; ++i) p.g_sh[(size_t)i * n + g] = 0.0f;
        if (p.g_mean2d) p.g_mean2d[g] = p.g_mean2d[n + g] = 0.0f;
        if (p.g_conic) p.g_conic[g] = p.g_conic[n + g] = p.g_conic[2 * n + g] = 0.0f;
        if (p.g_rgb) p.g_rgb[g] = p.g_rgb[n + g] = p.g_rgb[2 * n + g] = 0.0f;
        return;
    }
    float sg[kPairGrad];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) sg[c] = p.screen[(size_t)c * n + g];
    const float gu = sg[0], gv = sg[1], gA = sg[2], gB = sg[3], gC = sg[4];
    p.g_opacity[g] = sg[5];
    if (p.g_mean2d) { p.g_mean2d[g] = gu; p.g_mean2d[n + g] = gv; }
    if (p.g_conic) { p.g_conic[g] = gA; p.g_conic[n + g] = gB; p.g_conic[2 * n + g] = gC; }
    if (p.g_rgb) { p.g_rgb[g] = sg[6]; p.g_rgb[n + g] = sg[7]; p.g_rgb[2 * n + g] = sg[8]; }

    const float *W = p.R;
    const float mu[3] = {p.mean[g], p.mean[n + g], p.mean[2 * n + g]};
    const float q4[4] = {p.quat[g], p.quat[n + g], p.quat[2 * n + g], p.quat[3 * n + g]};

    // ---- forward quantities ----
    const float qn = sqrtf(q4[0] * q4[0] + q4[1] * q4[1] + q4[2] * q4[2] + q4[3] * q4[3]);
    const float qw = q4[0] / qn, qx = q4[1] / qn, qy = q4[2] / qn, qz = q4[3] / qn;
    float R[3][3];
    R[0][0] = 1.0f - 2.0f * (qy * qy + qz * qz);
    R[0][1] = 2.0f * (qx * qy - qw * qz);
    R[0][2] = 2.0f * (qx * qz + qw * qy);
    R[1][0] = 2.0f * (qx * qy + qw * qz);
    R[1][1] = 1.0f - 2.0f * (qx * qx + qz * qz);
    R[1][2] = 2.0f * (qy * qz - qw * qx);
    R[2][0] = 2.0f * (qx * qz - qw * qy);
    R[2][1] = 2.0f * (qy * qz + qw * qx);
    R[2][2] = 1.0f - 2.0f * (qx * qx + qy * qy);
    float s[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j] = expf(p.log_scale[j * n + g]);
    float M[3][3], S[3][3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) M[i][j] = R[i][j] * s[j];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) S[i][j] = M[i][0] * M[j][0] + M[i][1] * M[j][1] + M[i][2] * M[j][2];
    float t[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) t[i] = W[3 * i] * mu[0] + W[3 * i + 1] * mu[1] + W[3 * i + 2] * mu[2] + p.t[i];
    const float iz = 1.0f / t[2];
    const float j00 = p.fx * iz, j02 = -p.fx * t[0] * iz * iz;
    const float j11 = p.fy * iz, j12 = -p.fy * t[1] * iz * iz;
    float T0[3], T1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        T0[k] = j00 * W[k] + j02 * W[6 + k];
        T1[k] = j11 * W[3 + k] + j12 * W[6 + k];
    }
    float ST0[3], ST1[3];   // Sigma T0, Sigma T1
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        ST0[i] = S[i][0] * T0[0] + S[i][1] * T0[1] + S[i][2] * T0[2];
        ST1[i] = S[i][0] * T1[0] + S[i][1] * T1[1] + S[i][2] * T1[2];
    }
    const float a = T0[0] * ST0[0] + T0[1] * ST0[1] + T0[2] * ST0[2];
    const float b = T1[0] * ST0[0] + T1[1] * ST0[1] + T1[2] * ST0[2];
    const float c = T1[0] * ST1[0] + T1[1] * ST1[1] + T1[2] * ST1[2];
    const float idet = 1.0f / (a * c - b * b);
    const float idet2 = idet * idet;

    // ---- conic (A, B, C) = (c, -b, a) / det  ->  2D covariance ----
    const float ga = (-c * c * gA + b * c * gB - b * b * gC) * idet2;
    const float gb = (2.0f * b * c * gA - (a * c + b * b) * gB + 2.0f * a * b * gC) * idet2;
    const float gc = (-b * b * gA + a * b * gB - a * a * gC) * idet2;

    // ---- (a, b, c) = (T0.S.T0, T0.S.T1, T1.S.T1) -> T0, T1 and Sigma ----
    float gT0[3], gT1[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        gT0[i] = 2.0f * ga * ST0[i] + gb * ST1[i];
        gT1[i] = gb * ST0[i] + 2.0f * gc * ST1[i];
    }
    float gS[3][3];   // symmetric
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            gS[i][j] = ga * T0[i] * T0[j] + 0.5f * gb * (T0[i] * T1[j] + T1[i] * T0[j]) + gc * T1[i] * T1[j];

    // ---- T rows = J W  ->  J entries  ->  camera-space mean ----
    float gj00 = 0.0f, gj02 = 0.0f, gj11 = 0.0f, gj12 = 0.0f;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        gj00 += gT0[k] * W[k];
        gj02 += gT0[k] * W[6 + k];
        gj11 += gT1[k] * W[3 + k];
        gj12 += gT1[k] * W[6 + k];
    }
    const float iz2 = iz * iz, iz3 = iz2 * iz;
    float gt[3];
    gt[0] = -p.fx * iz2 * gj02 + p.fx * iz * gu;
    gt[1] = -p.fy * iz2 * gj12 + p.fy * iz * gv;
    gt[2] = -p.fx * iz2 * gj00 + 2.0f * p.fx * t[0] * iz3 * gj02 - p.fy * iz2 * gj11 +
            2.0f * p.fy * t[1] * iz3 * gj12 - p.fx * t[0] * iz2 * gu - p.fy * t[1] * iz2 * gv;
    float gmu[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) gmu[i] = W[i] * gt[0] + W[3 + i] * gt[1] + W[6 + i] * gt[2];

    // ---- Sigma = M M^T, M = R diag(s) ----
    float gR[3][3], gs[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const float gM = 2.0f * (gS[i][0] * M[0][j] + gS[i][1] * M[1][j] + gS[i][2] * M[2][j]);
            gR[i][j] = gM * s[j];
            gs[j] += gM * R[i][j];
        }
#pragma unroll
    for (int j = 0; j < 3; ++j) p.g_log_scale[j * n + g] = gs[j] * s[j];

    // ---- R of the unit quaternion, then the normalisation ----
    float gq[4];
    gq[0] = 2.0f * (qz * (gR[1][0] - gR[0][1]) + qy * (gR[0][2] - gR[2][0]) + qx * (gR[2][1] - gR[1][2]));
    gq[1] = 2.0f * (qy * (gR[0][1] + gR[1][0]) + qz * (gR[0][2] + gR[2][0]) + qw * (gR[2][1] - gR[1][2]) -
                    2.0f * qx * (gR[1][1] + gR[2][2]));
    gq[2] = 2.0f * (qx * (gR[0][1] + gR[1][0]) + qz * (gR[1][2] + gR[2][1]) + qw * (gR[0][2] - gR[2][0]) -
                    2.0f * qy * (gR[0][0] + gR[2][2]));
    gq[3] = 2.0f * (qx * (gR[0][2] + gR[2][0]) + qy * (gR[1][2] + gR[2][1]) + qw * (gR[1][0] - gR[0][1]) -
                    2.0f * qz * (gR[0][0] + gR[1][1]));
    const float qh[4] = {qw, qx, qy, qz};
    const float dot = qh[0] * gq[0] + qh[1] * gq[1] + qh[2] * gq[2] + qh[3] * gq[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) p.g_quat[i * n + g] = (gq[i] - qh[i] * dot) / qn;

    // ---- colour: rgb = sum_k Y_k(d) sh_k with d = (mean - C) / |mean - C| ----
    float dir[3] = {mu[0] - p.cam_pos[0], mu[1] - p.cam_pos[1], mu[2] - p.cam_pos[2]};
    const float idn = 1.0f / sqrtf(dir[0] * dir[0] + dir[1] * dir[1] + dir[2] * dir[2]);
    const float d[3] = {dir[0] * idn, dir[1] * idn, dir[2] * idn};
    float Y[K], wk[K];
    sh_basis_values<K>(d[0], d[1], d[2], Y);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float acc = 0.0f;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
            const size_t plane = (size_t)(k * 3 + ch) * n + g;
            p.g_sh[plane] = Y[k] * sg[6 + ch];
            acc += p.sh[plane] * sg[6 + ch];
        }
        wk[k] = acc;
    }
    float gd[3];
    sh_basis_vjp<K>(d[0], d[1], d[2], wk, gd);
    const float radial = gd[0] * d[0] + gd[1] * d[1] + gd[2] * d[2];
#pragma unroll
    for (int i = 0; i < 3; ++i) p.g_mean[i * n + g] = gmu[i] + (gd[i] - d[i] * radial) * idn;
}

}  // namespace

void launch_pair_base(const uint32_t *order, const uint32_t *offsets, int64_t n, uint32_t *pair_base,
                      hipStream_t s) {
    if (n <= 0) return;
    pair_base_kernel<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(order, offsets, n, pair_base);
}

void launch_composite_backward(const CompositeBackwardParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)(p.tiles_x * p.tiles_y);
    if (tiles == 0) return;
    composite_backward_kernel<<<tiles, kBwdThreads, 0, s>>>(p);
}

void launch_pair_reduce(const PairReduceParams &p, hipStream_t s) {
    if (p.n <= 0) return;
    launch_fill_u32(p.big_count, 0u, 1, s);
    pair_reduce_short_kernel<<<(unsigned)((p.n + kBlock - 1) / kBlock), kBlock, 0, s>>>(p);
    const int64_t groups = p.n < 2048 ? p.n : 2048;
    pair_reduce_long_kernel<<<(unsigned)groups, kBlock, 0, s>>>(p);
}

void launch_project_backward(const ProjectBackwardParams &p, hipStream_t s) {
    if (p.n <= 0) return;
    const dim3 grid((p.n + kBlock - 1) / kBlock);
    switch (p.sh_coeffs) {
        case 1: project_backward_kernel<1><<<grid, kBlock, 0, s>>>(p); break;
        case 4: project_backward_kernel<4><<<grid, kBlock, 0, s>>>(p); break;
        case 9: project_backward_kernel<9><<<grid, kBlock, 0, s>>>(p); break;
        default: project_backward_kernel<16><<<grid, kBlock, 0, s>>>(p); break;
    }
}

}  // namespace gsr
