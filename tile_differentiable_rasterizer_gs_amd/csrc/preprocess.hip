// Per-Gaussian projection, SH colour and tile rectangle (one thread per Gaussian).
//
// Method: lesson "3D Gaussian Splatting from scratch" (aiengineeringfromscratch.com),
// sections "Ce qu'un Gaussien porte" (parameters; Sigma = R S S^T R^T),
// "L'étape de projection" (mu' = project(mu), Sigma' = J W Sigma W^T J^T),
// "Étape 5: De la 2D à la 3D" (quaternion rotation, S = diag(exp(log_scale)),
// camera-space z as the sort depth) and "Étape 6" (SH colour in the view direction).
//
// Everything that decides an integer (visibility, depth bits, mean, radius, tile
// rectangle) is evaluated in fp32 with FMA contraction disabled, sums taken left to
// right, and the scale exponential taken in fp64 then rounded: the result is a
// function of the inputs alone, so tile counts and keys are reproducible bit for bit
// on any IEEE-754 implementation that follows the same operation order.
//
// Memory: structure-of-arrays planes, one coalesced fp32 load per plane per thread.
// Reads 56 B (SH0) .. 236 B (SH3) per Gaussian, writes 80 B (+8 B for the
// depth-first sort keys).  HBM-bound; no LDS, no MFMA.
#include "gs_internal.h"

namespace gsr {
namespace {

__device__ inline float clamp_nan_low(float x, float lo, float hi) {
    if (!(x > lo)) x = lo;   // NaN -> lo
    if (x > hi) x = hi;
    return x;
}

// Real SH basis, degree <= 3, at unit direction (x, y, z); index k = l^2 + l + m.
// Degrees 0-2 with the constants and signs of the lesson's "Étape 6" evaluator;
// degree 3 with the real-SH normalisation sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!),
// times sqrt(2) for m != 0, odd m entering negated as in the printed degree-1 band.
template <int K>
__device__ inline void sh_basis(float x, float y, float z, float Y[K]) {
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

// 3D covariance of Gaussian g (lesson, "Ce qu'un Gaussien porte": Sigma = R S S^T R^T with R
// from the normalised quaternion and S = diag(exp(log_scale))), upper triangle
// (xx, xy, xz, yy, yz, zz).  binary32 in this order, no contraction: the same bits wherever it is
// evaluated (the preprocess, or the covariance cache it may read instead).
__device__ __forceinline__ void covariance3d(const float *quat, const float *log_scale, int n, int g, float cov[6]) {
#pragma clang fp contract(off)
    const float qw = quat[g], qx = quat[n + g], qy = quat[2 * n + g], qz = quat[3 * n + g];
    const float l0 = log_scale[g], l1 = log_scale[n + g], l2 = log_scale[2 * n + g];
    // rotation from the normalised quaternion (w, x, y, z), Hamilton convention
    const float nq = sqrtf(((qw * qw + qx * qx) + qy * qy) + qz * qz);
    const float w = qw / nq, x = qx / nq, y = qy / nq, z = qz / nq;
    float r[3][3];
    r[0][0] = 1.0f - 2.0f * (y * y + z * z);
    r[0][1] = 2.0f * (x * y - w * z);
    r[0][2] = 2.0f * (x * z + w * y);
    r[1][0] = 2.0f * (x * y + w * z);
    r[1][1] = 1.0f - 2.0f * (x * x + z * z);
    r[1][2] = 2.0f * (y * z - w * x);
    r[2][0] = 2.0f * (x * z - w * y);
    r[2][1] = 2.0f * (y * z + w * x);
    r[2][2] = 1.0f - 2.0f * (x * x + y * y);
    const float s[3] = {scale_activation(l0), scale_activation(l1), scale_activation(l2)};
    // M = R diag(s); Sigma = M M^T
    float m[3][3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) m[i][j] = r[i][j] * s[j];
    int k = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = i; j < 3; ++j) cov[k++] = (m[i][0] * m[j][0] + m[i][1] * m[j][1]) + m[i][2] * m[j][2];
}

template <int K>
__global__ __launch_bounds__(kBlock) void preprocess_kernel(PreprocessParams p) {
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= p.n) return;
    const int n = p.n;
    const float mx = p.mean[g], my = p.mean[n + g], mz = p.mean[2 * n + g];
    const float opac = p.opacity[g];

    float tx, ty, tz, u, v, A, B, C, radius;
    uint32_t x0 = 0, x1 = 0, y0 = 0, y1 = 0;
    uint32_t kept = 0;   // tile count under the exact-footprint rule
    bool visible;
    {
#pragma clang fp contract(off)
        const float *W = p.R;
        tx = ((W[0] * mx + W[1] * my) + W[2] * mz) + p.t[0];
        ty = ((W[3] * mx + W[4] * my) + W[5] * mz) + p.t[1];
        tz = ((W[6] * mx + W[7] * my) + W[8] * mz) + p.t[2];

        float cv[6];
        if (p.cov) {   // cached by gs_cache_covariance for these parameters
#pragma unroll
            for (int k = 0; k < 6; ++k) cv[k] = p.cov[(size_t)k * n + g];
        } else {
            covariance3d(p.quat, p.log_scale, n, g, cv);
        }
        const float S[3][3] = {{cv[0], cv[1], cv[2]}, {cv[1], cv[3], cv[4]}, {cv[2], cv[4], cv[5]}};
        // Jacobian of (fx x/z + cx, fy y/z + cy) at the camera-space mean, times W
        const float j00 = p.fx / tz;
        const float j02 = -(p.fx * tx) / (tz * tz);
        const float j11 = p.fy / tz;
        const float j12 = -(p.fy * ty) / (tz * tz);
        float T0[3], T1[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            T0[k] = j00 * W[k] + j02 * W[6 + k];
            T1[k] = j11 * W[3 + k] + j12 * W[6 + k];
        }
        float U0[3], U1[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            U0[k] = (T0[0] * S[0][k] + T0[1] * S[1][k]) + T0[2] * S[2][k];
            U1[k] = (T1[0] * S[0][k] + T1[1] * S[1][k]) + T1[2] * S[2][k];
        }
        const float a = (U0[0] * T0[0] + U0[1] * T0[1]) + U0[2] * T0[2];
        const float b = (U0[0] * T1[0] + U0[1] * T1[1]) + U0[2] * T1[2];
        const float c = (U1[0] * T1[0] + U1[1] * T1[1]) + U1[2] * T1[2];
        const float det = a * c - b * b;
        const float mid = 0.5f * (a + c);
        const float hd = 0.5f * (a - c);
        const float lam = mid + sqrtf(hd * hd + b * b);
        radius = ceilf(3.0f * sqrtf(lam));
        u = p.fx * (tx / tz) + p.cx;
        v = p.fy * (ty / tz) + p.cy;
        A = c / det;
        B = -b / det;
        C = a / det;
        visible = (tz > p.znear) && (det > 0.0f);
        if (visible) {
            x0 = (uint32_t)clamp_nan_low(floorf((u - radius) * 0.0625f), 0.0f, (float)p.tiles_x);
            x1 = (uint32_t)clamp_nan_low(floorf((u + radius) * 0.0625f) + 1.0f, 0.0f, (float)p.tiles_x);
            y0 = (uint32_t)clamp_nan_low(floorf((v - radius) * 0.0625f), 0.0f, (float)p.tiles_y);
            y1 = (uint32_t)clamp_nan_low(floorf((v + radius) * 0.0625f) + 1.0f, 0.0f, (float)p.tiles_y);
            visible = (x1 > x0) && (y1 > y0);
        }
        if (!visible) x0 = x1 = y0 = y1 = 0;
        if (p.ellipse) {
            const EllipseRec E = make_ellipse(a, b, c, det, u, v);
            p.ellipse[g] = E;
            if (visible) {   // exact footprint: the sum of the row spans
                uint32_t count = 0, sa, sb;
                for (uint32_t row = y0; row < y1; ++row) {
                    row_span(E, x0, x1, row, sa, sb);
                    count += sb - sa;
                }
                kept = count;
                visible = count > 0;
            }
        }
    }

    // view-dependent colour: SH expansion in the direction camera centre -> mean
    float rgb[3] = {0.0f, 0.0f, 0.0f};
    {
        const float dx = mx - p.cam_pos[0], dy = my - p.cam_pos[1], dz = mz - p.cam_pos[2];
        const float inv = 1.0f / sqrtf(dx * dx + dy * dy + dz * dz);
        float Y[K];
        sh_basis<K>(dx * inv, dy * inv, dz * inv, Y);
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int ch = 0; ch < 3; ++ch) rgb[ch] += Y[k] * p.sh[(size_t)(k * 3 + ch) * n + g];
    }

    // record: what compositing reads first (conic pre-scaled so alpha = o * exp2(A' dx^2 + B' dx dy + C' dy^2)),
    // then the exact conic, radius and depth
    constexpr float kNegHalfLog2e = -0.72134752044448170f;   // -log2(e) / 2
    float4 *rec = reinterpret_cast<float4 *>(p.splat) + (size_t)g * 4;
    rec[0] = make_float4(u, v, opac, kNegHalfLog2e * A);
    rec[1] = make_float4(2.0f * kNegHalfLog2e * B, kNegHalfLog2e * C, rgb[0], rgb[1]);
    rec[2] = make_float4(rgb[2], radius, A, B);
    rec[3] = make_float4(C, tz, 0.0f, 0.0f);
    p.depth[g] = tz;
    p.rect[g] = make_uint2(x0 | (x1 << 16), y0 | (y1 << 16));
    const uint32_t tile_count = !visible ? 0u : (p.ellipse ? kept : (x1 - x0) * (y1 - y0));
    p.tile_count[g] = tile_count;
    if (p.packed_count) p.packed_count[g] = pack_counts(tile_count, make_uint2(x0 | (x1 << 16), y0 | (y1 << 16)));
    if (p.depth_key) {
        // Gaussians without pairs sort last: interleaved with the others they would dilute the
        // pair listing's rank windows (a 2048-entry block would meet thousands of empty ranks)
        p.depth_key[g] = visible ? __float_as_uint(tz) : kNoPairsKey;
        p.depth_index[g] = (uint32_t)g;
    }
    if (p.depth_range) {
        // the wave's smallest and largest depth bits among Gaussians with pairs (positive
        // floats order like their bit patterns) into one of kDepthSlots slots
        uint32_t lo = visible ? __float_as_uint(tz) : 0xffffffffu, hi = visible ? __float_as_uint(tz) : 0u;
        const uint64_t live = __ballot(1);   // lanes past n have left
        if (live == ~0ull) {
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) {
                lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
                hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
            }
        } else {
            uint32_t wl = 0xffffffffu, wh = 0u;
            for (uint64_t m = live; m; m &= m - 1) {
                const int l = __builtin_ctzll(m);
                wl = min(wl, (uint32_t)__builtin_amdgcn_readlane((int)lo, l));
                wh = max(wh, (uint32_t)__builtin_amdgcn_readlane((int)hi, l));
            }
            lo = wl;
            hi = wh;
        }
        const uint32_t lane = __builtin_amdgcn_mbcnt_hi((uint32_t)(live >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)live, 0u));
        if (lane == 0 && lo <= hi) {
            const uint32_t slot = (blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave) & (kDepthSlots - 1);
            atomicMin(&p.depth_range[slot], lo);
            atomicMax(&p.depth_range[kDepthSlots + slot], hi);
        }
    }
}

// cov[k][g] = the k-th upper-triangle element of Gaussian g's 3D covariance.
__global__ __launch_bounds__(kBlock) void covariance_kernel(const float *__restrict__ quat,
                                                             const float *__restrict__ log_scale, int n,
                                                             float *__restrict__ cov) {
    const int g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= n) return;
    float cv[6];
    covariance3d(quat, log_scale, n, g, cv);
#pragma unroll
    for (int k = 0; k < 6; ++k) cov[(size_t)k * n + g] = cv[k];
}

__global__ __launch_bounds__(kBlock) void scale_activation_kernel(const float *__restrict__ in,
                                                                   float *__restrict__ out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) out[i] = scale_activation(in[i]);
}

}  // namespace

void launch_scale_activation(const float *log_scale, float *scale, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    scale_activation_kernel<<<(unsigned)(blocks < 8192 ? blocks : 8192), kBlock, 0, s>>>(log_scale, scale, n);
}

void launch_covariance(const float *quat, const float *log_scale, int32_t n, float *cov, hipStream_t s) {
    if (n <= 0) return;
    covariance_kernel<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, s>>>(quat, log_scale, n, cov);
}

void launch_preprocess(const PreprocessParams &p, hipStream_t s) {
    if (p.n <= 0) return;
    const dim3 grid((p.n + kBlock - 1) / kBlock);
    switch (p.sh_coeffs) {
        case 1: preprocess_kernel<1><<<grid, kBlock, 0, s>>>(p); break;
        case 4: preprocess_kernel<4><<<grid, kBlock, 0, s>>>(p); break;
        case 9: preprocess_kernel<9><<<grid, kBlock, 0, s>>>(p); break;
        default: preprocess_kernel<16><<<grid, kBlock, 0, s>>>(p); break;
    }
}

}  // namespace gsr
