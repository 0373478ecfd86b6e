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
// 1. composite_backward_kernel: one wave64 per 16x16 tile, four pixels of a row per
//    lane.  The tile's list is walked back to front from the largest blended
//    count of its pixels.  A pixel recovers T_i = T_{i+1} / (1 - alpha_i) from the
//    forward's final transmittance, recomputing alpha_i exactly as the forward did,
//    and accumulates the colour behind entry i, B_{i-1} = alpha_i c_i + (1 - alpha_i) B_i
//    (only its product with dL/dC is needed, and carried):
//      dL/dc_i     = alpha_i T_i dL/dC
//      dL/dalpha_i = T_i (c_i - B_i) . dL/dC - T_final (bg . dL/dC) / (1 - alpha_i)
//    and, where alpha_i = o G is below the 0.99 clamp, with G = exp(-Q/2),
//    Q = A dx^2 + 2 B dx dy + C dy^2:
//      dL/do = G dL/dalpha,  dL/dQ = -alpha dL/dalpha / 2,
//      dL/du = -2 (A dx + B dy) dL/dQ,  dL/dv = -2 (B dx + C dy) dL/dQ,
//      dL/d(A, B, C) = (dx^2, 2 dx dy, dy^2) dL/dQ.
//    A lane sums its four pixels into three moments of d_i = alpha_i dL/dalpha_i
//    (sum d, sum d dx, sum d dx^2), from which the conic and mean terms follow linearly
//    with the Gaussian's conic; five moments (times powers of dy) and the opacity and
//    colour sums, nine values per entry, are summed over the wave through LDS and
//    written as one record at the pair's position in the
//    listing (Gaussian-major), so each Gaussian's records are contiguous.  Entries
//    past the last one any pixel of the tile blended contribute nothing and get no
//    record: the tile publishes the (depth bits, index) key of its deepest walked
//    entry, and the next stage reads exactly the records at or below it.
// 2. gaussian_backward_kernel: sum of each Gaussian's records (a 16-lane row per
//    Gaussian, reading consecutive records; the whole workgroup for a list longer than
//    512 records), then the chain rule through the projection
//    (conic <- 2D covariance <- J W Sigma W^T J^T <- R(q) diag(exp(log s)), mean2d <-
//    t) and the SH colour (sections "L'étape de projection", "Étape 5", "Étape 6"),
//    in fp32.  Records are laid out in Gaussian-index order (pair_base = exclusive
//    prefix of tile counts over the index), so this stage reads and writes the
//    parameter planes coalesced.
#include "gs_internal.h"
#include "wave_reduce.h"

namespace gsr {
namespace {

// ---------------------------------------------------------------------------
// compositing backward
// ---------------------------------------------------------------------------
// One wave64 per tile; lane l owns the four pixels (4i + (l & 3), l >> 2), i = 0..3,
// of one row, which share dy and the row terms of the exponent.
constexpr int kBwdThreads = kWave;
constexpr int kBwdPix = 4;         // pixels per lane
constexpr int kBwdBatch = 64;      // entries staged per LDS batch

// Per-lane state of the reverse walk: four pixels of one row.
struct BwdLane {
    float y;
    float x[kBwdPix], T[kBwdPix], gC[kBwdPix][3], bg_term[kBwdPix];
    float BgC[kBwdPix];    // B . dL/dC, B the colour behind the current entry
    uint32_t n[kBwdPix];   // entries the pixel blended in the forward

    // Entry idx of the tile list (staged f, f2, cn, cl): steps the four pixels back over it
    // and returns the lane's nine partial sums (S1, dy S0, S2, dy S1, dy^2 S0, opacity, r, g, b).
    __device__ __forceinline__ void entry(const float4 f, const float4 f2, const float4 cl,
                                          uint32_t idx, float v[kPairGrad]) {
        const float c[3] = {cl.w, cl.x, cl.y};
        const float dy = y - f.y;
        const float bdy = f.w * dy;
        const float row = splat_row_term(dy, f2.x, f2.y);
        // d_i = dL/dalpha_i * alpha_i where alpha is below the clamp (else 0);
        // S0 = sum d_i, S1 = sum d_i dx_i, S2 = sum d_i dx_i^2
        float S0 = 0.0f, S1 = 0.0f, S2 = 0.0f, So = 0.0f, Sc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < kBwdPix; ++i) {
            const float dx = x[i] - f.x;
            // raw = min(1, 2^q) = alpha / 0.99 (G itself when o = 0), as the forward computed it
            const float raw = splat_alpha_scaled(splat_exponent(dx, f.z, bdy, row));
            const bool active = idx < n[i];
            const float alpha = active ? f2.w * raw : 0.0f;
            const float rinv = __builtin_amdgcn_rcpf(1.0f - alpha);
            const float Ti = T[i] * rinv;
            // (c - B) . dL/dC, with B . dL/dC carried as one number: B_{i-1} = B_i + alpha (c - B_i)
            // gives B_{i-1} . dL/dC = B_i . dL/dC + alpha (c - B_i) . dL/dC
            const float dot = (c[0] * gC[i][0] + c[1] * gC[i][1] + c[2] * gC[i][2]) - BgC[i];
            // (an inactive pixel has alpha = 0, so 1/(1 - alpha) = 1 exactly and Ti = T; its
            // dL/dalpha is finite and reaches the sums only through `smooth`, which is false)
            const float d_alpha = __builtin_fmaf(Ti, dot, -bg_term[i] * rinv);
            const float w = alpha * Ti;
            Sc[0] = __builtin_fmaf(w, gC[i][0], Sc[0]);
            Sc[1] = __builtin_fmaf(w, gC[i][1], Sc[1]);
            Sc[2] = __builtin_fmaf(w, gC[i][2], Sc[2]);
            BgC[i] = __builtin_fmaf(alpha, dot, BgC[i]);
            T[i] = Ti;
            const bool smooth = active && raw < cl.z;
            So = __builtin_fmaf(smooth ? raw * f2.z : 0.0f, d_alpha, So);
            const float d = (smooth ? alpha : 0.0f) * d_alpha;
            S0 += d;
            const float t = d * dx;
            S1 += t;
            S2 = __builtin_fmaf(t, dx, S2);
        }
        // dL/dQ_i = -d_i / 2 with Q = A dx^2 + 2 B dx dy + C dy^2:
        //   dL/du = A S1 + B dy S0,  dL/dv = B S1 + C dy S0,
        //   dL/dA = -S2 / 2,  dL/dB = -dy S1,  dL/dC = -dy^2 S0 / 2
        // all linear in five moments with the Gaussian's own conic: the record carries the
        // moments (S1, dy S0, S2, dy S1, dy^2 S0) and the per-Gaussian stage applies the conic
        // once to their sum over the Gaussian's records
        const float dyS0 = dy * S0;
        v[0] = S1;
        v[1] = dyS0;
        v[2] = S2;
        v[3] = dy * S1;
        v[4] = dy * dyS0;
        v[5] = So;
        v[6] = Sc[0];
        v[7] = Sc[1];
        v[8] = Sc[2];
    }
};

// Wave sums of the nine partials, stored as one record.  The walk is bound by VALU issue,
// so the sums go through LDS rather than a butterfly: lane l writes its nine values to
// s_red[c][l]; then lane l adds the eight values of component l / 8 held by lanes
// 8 (l % 8) .. 8 (l % 8) + 7 (two 16-byte reads, a fixed add tree), and the same block of
// component 8; three row moves (lane ^ 1, lane ^ 2, lane i with 7 - i) finish each sum over
// its eight blocks.  About ten VALU instructions fewer per entry; the shuffling moves to the
// LDS pipe.  One wave per workgroup: its LDS accesses complete in order.
__device__ __forceinline__ float sum8(const float4 a, const float4 b) {
    return ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
}

__device__ __forceinline__ void store_record(const float v[kPairGrad], int lane, float *s_red /*[9][64]*/,
                                             float *rec) {
    // compiler-only ordering: the previous record's reads before these writes, the writes
    // before the reads of other lanes' values (the wave's LDS accesses run in program order)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) s_red[c * kWave + lane] = v[c];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const float4 *blk = reinterpret_cast<const float4 *>(s_red) + 2 * (lane & 7);
    const float4 *mine = blk + (lane >> 3) * (kWave / 4);
    const float4 *last = blk + 8 * (kWave / 4);
    float t = sum8(mine[0], mine[1]);
    float q = sum8(last[0], last[1]);
    t += dpp_moved<0xB1>(t);
    q += dpp_moved<0xB1>(q);
    t += dpp_moved<0x4E>(t);
    q += dpp_moved<0x4E>(q);
    t += dpp_moved<0x141>(t);
    q += dpp_moved<0x141>(q);
    // component j < 8 from lane 8 j, component 8 from lane 1
    const bool first = (lane & 7) == 0;
    if (first || lane == 1) rec[first ? lane >> 3 : 8] = first ? t : q;
}

__global__ __launch_bounds__(kBwdThreads) void composite_backward_kernel(CompositeBackwardParams p) {
    // staged entries: u, v, A', B' | C', log2(o / 0.99), 0.99 / o (1 when o = 0), alpha cap |
    // g, b, value of min(1, 2^q) below which alpha is smooth (1, or inf when o = 0), r
    __shared__ float4 s_fwd[kBwdBatch], s_fwd2[kBwdBatch];
    __shared__ float4 s_col[kBwdBatch];
    __shared__ uint32_t s_pos[kBwdBatch];
    __shared__ __align__(16) float s_red[kPairGrad * kWave];   // store_record's transpose

    const int tile = p.tile_order ? (int)p.tile_order[blockIdx.x] : (int)blockIdx.x;
    const int tile_x = tile % p.tiles_x, tile_y = tile / p.tiles_x;
    const int lane = threadIdx.x;
    const int iy = tile_y * kTile + (lane >> 2);

    BwdLane px;
    px.y = (float)iy;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kBwdPix; ++i) {
        const int ix = tile_x * kTile + 4 * i + (lane & 3);
        px.x[i] = (float)ix;
        px.T[i] = 0.0f;
        px.gC[i][0] = px.gC[i][1] = px.gC[i][2] = 0.0f;
        px.bg_term[i] = 0.0f;
        px.BgC[i] = 0.0f;
        px.n[i] = 0;
        if (ix < p.width && iy < p.height) {
            const size_t pix = (size_t)iy * p.width + ix;
            px.T[i] = p.final_T[pix];
            px.n[i] = p.n_blend[pix];
            px.gC[i][0] = p.grad_image[pix * 3 + 0];
            px.gC[i][1] = p.grad_image[pix * 3 + 1];
            px.gC[i][2] = p.grad_image[pix * 3 + 2];
            px.bg_term[i] = px.T[i] * (p.bg[0] * px.gC[i][0] + p.bg[1] * px.gC[i][1] + p.bg[2] * px.gC[i][2]);
        }
        m = max(m, px.n[i]);
    }
    const uint32_t start = p.ranges[2 * tile], end = p.ranges[2 * tile + 1];
    // entries no pixel reached need no work: start from the tile's largest count
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    const uint32_t n_max = min(m, end - start);

    const uint32_t ty = (uint32_t)tile_y, tx = (uint32_t)tile_x;
    // ... and contribute nothing: no record is written for them.  The list is sorted by
    // (depth bits, index), so the key of the deepest walked entry tells the per-Gaussian
    // stage which records exist.
    if (lane == 0) {
        unsigned long long cut = 0;
        if (n_max > 0) {
            const uint32_t g = p.values[start + n_max - 1];
            const float4 r3 = reinterpret_cast<const float4 *>(p.splat)[(size_t)g * 4 + 3];
            cut = ((unsigned long long)__float_as_uint(r3.y) << 32) | g;
        }
        p.cut[tile] = cut;
    }

    // The wave sum of an entry's partials is a chain of cross-lane steps; it is done one
    // entry late, so that it overlaps the pixel work of the next entry.
    float held[kPairGrad];
    uint32_t held_pos = 0;
    bool holding = false;
    for (int hi = (int)n_max; hi > 0; hi -= kBwdBatch) {
        const int lo = hi > kBwdBatch ? hi - kBwdBatch : 0;
        const int cnt = hi - lo;
        __syncthreads();   // the previous batch's staged entries are consumed
        if (lane < cnt) {
            const uint32_t e = start + (uint32_t)(lo + lane);
            const uint32_t g = p.values[e];
            const float4 *rec = reinterpret_cast<const float4 *>(p.splat) + (size_t)g * 4;
            const float4 r0 = rec[0], r1 = rec[1];
            const float b = reinterpret_cast<const float *>(rec)[8];
            const float o = r0.z;
            const bool zero_o = !(o > 0.0f);
            s_fwd[lane] = make_float4(r0.x, r0.y, r0.w, r1.x);
            // the exponent carries log2(o / 0.99) as in the forward, so min(1, 2^q) = alpha / 0.99
            // and G = min(1, 2^q) 0.99 / o below the clamp; o = 0: alpha is 0 and 2^q (with
            // the log term taken as 0) is G itself, never clamped
            s_fwd2[lane] = make_float4(r1.y, zero_o ? 0.0f : splat_log2_scaled_opacity(o),
                                       zero_o ? 1.0f : GS_ALPHA_MAX / o, zero_o ? 0.0f : GS_ALPHA_MAX);
            s_col[lane] = make_float4(r1.w, b, zero_o ? INFINITY : 1.0f, r1.z);
            const uint2 rc = p.rect[g];
            const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y0 = rc.y & 0xffffu;
            s_pos[lane] = p.pair_base[g] + (p.ellipse ? kept_index(p.ellipse[g], x0, x1, y0, tx, ty)
                                                      : (ty - y0) * (x1 - x0) + (tx - x0));
        }
        __syncthreads();
        int k = cnt - 1;
        if (!holding) {   // the tile's first entry
            px.entry(s_fwd[k], s_fwd2[k], s_col[k], (uint32_t)(lo + k), held);
            held_pos = s_pos[k];
            holding = true;
            --k;
        }
        for (; k >= 0; --k) {
            float v[kPairGrad];
            px.entry(s_fwd[k], s_fwd2[k], s_col[k], (uint32_t)(lo + k), v);
            store_record(held, lane, s_red, p.pair_grad + (size_t)held_pos * kPairStride);
#pragma unroll
            for (int c = 0; c < kPairGrad; ++c) held[c] = v[c];
            held_pos = s_pos[k];
        }
    }
    if (holding) store_record(held, lane, s_red, p.pair_grad + (size_t)held_pos * kPairStride);
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

// Activated scale in the chain's precision: binary32 expf, or the binary64 exp.
__device__ __forceinline__ float chain_scale(float ls, float) { return expf(ls); }
__device__ __forceinline__ double chain_scale(float ls, double) { return exp((double)ls); }

// Chain rule of one Gaussian, from its summed record (S1, dy S0, S2, dy S1, dy^2 S0,
// opacity, r, g, b) to its parameters.  A Gaussian in no tile list (live false, sums zero)
// gets zero gradients through the same stores, so that a wave writes each parameter plane
// with one store instruction: two partial-wave stores to the same lines cost extra HBM
// writes.
//
// Geometric part: the moments m (S1, dy S0, S2, dy S1, dy^2 S0) through the conic, the 2D
// covariance, Sigma and J to the scales, rotation and mean; writes dL/d(u, v) (optional
// plane), dL/dlog_scale and dL/dquat, returns the mean's share in gmu and a c / det.
// Real is the precision of the chain.  For a thin footprint the derivative of the conic
// (an inverse) and of Sigma' = T Sigma T^T cancel in proportion to the 2D covariance's
// condition: in binary32 that rounding alone outgrew a thin axis' log-scale gradient once
// a c / det passed ~100, so the binary32 pass queues such Gaussians for a binary64 one.
template <typename Real>
__device__ inline float geometric_vjp(const GaussianBackwardParams &p, int g, const float m[5], bool live,
                                      float gmu[3]) {
    const int n = p.n;
    auto out = [live](Real v) { return live ? (float)v : 0.0f; };   // culled Gaussians may give inf or NaN
    const float gA = -0.5f * m[2], gB = -m[3], gC = -0.5f * m[4];   // dL/d(A, B, C) of the conic
    const float mu[3] = {p.mean[g], p.mean[n + g], p.mean[2 * n + g]};
    Real W[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) W[i] = (Real)p.R[i];
    const Real q4[4] = {p.quat[g], p.quat[n + g], p.quat[2 * n + g], p.quat[3 * n + g]};
    const Real one = 1, two = 2, half = 0.5;

    // ---- forward quantities ----
    const Real qn = sqrt(q4[0] * q4[0] + q4[1] * q4[1] + q4[2] * q4[2] + q4[3] * q4[3]);
    const Real qw = q4[0] / qn, qx = q4[1] / qn, qy = q4[2] / qn, qz = q4[3] / qn;
    Real R[3][3];
    R[0][0] = one - two * (qy * qy + qz * qz);
    R[0][1] = two * (qx * qy - qw * qz);
    R[0][2] = two * (qx * qz + qw * qy);
    R[1][0] = two * (qx * qy + qw * qz);
    R[1][1] = one - two * (qx * qx + qz * qz);
    R[1][2] = two * (qy * qz - qw * qx);
    R[2][0] = two * (qx * qz - qw * qy);
    R[2][1] = two * (qy * qz + qw * qx);
    R[2][2] = one - two * (qx * qx + qy * qy);
    Real s[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j] = chain_scale(p.log_scale[j * n + g], Real(0));
    Real M[3][3], S[3][3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) M[i][j] = R[i][j] * s[j];
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) S[i][j] = M[i][0] * M[j][0] + M[i][1] * M[j][1] + M[i][2] * M[j][2];
    Real t[3];
#pragma unroll
    for (int i = 0; i < 3; ++i)
        t[i] = W[3 * i] * (Real)mu[0] + W[3 * i + 1] * (Real)mu[1] + W[3 * i + 2] * (Real)mu[2] + (Real)p.t[i];
    const Real fx = p.fx, fy = p.fy;
    const Real iz = one / t[2];
    const Real j00 = fx * iz, j02 = -fx * t[0] * iz * iz;
    const Real j11 = fy * iz, j12 = -fy * t[1] * iz * iz;
    Real T0[3], T1[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        T0[k] = j00 * W[k] + j02 * W[6 + k];
        T1[k] = j11 * W[3 + k] + j12 * W[6 + k];
    }
    Real ST0[3], ST1[3];   // Sigma T0, Sigma T1
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        ST0[i] = S[i][0] * T0[0] + S[i][1] * T0[1] + S[i][2] * T0[2];
        ST1[i] = S[i][0] * T1[0] + S[i][1] * T1[1] + S[i][2] * T1[2];
    }
    const Real a = T0[0] * ST0[0] + T0[1] * ST0[1] + T0[2] * ST0[2];
    const Real b = T1[0] * ST0[0] + T1[1] * ST0[1] + T1[2] * ST0[2];
    const Real c = T1[0] * ST1[0] + T1[1] * ST1[1] + T1[2] * ST1[2];
    const Real det = a * c - b * b;
    const Real idet = one / det;
    const Real idet2 = idet * idet;
    // dL/du = A S1 + B dy S0, dL/dv = B S1 + C dy S0 with the conic (A, B, C) = (c, -b, a) / det
    const Real cA = c * idet, cB = -b * idet, cC = a * idet;
    const Real gu = cA * (Real)m[0] + cB * (Real)m[1], gv = cB * (Real)m[0] + cC * (Real)m[1];
    if (p.g_mean2d) { p.g_mean2d[g] = out(gu); p.g_mean2d[n + g] = out(gv); }

    // ---- conic (A, B, C) = (c, -b, a) / det  ->  2D covariance ----
    const Real dA = gA, dB = gB, dC = gC;
    const Real ga = (-c * c * dA + b * c * dB - b * b * dC) * idet2;
    const Real gb = (two * b * c * dA - (a * c + b * b) * dB + two * a * b * dC) * idet2;
    const Real gc = (-b * b * dA + a * b * dB - a * a * dC) * idet2;

    // ---- (a, b, c) = (T0.S.T0, T0.S.T1, T1.S.T1) -> T0, T1 and Sigma ----
    Real gT0[3], gT1[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        gT0[i] = two * ga * ST0[i] + gb * ST1[i];
        gT1[i] = gb * ST0[i] + two * gc * ST1[i];
    }
    Real gS[3][3];   // symmetric
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            gS[i][j] = ga * T0[i] * T0[j] + half * gb * (T0[i] * T1[j] + T1[i] * T0[j]) + gc * T1[i] * T1[j];

    // ---- T rows = J W  ->  J entries  ->  camera-space mean ----
    Real gj00 = 0, gj02 = 0, gj11 = 0, gj12 = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        gj00 += gT0[k] * W[k];
        gj02 += gT0[k] * W[6 + k];
        gj11 += gT1[k] * W[3 + k];
        gj12 += gT1[k] * W[6 + k];
    }
    const Real iz2 = iz * iz, iz3 = iz2 * iz;
    Real gt[3];
    gt[0] = -fx * iz2 * gj02 + fx * iz * gu;
    gt[1] = -fy * iz2 * gj12 + fy * iz * gv;
    gt[2] = -fx * iz2 * gj00 + two * fx * t[0] * iz3 * gj02 - fy * iz2 * gj11 + two * fy * t[1] * iz3 * gj12 -
            fx * t[0] * iz2 * gu - fy * t[1] * iz2 * gv;
#pragma unroll
    for (int i = 0; i < 3; ++i) gmu[i] = (float)(W[i] * gt[0] + W[3 + i] * gt[1] + W[6 + i] * gt[2]);

    // ---- Sigma = M M^T, M = R diag(s) ----
    Real gR[3][3], gs[3] = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const Real gM = two * (gS[i][0] * M[0][j] + gS[i][1] * M[1][j] + gS[i][2] * M[2][j]);
            gR[i][j] = gM * s[j];
            gs[j] += gM * R[i][j];
        }
#pragma unroll
    for (int j = 0; j < 3; ++j) p.g_log_scale[j * n + g] = out(gs[j] * s[j]);

    // ---- R of the unit quaternion, then the normalisation ----
    Real gq[4];
    gq[0] = two * (qz * (gR[1][0] - gR[0][1]) + qy * (gR[0][2] - gR[2][0]) + qx * (gR[2][1] - gR[1][2]));
    gq[1] = two * (qy * (gR[0][1] + gR[1][0]) + qz * (gR[0][2] + gR[2][0]) + qw * (gR[2][1] - gR[1][2]) -
                   two * qx * (gR[1][1] + gR[2][2]));
    gq[2] = two * (qx * (gR[0][1] + gR[1][0]) + qz * (gR[1][2] + gR[2][1]) + qw * (gR[0][2] - gR[2][0]) -
                   two * qy * (gR[0][0] + gR[2][2]));
    gq[3] = two * (qx * (gR[0][2] + gR[2][0]) + qy * (gR[1][2] + gR[2][1]) + qw * (gR[1][0] - gR[0][1]) -
                   two * qz * (gR[0][0] + gR[1][1]));
    const Real qh[4] = {qw, qx, qy, qz};
    const Real dot = qh[0] * gq[0] + qh[1] * gq[1] + qh[2] * gq[2] + qh[3] * gq[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) p.g_quat[i * n + g] = out((gq[i] - qh[i] * dot) / qn);

    return (float)((a * c) / det);
}

// Colour part: dL/dsh from dL/drgb, and the mean's share through the view direction (gmu).
template <int K>
__device__ inline void colour_vjp(const GaussianBackwardParams &p, int g, const float sg[kPairGrad], bool live,
                                  float gmu[3]) {
    const int n = p.n;
    auto out = [live](float v) { return live ? v : 0.0f; };
    const float mu[3] = {p.mean[g], p.mean[n + g], p.mean[2 * n + g]};
    // ---- rgb = sum_k Y_k(d) sh_k with d = (mean - C) / |mean - C| ----
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
            p.g_sh[plane] = out(Y[k] * sg[6 + ch]);
            acc += p.sh[plane] * sg[6 + ch];
        }
        wk[k] = acc;
    }
    float gd[3];
    sh_basis_vjp<K>(d[0], d[1], d[2], wk, gd);
    const float radial = gd[0] * d[0] + gd[1] * d[1] + gd[2] * d[2];
#pragma unroll
    for (int i = 0; i < 3; ++i) gmu[i] = (gd[i] - d[i] * radial) * idn;
}

// Every gradient plane of Gaussian g.  Returns a c / det of its 2D covariance and the colour
// part of dL/dmean (col), which the binary64 geometric pass needs when it redoes the rest.
template <int K>
__device__ inline float gaussian_vjp(const GaussianBackwardParams &p, int g, const float sg[kPairGrad], bool live,
                                     float col[3]) {
    const int n = p.n;
    p.g_opacity[g] = sg[5];
    if (p.g_conic) { p.g_conic[g] = -0.5f * sg[2]; p.g_conic[n + g] = -sg[3]; p.g_conic[2 * n + g] = -0.5f * sg[4]; }
    if (p.g_rgb) { p.g_rgb[g] = sg[6]; p.g_rgb[n + g] = sg[7]; p.g_rgb[2 * n + g] = sg[8]; }
    float geo[3];
    const float kappa = geometric_vjp<float>(p, g, sg, live, geo);
    colour_vjp<K>(p, g, sg, live, col);
#pragma unroll
    for (int i = 0; i < 3; ++i) p.g_mean[i * n + g] = live ? geo[i] + col[i] : 0.0f;
    return kappa;
}

// ---------------------------------------------------------------------------
// per-Gaussian sums of the pair records + chain rule
// ---------------------------------------------------------------------------
// A wave owns 64 consecutive Gaussians.  In up to 16 rounds, each 16-lane row sums the
// records of one Gaussian (lane i takes records i, i + 16, ...: a row reads 16
// consecutive records, skipping those of tiles whose walk stopped before the
// Gaussian), reduces them with DPP row shifts and parks the nine sums in LDS; then
// every lane runs the chain rule of one Gaussian, so the parameter planes are read
// and written coalesced.
constexpr int kGaussPerWave = kWave;
constexpr int kRowLanes = 16;
// Lists longer than this (square rule) are left to the whole workgroup once the rows are
// done: a 16-lane row would otherwise walk a list of thousands of records (the large
// Gaussians of a scene) alone while the rest of the workgroup waits for it.
constexpr uint32_t kLongRecords = 512;

// Sum of the long list of Gaussian g (count records, square rule) by all threads of the
// workgroup: thread t adds records t, t + 256, ... that pass the cut test, then a
// fixed-order reduction over the waves, whose nine sums threads 0..8 store to out[0..8].
// Every thread of the workgroup must call it (two barriers).
__device__ __forceinline__ void long_list_sum(const GaussianBackwardParams &p, int64_t g,
                                              float (*s_part)[kPairGrad], float *out) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const uint32_t count = p.tile_count[g];
    const float *rec = p.pair_grad + (size_t)p.pair_base[g] * kPairStride;
    const uint2 rc = p.rect[g];
    const uint32_t x0 = rc.x & 0xffffu, w = (rc.x >> 16) - x0, y0 = rc.y & 0xffffu;
    const unsigned long long key = ((unsigned long long)__float_as_uint(p.depth[g]) << 32) | (uint64_t)g;
    float acc[kPairGrad];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) acc[c] = 0.0f;
    // record i's tile is (row, col) = divmod(i, w), stepped by divmod(256, w)
    uint32_t r = threadIdx.x / w, col = threadIdx.x - r * w;
    const uint32_t qs = kBlock / w, ss = kBlock - qs * w;
    for (uint32_t i = threadIdx.x; i < count; i += kBlock) {
        const uint32_t tile = (y0 + r) * (uint32_t)p.tiles_x + x0 + col;
        r += qs;
        col += ss;
        if (col >= w) {
            col -= w;
            ++r;
        }
        if (key > p.cut[tile]) continue;   // no pixel of that tile reached this Gaussian
        const float *q = rec + (size_t)i * kPairStride;
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) acc[c] += q[c];
    }
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) {
        const float v = wave_sum(acc[c]);
        if (lane == 0) s_part[wave][c] = v;
    }
    __syncthreads();
    if (threadIdx.x < kPairGrad) {
        float t = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kBlock / kWave; ++w2) t += s_part[w2][threadIdx.x];
        out[threadIdx.x] = t;
    }
    __syncthreads();
}

template <int K>
__global__ __launch_bounds__(kBlock) void gaussian_backward_kernel(GaussianBackwardParams p) {
    __shared__ float s_sum[kBlock / kWave][kGaussPerWave][kPairGrad + 1];
    __shared__ uint8_t s_long[kBlock / kWave][kGaussPerWave];   // per wave: lanes with a long list
    __shared__ int s_long_n[kBlock / kWave];
    __shared__ float s_part[kBlock / kWave][kPairGrad];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int row = lane / kRowLanes, li = lane & (kRowLanes - 1);
    const int64_t g0 = ((int64_t)blockIdx.x * (kBlock / kWave) + wave) * kGaussPerWave;
    // the 64 Gaussians' counts, record bases, rectangles and depth bits, one per lane (loaded
    // once, coalesced); each round's rows fetch theirs by shuffle
    const int64_t gm = g0 + lane;
    const uint32_t m_count = gm < p.n ? p.tile_count[gm] : 0u;
    const bool m_long = !p.ellipse && m_count > kLongRecords;
    const uint64_t longs = __ballot(m_long);
    if (m_long) s_long[wave][__builtin_amdgcn_mbcnt_hi((uint32_t)(longs >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)longs, 0u))] = (uint8_t)lane;
    if (lane == 0) s_long_n[wave] = __popcll(longs);
    uint32_t m_base = 0, m_rx = 0, m_ry = 0, m_depth = 0;
    if (m_count && !p.ellipse) {
        m_base = p.pair_base[gm];
        const uint2 rc = p.rect[gm];
        m_rx = rc.x;
        m_ry = rc.y;
        m_depth = __float_as_uint(p.depth[gm]);
    }
    // The rows take the wave's Gaussians in descending order of their list lengths (a bitonic
    // sort of (count, lane) over the wave; a long list counts as empty, the workgroup sums it),
    // so the four rows of a round walk lists of similar length; after the last Gaussian with a
    // list, the remaining rounds have nothing to do.
    uint32_t order = ((m_long ? 0u : min(m_count, 0xffffffu)) << 6) | (uint32_t)lane;
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t other = (uint32_t)__shfl_xor((int)order, j);
            const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
            order = keep_max ? max(order, other) : min(order, other);
        }
    for (int round = 0; round < kGaussPerWave / 4; ++round) {
        if ((__builtin_amdgcn_readlane((int)order, 4 * round) >> 6) == 0) break;
        const int gl = (int)((uint32_t)__shfl((int)order, 4 * round + row) & (kWave - 1));
        const int64_t g = g0 + gl;
        const uint32_t count = (uint32_t)__shfl((int)m_count, gl);
        const uint32_t base = (uint32_t)__shfl((int)m_base, gl), rx = (uint32_t)__shfl((int)m_rx, gl);
        const uint32_t ry = (uint32_t)__shfl((int)m_ry, gl), dbits = (uint32_t)__shfl((int)m_depth, gl);
        float acc[kPairGrad];
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) acc[c] = 0.0f;
        if (count && p.ellipse) {
            // exact footprint: records follow the row spans; the row's lanes take its tiles
            const float *rec = p.pair_grad + (size_t)p.pair_base[g] * kPairStride;
            const uint2 rc = p.rect[g];
            const uint32_t x0 = rc.x & 0xffffu, x1 = rc.x >> 16, y1 = rc.y >> 16;
            const EllipseRec E = p.ellipse[g];
            const unsigned long long key = ((unsigned long long)__float_as_uint(p.depth[g]) << 32) | (uint64_t)g;
            uint32_t k0 = 0, sa, sb;
            for (uint32_t ty = rc.y & 0xffffu; ty < y1; ++ty) {
                row_span(E, x0, x1, ty, sa, sb);
                for (uint32_t tx = sa + li; tx < sb; tx += kRowLanes) {
                    if (key > p.cut[ty * (uint32_t)p.tiles_x + tx]) continue;
                    const float *r = rec + (size_t)(k0 + tx - sa) * kPairStride;
#pragma unroll
                    for (int c = 0; c < kPairGrad; ++c) acc[c] += r[c];
                }
                k0 += sb - sa;
            }
        } else if (count > kLongRecords) {
            // summed by the whole workgroup below
        } else if (count) {
            const float *rec = p.pair_grad + (size_t)base * kPairStride;
            const uint32_t x0 = rx & 0xffffu, w = (rx >> 16) - x0, y0 = ry & 0xffffu;
            const unsigned long long key = ((unsigned long long)dbits << 32) | (uint64_t)g;
            // record i's tile is (row, col) = divmod(i, w), stepped by divmod(16, w) per record
            uint32_t r = li / w, col = li - r * w;
            const uint32_t q16 = kRowLanes / w, s16 = kRowLanes - q16 * w;
            for (uint32_t i = li; i < count; i += kRowLanes) {
                const uint32_t tile = (y0 + r) * (uint32_t)p.tiles_x + x0 + col;
                r += q16;
                col += s16;
                if (col >= w) {
                    col -= w;
                    ++r;
                }
                if (key > p.cut[tile]) continue;   // no pixel of that tile reached this Gaussian
                const float *q = rec + (size_t)i * kPairStride;
#pragma unroll
                for (int c = 0; c < kPairGrad; ++c) acc[c] += q[c];
            }
        }
#pragma unroll
        for (int c = 0; c < kPairGrad; ++c) {
            const float v = row_sum(acc[c]);
            if (li == kRowLanes - 1) s_sum[wave][gl][c] = v;
        }
    }
    __syncthreads();
    // the long lists of the workgroup's 256 Gaussians, one after another (the counts are in
    // LDS, so the branch and the loop are uniform over the workgroup)
    for (int w = 0; w < kBlock / kWave; ++w)
        for (int q = 0; q < s_long_n[w]; ++q) {
            const int l = s_long[w][q];
            long_list_sum(p, ((int64_t)blockIdx.x * (kBlock / kWave) + w) * kGaussPerWave + l, s_part, s_sum[w][l]);
        }
    const int64_t g = g0 + lane;
    if (g >= p.n) return;
    const bool live = m_count != 0;   // else in no tile list: zero gradients
    float sg[kPairGrad];
#pragma unroll
    for (int c = 0; c < kPairGrad; ++c) sg[c] = live ? s_sum[wave][lane][c] : 0.0f;
    float col[3];
    const float kappa = gaussian_vjp<K>(p, (int)g, sg, live, col);
    // ill-conditioned 2D covariances go to the binary64 pass: each wave compacts its queued
    // Gaussians into its own 64-entry segment and stores their number (no atomics)
    const bool queue = live && !(kappa <= kChainKappa);
    const uint64_t queued = __ballot(queue);
    const int64_t seg = g0 / kWave;
    if (queue) {
        const uint32_t slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(queued >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)queued, 0u));
        float *e = p.fix_list + (size_t)(seg * kWave + slot) * kFixStride;
        e[0] = __uint_as_float((uint32_t)g);
#pragma unroll
        for (int c = 0; c < 5; ++c) e[1 + c] = sg[c];
#pragma unroll
        for (int i = 0; i < 3; ++i) e[6 + i] = col[i];
    }
    if (lane == 0) p.fix_count[seg] = (uint32_t)__popcll(queued);   // lane 0 holds g0 < n
}

// The geometric chain again, in binary64, for the Gaussians the binary32 pass queued: it
// overwrites their mean, log-scale, quaternion and (u, v) gradients.  A wave takes
// kFixSegs consecutive segments (lane l < kFixSegs reads segment l's count), scans the
// counts, and its lanes take the queued entries of those segments one after another: at a
// few percent of Gaussians queued that is about one pass per wave with most lanes busy,
// over enough waves to hide the memory latency of the scattered parameter reads.  An entry
// holds the index, the five moments and the colour part of the mean gradient.
constexpr int kFixSegs = 8;
__global__ __launch_bounds__(kBlock) void gaussian_backward_fp64_kernel(GaussianBackwardParams p) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = p.n;
    const int64_t segs = ((int64_t)n + kWave - 1) / kWave;
    const int64_t seg0 = ((int64_t)blockIdx.x * (kBlock / kWave) + wave) * kFixSegs;
    // inclusive prefix of the kFixSegs counts, the same in every lane
    uint32_t incl[kFixSegs];
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < kFixSegs; ++j) {
        run += seg0 + j < segs ? p.fix_count[seg0 + j] : 0u;
        incl[j] = run;
    }
    for (uint32_t k = lane; k < run; k += kWave) {
        // the segment holding queued entry k: the first j with incl[j] > k
        uint32_t j = 0, before = 0;
#pragma unroll
        for (int i = 0; i + 1 < kFixSegs; ++i)
            if (k >= incl[i]) {
                j = i + 1;
                before = incl[i];
            }
        const float *e = p.fix_list + (size_t)((seg0 + j) * kWave + (k - before)) * kFixStride;
        const int g = (int)__float_as_uint(e[0]);
        const float m[5] = {e[1], e[2], e[3], e[4], e[5]};
        float geo[3];
        (void)geometric_vjp<double>(p, g, m, true, geo);
#pragma unroll
        for (int c = 0; c < 3; ++c) p.g_mean[c * n + g] = geo[c] + e[6 + c];
    }
}

}  // namespace

void launch_composite_backward(const CompositeBackwardParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)(p.tiles_x * p.tiles_y);
    if (tiles == 0) return;
    composite_backward_kernel<<<tiles, kBwdThreads, 0, s>>>(p);
}

void launch_gaussian_backward(const GaussianBackwardParams &p, hipStream_t s) {
    if (p.n <= 0) return;
    constexpr int per_group = (kBlock / kWave) * kGaussPerWave;
    const dim3 grid((p.n + per_group - 1) / per_group);
    switch (p.sh_coeffs) {
        case 1: gaussian_backward_kernel<1><<<grid, kBlock, 0, s>>>(p); break;
        case 4: gaussian_backward_kernel<4><<<grid, kBlock, 0, s>>>(p); break;
        case 9: gaussian_backward_kernel<9><<<grid, kBlock, 0, s>>>(p); break;
        default: gaussian_backward_kernel<16><<<grid, kBlock, 0, s>>>(p); break;
    }
    const int64_t segs = ((int64_t)p.n + kWave - 1) / kWave;       // 64-Gaussian queue segments
    const int64_t per_fix_group = (int64_t)(kBlock / kWave) * kFixSegs;   // segments per workgroup
    gaussian_backward_fp64_kernel<<<(unsigned)((segs + per_fix_group - 1) / per_fix_group), kBlock, 0, s>>>(p);
}

}  // namespace gsr
