// Front-to-back alpha compositing, one 128-thread workgroup (two wave64) per 16x16 tile.
//
// Lesson "3D Gaussian Splatting from scratch", section "La règle de composition
// alpha": C = sum_i alpha_i T_i c_i with T_i = prod_{j<i} (1 - alpha_j) and
// alpha_i = o_i exp(-d^T Sigma'^-1 d / 2); section "Étape 2" clamps alpha to at
// most 0.99 and samples pixel (row i, column j) at (x = j, y = i).
//
// The tile's depth-sorted list is walked in batches of 128 splats.  The workgroup
// gathers a batch into LDS (double-buffered: the global loads of the next batch are
// in flight while the current one is blended) and every lane reads each splat back
// as a wave-wide LDS broadcast.  A lane owns the two pixels (x, y) and (x + 8, y);
// the row terms B'dy and C'dy^2 + log2(o / 0.99) are computed once per (splat, row) and
// shared through a swizzle, so a pair costs 11 VALU ops:
//   q = (A' dx + B' dy) dx + C' dy^2 + log2(o / 0.99),  alpha = 0.99 min(1, 2^q)
// with (A', B', C') = -log2(e)/2 (A, 2B, C); the min is the exp's output clamp and the
// factor 0.99 rides on the staged colours and the T update.  A pixel stops after the blend that
// brings T below GS_T_EPS; the blend is branchless (a stopped pixel blends with T
// masked to 0).  Every 8 splats a wave counts its live pixels: with none left it
// stops blending for the rest of the list; with 64 or fewer it packs them one per
// lane (cross-lane permutes, no LDS) and blends the rest of the list one pixel per
// lane, since a lane of two stopped pixels would otherwise spend its issue slots on
// nothing.  The workgroup leaves the list when a barrier count finds no live pixel.
// Pure VALU work (one v_exp_f32 per pair): no dense contraction, so no MFMA.
#include "gs_internal.h"

namespace gsr {
namespace {

// Workgroup shape by pixels per lane: two (two waves of 16 x 8 pixels: the row terms shared by a
// lane's pixels; the default) or one (four waves of 16 x 4: twice the waves on a tile, for images
// of few tiles, where the frame waits on its heaviest tiles' serial blend chains).
template <int kPix>
struct Shape {
    static constexpr int kThreads = kTile * kTile / kPix;   // 128 or 256
    static constexpr int kBatch = 128 * (3 - kPix);         // splats per LDS batch (9.5 KB of LDS per
                                                            // two-pixel workgroup: 6 waves per SIMD)
    static constexpr int kLoads = kBatch / kThreads;        // records gathered per thread per batch
    static constexpr int kRowsPerWave = kWave * kPix / kTile;
};
constexpr int kFewTiles = 4096;              // images with fewer tiles take one pixel per lane
constexpr int kUnroll = 8;                   // splats between wave exit tests
static_assert(Shape<1>::kLoads == 1 && Shape<2>::kLoads == 1, "one record per thread per batch");

// A staged splat: what the per-pixel blend reads (a, c) apart from what only the per-row
// terms need (b), so that the blend reads two LDS words per splat.
template <int kLoads>
struct Staged {
    float4 a[kLoads];   // u, A', 0.99 r, 0.99 g
    float4 b[kLoads];   // v, log2(o / 0.99), B', C'
    float c[kLoads];    // 0.99 b
};

template <int kThreads, int kLoads>
__device__ __forceinline__ void gather(Staged<kLoads> &st, const float *__restrict__ splat,
                                       const uint32_t *__restrict__ values, uint32_t base, uint32_t end) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const uint32_t idx = base + k * kThreads + threadIdx.x;
        if (idx < end) {
            const float4 *rec = reinterpret_cast<const float4 *>(splat) + (size_t)values[idx] * 4;
            const float4 r0 = rec[0], r1 = rec[1];
            // alpha = GS_ALPHA_MAX min(1, 2^q): the exponent carries log2(o / GS_ALPHA_MAX) and
            // the colours carry the factor GS_ALPHA_MAX, which leaves the clamp to the exp
            st.a[k] = make_float4(r0.x, r0.w, GS_ALPHA_MAX * r1.z, GS_ALPHA_MAX * r1.w);
            st.b[k] = make_float4(r0.y, splat_log2_scaled_opacity(r0.z), r1.x, r1.y);
            st.c[k] = GS_ALPHA_MAX * rec[2].x;
        }
    }
}

// Value of lane 8 (l / 8) + u for lane l (within each group of 8 lanes), by ds_swizzle in
// its bit mode: source lane = (l & 0x18) | u inside each half-wave of 32.
template <int u>
__device__ __forceinline__ float group8_get(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x18 | (u << 5)));
}

// Position of the k-th (from 0) set bit of m, for k < popcount(m).
__device__ __forceinline__ uint32_t nth_set_bit(uint64_t m, uint32_t k) {
    uint32_t pos = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const uint32_t c = (uint32_t)__popcll(m & ((1ull << w) - 1));
        if (k >= c) {
            k -= c;
            m >>= w;
            pos += w;
        }
    }
    return pos;
}

__device__ __forceinline__ float lane_pull(int src, float v) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

template <bool kAux, int kPix>
struct Pixels {
    float x0, x1, y;   // x1: the second pixel's column (kPix == 2)
    float T[kPix], r[kPix], g[kPix], b[kPix];
    uint32_t blended[kPix];

    __device__ __forceinline__ void blend(const float4 a, const float4 b4, const float c) {
        const float dy = y - b4.x;
        blend_row(a, c, b4.z * dy, splat_row_term(dy, b4.w, b4.y));
    }
    // the same, given the splat's row terms B' dy and C' dy^2 + log2(o / 0.99) for this lane's row
    __device__ __forceinline__ void blend_row(const float4 a, const float c, const float bdy, const float e) {
#pragma unroll
        for (int i = 0; i < kPix; ++i) {
            const float dx = (i ? x1 : x0) - a.x;
            // alpha / GS_ALPHA_MAX; the colours are staged times GS_ALPHA_MAX
            const float as = splat_alpha_scaled(splat_exponent(dx, a.y, bdy, e));
            const bool live = T[i] >= GS_T_EPS;
            const float w = (live ? T[i] : 0.0f) * as;   // T alpha / GS_ALPHA_MAX
            r[i] += w * a.z;
            g[i] += w * a.w;
            b[i] += w * c;
            T[i] = __builtin_fmaf(-GS_ALPHA_MAX, w, T[i]);
            if (kAux) blended[i] += live ? 1u : 0u;
        }
    }
    // One pixel per lane (slot 0) after the wave has packed its live pixels: the row terms
    // are this lane's own, computed by the same operations as the shared ones.
    __device__ __forceinline__ void blend_one(const float4 a, const float4 b4, const float c) {
        const float dy = y - b4.x;
        const float bdy = b4.z * dy, e = splat_row_term(dy, b4.w, b4.y);
        const float as = splat_alpha_scaled(splat_exponent(x0 - a.x, a.y, bdy, e));
        const bool live = T[0] >= GS_T_EPS;
        const float w = (live ? T[0] : 0.0f) * as;
        r[0] += w * a.z;
        g[0] += w * a.w;
        b[0] += w * c;
        T[0] = __builtin_fmaf(-GS_ALPHA_MAX, w, T[0]);
        if (kAux) blended[0] += live ? 1u : 0u;
    }
    __device__ __forceinline__ bool live() const {
        bool any = false;
#pragma unroll
        for (int i = 0; i < kPix; ++i) any |= T[i] >= GS_T_EPS;
        return any;
    }
};

// Output of one pixel: C + T bg, and the per-pixel state the backward reads.
template <bool kAux>
__device__ __forceinline__ void write_pixel(const CompositeParams &p, int x, int y, float r, float g, float b,
                                            float T, uint32_t blended) {
    if (x < p.width && y < p.height) {
        const size_t pix = (size_t)y * p.width + x;
        p.image[pix * 3 + 0] = r + T * p.bg[0];
        p.image[pix * 3 + 1] = g + T * p.bg[1];
        p.image[pix * 3 + 2] = b + T * p.bg[2];
        if (kAux) {
            if (p.final_T) p.final_T[pix] = T;
            if (p.n_blend) p.n_blend[pix] = blended;
        }
    }
}

template <bool kAux, int kPix>
__global__ __launch_bounds__(Shape<kPix>::kThreads) void composite_kernel(CompositeParams p) {
    constexpr int kThreads = Shape<kPix>::kThreads, kBatch = Shape<kPix>::kBatch, kLoads = Shape<kPix>::kLoads;
    constexpr int kPerRow = kTile / kPix;   // lanes of a pixel row (16 or 8): groups of 8 share its row terms
    __shared__ float4 s_a[2][kBatch], s_b[2][kBatch];
    __shared__ float s_c[2][kBatch];
    const float *__restrict__ splat = p.splat;
    const uint32_t *__restrict__ values = p.values;
    const int tile = p.tile_order ? (int)p.tile_order[blockIdx.x] : (int)blockIdx.x;
    const int tile_x = tile % p.tiles_x, tile_y = tile / p.tiles_x;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int ix = tile_x * kTile + (lane % kPerRow);
    const int iy = tile_y * kTile + wave * Shape<kPix>::kRowsPerWave + lane / kPerRow;

    Pixels<kAux, kPix> px;
    px.x0 = (float)ix;
    px.x1 = (float)(ix + 8);
    px.y = (float)iy;
#pragma unroll
    for (int i = 0; i < kPix; ++i) {
        px.T[i] = (ix + 8 * i < p.width && iy < p.height) ? 1.0f : 0.0f;
        px.r[i] = px.g[i] = px.b[i] = 0.0f;
        px.blended[i] = 0u;
    }

    const uint32_t start = p.ranges[2 * tile], end = p.ranges[2 * tile + 1];
    Staged<kLoads> st;
    int buf = 0;
    if (start < end) {
        gather<kThreads, kLoads>(st, splat, values, start, end);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            s_a[0][k * kThreads + threadIdx.x] = st.a[k];
            s_b[0][k * kThreads + threadIdx.x] = st.b[k];
            s_c[0][k * kThreads + threadIdx.x] = st.c[k];
        }
    }
    __syncthreads();
    // Wave-uniform state: 'single' once the wave has packed its live pixels one per lane
    // (slot 0 holds the pixel at (sx, sy), 'held' says the lane got one), 'done' once none
    // is left.  Pixels that were no longer live when the wave packed are written then.
    bool single = false, done = false, held = false;
    int sx = 0, sy = 0;
    uint32_t total = 0;
    for (uint32_t base = start; base < end; base += kBatch) {
        const uint32_t next = base + kBatch;
        if (next < end) gather<kThreads, kLoads>(st, splat, values, next, end);   // in flight during the blends below
        const int count = (int)min<uint32_t>(kBatch, end - base);
        const float4 *sa = s_a[buf];
        const float4 *sb = s_b[buf];
        const float *sc = s_c[buf];
        int j = 0;
        if (!done && !single) {
            for (; j + kUnroll <= count;) {
                // The row terms of the next 8 splats, computed once per (splat, row): lane l takes
                // splat j + l % 8 at its own row (lanes 8r .. 8r + 7 share row r), then each lane
                // fetches splat u's terms from lane 8 (l / 8) + u of its group with a swizzle,
                // which runs on the LDS pipe; the blend itself is bound by VALU issue.
                const float4 rb = sb[j + (lane & 7)];
                const float rdy = px.y - rb.x;
                const float r_bdy = rb.z * rdy, r_e = splat_row_term(rdy, rb.w, rb.y);
                static_assert(kUnroll == 8, "one splat per lane of an 8-lane group");
#define GS_BLEND_ROW(u) px.blend_row(sa[j + u], sc[j + u], group8_get<u>(r_bdy), group8_get<u>(r_e))
                GS_BLEND_ROW(0);
                GS_BLEND_ROW(1);
                GS_BLEND_ROW(2);
                GS_BLEND_ROW(3);
                GS_BLEND_ROW(4);
                GS_BLEND_ROW(5);
                GS_BLEND_ROW(6);
                GS_BLEND_ROW(7);
#undef GS_BLEND_ROW
                j += kUnroll;
                if constexpr (kPix == 1) {
                    if (!__any(px.T[0] >= GS_T_EPS)) {
                        done = true;
                        break;
                    }
                } else {
                    const uint64_t m0 = __ballot(px.T[0] >= GS_T_EPS), m1 = __ballot(px.T[kPix - 1] >= GS_T_EPS);
                    if ((m0 | m1) == 0) {
                        done = true;
                        break;
                    }
                    const uint32_t n0 = (uint32_t)__popcll(m0), n = n0 + (uint32_t)__popcll(m1);
                    if (n <= (uint32_t)kWave) {
                        // Pack: lane k takes the wave's k-th live pixel, slot 0 ones (in lane order)
                        // before slot 1 ones.  First write this lane's pixels that are not live.
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            if (!(px.T[i] >= GS_T_EPS)) {
                                write_pixel<kAux>(p, ix + 8 * i, iy, px.r[i], px.g[i], px.b[i], px.T[i], px.blended[i]);
                                total += px.blended[i];
                            }
                        const uint32_t k = (uint32_t)lane;
                        const bool second = k >= n0;
                        held = k < n;
                        const int src = held ? (int)(second ? nth_set_bit(m1, k - n0) : nth_set_bit(m0, k)) : lane;
                        float v[2][4];
                        uint32_t nb[2];
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            v[i][0] = lane_pull(src, px.T[i]);
                            v[i][1] = lane_pull(src, px.r[i]);
                            v[i][2] = lane_pull(src, px.g[i]);
                            v[i][3] = lane_pull(src, px.b[i]);
                            nb[i] = kAux ? (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)px.blended[i]) : 0u;
                        }
                        const int i = second ? 1 : 0;
                        sx = tile_x * kTile + (src & 7) + 8 * i;
                        sy = tile_y * kTile + wave * 8 + (src >> 3);
                        px.T[0] = held ? (second ? v[1][0] : v[0][0]) : 0.0f;
                        px.r[0] = second ? v[1][1] : v[0][1];
                        px.g[0] = second ? v[1][2] : v[0][2];
                        px.b[0] = second ? v[1][3] : v[0][3];
                        px.blended[0] = second ? nb[1] : nb[0];
                        px.T[1] = 0.0f;
                        px.x0 = (float)sx;
                        px.y = (float)sy;
                        single = true;
                        break;
                    }
                }
            }
            if (!done && !single)
                for (; j < count; ++j) px.blend(sa[j], sb[j], sc[j]);
        }
        if (!done && single) {
            for (; j + kUnroll <= count; j += kUnroll) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) px.blend_one(sa[j + u], sb[j + u], sc[j + u]);
                if (!__any(px.T[0] >= GS_T_EPS)) {
                    done = true;
                    break;
                }
            }
            if (!done)
                for (; j < count; ++j) px.blend_one(sa[j], sb[j], sc[j]);
        }
        if (next < end) {
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                s_a[buf ^ 1][k * kThreads + threadIdx.x] = st.a[k];
                s_b[buf ^ 1][k * kThreads + threadIdx.x] = st.b[k];
                s_c[buf ^ 1][k * kThreads + threadIdx.x] = st.c[k];
            }
        }
        if (__syncthreads_count(px.live()) == 0) break;
        buf ^= 1;
    }

    if (!single) {
#pragma unroll
        for (int i = 0; i < kPix; ++i) {
            write_pixel<kAux>(p, ix + 8 * i, iy, px.r[i], px.g[i], px.b[i], px.T[i], px.blended[i]);
            total += px.blended[i];
        }
    } else if (held) {
        write_pixel<kAux>(p, sx, sy, px.r[0], px.g[0], px.b[0], px.T[0], px.blended[0]);
        total += px.blended[0];
    }
    if (kAux && p.blend_total) {
        __shared__ unsigned long long s_sum;
        if (threadIdx.x == 0) s_sum = 0;
        __syncthreads();
        atomicAdd(&s_sum, (unsigned long long)total);
        __syncthreads();
        if (threadIdx.x == 0 && s_sum) atomicAdd(p.blend_total, s_sum);
    }
}

template <int kPix>
void launch_shape(const CompositeParams &p, unsigned tiles, hipStream_t s) {
    if (p.final_T || p.n_blend || p.blend_total)
        composite_kernel<true, kPix><<<tiles, Shape<kPix>::kThreads, 0, s>>>(p);
    else
        composite_kernel<false, kPix><<<tiles, Shape<kPix>::kThreads, 0, s>>>(p);
}

}  // namespace

void launch_composite(const CompositeParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)(p.tiles_x * p.tiles_y);
    if (tiles == 0) return;
    if (tiles < (unsigned)kFewTiles)
        launch_shape<1>(p, tiles, s);
    else
        launch_shape<2>(p, tiles, s);
}

}  // namespace gsr
