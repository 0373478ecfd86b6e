// Front-to-back alpha compositing, one 128-thread workgroup (two wave64) per 16x16 tile.
//
// Lesson "3D Gaussian Splatting from scratch", section "La règle de composition
// alpha": C = sum_i alpha_i T_i c_i with T_i = prod_{j<i} (1 - alpha_j) and
// alpha_i = o_i exp(-d^T Sigma'^-1 d / 2); section "Étape 2" clamps alpha to at
// most 0.99 and samples pixel (row i, column j) at (x = j, y = i).
//
// The tile's depth-sorted list is walked in batches of 256 splats.  The workgroup
// gathers a batch into LDS (double-buffered: the global loads of the next batch are
// in flight while the current one is blended) and every lane reads each splat back
// as a wave-wide LDS broadcast.  A lane owns the two pixels (x, y) and (x + 8, y);
// the row terms B'dy and C'dy^2 + log2(o / 0.99) are computed once per (splat, row) and
// shared through a swizzle, so a pair costs 11 VALU ops:
//   q = (A' dx + B' dy) dx + C' dy^2 + log2(o / 0.99),  alpha = 0.99 min(1, 2^q)
// with (A', B', C') = -log2(e)/2 (A, 2B, C); the min is the exp's output clamp and the
// factor 0.99 rides on the staged colours and the T update.  A pixel stops after the blend that
// brings T below GS_T_EPS; the blend is branchless (a stopped pixel blends with T
// masked to 0).  A wave leaves a batch once none of its 128 pixels is live (tested
// every 8 splats) and the workgroup leaves the list when a barrier count finds no
// live pixel.  Pure VALU work (one v_exp_f32 per pair): no dense contraction, so
// no MFMA.
#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kThreads = 128;                // 64 lanes x 2 pixels = one 16x8 half tile per wave
constexpr int kBatch = 256;                  // splats per LDS batch
constexpr int kLoads = kBatch / kThreads;    // records gathered per thread per batch
constexpr int kUnroll = 8;                   // splats between wave exit tests

// A staged splat: what the per-pixel blend reads (a, c) apart from what only the per-row
// terms need (b), so that the blend reads two LDS words per splat.
struct Staged {
    float4 a[kLoads];   // u, A', 0.99 r, 0.99 g
    float4 b[kLoads];   // v, log2(o / 0.99), B', C'
    float c[kLoads];    // 0.99 b
};

__device__ __forceinline__ void gather(Staged &st, const float *__restrict__ splat,
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

template <bool kAux>
struct Pixels {
    float x0, x1, y;
    float T[2], r[2], g[2], b[2];
    uint32_t blended[2];

    __device__ __forceinline__ void blend(const float4 a, const float4 b4, const float c) {
        const float dy = y - b4.x;
        blend_row(a, c, b4.z * dy, splat_row_term(dy, b4.w, b4.y));
    }
    // the same, given the splat's row terms B' dy and C' dy^2 + log2(o / 0.99) for this lane's row
    __device__ __forceinline__ void blend_row(const float4 a, const float c, const float bdy, const float e) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
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
    __device__ __forceinline__ bool live() const { return (T[0] >= GS_T_EPS) | (T[1] >= GS_T_EPS); }
};

template <bool kAux>
__global__ __launch_bounds__(kThreads) void composite_kernel(CompositeParams p) {
    __shared__ float4 s_a[2][kBatch], s_b[2][kBatch];
    __shared__ float s_c[2][kBatch];
    const float *__restrict__ splat = p.splat;
    const uint32_t *__restrict__ values = p.values;
    const int tile = p.tile_order ? (int)p.tile_order[blockIdx.x] : (int)blockIdx.x;
    const int tile_x = tile % p.tiles_x, tile_y = tile / p.tiles_x;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int ix = tile_x * kTile + (lane & 7);
    const int iy = tile_y * kTile + wave * 8 + (lane >> 3);

    Pixels<kAux> px;
    px.x0 = (float)ix;
    px.x1 = (float)(ix + 8);
    px.y = (float)iy;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        px.T[i] = (ix + 8 * i < p.width && iy < p.height) ? 1.0f : 0.0f;
        px.r[i] = px.g[i] = px.b[i] = 0.0f;
        px.blended[i] = 0u;
    }

    const uint32_t start = p.ranges[2 * tile], end = p.ranges[2 * tile + 1];
    Staged st;
    int buf = 0;
    if (start < end) {
        gather(st, splat, values, start, end);
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            s_a[0][k * kThreads + threadIdx.x] = st.a[k];
            s_b[0][k * kThreads + threadIdx.x] = st.b[k];
            s_c[0][k * kThreads + threadIdx.x] = st.c[k];
        }
    }
    __syncthreads();
    for (uint32_t base = start; base < end; base += kBatch) {
        const uint32_t next = base + kBatch;
        if (next < end) gather(st, splat, values, next, end);   // in flight during the blends below
        const int count = (int)min<uint32_t>(kBatch, end - base);
        const float4 *sa = s_a[buf];
        const float4 *sb = s_b[buf];
        const float *sc = s_c[buf];
        int j = 0;
        bool wave_live = true;
        for (; j + kUnroll <= count; j += kUnroll) {
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
            if (!__any(px.live())) {
                wave_live = false;
                break;
            }
        }
        if (wave_live)
            for (; j < count; ++j) px.blend(sa[j], sb[j], sc[j]);
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

    uint32_t total = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int x = ix + 8 * i;
        if (x < p.width && iy < p.height) {
            const size_t pix = (size_t)iy * p.width + x;
            p.image[pix * 3 + 0] = px.r[i] + px.T[i] * p.bg[0];
            p.image[pix * 3 + 1] = px.g[i] + px.T[i] * p.bg[1];
            p.image[pix * 3 + 2] = px.b[i] + px.T[i] * p.bg[2];
            if (kAux) {
                if (p.final_T) p.final_T[pix] = px.T[i];
                if (p.n_blend) p.n_blend[pix] = px.blended[i];
            }
        }
        total += px.blended[i];
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

}  // namespace

void launch_composite(const CompositeParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)(p.tiles_x * p.tiles_y);
    if (tiles == 0) return;
    if (p.final_T || p.n_blend || p.blend_total)
        composite_kernel<true><<<tiles, kThreads, 0, s>>>(p);
    else
        composite_kernel<false><<<tiles, kThreads, 0, s>>>(p);
}

}  // namespace gsr
