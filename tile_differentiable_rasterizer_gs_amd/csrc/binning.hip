// Per-tile lists through super-tiles: the depth-ranked Gaussians expanded into their tiles
// without sorting the (Gaussian, tile) pairs.
//
// Lesson "3D Gaussian Splatting from scratch", flowchart steps "Assign to tiles (16x16
// screen-space)" and "Depth-sort per tile": each tile gets the Gaussians whose footprint
// meets it, nearest first (ties by index).  The Gaussians arrive in that order (depth ranks).
// Tiles are grouped 8 x 8 into super-tiles; every Gaussian is listed once per super-tile of
// its rectangle, with its part of the rectangle inside that super-tile in the key, and that
// short list (about two entries per Gaussian at 1080p) is sorted stably by super-tile in one
// 8-bit radix pass (sort.hip), so each super-tile's list keeps the depth order.  Here each
// super-tile's list is cut into segments of kSegment entries, one wave each (one per lane);
// a workgroup's waves take consecutive segments and share the segment table that its first
// wave builds in LDS.  An entry's tiles inside its
// super-tile form a 64-bit mask (bit 8 r + c: tile column c, row r of the super-tile), one
// row span per tile row: the rectangle's columns, or the exact-footprint rule's span.
//   super_count_kernel   pairs per (segment, tile): the wave's 64 entry masks transposed, popcounts
//   super_column_kernel  per super-tile: tile totals, the pairs of each of its tile rows (row
//                        parts), and each segment's offset in each tile counted from the start
//                        of the tile's row part (the tiles left of it, then earlier segments)
//   row_offsets_kernel   exclusive scan of the row parts in tile order (one workgroup)
//   super_place_kernel   per tile of the super-tile, a ballot ranks the segment's entries
//                        that meet it, and they write at the row part's offset plus the
//                        segment's offset plus their rank; the kernel's first workgroup
//                        completes the tile ranges and builds the launch order (order_tiles)
// The lists equal those of a stable sort of the pairs by tile, and each pair is written once,
// 4 bytes (plus 8 when the 64-bit keys are asked for).
#include "gs_internal.h"

namespace gsr {
namespace {

constexpr int kXcds = 8;              // XCDs of the chip (workgroups are dealt to them round-robin)
constexpr int kColumnWaves = 16;      // super_column_kernel: waves per super-tile ...
constexpr int kColumnBatch = 8;       // ... and segment counts each lane loads per round trip
// Segments (one a wave) per workgroup, which share the workgroup's segment table: the count
// kernel takes 4; the place kernel 4, or 16 from kPlaceWideSegs segments on (a larger grid
// hides the table's build better in bigger workgroups).
constexpr int kCountWaves = 4;
constexpr int kPlaceWaves = 4, kPlaceWideWaves = 16;
constexpr uint32_t kPlaceWideSegs = 1u << 16;

// Segment geometry from the super-tile totals, built by the first wave of each workgroup:
// super-tile s owns segments [first[s], first[s + 1]) and entries [start[s], start[s + 1]) of
// the sorted super list.
struct SegmentTable {
    uint32_t first[kMaxSuper + 1];
    uint32_t start[kMaxSuper + 1];
};

__device__ void build_segment_table(const SuperBinParams &p, SegmentTable &t) {
    constexpr int kPer = kMaxSuper / kWave;
    const int lane = threadIdx.x;
    const int supers = p.super_x * p.super_y;
    if (lane < kWave) {   // the first wave builds it
        uint32_t n[kPer], segs[kPer], sum_n = 0, sum_s = 0;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int s = lane * kPer + k;
            n[k] = s < supers ? p.super_totals[s] : 0u;
            segs[k] = (n[k] + kSegment - 1) / kSegment;
            sum_n += n[k];
            sum_s += segs[k];
        }
        uint32_t inc_n = sum_n, inc_s = sum_s;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t a = (uint32_t)__shfl_up((int)inc_n, d), b = (uint32_t)__shfl_up((int)inc_s, d);
            if (lane >= d) {
                inc_n += a;
                inc_s += b;
            }
        }
        uint32_t run_n = inc_n - sum_n, run_s = inc_s - sum_s;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            t.start[lane * kPer + k] = run_n;
            t.first[lane * kPer + k] = run_s;
            run_n += n[k];
            run_s += segs[k];
        }
        if (lane == kWave - 1) {
            t.start[kMaxSuper] = run_n;
            t.first[kMaxSuper] = run_s;
        }
    }
    __syncthreads();
}

// Super-tile of segment seg (< first[kMaxSuper]): the last s with first[s] <= seg; super-tiles
// without entries own no segment and share the next one's first.
__device__ inline int segment_super(const SegmentTable &t, uint32_t seg) {
    int lo = 0, hi = kMaxSuper - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t.first[mid] <= seg) lo = mid; else hi = mid - 1;
    }
    return lo;
}

struct SegmentRange {
    int sx, sy;
    uint32_t a, b;   // entries [a, b) of the sorted super list
};

__device__ inline SegmentRange segment_range(const SuperBinParams &p, const SegmentTable &t, uint32_t seg) {
    const int s = segment_super(t, seg);
    SegmentRange r;
    r.sx = s % p.super_x;
    r.sy = s / p.super_x;
    r.a = t.start[s] + (seg - t.first[s]) * (uint32_t)kSegment;
    r.b = min(t.start[s + 1], r.a + (uint32_t)kSegment);
    return r;
}

// An entry's part of its rectangle inside the super-tile, from its key: columns [a, b),
// rows [r0, r1), relative to the super-tile's first tile.
struct LocalRect {
    uint32_t a, b, r0, r1;
};
__device__ inline LocalRect local_rect(uint32_t key) {
    return LocalRect{(key >> 8) & 15u, (key >> 12) & 15u, (key >> 16) & 15u, (key >> 20) & 15u};
}

// The exact-footprint rule's kept columns [sa, sb) of local row `row` (relative, like lr):
// the row span within the entry's columns of the super-tile, which equals the span within
// the whole rectangle clamped to the super-tile.
__device__ inline void local_span(const EllipseRec &E, const LocalRect &lr, uint32_t cx, uint32_t cy, uint32_t row,
                                  uint32_t &sa, uint32_t &sb) {
    row_span(E, cx + lr.a, cx + lr.b, cy + row, sa, sb);
    sa -= cx;
    sb -= cx;
}

// An entry's tiles inside super-tile (sx, sy) as a 64-bit mask (bit 8 r + c for tile column
// c, row r of the super-tile): the square rule's rectangle, or each row's span.
__device__ inline uint64_t entry_mask(const SuperBinParams &p, uint32_t key, uint32_t g, int sx, int sy) {
    const LocalRect lr = local_rect(key);
    uint64_t mask = 0;
    if (p.ellipse) {
        const EllipseRec E = p.ellipse[g];
        const uint32_t cx = (uint32_t)sx * kSuperSide, cy = (uint32_t)sy * kSuperSide;
        for (uint32_t row = lr.r0; row < lr.r1; ++row) {
            uint32_t sa, sb;
            local_span(E, lr, cx, cy, row, sa, sb);
            if (sa < sb) mask |= ((1ull << (sb - sa)) - 1ull) << (kSuperSide * row + sa);
        }
    } else if (lr.a < lr.b && lr.r0 < lr.r1) {
        // the row's bits repeated on rows r0 .. r1 - 1 (one byte per row: no carries)
        const uint64_t rows = (0x0101010101010101ull >> (kSuperSide * (kSuperSide - (lr.r1 - lr.r0)))) << (kSuperSide * lr.r0);
        mask = (((1ull << (lr.b - lr.a)) - 1ull) << lr.a) * rows;
    }
    return mask;
}

static_assert(kSegment == kWave, "one entry per lane");

// Lane e's 64-bit word is row e of a 64 x 64 bit matrix; returns column `lane`: bit e set when
// row e has bit `lane`.  Six exchanges between lanes l and l ^ j (j = 32, 16, .., 1), each
// swapping bit j of the row and column indices: the lane whose bit j is clear keeps the bits
// at positions with bit j clear and takes its partner's such bits moved up by j; the other
// keeps the positions with bit j set and takes its partner's such bits moved down by j.
__device__ inline uint64_t transpose_bits(uint64_t row, uint32_t lane) {
    uint32_t lo = (uint32_t)row, hi = (uint32_t)(row >> 32);
    {   // j = 32: whole halves
        const bool up = (lane & 32u) != 0u;
        const uint32_t got = (uint32_t)__shfl_xor((int)(up ? lo : hi), 32);
        if (up)
            lo = got;
        else
            hi = got;
    }
    constexpr uint32_t kKeep[5] = {0x0000ffffu, 0x00ff00ffu, 0x0f0f0f0fu, 0x33333333u, 0x55555555u};
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int j = 16 >> k;
        const uint32_t m = kKeep[k];
        const bool up = (lane & (uint32_t)j) != 0u;
        // what the partner takes: the set lane's kept bits, the clear lane's upper bits moved down
        const uint32_t slo = (up ? lo : lo >> j) & m, shi = (up ? hi : hi >> j) & m;
        const uint32_t glo = (uint32_t)__shfl_xor((int)slo, j), ghi = (uint32_t)__shfl_xor((int)shi, j);
        lo = up ? (glo | (lo & ~m)) : ((lo & m) | (glo << j));
        hi = up ? (ghi | (hi & ~m)) : ((hi & m) | (ghi << j));
    }
    return ((uint64_t)hi << 32) | lo;
}

// Pairs per (segment, tile of its super-tile): each lane builds its entry's tile mask (the
// rectangle's part in the super-tile, or each row span of the exact-footprint rule), the
// wave transposes the 64 masks, and lane k's popcount is the number of entries meeting tile k.
// The square rule reads the keys only.
__global__ __launch_bounds__(kCountWaves * kWave) void super_count_kernel(SuperBinParams p) {
    __shared__ SegmentTable t;
    build_segment_table(p, t);
    const uint32_t lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t seg = blockIdx.x * kCountWaves + wave;
    if (seg >= t.first[kMaxSuper]) return;   // the whole wave; no barrier follows
    const SegmentRange r = segment_range(p, t, seg);
    const uint32_t e = r.a + lane;
    const bool valid = e < r.b;
    const uint32_t key = p.keys[valid ? e : r.a];   // a lane past the segment meets no tile
    const uint32_t g = p.ellipse ? p.gauss[valid ? e : r.a] : 0u;
    const uint64_t mask = valid ? entry_mask(p, key, g, r.sx, r.sy) : 0ull;
    p.seg_tiles[(size_t)seg * kWave + lane] = (uint32_t)__popcll(transpose_bits(mask, lane));
}

// One workgroup per super-tile; lane k of each wave owns tile k.  The super-tile's segments are
// split into kColumnWaves contiguous blocks, one per wave: each wave sums its block's counts,
// the waves' sums are scanned through LDS, and each wave then replaces every count of its
// block by the pairs of the tile in the segments before it.  The total is the tile's.
__global__ __launch_bounds__(kColumnWaves * kWave) void super_column_kernel(SuperBinParams p) {
    __shared__ SegmentTable t;
    __shared__ uint32_t s_sum[kColumnWaves][kWave];
    build_segment_table(p, t);
    const int s = blockIdx.x;
    if (s >= p.super_x * p.super_y) return;
    const uint32_t lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t j0 = t.first[s], j1 = t.first[s + 1];
    const uint32_t per = (j1 - j0 + kColumnWaves - 1) / kColumnWaves;
    const uint32_t lo = min(j1, j0 + wave * per), hi = min(j1, lo + per);
    uint32_t sum = 0;
    for (uint32_t j = lo; j < hi; j += kColumnBatch) {
        uint32_t c[kColumnBatch];
#pragma unroll
        for (int q = 0; q < kColumnBatch; ++q) c[q] = j + q < hi ? p.seg_tiles[(size_t)(j + q) * kWave + lane] : 0u;
#pragma unroll
        for (int q = 0; q < kColumnBatch; ++q) sum += c[q];
    }
    s_sum[wave][lane] = sum;
    __syncthreads();
    uint32_t off = 0, total = 0;
    for (uint32_t w = 0; w < (uint32_t)kColumnWaves; ++w) {
        const uint32_t v = s_sum[w][lane];
        off += w < wave ? v : 0u;
        total += v;
    }
    // the pairs of the tiles left of this one in its row of the super-tile (lanes 8 r .. 8 r + 7
    // hold row r; tiles past the image's edge have none): offsets count from the row part's start
    uint32_t incl = total;
#pragma unroll
    for (int d = 1; d < kSuperSide; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, d, kSuperSide);
        if ((int)(lane % kSuperSide) >= d) incl += y;
    }
    const uint32_t left = incl - total;
    off += left;
    for (uint32_t j = lo; j < hi; j += kColumnBatch) {
        uint32_t c[kColumnBatch];
#pragma unroll
        for (int q = 0; q < kColumnBatch; ++q) c[q] = j + q < hi ? p.seg_tiles[(size_t)(j + q) * kWave + lane] : 0u;
#pragma unroll
        for (int q = 0; q < kColumnBatch; ++q) {
            if (j + q < hi) p.seg_tiles[(size_t)(j + q) * kWave + lane] = off;
            off += c[q];
        }
    }
    const int sx = s % p.super_x;
    const int tx = sx * kSuperSide + (int)lane % kSuperSide;
    const int ty = (s / p.super_x) * kSuperSide + (int)lane / kSuperSide;
    if (wave == 0) {
        // the tile's total, its range from the row part's start ((0, 0) without pairs; the place
        // kernel adds the row part's offset), and the row part (the last lane of each row)
        if (tx < p.tiles_x && ty < p.tiles_y) {
            p.tile_total[ty * p.tiles_x + tx] = total;
            reinterpret_cast<uint2 *>(p.ranges)[ty * p.tiles_x + tx] = total ? make_uint2(left, incl) : make_uint2(0u, 0u);
        }
        if (lane % kSuperSide == kSuperSide - 1 && ty < p.tiles_y) p.rows[ty * p.super_x + sx] = incl;
    }
}

// The row parts into the pairs before each of them in tile order (row by row, and left to
// right within a row): one workgroup, an exclusive scan of at most 8 kMaxSuper values, two
// consecutive ones per thread, written row_stride words apart.
constexpr int kRowThreads = 1024;
__global__ __launch_bounds__(kRowThreads) void row_offsets_kernel(SuperBinParams p) {
    static_assert(kRowThreads * 2 >= kSuperSide * kMaxSuper, "two row parts per thread");
    __shared__ uint32_t s_tot[kRowThreads / kWave];
    const uint32_t lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const uint32_t parts = (uint32_t)(p.tiles_y * p.super_x), i0 = 2 * threadIdx.x;
    const uint2 v = i0 + 1 < parts ? reinterpret_cast<const uint2 *>(p.rows)[threadIdx.x]
                                   : make_uint2(i0 < parts ? p.rows[i0] : 0u, 0u);
    uint32_t inc = v.x + v.y;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)inc, d);
        if ((int)lane >= d) inc += y;
    }
    if (lane == kWave - 1) s_tot[wave] = inc;
    __syncthreads();
    uint32_t before = inc - v.x - v.y;
    for (uint32_t w = 0; w < wave; ++w) before += s_tot[w];
    if (i0 < parts) p.row_start[i0 * (uint32_t)p.row_stride] = before;
    if (i0 + 1 < parts) p.row_start[(i0 + 1) * (uint32_t)p.row_stride] = before + v.x;
}

// The super list in rank order: a thread per ranked Gaussian writes its entries, one per
// super-tile of its tile rectangle (row-major over the super-tiles), at its offset from the
// prefix sum; how many is the distance to the next rank's offset (a Gaussian without pairs
// owns none, whatever its rectangle).  With about two entries per Gaussian a thread per rank
// is balanced enough and needs no partition table or staged rank window; a rank of more than
// kSuperListSolo entries (a large footprint) is written by its whole wave instead, one entry
// per lane.  Entries past the buffer's capacity are not written (a launch on buffers sized
// for an earlier frame, which the host then repeats).
constexpr uint32_t kSuperListSolo = 16;

__device__ inline void super_entry(const DuplicateParams &p, int64_t k, uint32_t j, uint32_t g, uint2 rc) {
    const uint32_t tx0 = rc.x & 0xffffu, tx1 = rc.x >> 16, ty0 = rc.y & 0xffffu, ty1 = rc.y >> 16;
    const uint32_t sx0 = tx0 >> kSuperShift, sw = ((tx1 - 1) >> kSuperShift) + 1 - sx0, sy0 = ty0 >> kSuperShift;
    const uint32_t row = j / sw, sx = sx0 + (j - row * sw), sy = sy0 + row;
    const uint32_t cx = sx << kSuperShift, cy = sy << kSuperShift;
    p.tile_keys[k] = super_key(sy * (uint32_t)p.tiles_x + sx, max(tx0, cx) - cx, min(tx1, cx + kSuperSide) - cx,
                               max(ty0, cy) - cy, min(ty1, cy + kSuperSide) - cy);
    p.values[k] = g;
}

__global__ __launch_bounds__(kBlock) void super_list_kernel(DuplicateParams p) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int64_t k0 = 0, stop = 0;
    uint32_t g = 0;
    uint2 rc = make_uint2(0u, 0u);
    if (i < p.n_items) {
        const int64_t total = (int64_t)*p.num_dups;
        stop = min<int64_t>(p.capacity, i + 1 < p.n_items ? (int64_t)p.offsets[i + 1] : total);
        k0 = p.offsets[i];
        if (k0 < stop) {
            g = p.order ? p.order[i] : (uint32_t)i;
            rc = p.rect_ranked ? p.rect_ranked[i] : p.rect[g];
        }
    }
    const bool solo = stop - k0 > (int64_t)kSuperListSolo;
    if (!solo)
        for (int64_t k = k0; k < stop; ++k) super_entry(p, k, (uint32_t)(k - k0), g, rc);
    // the wave writes each large rank's entries together
    const uint32_t lane = threadIdx.x & (kWave - 1);
    for (uint64_t m = __ballot(solo); m; m &= m - 1) {
        const int l = __builtin_ctzll(m);
        const int64_t a = ((int64_t)__builtin_amdgcn_readlane((int)(k0 >> 32), l) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)k0, l);
        const int64_t b = ((int64_t)__builtin_amdgcn_readlane((int)(stop >> 32), l) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)stop, l);
        const uint32_t gl = (uint32_t)__builtin_amdgcn_readlane((int)g, l);
        const uint2 rl = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)rc.x, l),
                                    (uint32_t)__builtin_amdgcn_readlane((int)rc.y, l));
        for (int64_t k = a + lane; k < b; k += kWave) super_entry(p, k, (uint32_t)(k - a), gl, rl);
    }
}

// The segment's entries, one per lane, in list order.  For each tile k of the super-tile (a
// uniform loop): the ballot of the lanes whose entry meets tile k gives each such lane its
// rank among them, and they write their Gaussians at the tile's position for this segment
// (its start plus the segment's offset, held by lane k and read with readlane) plus the rank:
// one store instruction writes a contiguous run.  When the frame has more pairs than the
// value buffer holds (a launch on buffers sized for an earlier frame, which the host then
// repeats) nothing is written.  kKeys: also the 64-bit keys.  kNarrow: positions below 2^30,
// so a store's address is the buffer plus a 32-bit byte offset.
template <int kWaves>
union PlaceShared {
    SegmentTable t;
    struct {
        uint32_t count[kOrderBuckets];
        uint32_t wave[kWaves];
    } order;
};

template <bool kKeys, bool kNarrow, int kWaves>
__global__ __launch_bounds__(kWaves * kWave) void super_place_kernel(SuperBinParams p) {
    __shared__ PlaceShared<kWaves> sh;
    SegmentTable &t = sh.t;
    // Workgroup 0 completes the ranges (the row parts' offsets added to the column kernel's
    // row-relative ones) and builds the launch order when asked for, from the tile totals, while
    // the others place the pairs; it starts first and hides under them.
    if (blockIdx.x == 0) {
        const int tiles = p.tiles_x * p.tiles_y;
        uint2 *ranges = reinterpret_cast<uint2 *>(p.ranges);
        for (int i = threadIdx.x; i < tiles; i += kWaves * kWave) {
            const uint2 r = ranges[i];
            if (r.y != 0u) {   // a tile with pairs
                const uint32_t add = p.row_start[((i / p.tiles_x) * p.super_x + (i % p.tiles_x) / kSuperSide) * p.row_stride];
                ranges[i] = make_uint2(r.x + add, r.y + add);
            }
        }
        if (p.order) {
            const TileOrderParams o{tiles, nullptr, p.tile_total, p.order};
            order_tiles<kWaves * kWave>(o, sh.order.count, sh.order.wave);
        }
        return;
    }
    const uint32_t block = blockIdx.x - 1;
    if ((int64_t)*p.num_dups > p.capacity) return;
    build_segment_table(p, t);
    // Workgroups go round-robin to the eight XCDs, each with its own L2: the XCD of `block`
    // (counted after workgroup 0) is fixed by block % 8, and XCD x takes the x-th contiguous
    // block of segments, so the short runs that consecutive segments write into one tile's
    // list meet in one L2 and leave it as whole lines.
    const uint32_t per_xcd = (gridDim.x - 1) / kXcds;   // a multiple of kXcds
    const uint32_t seg = ((block % kXcds) * per_xcd + block / kXcds) * kWaves + threadIdx.x / kWave;
    if (seg >= t.first[kMaxSuper]) return;
    const SegmentRange r = segment_range(p, t, seg);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t e = r.a + lane;
    const bool valid = e < r.b;
    const uint32_t key = p.keys[valid ? e : r.a];   // a lane past the segment meets no tile
    const uint32_t g = p.gauss[valid ? e : r.a];
    const uint32_t tx = (uint32_t)r.sx * kSuperSide + lane % kSuperSide;
    const uint32_t ty = (uint32_t)r.sy * kSuperSide + lane / kSuperSide;
    const bool have_tile = tx < (uint32_t)p.tiles_x && ty < (uint32_t)p.tiles_y;
    // the tile's position for this segment: its row part's offset in tile order plus the
    // segment's offset within the row part
    const uint32_t at = have_tile ? p.row_start[(ty * (uint32_t)p.super_x + (uint32_t)r.sx) * (uint32_t)p.row_stride] +
                                        p.seg_tiles[(size_t)seg * kWave + lane]
                                  : 0u;
    const uint64_t mask = valid ? entry_mask(p, key, g, r.sx, r.sy) : 0ull;
    const uint32_t mlo = (uint32_t)mask, mhi = (uint32_t)(mask >> 32);
    const uint32_t dbits = kKeys ? __float_as_uint(p.depth[g]) : 0u;
    const uint32_t tile0 = (uint32_t)r.sy * kSuperSide * p.tiles_x + (uint32_t)r.sx * kSuperSide;
    // Every load has landed here.  Said explicitly: otherwise the compiler counts the Gaussian's
    // load (skipped on some paths) as pending at each store below, and since the counter also
    // counts stores, each store would wait for all the earlier ones.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int k = 0; k < kWave; ++k) {
        if (__builtin_amdgcn_ubfe(k < 32 ? mlo : mhi, (uint32_t)(k & 31), 1u) != 0u) {
            // the lanes here are the entries meeting tile k (one bit test serves as the branch
            // and, through the active lanes, as the ballot)
            const uint64_t bk = __ballot(1);
            const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)at, k);
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bk, 0u));
            if (kNarrow) {
                *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(p.values) + ((rank << 2) + (base << 2))) = g;
            } else {
                p.values[(size_t)base + rank] = g;
            }
            if (kKeys) {
                const uint32_t tile = tile0 + (uint32_t)(k / kSuperSide) * p.tiles_x + (uint32_t)(k % kSuperSide);
                p.keys_out[(size_t)base + rank] = ((uint64_t)tile << 32) | dbits;
            }
        }
    }
}

}  // namespace

int64_t super_segment_capacity(int64_t entries) { return entries / kSegment + kMaxSuper + 1; }

void launch_super_list(const DuplicateParams &p, hipStream_t s) {
    if (p.n_items <= 0 || p.capacity <= 0) return;
    super_list_kernel<<<(unsigned)((p.n_items + kBlock - 1) / kBlock), kBlock, 0, s>>>(p);
}

template <int kWaves>
void launch_place(const SuperBinParams &p, unsigned segs, hipStream_t s) {
    // every segment below the capacity has a wave; the placing workgroups are a multiple of
    // kXcds, after workgroup 0
    const unsigned groups = ((segs + kWaves - 1) / kWaves + kXcds - 1) / kXcds * kXcds + 1;
    if (p.keys_out)
        super_place_kernel<true, false, kWaves><<<groups, kWaves * kWave, 0, s>>>(p);
    else if (p.capacity <= ((int64_t)1 << 30))
        super_place_kernel<false, true, kWaves><<<groups, kWaves * kWave, 0, s>>>(p);
    else
        super_place_kernel<false, false, kWaves><<<groups, kWaves * kWave, 0, s>>>(p);
}

void launch_super_binning(const SuperBinParams &params, hipStream_t s) {
    const unsigned segs = (unsigned)params.seg_capacity;
    SuperBinParams p = params;
    p.row_stride = segs >= kPlaceWideSegs ? kRowStride : 1;
    super_count_kernel<<<(segs + kCountWaves - 1) / kCountWaves, kCountWaves * kWave, 0, s>>>(p);
    super_column_kernel<<<(unsigned)(p.super_x * p.super_y), kColumnWaves * kWave, 0, s>>>(p);
    row_offsets_kernel<<<1, kRowThreads, 0, s>>>(p);
    if (segs >= kPlaceWideSegs)
        launch_place<kPlaceWideWaves>(p, segs, s);
    else
        launch_place<kPlaceWaves>(p, segs, s);
}

}  // namespace gsr
