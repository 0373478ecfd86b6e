"""Host emulation of the exact-footprint pair listing's index arithmetic (CPU only).

The exact-footprint rule lists a Gaussian in the tiles of its square whose pixel-centre
box meets its 3-sigma ellipse (the lesson's projection step draws that ellipse; the
flowchart's "Assign to tiles (16x16 screen-space)" step lists the pairs).  The GPU
listing (partition table, 2048-entry blocks, staged rank windows, a first-entry walk
over each rank's row spans, then a per-thread walk with rank steps), the backward's
record index of a pair (kept tiles in the rows above plus the column in the span) and
the per-Gaussian span walk are re-enacted here step by step on the host, with every
index checked against the size of what it addresses, and the listing compared with
the oracle's pairs.  The spans come from the oracle's binary32 row_span, which gives
the same spans as the device (the GPU parity tests compare tile counts and pairs bit
for bit).  Inputs: a 40 x 3000 view with wide, flat footprints whose squares are up to
188 tile rows high (most rows of the square empty), and elongated footprints.
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import scenes


def tall_input():
    n, nw = 4000, 200
    s = scenes.random_scene(64, n, 0, 40, 3000)
    a = s.arrays()
    rng = np.random.default_rng(10)
    ls = rng.uniform(-3.5, -2.5, (n, 3))
    ls[n - nw:] = np.c_[rng.uniform(-1.5, -0.3, nw), rng.uniform(-6.0, -5.0, nw), rng.uniform(-6.0, -5.0, nw)]
    a["log_scale"] = np.ascontiguousarray(ls.T.astype(np.float32))
    return a, s.cameras[0]


def elongated_input():
    rng = np.random.default_rng(5)
    n = 400
    s = scenes.random_scene(61, n, 1, 180, 120)
    a = s.arrays()
    a["log_scale"] = np.ascontiguousarray(np.c_[rng.uniform(-3.0, -0.8, n), rng.uniform(-6.0, -4.0, n),
                                                rng.uniform(-6.0, -4.0, n)].T.astype(np.float32))
    a["sh"] = np.ascontiguousarray(a["sh"][:3])
    return a, s.cameras[0]


def emulate(a, cam, mode, kItems=8, kBlock=256, kDupWindow=1025):
    deg = {1: 0, 4: 1}[a["sh"].shape[0] // 3]
    p = oracle.preprocess(a, deg, cam, tile_test=1)
    n = p["depth"].shape[0]
    tiles_x, tiles_y = oracle.tiles_for(cam)
    tiles = tiles_x * tiles_y
    rect = p["rect"].astype(np.int64)            # x0, x1, y0, y1
    cnt = p["tile_count"].astype(np.int64)
    spans = {}
    def row_span(g, ty):
        key = (g, ty)
        if key not in spans:
            spans[key] = oracle.row_span(p["mean2d"][0, g], p["mean2d"][1, g], p["ellipse"][:, g],
                                         rect[0, g], rect[1, g], ty)
        return spans[key]
    # preprocess count = sum of row spans (as the kernel sums them)
    for g in range(n):
        if cnt[g]:
            s = sum(row_span(g, ty)[1] - row_span(g, ty)[0] for ty in range(rect[2, g], rect[3, g]))
            assert s == cnt[g], ("count", g)
    # rank order
    if mode == 0:
        key = np.where(cnt > 0, p["depth"].view(np.uint32), np.uint32(0xffffffff)).astype(np.uint64)
        order = np.lexsort((np.arange(n), key))
    else:
        order = np.arange(n)
    c_r = cnt[order]
    off = np.concatenate([[0], np.cumsum(c_r)[:-1]]).astype(np.int64)
    M = int(c_r.sum())
    kTile = kBlock * kItems
    blocks = (M + kTile - 1) // kTile
    # partition table
    part = np.full(blocks + 1, -1, np.int64)
    for i in range(n):
        start = off[i]
        end = min(off[i + 1] if i + 1 < n else M, M)
        b = (start + kTile - 1) // kTile
        while b * kTile < end:
            part[b] = i; b += 1
        if start < end and end == M:
            part[(M + kTile - 1) // kTile] = i
    assert (part >= 0).all(), "partition table hole"
    tiles_out = np.full(M, -1, np.int64); vals_out = np.full(M, -1, np.int64)
    max_walk_rows = 0; unstaged = 0; max_window = 0
    for blk in range(blocks):
        first = blk * kTile
        lo, hi = part[blk], part[blk + 1]
        window = hi - lo + 1
        max_window = max(max_window, window)
        staged = window <= kDupWindow
        unstaged += not staged
        s_rank = np.full(kBlock, -1, np.int64)
        if staged:
            for k in range(window):
                A = off[lo + k] - first
                B = off[lo + k + 1] - first if k + 1 < window else kTile
                t0 = 0 if A <= 0 else (A + kItems - 1) // kItems
                t1 = min(kBlock, 0 if B <= 0 else (B + kItems - 1) // kItems)
                for t in range(t0, t1):
                    assert 0 <= t < kBlock
                    s_rank[t] = k
        last = hi - lo
        def rank_offset(k):
            assert 0 <= k <= last, ("rank_offset", k, last)
            return off[lo + k]
        def next_rank(i, e_next):
            i += 1
            assert i <= last, ("next_rank past window", i, last)
            if i >= last or rank_offset(i + 1) > e_next:
                return i
            a_, b_ = i + 1, last
            while a_ < b_:
                mid = a_ + (b_ - a_ + 1) // 2
                if rank_offset(mid) <= e_next: a_ = mid
                else: b_ = mid - 1
            return a_
        for t in range(kBlock):
            e0 = first + t * kItems
            if e0 >= M: break
            n_here = min(kItems, M - e0)
            if staged:
                i = s_rank[t]
                assert 0 <= i < window, ("s_rank unset", blk, t, i)
            else:
                lo_, hi_ = lo, hi
                while lo_ < hi_:
                    mid = lo_ + (hi_ - lo_ + 1) // 2
                    if off[mid] <= e0: lo_ = mid
                    else: hi_ = mid - 1
                i = lo_ - lo
            g = order[lo + i]; o = off[lo + i]
            x0, x1, y0, y1 = rect[:, g]
            ty = y0
            j = e0 - o
            assert 0 <= j < cnt[g], ("first entry outside rank", j, cnt[g])
            sa, sb = row_span(g, ty)
            walked = 0
            while j >= sb - sa:
                j -= sb - sa
                ty += 1; walked += 1
                assert ty < y1, ("first-entry walk past the rectangle", g, ty, y1)
                sa, sb = row_span(g, ty)
            max_walk_rows = max(max_walk_rows, walked)
            tx = sa + j
            for k in range(n_here):
                tid = ty * tiles_x + tx
                assert 0 <= tid < tiles and x0 <= tx < x1 and y0 <= ty < y1, ("tile id", g, tx, ty)
                assert tiles_out[e0 + k] == -1
                tiles_out[e0 + k] = tid; vals_out[e0 + k] = g
                tx += 1
                if tx == sb and k + 1 < n_here:
                    while True:
                        ty += 1
                        if ty == y1:
                            i = next_rank(i, e0 + k + 1)
                            g = order[lo + i]
                            x0, x1, y0, y1 = rect[:, g]
                            ty = y0
                            assert cnt[g] > 0
                        assert ty < y1
                        sa, sb = row_span(g, ty)
                        if sa != sb: break
                    tx = sa
    assert (tiles_out >= 0).all()
    # listing equals the oracle's unsorted pair list (key64 mode order = index order)
    b = oracle.bin_pairs(p, want_unsorted=True)
    if mode == 1:
        assert np.array_equal(tiles_out, (b["keys_unsorted"] >> np.uint64(32)).astype(np.int64))
        assert np.array_equal(vals_out, b["values_unsorted"].astype(np.int64))
    # backward: kept_index of every listed pair, and the per-Gaussian span walk
    pair_base = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    for e in range(M):
        g = vals_out[e]; tid = tiles_out[e]
        tx, ty = tid % tiles_x, tid // tiles_x
        x0, x1, y0, y1 = rect[:, g]
        assert y0 <= ty < y1
        k = sum(row_span(g, r)[1] - row_span(g, r)[0] for r in range(y0, ty))
        sa, sb = row_span(g, ty)
        assert sa <= tx < sb
        idx = k + tx - sa
        assert 0 <= idx < cnt[g] and pair_base[g] + idx < M
    for g in range(n):
        if not cnt[g]: continue
        k0 = 0
        for ty in range(rect[2, g], rect[3, g]):
            sa, sb = row_span(g, ty)
            for tx in range(sa, sb):
                assert 0 <= ty * tiles_x + tx < tiles and k0 + tx - sa < cnt[g]
            k0 += sb - sa
        assert k0 == cnt[g]
    rows = (rect[3] - rect[2])[cnt > 0]
    return dict(M=M, blocks=blocks, max_window=max_window, unstaged=unstaged, max_walk_rows=max_walk_rows,
                max_rows=int(rows.max()), tiles=tiles)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("which", ["tall", "elongated"])
def test_listing_indices_stay_in_bounds(which, mode):
    a, cam = tall_input() if which == "tall" else elongated_input()
    st = emulate(a, cam, mode)
    assert st["M"] > 0 and st["unstaged"] == 0
    if which == "tall":
        assert st["max_rows"] > 100 and st["max_walk_rows"] > 50


def test_listing_unstaged_windows():
    """Blocks meeting more ranks than the staged window search them in global memory."""
    a, cam = tall_input()
    st = emulate(a, cam, 1, kDupWindow=16)
    assert st["unstaged"] > 0
