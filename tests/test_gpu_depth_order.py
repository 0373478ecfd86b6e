"""Bucketed depth order (GS_DEPTH_ORDER_BUCKETS, the default) against the four-pass radix sort
of the depth bits (GS_DEPTH_ORDER_RADIX) and the oracle (needs an MI355X).

Both produce the order of the lesson's flowchart step "Depth-sort per tile": Gaussians by
(camera-space depth, index), from which the per-tile lists are built.  The bucketed order
distributes the Gaussians into buckets linear in depth and sorts each bucket in LDS; a
bucket too large for that makes the host redo the frame with the radix sort.  Values,
ranges, keys, images, final transmittance and blend counts must be identical bit for bit,
and the lists equal the oracle's.  gs_binning.depth_buckets shows which path produced the
order: the bucket count, or 0 for the radix sort (also after a fallback).
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import binding, scenes

from gs_util import check_binning, gpu_run, note, plane_scene

pytestmark = pytest.mark.gpu

FIELDS = ("num_dups", "values", "ranges", "keys", "image", "T", "n_blend", "blend_total")


def _run(arrays, deg, cam, order, binning=binding.GS_BINNING_AUTO, bg=(0.0, 0.0, 0.0)):
    r = binding.Rasterizer(depth_order=order, binning=binning)
    out = gpu_run(arrays, deg, cam, bg=bg, rast=r)
    r.close()
    return out, out["depth_buckets"]


def _buckets(n):
    # the library's choice: 256 .. 8192 buckets, about 512 Gaussians each
    b = 8
    while b < 13 and (1 << b) * 512 < n:
        b += 1
    return 1 << b


def _same(a, b, what):
    for k in FIELDS:
        x, y = a[k], b[k]
        if isinstance(x, np.ndarray):
            assert x.dtype == y.dtype and x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
                f"{what}: {k} differs"
        else:
            assert x == y, f"{what}: {k} {x} vs {y}"


def _check(arrays, deg, cam, what, fallback=False, binning=binding.GS_BINNING_AUTO, bg=(0.0, 0.0, 0.0)):
    n = arrays["opacity"].shape[0]
    bk, nb = _run(arrays, deg, cam, binding.GS_DEPTH_ORDER_BUCKETS, binning, bg)
    rd, rb = _run(arrays, deg, cam, binding.GS_DEPTH_ORDER_RADIX, binning, bg)
    assert rb == 0 and nb == (0 if fallback else _buckets(n)), (nb, rb)
    _same(bk, rd, what)
    check_binning(bk, oracle.bin_pairs(oracle.preprocess(arrays, deg, cam)))
    note(f"{what}: {bk['num_dups']} pairs identical under both depth orders and to the oracle "
         f"({nb} buckets)")
    return bk


# (width, height, Gaussians, SH degree, log-scale range): 256 to 1024 buckets, ragged groups
CASES = [
    (211, 139, 4000, 2, (-4.0, -1.8)),
    (320, 240, 25000, 0, (-4.5, -2.5)),
    (640, 360, 60001, 1, (-4.5, -3.0)),
    (96, 64, 3, 0, (-2.0, -1.0)),
    (640, 360, 300007, 0, (-5.0, -3.5)),
    (512, 384, 262144, 0, (-5.0, -3.5)),   # exactly 64 counting groups: the group-major count table
    (512, 384, 258047, 0, (-5.0, -3.5)),   # 63 groups: the bucket-major one
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bucket_order_matches_radix_and_oracle(case):
    w, h, n, deg, ls = CASES[case]
    s = scenes.random_scene(300 + case, n, deg, w, h, log_scale_range=ls)
    _check(s.arrays(), deg, s.cameras[0], f"{w}x{h} n={n}", bg=(0.1, 0.2, 0.3))


def test_bucket_order_with_super_tile_binning():
    s = scenes.random_scene(310, 20000, 1, 400, 300, log_scale_range=(-4.0, -2.0))
    _check(s.arrays(), 1, s.cameras[0], "super-tile binning", binning=binding.GS_BINNING_SUPER_TILE)


@pytest.mark.parametrize("depths,n,fallback", [
    ((5.0,), 6000, True),               # one depth: one bucket of 6000, the radix sort takes over
    ((3.0, 4.0, 5.0), 15000, True),     # three buckets of ~5000
    ((3.0, 4.0, 5.0), 9000, False),     # ~3000 equal depths per bucket: the widest network
])
def test_bucket_order_crowded_depths(depths, n, fallback):
    arrays, cam = plane_scene(320 + n, n, depths)
    _check(arrays, 0, cam, f"depths {depths} n={n}", fallback=fallback)


def test_bucket_order_culled_and_tiny_scenes():
    # half the Gaussians behind the camera (no pairs: the output tail); then n = 2
    s = scenes.random_scene(330, 8000, 0, 128, 96, log_scale_range=(-4.0, -2.5))
    a = s.arrays()
    cam = s.cameras[0]
    centre = -np.asarray(cam["R"], np.float64).reshape(3, 3).T @ np.asarray(cam["t"], np.float64)
    a["mean"][:, ::2] = centre[:, None].astype(np.float32)
    _check(a, 0, cam, "half culled")
    s = scenes.random_scene(331, 2, 0, 64, 48, log_scale_range=(-2.0, -1.0))
    _check(s.arrays(), 0, s.cameras[0], "n=2")


@pytest.mark.parametrize("name", ["c1_10k_sh0_256", "c2_100k_sh3_800", "c3_1m_sh3_1080p"])
def test_bucket_order_workloads(name):
    s = scenes.make_scene(name)
    cam = s.cameras[0]
    bk, nb = _run(s.arrays(), s.sh_degree, cam, binding.GS_DEPTH_ORDER_BUCKETS)
    rd, rb = _run(s.arrays(), s.sh_degree, cam, binding.GS_DEPTH_ORDER_RADIX)
    assert nb == _buckets(s.n) and rb == 0
    _same(bk, rd, name)
    note(f"{name}: {bk['num_dups']} pairs, both depth orders identical")


def test_bucket_order_sequence_on_one_context():
    # one context through scenes that grow, shrink and fall back: the bound slots are emptied
    # after every order, buffers are reused, and a fallback frame leaves the next one exact
    r = binding.Rasterizer()
    frames = []
    for seed, n in ((340, 3000), (341, 40000), (342, 700)):
        s = scenes.random_scene(seed, n, 0, 301, 197, log_scale_range=(-4.0, -2.0))
        frames.append((s.arrays(), s.cameras[0]))
    frames.insert(2, plane_scene(343, 7000, (5.0,)))   # one bucket of 7000: the fallback
    for arrays, cam in frames:
        g = gpu_run(arrays, 0, cam, rast=r)
        check_binning(g, oracle.bin_pairs(oracle.preprocess(arrays, 0, cam)))
    r.close()


def test_larger_bucket_kernel_follows_the_last_frame():
    # the larger-bucket kernel runs only while the last bucketed frame met a bucket of more than
    # 2048 Gaussians; a frame that meets one without it is redone by the radix sort (reported as
    # 0 buckets) and exact, and the frame after it runs the kernel again
    r = binding.Rasterizer()
    small = scenes.random_scene(350, 20000, 0, 301, 197, log_scale_range=(-4.0, -2.0))
    crowded = plane_scene(351, 9000, (3.0, 4.0, 5.0))   # ~3000 Gaussians per occupied bucket
    seq = [(small.arrays(), small.cameras[0], _buckets(20000)),   # first frame: the kernel runs
           (small.arrays(), small.cameras[0], _buckets(20000)),   # left out: no larger bucket
           (crowded[0], crowded[1], 0),                            # met without it: redone
           (crowded[0], crowded[1], _buckets(9000)),               # run again
           (small.arrays(), small.cameras[0], _buckets(20000)),
           (crowded[0], crowded[1], 0)]
    for i, (arrays, cam, want) in enumerate(seq):
        g = gpu_run(arrays, 0, cam, rast=r)
        assert g["depth_buckets"] == want, (i, g["depth_buckets"], want)
        check_binning(g, oracle.bin_pairs(oracle.preprocess(arrays, 0, cam)))
    r.close()
    note("larger-bucket kernel launched after frames that met such buckets; other frames redone exactly")
