"""Super-tile binning (GS_BINNING_SUPER_TILE) against the two-pass radix tile sort (GS_BINNING_RADIX)
and the oracle (needs an MI355X); GS_BINNING_AUTO picks one of them by scene size.

Both build the per-tile lists of the lesson's flowchart ("Assign to tiles (16x16
screen-space)", then "Depth-sort per tile"): every tile's Gaussians in (depth, index)
order.  The super-tile path lists each Gaussian once per 8 x 8-tile super-tile, sorts that
short list by super-tile and expands it into tiles with per-tile ballots; the radix path
sorts every (Gaussian, tile) pair.  Values, ranges, 64-bit keys, images, final
transmittance and blend counts must be identical bit for bit, and the lists equal the
oracle's.
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import binding, scenes

from gs_util import check_binning, gpu_run, note

pytestmark = pytest.mark.gpu

FIELDS = ("num_dups", "values", "ranges", "keys", "image", "T", "n_blend", "blend_total")


def _both(arrays, deg, cam, bg=(0.0, 0.0, 0.0), tile_test=0):
    out = []
    for mode in (binding.GS_BINNING_SUPER_TILE, binding.GS_BINNING_RADIX):
        r = binding.Rasterizer(tile_test=tile_test, binning=mode)
        out.append(gpu_run(arrays, deg, cam, bg=bg, rast=r))
        r.close()
    return out


def _same(a, b, what):
    for k in FIELDS:
        x, y = a[k], b[k]
        if isinstance(x, np.ndarray):
            assert x.dtype == y.dtype and x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), \
                f"{what}: {k} differs"
        else:
            assert x == y, f"{what}: {k} {x} vs {y}"


def _check(arrays, deg, cam, what, bg=(0.0, 0.0, 0.0), tile_test=0):
    sup, rad = _both(arrays, deg, cam, bg=bg, tile_test=tile_test)
    _same(sup, rad, what)
    o = oracle.preprocess(arrays, deg, cam, tile_test=tile_test)
    check_binning(sup, oracle.bin_pairs(o))
    note(f"{what}: {sup['num_dups']} pairs identical in both binnings and to the oracle")
    return sup


# (width, height, Gaussians, SH degree, log-scale range): grids whose super-tiles are partial on
# both axes, exactly one super-tile, a tall strip, and footprints spanning many super-tiles
CASES = [
    (211, 139, 4000, 2, (-4.0, -1.8)),
    (128, 128, 3000, 0, (-4.5, -2.5)),
    (37, 1000, 2000, 1, (-3.5, -1.5)),
    (400, 300, 600, 0, (-1.5, 0.0)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_super_tile_binning_matches_radix_and_oracle(case):
    w, h, n, deg, ls = CASES[case]
    s = scenes.random_scene(70 + case, n, deg, w, h, log_scale_range=ls)
    _check(s.arrays(), deg, s.cameras[0], f"{w}x{h} n={n}", bg=(0.1, 0.2, 0.3))


@pytest.mark.parametrize("elongated", [False, True])
def test_super_tile_binning_exact_footprint(elongated):
    n = 3000
    s = scenes.random_scene(80 + elongated, n, 1, 233, 171, log_scale_range=(-4.0, -1.5))
    a = s.arrays()
    if elongated:
        rng = np.random.default_rng(6)
        a["log_scale"] = np.ascontiguousarray(np.c_[rng.uniform(-3.0, -0.8, n), rng.uniform(-6.0, -4.0, n),
                                                    rng.uniform(-6.0, -4.0, n)].T.astype(np.float32))
    _check(a, 1, s.cameras[0], f"ellipse elongated={elongated}", tile_test=1)


def test_super_tile_binning_culled_and_tiny_scenes():
    # every mean at the camera centre (depth 0, inside the near plane); two Gaussians; one
    # Gaussian (the radix path: a single rank)
    s = scenes.random_scene(90, 50, 0, 64, 48)
    a = s.arrays()
    cam = s.cameras[0]
    centre = -np.asarray(cam["R"], np.float64).reshape(3, 3).T @ np.asarray(cam["t"], np.float64)
    a["mean"] = np.ascontiguousarray(np.repeat(centre[:, None], 50, axis=1).astype(np.float32))
    sup, rad = _both(a, 0, cam)
    _same(sup, rad, "all culled")
    assert sup["num_dups"] == 0 and not sup["ranges"].any()
    for n in (1, 2):
        s = scenes.random_scene(91 + n, n, 0, 64, 48, log_scale_range=(-2.0, -1.0))
        _check(s.arrays(), 0, s.cameras[0], f"n={n}")


@pytest.mark.parametrize("name", ["c1_10k_sh0_256", "c2_100k_sh3_800", "c3_1m_sh3_1080p"])
def test_super_tile_binning_workloads(name):
    s = scenes.make_scene(name)
    cam = s.cameras[0]
    sup, rad = _both(s.arrays(), s.sh_degree, cam)
    _same(sup, rad, name)
    note(f"{name}: {sup['num_dups']} pairs, both binnings identical")


def test_super_tile_binning_growth_on_one_context():
    # one context through scenes whose pair and super-list counts grow and shrink: the
    # speculative launch on too-small buffers must be redone, and reuse must stay exact
    r = binding.Rasterizer(binning=binding.GS_BINNING_SUPER_TILE)
    for seed, n, ls in ((100, 500, (-4.0, -2.0)), (101, 6000, (-2.5, -0.5)), (102, 300, (-4.5, -3.0)),
                        (103, 8000, (-2.0, 0.0))):
        s = scenes.random_scene(seed, n, 0, 301, 197, log_scale_range=ls)
        g = gpu_run(s.arrays(), 0, s.cameras[0], rast=r)
        o = oracle.preprocess(s.arrays(), 0, s.cameras[0])
        check_binning(g, oracle.bin_pairs(o))
    r.close()
