"""The exact-footprint tile rule (GS_TILE_ELLIPSE) through the C ABI vs the oracle (needs an MI355X).

With the rule on, a Gaussian is listed only in the tiles of its square whose pixel-centre box
meets its 3-sigma ellipse; the oracle states the same rule (tests/test_oracle_ellipse.py pins
it against a binary64 definition).  Tile counts, sorted keys and values, and tile ranges must
be bit-identical; the image within 2e-4; the gradients within the backward bound.
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import scenes

from gs_util import IMAGE_TOL, check_binning, check_preprocess, gpu_run, image_error, note
from test_gpu_backward import check_grads, gpu_grads

pytestmark = pytest.mark.gpu
ELL = 1


def _check(arrays, deg, cam, mode=0, bg=(0.0, 0.0, 0.0), pixels=None):
    g = gpu_run(arrays, deg, cam, bg=bg, sort_mode=mode, tile_test=ELL)
    o = oracle.preprocess(arrays, deg, cam, tile_test=ELL)
    check_preprocess(g, o)
    sq = oracle.preprocess(arrays, deg, cam)
    assert o["tile_count"].sum() < sq["tile_count"].sum()
    ob = oracle.bin_pairs(o, want_unsorted=(mode == 1))
    check_binning(g, ob)
    if mode == 1:
        assert np.array_equal(g["keys_unsorted"], ob["keys_unsorted"]), "unsorted keys"
    if pixels is None:
        oimg, _, ocnt = oracle.composite(o, cam, bg=bg)
        err = image_error(g["image"], oimg)
        assert np.mean(g["n_blend"] != ocnt) < 1e-3
    else:
        oimg, _, _ = oracle.composite(o, cam, bg=bg, pixels=pixels)
        err = image_error(g["image"].reshape(-1, 3)[pixels], oimg)
    assert err <= IMAGE_TOL, f"image err {err}"
    return g, o, err


@pytest.mark.parametrize("deg", [0, 3])
@pytest.mark.parametrize("mode", [0, 1])
def test_ellipse_random_ragged(deg, mode):
    w, h = 211 + deg, 139 + 3 * deg
    s = scenes.random_scene(60 + deg, 4000, deg, w, h, log_scale_range=(-4.0, -1.8))
    note(f"ellipse random deg={deg} mode={mode}")
    g, o, err = _check(s.arrays(), deg, s.cameras[0], mode=mode, bg=(0.1, 0.2, 0.3))
    note(f"  pairs {g['num_dups']} image err {err:.2e}")


@pytest.mark.parametrize("mode", [0, 1])
def test_ellipse_elongated_large(mode):
    rng = np.random.default_rng(5)
    n = 400
    s = scenes.random_scene(61, n, 1, 180, 120)
    a = s.arrays()
    a["log_scale"] = np.ascontiguousarray(np.c_[rng.uniform(-3.0, -0.8, n), rng.uniform(-6.0, -4.0, n),
                                                rng.uniform(-6.0, -4.0, n)].T.astype(np.float32))
    note(f"ellipse elongated mode={mode}")
    _check(a, 1, s.cameras[0], mode=mode)


@pytest.mark.skip(reason="a GPU run that included this case, together with a since-removed listing variant, "
                         "ended in a device fault whose cause was never shown; the host emulation of the current "
                         "kernels on this input (test_ellipse_listing_emulation.py) keeps every index in bounds, "
                         "but the case stays off the GPU until a cause is shown")
@pytest.mark.parametrize("mode", [0, 1])
def test_ellipse_tall_view_flat_footprints(mode):
    # a 40 x 3000 view: small Gaussians plus 200 wide, flat ones whose squares are up to
    # 188 tile rows high with only a few kept tiles (most rows of the square are empty)
    n, nw = 4000, 200
    s = scenes.random_scene(64, n, 0, 40, 3000)
    a = s.arrays()
    rng = np.random.default_rng(10)
    ls = rng.uniform(-3.5, -2.5, (n, 3))
    ls[n - nw:] = np.c_[rng.uniform(-1.5, -0.3, nw), rng.uniform(-6.0, -5.0, nw), rng.uniform(-6.0, -5.0, nw)]
    a["log_scale"] = np.ascontiguousarray(ls.T.astype(np.float32))
    o = oracle.preprocess(a, 0, s.cameras[0], tile_test=ELL)
    kept = o["tile_count"] > 0
    rows = (o["rect"][3] - o["rect"][2])[kept]
    assert rows.max() > 100 and (rows > 4 * o["tile_count"][kept]).any()
    note(f"ellipse tall view mode={mode}")
    _check(a, 0, s.cameras[0], mode=mode)


def test_ellipse_c1_and_headline_sampled():
    s = scenes.make_scene("c1_10k_sh0_256")
    note("ellipse c1")
    _check(s.arrays(), s.sh_degree, s.cameras[0])
    s = scenes.make_scene(scenes.HEADLINE)
    cam = s.cameras[0]
    pix = np.random.default_rng(8).choice(cam["width"] * cam["height"], 4096, replace=False)
    note("ellipse headline")
    g, o, err = _check(s.arrays(), s.sh_degree, cam, pixels=pix)
    note(f"  headline pairs {g['num_dups']} ({g['num_dups'] / oracle.preprocess(s.arrays(), 3, cam)['tile_count'].sum():.3f} of the square) image err {err:.2e}")


@pytest.mark.parametrize("mode", [0, 1])
def test_ellipse_backward(mode):
    from tile_differentiable_rasterizer_gs_amd import binding

    s = scenes.random_scene(62, 2000, 2, 170, 110, log_scale_range=(-3.6, -1.9))
    cam = s.cameras[0]
    gimg = np.random.default_rng(3).normal(size=(cam["height"], cam["width"], 3))
    note(f"ellipse backward mode={mode}")
    r = binding.Rasterizer(sort_mode=mode, emit_keys=False, tile_test=ELL)
    g = gpu_grads(s.arrays(), 2, cam, gimg, bg=(0.3, 0.1, 0.2), rast=r)
    r.close()
    o = oracle.render_backward(s.arrays(), 2, cam, gimg, bg=(0.3, 0.1, 0.2), tile_test=ELL)
    check_grads(g, o, f"ellipse backward mode={mode}")
