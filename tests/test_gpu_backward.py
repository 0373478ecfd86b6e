"""Backward pass through the C ABI (gs_backward) vs the gradient oracle (needs an MI355X).

The oracle (oracle/gs_oracle_grad.c, pinned by finite differences in
test_oracle_grad.py) differentiates the same fixed lists in binary64.  The HIP
path works in fp32: every alpha and transmittance carries a relative error of a
few 1e-7, transmittance is recovered by division on the way back (one more such
error per step), and each gradient is a sum of up to hundreds of per-pixel terms of
both signs.  The bound below is therefore relative to the largest gradient of each
kind (terms cancel, so small entries can lose relative precision) plus a relative
part for the large ones:
    |gpu - oracle| <= GRAD_RTOL |oracle| + GRAD_ATOL max|oracle|
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import scenes

from gs_util import note

pytestmark = pytest.mark.gpu

GRAD_RTOL = 2e-3
GRAD_ATOL = 2e-5
PARAMS = ("mean", "quat", "log_scale", "opacity", "sh")
SCREEN = (("screen_mean2d", "mean2d"), ("screen_conic", "conic"), ("screen_rgb", "rgb"),
          ("screen_opacity", "opacity"))


def gpu_grads(arrays, deg, cam, g_image, bg=(0.0, 0.0, 0.0), mode=0, screen=True, rast=None):
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = rast or binding.Rasterizer(sort_mode=mode, emit_keys=False)
    dev = binding.gaussians_to_device(arrays)
    pr = r.preprocess(dev, deg, cam)
    bn = r.bin_and_sort(pr, cam)
    H, W = cam["height"], cam["width"]
    T = torch.empty((H, W), dtype=torch.float32, device="cuda")
    nb = torch.empty((H, W), dtype=torch.int32, device="cuda")
    img = r.composite(pr, bn, cam, bg=bg, final_T=T, n_blend=nb)
    gi = torch.from_numpy(np.ascontiguousarray(g_image, np.float32)).cuda()
    gr = r.backward(dev, deg, cam, pr, bn, T, nb, gi, bg=bg, screen=screen)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in gr.items()}
    out["image"] = img.cpu().numpy()
    out["n_blend"] = nb.cpu().numpy()
    if rast is None:
        r.close()
    return out


def grad_ratio(gpu, ref):
    """Largest |gpu - ref| / (GRAD_RTOL |ref| + GRAD_ATOL max|ref|); <= 1 passes."""
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    if scale == 0.0:
        return 0.0 if np.abs(gpu).max() == 0.0 else np.inf
    bound = GRAD_RTOL * np.abs(ref) + GRAD_ATOL * scale
    return float((np.abs(np.asarray(gpu, np.float64) - ref) / bound).max())


def check_grads(g, o, tag, screen=True):
    worst = {}
    for k in PARAMS:
        worst[k] = grad_ratio(g[k], o[k])
    if screen:
        for ko, kg in SCREEN:
            worst[kg + "(screen)" if kg == "opacity" else kg] = grad_ratio(g[kg], o[ko])
    note(f"{tag}: " + " ".join(f"{k}={v:.3f}" for k, v in worst.items()))
    bad = {k: v for k, v in worst.items() if not v <= 1.0}
    assert not bad, f"{tag}: gradients outside tolerance {bad}"


def _cotangent(cam, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(cam["height"], cam["width"], 3))


@pytest.mark.parametrize("deg", [0, 1, 2, 3])
def test_backward_random_ragged(deg):
    w, h = 150 + 9 * deg, 107 + 5 * deg
    sc = scenes.random_scene(100 + deg, 1500, deg, w, h)
    cam = sc.cameras[0]
    gimg = _cotangent(cam, deg)
    bg = (0.2, -0.1, 0.4)
    note(f"backward random deg={deg} {w}x{h}")
    g = gpu_grads(sc.arrays(), deg, cam, gimg, bg=bg)
    o = oracle.render_backward(sc.arrays(), deg, cam, gimg, bg=bg)
    check_grads(g, o, f"random deg={deg}")


@pytest.mark.parametrize("mode", [0, 1])
def test_backward_c1(mode):
    s = scenes.make_scene("c1_10k_sh0_256")
    cam = s.cameras[0]
    gimg = _cotangent(cam, 7)
    note(f"backward c1 mode={mode}")
    g = gpu_grads(s.arrays(), s.sh_degree, cam, gimg, mode=mode)
    o = oracle.render_backward(s.arrays(), s.sh_degree, cam, gimg)
    check_grads(g, o, f"c1 mode={mode}")


def test_backward_long_pair_lists():
    # large Gaussians: many cover more than 32 tiles (several passes of a 16-lane row)
    sc = scenes.random_scene(7, 300, 3, 240, 176, log_scale_range=(-1.6, -0.9))
    cam = sc.cameras[0]
    tc = oracle.preprocess(sc.arrays(), 3, cam)["tile_count"]
    assert (tc > 32).sum() > 20 and (tc > 0).sum() > (tc > 32).sum()
    gimg = _cotangent(cam, 3)
    note("backward long lists")
    g = gpu_grads(sc.arrays(), 3, cam, gimg, bg=(0.5, 0.5, 0.5))
    o = oracle.render_backward(sc.arrays(), 3, cam, gimg, bg=(0.5, 0.5, 0.5))
    check_grads(g, o, "long lists")


@pytest.mark.parametrize("mode", [0, 1])
def test_backward_lists_longer_than_a_row_takes(mode):
    # hundreds of Gaussians with more than 512 records: their lists are summed by a whole
    # workgroup before the per-Gaussian pass, the others by 16-lane rows
    sc = scenes.random_scene(23, 400, 3, 640, 480, log_scale_range=(-1.2, -0.4))
    cam = sc.cameras[0]
    tc = oracle.preprocess(sc.arrays(), 3, cam)["tile_count"]
    assert (tc > 512).sum() > 100 and ((tc > 0) & (tc <= 512)).sum() > 20
    gimg = _cotangent(cam, 4)
    note(f"backward lists over 512 mode={mode}")
    g = gpu_grads(sc.arrays(), 3, cam, gimg, bg=(0.2, 0.3, 0.4), mode=mode)
    o = oracle.render_backward(sc.arrays(), 3, cam, gimg, bg=(0.2, 0.3, 0.4))
    check_grads(g, o, f"lists over 512 mode={mode}")


def test_backward_opacity_zero_and_clamped():
    sc = scenes.random_scene(8, 800, 2, 128, 96, log_scale_range=(-2.8, -2.0))
    a = sc.arrays()
    idx = np.arange(sc.n)
    a["opacity"] = np.where(idx % 5 == 0, 0.0, np.where(idx % 5 == 1, 1.0, a["opacity"])).astype(np.float32)
    cam = sc.cameras[0]
    gimg = _cotangent(cam, 11)
    note("backward opacity 0 / 1")
    g = gpu_grads(a, 2, cam, gimg)
    o = oracle.render_backward(a, 2, cam, gimg)
    check_grads(g, o, "opacity 0/1")
    # an opacity-0 Gaussian still gets an opacity gradient (alpha = o G is linear in o)
    vis0 = (idx % 5 == 0) & (np.abs(o["opacity"]) > 0)
    assert vis0.any()


def test_backward_deterministic_and_modes_agree():
    sc = scenes.random_scene(9, 2000, 3, 200, 150)
    cam = sc.cameras[0]
    gimg = _cotangent(cam, 2)
    note("backward determinism")
    a = gpu_grads(sc.arrays(), 3, cam, gimg, mode=0)
    b = gpu_grads(sc.arrays(), 3, cam, gimg, mode=0)
    c = gpu_grads(sc.arrays(), 3, cam, gimg, mode=1)
    for k in PARAMS + ("mean2d", "conic", "rgb"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), f"run-to-run {k}"
        assert np.array_equal(a[k].view(np.uint32), c[k].view(np.uint32)), f"sort modes {k}"


def test_backward_reused_context_matches_fresh():
    # a context that served a larger scene before must give the same gradients as a fresh
    # one: every per-pair record is rewritten each call, including tile entries no pixel
    # reached (occluded Gaussians)
    from tile_differentiable_rasterizer_gs_amd import binding

    big = scenes.random_scene(21, 3000, 2, 180, 130, log_scale_range=(-2.2, -1.2))
    small = scenes.random_scene(22, 1200, 2, 180, 130)
    cam_b, cam_s = big.cameras[0], small.cameras[0]
    r = binding.Rasterizer(emit_keys=False)
    gpu_grads(big.arrays(), 2, cam_b, _cotangent(cam_b, 1), rast=r)
    gimg = _cotangent(cam_s, 2)
    reused = gpu_grads(small.arrays(), 2, cam_s, gimg, rast=r)
    r.close()
    fresh = gpu_grads(small.arrays(), 2, cam_s, gimg)
    for k in PARAMS:
        assert np.array_equal(reused[k].view(np.uint32), fresh[k].view(np.uint32)), k
    check_grads(fresh, oracle.render_backward(small.arrays(), 2, cam_s, gimg), "reused context")


def test_backward_empty_and_culled():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    cam = scenes.random_scene(1, 10, 0, 64, 48).cameras[0]
    gimg = _cotangent(cam, 1)
    e = scenes.empty_arrays(1)
    g = gpu_grads(e, 1, cam, gimg)
    assert g["mean"].shape == (3, 0)
    # everything behind the camera: all gradients exactly zero
    sc = scenes.random_scene(2, 50, 1, 64, 48)
    a = sc.arrays()
    R = np.asarray(cam["R"], np.float64).reshape(3, 3)
    behind = -R.T @ np.asarray(cam["t"], np.float64) - 10.0 * R[2]
    a["mean"] = np.repeat(behind[:, None], sc.n, axis=1).astype(np.float32)
    g = gpu_grads(a, 1, sc.cameras[0], _cotangent(sc.cameras[0], 1))
    for k in PARAMS:
        assert np.all(g[k] == 0.0), k
    torch.cuda.synchronize()
    assert binding is not None


def test_autograd_function_matches_direct_backward():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    sc = scenes.random_scene(12, 1000, 3, 96, 80)
    cam = sc.cameras[0]
    gimg = _cotangent(cam, 5).astype(np.float32)
    direct = gpu_grads(sc.arrays(), 3, cam, gimg, screen=False)
    r = binding.Rasterizer(emit_keys=False)
    params = {k: v.clone().requires_grad_(True) for k, v in binding.gaussians_to_device(sc.arrays()).items()}
    img = binding.render_differentiable(r, params, 3, cam)
    loss = (img * torch.from_numpy(gimg).cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    for k in PARAMS:
        assert np.array_equal(params[k].grad.cpu().numpy().view(np.uint32), direct[k].view(np.uint32)), k
    r.close()


def test_backward_headline_scene_sampled_pixels():
    # the 1M-Gaussian SH3 1080p frame in the bench's launch configuration; the loss
    # reads 48 random pixels, which the oracle can differentiate one by one
    s = scenes.make_scene(scenes.HEADLINE)
    cam = s.cameras[0]
    H, W = cam["height"], cam["width"]
    rng = np.random.default_rng(17)
    pix = rng.choice(H * W, 48, replace=False)
    gimg = np.zeros((H * W, 3))
    gimg[pix] = rng.normal(size=(48, 3))
    gimg = gimg.reshape(H, W, 3)
    note("backward headline scene")
    g = gpu_grads(s.arrays(), s.sh_degree, cam, gimg)
    o = oracle.render_backward(s.arrays(), s.sh_degree, cam, gimg, pixels=pix)
    touched = np.abs(o["opacity"]) > 0
    note(f"headline: {int(touched.sum())} Gaussians reach the sampled pixels")
    assert touched.sum() > 100
    check_grads(g, o, "headline sampled")


# log-scale ranges of the long axis and of the two short axes: 2D covariances with
# a c / det up to ~160 ("moderate") and ~2100 ("thin"); c3's footprints reach ~100.
# The last number is a condition that at least 20 footprints of the scene exceed.
ANISO = {"moderate": ((-3.0, -1.2), (-5.0, -3.5), 30.0), "thin": ((-3.0, -0.8), (-6.0, -4.0), 300.0)}
# Above this a c / det the gradients of a thin axis' log-scale (and through it of the
# quaternion and the mean) are amplified from the screen-space gradients by about that
# condition number: the binary32 sums of the screen-space moments can no longer resolve
# them to the bound above, whatever the precision of the chain after them.  Such Gaussians
# are reported, not asserted.
KAPPA_MAX = 200.0


@pytest.mark.parametrize("aniso", ["moderate", "thin"])
@pytest.mark.parametrize("tile_test", [0, 1])
def test_backward_elongated_footprints(tile_test, aniso):
    # rotated Gaussians with one axis much longer than the other two: the 2D covariance's
    # determinant cancels, so the chain from the conic back to the parameters is ill-conditioned
    from tile_differentiable_rasterizer_gs_amd import binding

    rng = np.random.default_rng(15)
    n = 600
    (l0, l1), (t0, t1), k_min = ANISO[aniso]
    sc = scenes.random_scene(16, n, 1, 180, 130)
    a = sc.arrays()
    a["log_scale"] = np.ascontiguousarray(np.c_[rng.uniform(l0, l1, n), rng.uniform(t0, t1, n),
                                                rng.uniform(t0, t1, n)].T.astype(np.float32))
    cam = sc.cameras[0]
    gimg = _cotangent(cam, 11)
    bg = (0.1, 0.3, -0.2)
    note(f"backward elongated {aniso} tile_test={tile_test}")
    r = binding.Rasterizer(emit_keys=False, tile_test=tile_test)
    g = gpu_grads(a, 1, cam, gimg, bg=bg, rast=r)
    r.close()
    o = oracle.render_backward(a, 1, cam, gimg, bg=bg, tile_test=tile_test)
    p = oracle.preprocess(a, 1, cam, tile_test=tile_test)
    ca, cb, cc = (p["cov2d"][i].astype(np.float64) for i in range(3))
    kappa = np.where(p["tile_count"] > 0, ca * cc / (ca * cc - cb * cb), 1.0)
    keep = kappa <= KAPPA_MAX
    assert (kappa > k_min).sum() > 20
    sub = lambda d, ks: {k: d[k][..., keep] for k in ks}
    check_grads(sub(g, PARAMS + tuple(kg for _, kg in SCREEN)), sub(o, PARAMS + tuple(ko for ko, _ in SCREEN)),
                f"elongated {aniso} tile_test={tile_test}, a c / det <= {KAPPA_MAX:g} ({keep.sum()} Gaussians)")
    if not keep.all():
        worst = {k: grad_ratio(g[k][..., ~keep], o[k][..., ~keep]) for k in PARAMS}
        note(f"  a c / det > {KAPPA_MAX:g} ({(~keep).sum()} Gaussians, not asserted): " +
             " ".join(f"{k}={v:.2f}" for k, v in worst.items()))
