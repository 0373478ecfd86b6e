"""gs_render_noalloc (buffers in the library's static scratch, no allocation) against gs_render.

Needs an MI355X.  The allocation-free entry point runs the same kernels as gs_render, so the
images must be identical bit for bit; two calls in a row (the second with a smaller scene)
check that nothing of the first call's scratch contents leaks into the second.
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import scenes

from gs_util import IMAGE_TOL, image_error, note, plane_scene

pytestmark = pytest.mark.gpu


def test_noalloc_render_matches_render_twice_then_smaller():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    big = scenes.random_scene(seed=201, n=20000, sh_degree=2, width=333, height=250)
    small = scenes.random_scene(seed=202, n=3000, sh_degree=3, width=97, height=71)
    r = binding.Rasterizer()
    for tag, sc, bg in (("big", big, (0.1, 0.2, 0.3)), ("small", small, (0.4, 0.0, 0.2))):
        note(f"noalloc {tag}: n={sc.n} {sc.cameras[0]['width']}x{sc.cameras[0]['height']}")
        dev = binding.gaussians_to_device(sc.arrays())
        cam = sc.cameras[0]
        ref = r.render(dev, sc.sh_degree, cam, bg=bg).clone()
        got = r.render_noalloc(dev, sc.sh_degree, cam, bg=bg)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), tag
        o = oracle.preprocess(sc.arrays(), sc.sh_degree, cam)
        oimg, _, _ = oracle.composite(o, cam, bg=bg)
        err = image_error(got.cpu().numpy(), oimg)
        note(f"  identical to gs_render; image err vs oracle {err:.2e}")
        assert err <= IMAGE_TOL
    # the context's own workspace is untouched: staged calls still work afterwards
    dev = binding.gaussians_to_device(small.arrays())
    pr = r.preprocess(dev, small.sh_degree, small.cameras[0])
    bn = r.bin_and_sort(pr, small.cameras[0])
    img = r.composite(pr, bn, small.cameras[0], bg=(0.4, 0.0, 0.2))
    assert torch.equal(img, got)
    r.close()


def test_noalloc_crowded_depths_fall_back_inside_the_scratch():
    # every depth equal: the bucketed depth order overflows and the frame is redone with the
    # radix sort, whose buffers then come from the scratch too; twice, then a normal frame
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = binding.Rasterizer()
    for seed, n, depths in ((210, 7000, (5.0,)), (211, 5000, (3.0,)), (212, 4000, (2.0, 3.0, 4.0, 6.0))):
        arrays, cam = plane_scene(seed, n, depths)
        note(f"noalloc crowded: n={n} depths={depths}")
        dev = binding.gaussians_to_device(arrays)
        ref = r.render(dev, 0, cam, bg=(0.3, 0.3, 0.1)).clone()
        got = r.render_noalloc(dev, 0, cam, bg=(0.3, 0.3, 0.1))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), depths
    r.close()


def test_noalloc_rejects_what_does_not_fit():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = binding.Rasterizer()
    # too many Gaussians for half the scratch: refused before anything is enqueued
    n = 400_000
    many = {k: torch.zeros(s, dtype=torch.float32, device="cuda")
            for k, s in (("mean", (3, n)), ("quat", (4, n)), ("log_scale", (3, n)), ("opacity", (n,)),
                         ("sh", (3, n)))}
    cam = scenes.look_at_camera((0.0, 0.0, -4.0), (0, 0, 0), 500.0, 640, 480)
    with pytest.raises(binding.GsError) as e:
        r.render_noalloc(many, 0, cam)
    assert e.value.status == binding.GS_ERR_CAPACITY
    # too many pairs: refused once the pair count is known
    sc = scenes.random_scene(seed=93, n=30000, sh_degree=0, width=1280, height=720, log_scale_range=(-1.2, -0.4))
    dev = binding.gaussians_to_device(sc.arrays())
    note("noalloc pair capacity")
    with pytest.raises(binding.GsError) as e:
        r.render_noalloc(dev, 0, sc.cameras[0])
    assert e.value.status == binding.GS_ERR_CAPACITY
    # the context recovers: a frame that fits renders as gs_render does
    small = scenes.random_scene(seed=203, n=2000, sh_degree=1, width=64, height=48)
    d2 = binding.gaussians_to_device(small.arrays())
    ref = r.render(d2, 1, small.cameras[0]).clone()
    got = r.render_noalloc(d2, 1, small.cameras[0])
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    r.close()
