"""gs_cache_covariance (the view-independent 3D covariance computed once for several views)
against the uncached preprocess (needs an MI355X).

The lesson's "Ce qu'un Gaussien porte" builds Sigma = R S S^T R^T from the quaternion and the
scales alone, so every view of a scene shares it.  With the cache held, gs_preprocess reads the
six stored values instead of recomputing them; the projection, binning and image must be the
same bits as without it, for every view of an orbit.  The cache applies only to the Gaussians
whose quat / log_scale tensors it was built from, and is rebuilt or dropped on request.
"""
import numpy as np
import pytest

import oracle
from tile_differentiable_rasterizer_gs_amd import binding, scenes

from gs_util import check_binning, check_preprocess, note

pytestmark = pytest.mark.gpu


def _frame(r, dev, deg, cam):
    import torch

    pr = r.preprocess(dev, deg, cam)
    bn = r.bin_and_sort(pr, cam)
    img = r.composite(pr, bn, cam, bg=(0.2, 0.1, 0.0))
    pt = r.projected_tensors(pr)
    bt = r.binning_tensors(bn)
    torch.cuda.synchronize()
    return dict(splat=pt["splat"].cpu().numpy(), rect=pt["rect"].cpu().numpy(), image=img.cpu().numpy(),
                values=bt["values"].cpu().numpy(), ranges=bt["ranges"].cpu().numpy())


def _same(a, b, what):
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{what}: {k} differs"


def test_cached_covariance_gives_the_same_bits_on_every_view():
    s = scenes.random_scene(400, 20000, 2, 320, 240, log_scale_range=(-4.0, -2.0))
    # four views on an orbit around the scene
    s.cameras = [scenes.look_at_camera(scenes.orbit_position(4.0, 0.7 * k, 0.3), (0.0, 0.0, 0.0), 300.0, 320, 240)
                 for k in range(4)]
    dev = binding.gaussians_to_device(s.arrays())
    plain, cached = binding.Rasterizer(), binding.Rasterizer()
    cached.cache_covariance(dev, s.sh_degree)
    for i, cam in enumerate(s.cameras):
        a, b = _frame(plain, dev, s.sh_degree, cam), _frame(cached, dev, s.sh_degree, cam)
        _same(a, b, f"view {i}")
    # and the cached path against the oracle on one view
    pr = cached.preprocess(dev, s.sh_degree, s.cameras[1])
    pt = cached.projected_tensors(pr)
    o = oracle.preprocess(s.arrays(), s.sh_degree, s.cameras[1])
    check_preprocess(dict(splat=pt["splat"].cpu().numpy(), depth=pt["depth"].cpu().numpy(),
                          rect=pt["rect"].cpu().numpy().view(np.uint16).astype(np.int32),
                          tile_count=pt["tile_count"].cpu().numpy().view(np.uint32)), o)
    note(f"covariance cache: {len(s.cameras)} views bit-identical, preprocess equal to the oracle")
    plain.close()
    cached.close()


def test_cache_follows_the_parameter_tensors():
    import torch

    s = scenes.random_scene(401, 5000, 1, 256, 192, log_scale_range=(-3.5, -2.0))
    cam = s.cameras[0]
    dev = binding.gaussians_to_device(s.arrays())
    r, ref = binding.Rasterizer(), binding.Rasterizer()
    r.cache_covariance(dev, s.sh_degree)
    # other tensors with other values: the cache does not apply to them
    other = binding.gaussians_to_device(scenes.random_scene(402, 5000, 1, 256, 192).arrays())
    _same(_frame(r, other, s.sh_degree, cam), _frame(ref, other, s.sh_degree, cam), "other tensors")
    # parameters changed in place, cache rebuilt: the new covariances are used
    with torch.no_grad():
        dev["quat"].add_(0.3 * torch.randn_like(dev["quat"]))
        dev["log_scale"].add_(0.2)
    r.cache_covariance(dev, s.sh_degree)
    _same(_frame(r, dev, s.sh_degree, cam), _frame(ref, dev, s.sh_degree, cam), "rebuilt")
    # dropped: the uncached path again (same bits)
    r.cache_covariance(None)
    _same(_frame(r, dev, s.sh_degree, cam), _frame(ref, dev, s.sh_degree, cam), "dropped")
    # the image of a cached frame matches the oracle's binning too
    r.cache_covariance(dev, s.sh_degree)
    g = {k: v.detach().cpu().numpy() for k, v in dev.items()}
    pr = r.preprocess(dev, s.sh_degree, cam)
    bn = r.bin_and_sort(pr, cam)
    bt = r.binning_tensors(bn)
    torch.cuda.synchronize()
    check_binning(dict(num_dups=bt["num_dups"], values=bt["values"].cpu().numpy().view(np.uint32),
                       ranges=bt["ranges"].cpu().numpy().view(np.uint32),
                       keys=None if bt["keys"] is None else bt["keys"].cpu().numpy().view(np.uint64)),
                  oracle.bin_pairs(oracle.preprocess(g, s.sh_degree, cam)))
    r.close()
    ref.close()
