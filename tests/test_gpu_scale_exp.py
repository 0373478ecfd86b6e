"""Exhaustive check of the scale activation, the one transcendental on the integer key path (needs an MI355X).

The preprocess turns each log-scale into exp(log_scale) rounded to binary32 (lesson, sections "Ce qu'un
Gaussien porte" and "Étape 5"); the 2D covariance, radius, tile rectangle and count all follow from
those bits, so the device (ROCm's binary64 exp) and the oracle (the host libm's binary64 exp) must
round every log-scale to the same float.  This test runs gs_scale_activation over every binary32
value in [-16, 4] (2.18e9 inputs; every workload draws its log-scales from [-6, 0], and e^-16 to e^4
spans scales far beyond any scene's) and compares each result bit for bit with the oracle's.
"""
import numpy as np
import pytest

import oracle

from gs_util import note

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def _bits(x: float) -> int:
    return int(np.array(x, np.float32).view(np.uint32))


def _runs():
    """Bit-pattern runs covering [-16, 4]: -0.0 down to -16 (patterns grow with |x|), 0 up to 4."""
    return [(_bits(-0.0), _bits(-16.0)), (_bits(0.0), _bits(4.0))]


def test_scale_activation_matches_host_exp_on_every_float_in_minus16_4():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = binding.Rasterizer(emit_keys=False)
    dev_in = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    dev_out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    total = sum(b - a + 1 for a, b in _runs())
    bad = []
    done = 0
    for first, last in _runs():
        for lo in range(first, last + 1, CHUNK):
            hi = min(lo + CHUNK, last + 1)
            x = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
            m = x.size
            dev_in[:m].copy_(torch.from_numpy(x))
            r.scale_activation(dev_in[:m], out=dev_out[:m])
            got = dev_out[:m].cpu().numpy()
            want = oracle.scale_activation(x)
            diff = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
            bad.extend((float(x[i]), float(got[i]), float(want[i])) for i in diff[:20])
            done += m
            note(f"scale activation: {done} of {total} inputs, {len(bad)} differing so far")
    r.close()
    assert done == total
    assert not bad, f"device and host exp round differently: {bad[:10]}"
