"""The lesson's 2D splat-fitting workload on the HIP rasteriser.

Lesson "3D Gaussian Splatting from scratch", sections "Étape 3: Une scène de splat
2D entraînable" and "Étape 4: Adaptez les Gaussiens 2D à une image cible": a set of
2D splats with unconstrained parameters (mean, per-axis log-scale, one rotation
angle, colour and opacity logits, a depth scalar that only orders them), mapped at
render time to a covariance R diag(exp(log_scale))^2 R^T, sigmoid colours and
sigmoid opacities, is fitted to a synthetic target image (a red disc and a blue
square on black) by Adam on the mean squared error.

The rasteriser (forward and gradient) runs in `libgsrast.so` (gs_splat2d_forward /
gs_splat2d_backward); the parameter activations, the loss and the optimiser are
ordinary torch operations on the device.
"""
from __future__ import annotations

import math

import torch

from . import binding


def make_target(size: int = 64, device="cuda") -> torch.Tensor:
    """[size, size, 3] target: a red disc (centre (20, 20), radius 10, colour (1, 0.2, 0.2))
    and a blue square (centre (45, 40), half-width 8 exclusive, colour (0.2, 0.3, 1)) on black."""
    y, x = torch.meshgrid(torch.arange(size, device=device), torch.arange(size, device=device), indexing="ij")
    img = torch.zeros((size, size, 3), dtype=torch.float32, device=device)
    disc = (x - 20) ** 2 + (y - 20) ** 2 < 100
    square = ((x - 45).abs() < 8) & ((y - 40).abs() < 8)
    img[disc] = torch.tensor([1.0, 0.2, 0.2], device=device)
    img[square] = torch.tensor([0.2, 0.3, 1.0], device=device)
    return img


def init_splats(n: int = 64, size: int = 64, seed: int = 0, device="cuda") -> dict:
    """Initial unconstrained parameters: means uniform over the image, log-scales log 2
    (a 2-pixel standard deviation), rotation 0, colour logits N(0, 0.5^2), opacity
    logits 0 (opacity 1/2), depths uniform in [0, 1)."""
    g = torch.Generator().manual_seed(seed)
    p = dict(mean=torch.rand(n, 2, generator=g) * size,
             log_scale=torch.full((n, 2), math.log(2.0)),
             angle=torch.zeros(n),
             colour_logit=0.5 * torch.randn(n, 3, generator=g),
             opacity_logit=torch.zeros(n),
             depth=torch.rand(n, generator=g))
    return {k: v.to(device).requires_grad_(k != "depth") for k, v in p.items()}


def splat_arrays(p: dict):
    """(means, covs, colours, opacities, depths) the rasteriser takes, from the parameters."""
    s2 = torch.exp(2.0 * p["log_scale"])
    c, s = torch.cos(p["angle"]), torch.sin(p["angle"])
    # R diag(s^2) R^T written out for R = [[c, -s], [s, c]]
    a = c * c * s2[:, 0] + s * s * s2[:, 1]
    b = c * s * (s2[:, 0] - s2[:, 1])
    d = s * s * s2[:, 0] + c * c * s2[:, 1]
    covs = torch.stack([torch.stack([a, b], -1), torch.stack([b, d], -1)], -2)
    return p["mean"], covs, torch.sigmoid(p["colour_logit"]), torch.sigmoid(p["opacity_logit"]), p["depth"]


def render(rasterizer: binding.Rasterizer, p: dict, size: int) -> torch.Tensor:
    return binding.rasterise_2d(rasterizer, *splat_arrays(p), (size, size))


def fit(rasterizer: binding.Rasterizer | None = None, n: int = 64, size: int = 64, steps: int = 200,
        lr: float = 0.05, seed: int = 0, record_every: int = 1) -> dict:
    """Fits n splats to make_target(size) with Adam(lr) for `steps` steps.  Returns the loss
    history (every `record_every` steps, plus the last), the final parameters and image."""
    r = rasterizer or binding.Rasterizer(emit_keys=False)
    target = make_target(size)
    p = init_splats(n, size, seed)
    opt = torch.optim.Adam([v for k, v in p.items() if k != "depth"], lr=lr)
    losses = []
    for step in range(steps):
        img = render(r, p, size)
        loss = torch.mean((img - target) ** 2)
        opt.zero_grad()
        loss.backward()
        opt.step()
        if step % record_every == 0 or step == steps - 1:
            losses.append((step, loss.detach()))
    with torch.no_grad():
        final = render(r, p, size)
        final_loss = torch.mean((final - target) ** 2)
    out = dict(losses=[(s, float(l)) for s, l in losses], final_loss=float(final_loss), params=p, image=final)
    if rasterizer is None:
        r.close()
    return out
