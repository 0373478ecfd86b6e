"""Seeded synthetic scenes and cameras for the forward Gaussian-splatting rasterizer.

This module only draws inputs: it holds none of the rasterizer's arithmetic
(no covariance, projection, colour or compositing step). Both the HIP path and
the CPU oracle consume what it returns.

Scale and content follow the lesson "3D Gaussian Splatting from scratch"
(aiengineeringfromscratch.com), section "Ce qu'un Gaussien porte": a Gaussian
carries a position (3), a unit quaternion (4), per-axis log-scales (3), an
opacity already in [0, 1] (1) and 3*(L+1)^2 spherical-harmonic coefficients;
scenes hold 1-5 million Gaussians, and SH degree 3 is the default (the lesson's
spherical-harmonics paragraph). No trained scene or dataset is available, so
these seeded distributions stand in for one.

Layout returned (structure of arrays, float32, C-contiguous):
    mean      [3, n]           world position
    quat      [4, n]           (w, x, y, z), normalised here
    log_scale [3, n]
    opacity   [n]              post-sigmoid
    sh        [K*3, n]         plane k*3 + c holds coefficient k of channel c,
                               K = (sh_degree + 1)^2
Cameras are dicts: R (3x3 world->camera, row-major, x right / y down /
z forward), t (3,), fx, fy, cx, cy, znear, width, height.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ZNEAR = 0.2

# The five workloads: small sanity case, mid-size SH3 case, the 1M SH3 1080p
# headline, the 5M stress case with 2 % large Gaussians, and a 3M 32-view orbit.
CONFIGS = {
    "c1_10k_sh0_256": dict(seed=1, n=10_000, sh_degree=0, width=256, height=256, layout="uniform"),
    "c2_100k_sh3_800": dict(seed=2, n=100_000, sh_degree=3, width=800, height=800, layout="uniform"),
    "c3_1m_sh3_1080p": dict(seed=3, n=1_000_000, sh_degree=3, width=1920, height=1080, layout="clusters"),
    "c4_5m_sh3_1080p_large": dict(seed=4, n=5_000_000, sh_degree=3, width=1920, height=1080,
                                  layout="clusters", large_frac=0.02),
    "c5_3m_sh3_1080p_orbit32": dict(seed=5, n=3_000_000, sh_degree=3, width=1920, height=1080,
                                    layout="clusters", views=32),
}
HEADLINE = "c3_1m_sh3_1080p"


def sh_coeff_count(sh_degree: int) -> int:
    return (sh_degree + 1) ** 2


def look_at_camera(position, target, f, width, height, znear=ZNEAR) -> dict:
    """Pinhole camera at `position` looking at `target` with world +y as up.

    Rows of R are the camera axes in world coordinates: z toward the target,
    x = normalise(z x up), y = z x x (so y points down in the image).
    """
    c = np.asarray(position, dtype=np.float64)
    z = np.asarray(target, dtype=np.float64) - c
    z /= np.linalg.norm(z)
    x = np.cross(z, np.array([0.0, 1.0, 0.0]))
    x /= np.linalg.norm(x)
    y = np.cross(z, x)
    R = np.stack([x, y, z]).astype(np.float32)
    t = (-(R.astype(np.float64) @ c)).astype(np.float32)
    return dict(R=R, t=t, fx=float(np.float32(f)), fy=float(np.float32(f)),
                cx=float(np.float32(width / 2.0)), cy=float(np.float32(height / 2.0)),
                znear=float(np.float32(znear)), width=int(width), height=int(height))


def orbit_position(radius: float, azimuth: float, elevation: float) -> np.ndarray:
    ce = math.cos(elevation)
    return np.array([radius * ce * math.sin(azimuth), radius * math.sin(elevation),
                     -radius * ce * math.cos(azimuth)])


def _random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Haar-random rotation via QR of a Gaussian matrix (sign-fixed, det +1)."""
    a = rng.standard_normal((3, 3))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def _cluster_means(rng: np.random.Generator, n: int) -> np.ndarray:
    """90 % from 64 anisotropic clusters inside [-3,3]^3, 10 % on a radius-8 shell."""
    n_shell = n // 10
    n_clu = n - n_shell
    n_clusters = 64
    centres = rng.uniform(-2.0, 2.0, size=(n_clusters, 3))
    stds = rng.uniform(0.05, 0.5, size=(n_clusters, 3))
    frames = np.stack([_random_rotation(rng) for _ in range(n_clusters)])
    assign = rng.integers(0, n_clusters, size=n_clu)
    pts = np.empty((n_clu, 3))
    todo = np.arange(n_clu)
    while todo.size:
        k = assign[todo]
        local = rng.standard_normal((todo.size, 3)) * stds[k]
        p = centres[k] + np.einsum("nij,nj->ni", frames[k], local)
        ok = np.all(np.abs(p) <= 3.0, axis=1)
        pts[todo[ok]] = p[ok]
        todo = todo[~ok]
    shell = rng.standard_normal((n_shell, 3))
    shell = 8.0 * shell / np.linalg.norm(shell, axis=1, keepdims=True)
    out = np.concatenate([pts, shell], axis=0)
    return out[rng.permutation(n)]


@dataclass
class Scene:
    name: str
    n: int
    sh_degree: int
    mean: np.ndarray
    quat: np.ndarray
    log_scale: np.ndarray
    opacity: np.ndarray
    sh: np.ndarray
    cameras: list

    def arrays(self) -> dict:
        return dict(mean=self.mean, quat=self.quat, log_scale=self.log_scale,
                    opacity=self.opacity, sh=self.sh)

    @property
    def param_bytes(self) -> int:
        return sum(a.nbytes for a in self.arrays().values())


def _soa(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.T.astype(np.float32))


def make_scene(name: str, n: int | None = None) -> Scene:
    """Build one of CONFIGS; `n` overrides the Gaussian count (same recipe)."""
    cfg = CONFIGS[name]
    n = cfg["n"] if n is None else int(n)
    rng = np.random.default_rng(cfg["seed"])
    deg = cfg["sh_degree"]
    K = sh_coeff_count(deg)
    clusters = cfg["layout"] == "clusters"
    # fixed draw order: means, quats, log-scales, opacity normals, SH DC, SH rest, camera
    means = _cluster_means(rng, n) if clusters else rng.uniform(-1.0, 1.0, size=(n, 3))
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    if clusters:
        ls = rng.uniform(-6.0, -3.0, size=(n, 3))
        large = cfg.get("large_frac", 0.0)
        if large:
            idx = rng.choice(n, size=int(math.floor(large * n)), replace=False)
            ls[idx] = rng.uniform(-1.5, 0.0, size=(idx.size, 3))
        op = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.5, size=n)))
    else:
        ls = rng.uniform(-4.5, -2.5, size=(n, 3))
        op = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, size=n)))
    sh = np.zeros((n, K, 3))
    sh[:, 0, :] = rng.normal(0.0, 0.5, size=(n, 3))
    if K > 1:
        sh[:, 1:, :] = rng.normal(0.0, 0.1, size=(n, K - 1, 3))
    w, h = cfg["width"], cfg["height"]
    if name.startswith("c1"):
        cams = [look_at_camera((0.0, 0.0, -4.0), (0.0, 0.0, 0.0), 256.0, w, h)]
    elif name.startswith("c2"):
        az = rng.uniform(0.0, 2.0 * math.pi)
        el = rng.uniform(-math.pi / 4, math.pi / 4)
        cams = [look_at_camera(orbit_position(4.0, az, el), (0, 0, 0), 1100.0, w, h)]
    elif "views" in cfg:
        el = math.radians(15.0)
        cams = [look_at_camera(orbit_position(5.0, 2 * math.pi * k / cfg["views"], el), (0, 0, 0),
                               1500.0, w, h) for k in range(cfg["views"])]
    else:
        cams = [look_at_camera((0.0, 0.0, -5.0), (0.0, 0.0, 0.0), 1500.0, w, h)]
    return Scene(name=name, n=n, sh_degree=deg,
                 mean=_soa(means), quat=_soa(q), log_scale=_soa(ls),
                 opacity=np.ascontiguousarray(op.astype(np.float32)),
                 sh=np.ascontiguousarray(sh.reshape(n, K * 3).T.astype(np.float32)),
                 cameras=cams)


def random_scene(seed: int, n: int, sh_degree: int, width: int, height: int,
                 f: float | None = None, spread: float = 1.0,
                 log_scale_range=(-4.5, -2.5), camera_distance: float = 4.0) -> Scene:
    """Small seeded scene for parity tests (uniform cube, random orbit camera)."""
    rng = np.random.default_rng(seed)
    K = sh_coeff_count(sh_degree)
    means = rng.uniform(-spread, spread, size=(n, 3))
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    ls = rng.uniform(log_scale_range[0], log_scale_range[1], size=(n, 3))
    op = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, size=n)))
    sh = np.zeros((n, K, 3))
    sh[:, 0, :] = rng.normal(0.0, 0.5, size=(n, 3))
    if K > 1:
        sh[:, 1:, :] = rng.normal(0.0, 0.1, size=(n, K - 1, 3))
    az = rng.uniform(0.0, 2.0 * math.pi)
    el = rng.uniform(-math.pi / 4, math.pi / 4)
    f = float(max(width, height)) if f is None else f
    cam = look_at_camera(orbit_position(camera_distance, az, el), (0, 0, 0), f, width, height)
    return Scene(name=f"random_{seed}", n=n, sh_degree=sh_degree,
                 mean=_soa(means), quat=_soa(q), log_scale=_soa(ls),
                 opacity=np.ascontiguousarray(op.astype(np.float32)),
                 sh=np.ascontiguousarray(sh.reshape(n, K * 3).T.astype(np.float32)),
                 cameras=[cam])


def empty_arrays(sh_degree: int) -> dict:
    K = sh_coeff_count(sh_degree)
    z = lambda r: np.zeros((r, 0), dtype=np.float32)
    return dict(mean=z(3), quat=z(4), log_scale=z(3), opacity=np.zeros(0, np.float32), sh=z(K * 3))
