"""CPU oracle for the forward Gaussian-splatting rasterizer.

TEST INFRASTRUCTURE ONLY: imported by `tests/`, by `__graft_entry__.smoke()`
and by the benchmark's `cpu_baseline` leg, never by the product package.

Independent pieces:
  * `gs_oracle.c` (built with `gs_oracle_grad.c` into `liboracle.so` by gcc,
    OpenMP, -ffp-contract=off): projection in binary32 following a fixed
    operation order, binning, and per-pixel binary64 compositing over all
    depth-sorted Gaussians;
  * `gs_oracle_grad.c`: the same projection and compositing in binary64 over
    fixed per-pixel lists, and their vector-Jacobian products written out by
    hand (the gradients of the lesson's section "Pourquoi est-ce
    différenciable");
  * `composite_2d` below: the dense 2D rasteriser of the lesson
    "3D Gaussian Splatting from scratch", section "Étape 2: Rasteriser à
    éclaboussure en 2D", in numpy binary64 (every Gaussian at every pixel,
    alpha clamped to 0.99, ordered by depth, no early stop).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
_SRC_GRAD = os.path.join(_HERE, "gs_oracle_grad.c")
_LIB = os.path.join(_HERE, "liboracle.so")
TILE = 16


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (binary32 semantics: no contraction, no fast-math)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in (_SRC, _SRC_GRAD))
    if force or stale:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
                               "-o", tmp, _SRC, _SRC_GRAD, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Camera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3),
                ("fx", ctypes.c_float), ("fy", ctypes.c_float), ("cx", ctypes.c_float),
                ("cy", ctypes.c_float), ("znear", ctypes.c_float),
                ("width", ctypes.c_int32), ("height", ctypes.c_int32)]


class _Projected(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("depth", "mean2d", "cov2d", "conic", "radius", "cov3d", "rect", "tile_count", "rgb", "ellipse")]


TILE_SQUARE, TILE_ELLIPSE = 0, 1   # tile membership rules (the library's GS_OPT_TILE_TEST)


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.oracle_preprocess.argtypes = [i64, i32, P, P, P, P, P, ctypes.POINTER(_Camera),
                                          ctypes.POINTER(_Projected)]
        lib.oracle_preprocess.restype = None
        lib.oracle_preprocess_ex.argtypes = [i64, i32, P, P, P, P, P, ctypes.POINTER(_Camera), i32,
                                             ctypes.POINTER(_Projected)]
        lib.oracle_preprocess_ex.restype = None
        lib.oracle_bin.argtypes = [i64, P, P, P, i32, i32, P, P, P, P, P]
        lib.oracle_bin.restype = None
        lib.oracle_bin_ex.argtypes = [i64, P, P, P, i32, i32, P, P, i32, P, P, P, P, P]
        lib.oracle_bin_ex.restype = None
        lib.oracle_composite_ex.argtypes = [i64, P, P, P, P, P, P, P, P, i32, i32, i32, P, i32, ctypes.c_double,
                                            P, i64, P, P, P]
        lib.oracle_composite_ex.restype = None
        lib.oracle_row_span.argtypes = [ctypes.c_float, ctypes.c_float, P, i32, i32, i32,
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.oracle_row_span.restype = None
        lib.oracle_total_pairs.argtypes = [i64, P]
        lib.oracle_total_pairs.restype = i64
        lib.oracle_composite.argtypes = [i64, P, P, P, P, P, P, P, i32, i32, P, i32, ctypes.c_double,
                                         P, i64, P, P, P]
        lib.oracle_composite.restype = None
        lib.oracle_cov3d.argtypes = [P, P, P]
        lib.oracle_scale_activation.argtypes = [i64, P, P]
        lib.oracle_cov3d.restype = None
        lib.oracle_sh_basis.argtypes = [ctypes.c_double] * 3 + [P]
        lib.oracle_sh_basis.restype = None
        lib.oracle_project64.argtypes = [i64, i32, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_project64.restype = None
        lib.oracle_project_backward.argtypes = [i64, i32, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_project_backward.restype = None
        lib.oracle_composite_fixed.argtypes = [i64, P, P, P, P, P, P, P, i32, P, i64, i32, i32, P, P,
                                               ctypes.c_double, P, P, P]
        lib.oracle_composite_fixed.restype = None
        lib.oracle_composite_backward.argtypes = [i64, P, P, P, P, P, P, P, i32, P, i64, i32, i32, P, P,
                                                  ctypes.c_double, P, P, i64, P, P, P, P]
        lib.oracle_composite_backward.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def tiles_for(camera: dict) -> tuple[int, int]:
    return (camera["width"] + TILE - 1) // TILE, (camera["height"] + TILE - 1) // TILE


def _camera(camera: dict) -> _Camera:
    c = _Camera()
    c.R[:] = [float(v) for v in np.asarray(camera["R"], np.float32).reshape(9)]
    c.t[:] = [float(v) for v in np.asarray(camera["t"], np.float32).reshape(3)]
    for k in ("fx", "fy", "cx", "cy", "znear"):
        setattr(c, k, float(np.float32(camera[k])))
    c.width, c.height = int(camera["width"]), int(camera["height"])
    return c


def preprocess(arrays: dict, sh_degree: int, camera: dict, tile_test: int = TILE_SQUARE) -> dict:
    """Per-Gaussian projection record (numpy planes, index g last).  tile_test selects the tile
    membership rule (the pages' square, or its part that meets the exact 3-sigma ellipse)."""
    lib = _load()
    mean, quat = _f32(arrays["mean"]), _f32(arrays["quat"])
    ls, op, sh = _f32(arrays["log_scale"]), _f32(arrays["opacity"]), _f32(arrays["sh"])
    n = mean.shape[1]
    out = dict(depth=np.zeros(n, np.float32), mean2d=np.zeros((2, n), np.float32),
               cov2d=np.zeros((3, n), np.float32), conic=np.zeros((3, n), np.float32),
               radius=np.zeros(n, np.float32), cov3d=np.zeros((6, n), np.float32),
               rect=np.zeros((4, n), np.int32), tile_count=np.zeros(n, np.uint32),
               rgb=np.zeros((3, n), np.float64), ellipse=np.zeros((5, n), np.float32))
    pr = _Projected(**{k: _ptr(v).value for k, v in out.items()})
    cam = _camera(camera)
    lib.oracle_preprocess_ex(n, sh_degree, _ptr(mean), _ptr(quat), _ptr(ls), _ptr(op), _ptr(sh),
                             ctypes.byref(cam), int(tile_test), ctypes.byref(pr))
    out["opacity"] = op
    out["tiles"] = tiles_for(camera)
    out["tile_test"] = int(tile_test)
    return out


def row_span(u: float, v: float, ellipse5, x0: int, x1: int, ty: int) -> tuple[int, int]:
    """Kept tiles [a, b) of tile row ty under the exact-footprint rule (binary32)."""
    lib = _load()
    E = _f32(ellipse5).reshape(5)
    a, b = ctypes.c_int32(), ctypes.c_int32()
    lib.oracle_row_span(float(np.float32(u)), float(np.float32(v)), _ptr(E), int(x0), int(x1), int(ty),
                        ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def bin_pairs(proj: dict, want_unsorted: bool = True) -> dict:
    """Duplicated (tile, depth) keys, their sorted order and per-tile ranges."""
    lib = _load()
    tx, ty = proj["tiles"]
    n = proj["depth"].shape[0]
    m = int(lib.oracle_total_pairs(n, _ptr(proj["tile_count"])))
    ku = np.zeros(m, np.uint64) if want_unsorted else None
    vu = np.zeros(m, np.uint32) if want_unsorted else None
    ks, vs = np.zeros(m, np.uint64), np.zeros(m, np.uint32)
    ranges = np.zeros((tx * ty, 2), np.uint32)
    lib.oracle_bin_ex(n, _ptr(proj["depth"]), _ptr(proj["rect"]), _ptr(proj["tile_count"]), tx, ty,
                      _ptr(proj["mean2d"]), _ptr(proj["ellipse"]), int(proj.get("tile_test", TILE_SQUARE)),
                      _ptr(ku), _ptr(vu), _ptr(ks), _ptr(vs), _ptr(ranges))
    return dict(num_dups=m, keys_unsorted=ku, values_unsorted=vu, keys=ks, values=vs, ranges=ranges)


def composite(proj: dict, camera: dict, bg=(0.0, 0.0, 0.0), pixels=None, support_all=False,
              t_eps: float = 1e-4):
    """Image (binary64). Returns (rgb[n_pix,3] or [H,W,3], T, blended-pair counts)."""
    lib = _load()
    n = proj["depth"].shape[0]
    W, H = camera["width"], camera["height"]
    if pixels is None:
        npx = W * H
        pix = None
    else:
        pix = np.ascontiguousarray(pixels, dtype=np.int64)
        npx = pix.shape[0]
    out = np.zeros((npx, 3), np.float64)
    T = np.zeros(npx, np.float64)
    cnt = np.zeros(npx, np.int64)
    bgv = np.asarray(bg, np.float64)
    rgb = np.ascontiguousarray(proj["rgb"], np.float64)
    lib.oracle_composite_ex(n, _ptr(proj["mean2d"]), _ptr(proj["conic"]), _ptr(_f32(proj["opacity"])),
                            _ptr(rgb), _ptr(proj["depth"]), _ptr(proj["rect"]), _ptr(proj["tile_count"]),
                            _ptr(proj["ellipse"]), int(proj.get("tile_test", TILE_SQUARE)),
                            W, H, _ptr(bgv), 1 if support_all else 0, float(t_eps), _ptr(pix), npx,
                            _ptr(out), _ptr(T), _ptr(cnt))
    if pixels is None:
        return out.reshape(H, W, 3), T.reshape(H, W), cnt.reshape(H, W)
    return out, T, cnt


def render(arrays: dict, sh_degree: int, camera: dict, bg=(0.0, 0.0, 0.0), pixels=None):
    proj = preprocess(arrays, sh_degree, camera)
    return composite(proj, camera, bg=bg, pixels=pixels)


def cov3d(quat4, log_scale3) -> np.ndarray:
    lib = _load()
    q, s = _f32(quat4).reshape(4), _f32(log_scale3).reshape(3)
    out = np.zeros(6, np.float32)
    lib.oracle_cov3d(_ptr(q), _ptr(s), _ptr(out))
    return out


def scale_activation(log_scale) -> np.ndarray:
    """(float)exp((double)log_scale) elementwise, the host's libm exp (binary32 array in, out)."""
    lib = _load()
    ls = np.ascontiguousarray(log_scale, dtype=np.float32).ravel()
    out = np.empty_like(ls)
    lib.oracle_scale_activation(ls.size, _ptr(ls), _ptr(out))
    return out


def sh_basis(direction) -> np.ndarray:
    lib = _load()
    out = np.zeros(16, np.float64)
    x, y, z = (float(v) for v in direction)
    lib.oracle_sh_basis(x, y, z, _ptr(out))
    return out


def _splat2d_terms(means, covs, colours, opacities, depths, H, W):
    """Per-splat quantities of the dense 2D rasteriser over an H x W grid, splats ranked by
    (depth, index): rank, mean, colour, opacity, offsets dx [n,1,W] and dy [n,H,1] of the
    pixel positions (x = column, y = row) from the mean, the closed-form inverse P [n,2,2] of
    the 2x2 covariance, the density exp(-q/2) and the unclamped o * density [n, H*W]."""
    means = np.asarray(means, np.float64).reshape(-1, 2)
    covs = np.asarray(covs, np.float64).reshape(-1, 2, 2)
    colours = np.asarray(colours, np.float64).reshape(-1, 3)
    opacities = np.asarray(opacities, np.float64).reshape(-1)
    n = len(opacities)
    rank = np.lexsort((np.arange(n), np.asarray(depths, np.float64).reshape(-1)))
    m, S = means[rank], covs[rank]
    det = S[:, 0, 0] * S[:, 1, 1] - S[:, 0, 1] * S[:, 1, 0]
    P = np.empty_like(S)
    P[:, 0, 0], P[:, 0, 1] = S[:, 1, 1] / det, -S[:, 0, 1] / det
    P[:, 1, 0], P[:, 1, 1] = -S[:, 1, 0] / det, S[:, 0, 0] / det
    dx = np.arange(W, dtype=np.float64)[None, None, :] - m[:, 0, None, None]
    dy = np.arange(H, dtype=np.float64)[None, :, None] - m[:, 1, None, None]
    p = lambda i, j: P[:, i, j, None, None]
    q = p(0, 0) * dx * dx + (p(0, 1) + p(1, 0)) * dx * dy + p(1, 1) * dy * dy
    dens = np.exp(-0.5 * q).reshape(n, H * W)
    raw = opacities[rank][:, None] * dens
    return dict(rank=rank, col=colours[rank], dx=dx, dy=dy, P=P, dens=dens, raw=raw)


def composite_2d(means, covs, colours, opacities, depths, image_size, bg=None):
    """Dense 2D splat rasteriser in binary64.

    The lesson "3D Gaussian Splatting from scratch", sections "Étape 1: Un
    gaussien 2D" (density of one splat at a pixel) and "Étape 2: Rasteriser à
    éclaboussure en 2D" (every splat at every pixel, opacity times density
    clamped to [0, 0.99], ascending depth, front-to-back blend, no early stop;
    pixel (i, j) sits at x = j, y = i).  Written here as the closed form of the
    blend: with the splats of pixel p ranked k = 0, 1, ... by (depth, index),
        C(p) = sum_k c_k a_k(p) prod_{j<k} (1 - a_j(p)),   T(p) = prod_k (1 - a_k(p)),
    a_k(p) = min(0.99, max(0, o_k exp(-q_k(p) / 2))), q_k(p) = d^T cov_k^-1 d with
    d = p - mean_k and the 2x2 inverse in closed form.  Returns (H, W, 3) and T (H, W).
    """
    H, W = image_size
    s = _splat2d_terms(means, covs, colours, opacities, depths, H, W)
    a = np.clip(s["raw"], 0.0, 0.99)
    after = np.cumprod(1.0 - a, axis=0)              # transmittance behind each ranked splat
    before = np.vstack([np.ones((1, H * W)), after[:-1]]) if len(a) else after
    rgb = (a * before).T @ s["col"]                  # [H*W, 3]
    T = after[-1] if len(a) else np.ones(H * W)
    if bg is not None:
        rgb = rgb + T[:, None] * np.asarray(bg, np.float64)[None, :]
    return rgb.reshape(H, W, 3), T.reshape(H, W)


def composite_2d_backward(means, covs, colours, opacities, depths, image_size, g_image, bg=None) -> dict:
    """Vector-Jacobian product of composite_2d in binary64, written out by hand.

    For each pixel the forward walk gives T_i before entry i; walking back with the
    colour behind B_i (B_{i-1} = a_i c_i + (1 - a_i) B_i):
        dL/dc_i = a_i T_i dL/dC,   dL/da_i = T_i (c_i - B_i) . dL/dC - T_final (bg . dL/dC) / (1 - a_i)
    a = clamp(o G, 0, 0.99) passes the derivative where 0 <= o G <= 0.99 (the clamp's
    own convention at its ends); G = exp(-q/2), q = d^T P d with d = pixel - mean and
    P = cov^-1, so dL/dq = -o G dL/da / 2, dL/dmean = -(P + P^T) d dL/dq summed over
    pixels, and with M = sum_pixels dL/dq d d^T the covariance gets dL/dcov = -P^T M P^T.
    Returns means (G,2), covs (G,2,2), colours (G,3), opacities (G,).
    """
    H, W = image_size
    s = _splat2d_terms(means, covs, colours, opacities, depths, H, W)
    rank, col, P, dens, raw = s["rank"], s["col"], s["P"], s["dens"], s["raw"]
    n = len(rank)
    gC = np.asarray(g_image, np.float64).reshape(H * W, 3)
    dx = np.broadcast_to(s["dx"], (n, H, W)).reshape(n, H * W)
    dy = np.broadcast_to(s["dy"], (n, H, W)).reshape(n, H * W)
    a = np.clip(raw, 0.0, 0.99)
    smooth = (raw >= 0.0) & (raw <= 0.99)
    T = np.ones(H * W)
    Ts = np.empty((n, H * W))
    for k in range(n):
        Ts[k] = T
        T = T * (1.0 - a[k])
    bg_term = np.zeros(H * W) if bg is None else T * (gC @ np.asarray(bg, np.float64))
    ranked = dict(means=np.zeros((n, 2)), covs=np.zeros((n, 2, 2)), colours=np.zeros((n, 3)), opacities=np.zeros(n))
    B = np.zeros((H * W, 3))
    for k in range(n - 1, -1, -1):
        ranked["colours"][k] = (a[k] * Ts[k]) @ gC
        d_a = Ts[k] * ((col[k][None, :] - B) * gC).sum(axis=1) - bg_term / (1.0 - a[k])
        B = a[k][:, None] * col[k][None, :] + (1.0 - a[k])[:, None] * B
        d_a = np.where(smooth[k], d_a, 0.0)
        ranked["opacities"][k] = dens[k] @ d_a
        d_q = -0.5 * raw[k] * d_a
        Ps = P[k] + P[k].T
        ranked["means"][k, 0] = -(d_q * (Ps[0, 0] * dx[k] + Ps[0, 1] * dy[k])).sum()
        ranked["means"][k, 1] = -(d_q * (Ps[1, 0] * dx[k] + Ps[1, 1] * dy[k])).sum()
        M = np.array([[d_q @ (dx[k] * dx[k]), d_q @ (dx[k] * dy[k])],
                      [d_q @ (dy[k] * dx[k]), d_q @ (dy[k] * dy[k])]])
        ranked["covs"][k] = -P[k].T @ M @ P[k].T
    out = {}
    for key, v in ranked.items():
        out[key] = np.zeros_like(v)
        out[key][rank] = v
    return out


# ---------------------------------------------------------------------------
# gradients (gs_oracle_grad.c)
# ---------------------------------------------------------------------------
def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def camera64(camera: dict) -> np.ndarray:
    """R[9], t[3], fx, fy, cx, cy as binary64 copies of the binary32 camera values."""
    vals = list(np.asarray(camera["R"], np.float32).reshape(9)) + list(np.asarray(camera["t"], np.float32).reshape(3))
    vals += [np.float32(camera[k]) for k in ("fx", "fy", "cx", "cy")]
    return np.array([float(v) for v in vals], np.float64)


def project64(arrays: dict, sh_degree: int, camera: dict) -> dict:
    """binary64 projection with no culling: mean2d, conic, rgb, cov2d, depth."""
    lib = _load()
    mean, quat, ls, sh = (_f64(arrays[k]) for k in ("mean", "quat", "log_scale", "sh"))
    n = mean.shape[1]
    K = (sh_degree + 1) ** 2
    out = dict(mean2d=np.zeros((2, n)), conic=np.zeros((3, n)), rgb=np.zeros((3, n)), cov2d=np.zeros((3, n)),
               depth=np.zeros(n))
    lib.oracle_project64(n, K, _ptr(mean), _ptr(quat), _ptr(ls), _ptr(sh), _ptr(camera64(camera)),
                         _ptr(out["mean2d"]), _ptr(out["conic"]), _ptr(out["rgb"]), _ptr(out["cov2d"]),
                         _ptr(out["depth"]))
    return out


def project_backward(arrays: dict, sh_degree: int, camera: dict, g_mean2d=None, g_conic=None, g_rgb=None) -> dict:
    """Vector-Jacobian product of project64: gradients for mean, quat, log_scale, sh."""
    lib = _load()
    mean, quat, ls, sh = (_f64(arrays[k]) for k in ("mean", "quat", "log_scale", "sh"))
    n = mean.shape[1]
    K = (sh_degree + 1) ** 2
    out = dict(mean=np.zeros((3, n)), quat=np.zeros((4, n)), log_scale=np.zeros((3, n)), sh=np.zeros((K * 3, n)))
    gm = None if g_mean2d is None else _f64(g_mean2d)
    gc = None if g_conic is None else _f64(g_conic)
    gr = None if g_rgb is None else _f64(g_rgb)
    lib.oracle_project_backward(n, K, _ptr(mean), _ptr(quat), _ptr(ls), _ptr(sh), _ptr(camera64(camera)),
                                _ptr(gm), _ptr(gc), _ptr(gr), _ptr(out["mean"]), _ptr(out["quat"]),
                                _ptr(out["log_scale"]), _ptr(out["sh"]))
    return out


def depth_order(depth, tile_count) -> np.ndarray:
    """Gaussians with tile_count > 0 in ascending (binary32 depth, index)."""
    g = np.nonzero(np.asarray(tile_count) > 0)[0]
    d = np.asarray(depth, np.float32)[g]
    return np.ascontiguousarray(g[np.lexsort((g, d))], dtype=np.int64)


def _list_rule(proj32):
    """(mean2d32, ellipse, tile_test) of a binary32 projection, or the plain rectangle rule."""
    if proj32 is None or proj32.get("tile_test", TILE_SQUARE) == TILE_SQUARE:
        return None, None, TILE_SQUARE
    return _f32(proj32["mean2d"]), _f32(proj32["ellipse"]), int(proj32["tile_test"])


def composite_fixed(screen: dict, rect, order, camera: dict, bg=(0.0, 0.0, 0.0), n_limit=None, t_eps=1e-4,
                    proj32=None):
    """binary64 compositing over fixed lists; returns (rgb [H,W,3], T [H,W], count [H,W]).
    proj32 (a `preprocess` result) supplies the tile membership rule when it is not the rectangle."""
    lib = _load()
    m32, ell, tt = _list_rule(proj32)
    W, H = camera["width"], camera["height"]
    n = np.asarray(screen["opacity"]).shape[0]
    m2, co, op, rgb = (_f64(screen[k]) for k in ("mean2d", "conic", "opacity", "rgb"))
    rect = np.ascontiguousarray(rect, np.int32)
    order = np.ascontiguousarray(order, np.int64)
    lim = None if n_limit is None else np.ascontiguousarray(n_limit, np.int64).reshape(-1)
    out, T, cnt = np.zeros(H * W * 3), np.zeros(H * W), np.zeros(H * W, np.int64)
    lib.oracle_composite_fixed(n, _ptr(m2), _ptr(co), _ptr(op), _ptr(rgb), _ptr(rect), _ptr(m32), _ptr(ell), tt,
                               _ptr(order), order.shape[0], W, H, _ptr(_f64(bg)), _ptr(lim), float(t_eps),
                               _ptr(out), _ptr(T), _ptr(cnt))
    return out.reshape(H, W, 3), T.reshape(H, W), cnt.reshape(H, W)


def composite_backward(screen: dict, rect, order, camera: dict, g_image, bg=(0.0, 0.0, 0.0), n_limit=None,
                       t_eps=1e-4, pixels=None, proj32=None) -> dict:
    """Vector-Jacobian product of composite_fixed: gradients for mean2d, conic, opacity, rgb.

    pixels: optional flat indices y*W+x; only their cotangents are taken (the rest count as 0).
    """
    lib = _load()
    m32, ell, tt = _list_rule(proj32)
    W, H = camera["width"], camera["height"]
    n = np.asarray(screen["opacity"]).shape[0]
    m2, co, op, rgb = (_f64(screen[k]) for k in ("mean2d", "conic", "opacity", "rgb"))
    rect = np.ascontiguousarray(rect, np.int32)
    order = np.ascontiguousarray(order, np.int64)
    lim = None if n_limit is None else np.ascontiguousarray(n_limit, np.int64).reshape(-1)
    gi = _f64(g_image).reshape(-1)
    assert gi.shape[0] == H * W * 3
    out = dict(mean2d=np.zeros((2, n)), conic=np.zeros((3, n)), opacity=np.zeros(n), rgb=np.zeros((3, n)))
    pix = None if pixels is None else np.ascontiguousarray(pixels, np.int64)
    lib.oracle_composite_backward(n, _ptr(m2), _ptr(co), _ptr(op), _ptr(rgb), _ptr(rect), _ptr(m32), _ptr(ell),
                                  tt, _ptr(order), order.shape[0], W, H, _ptr(_f64(bg)), _ptr(lim), float(t_eps),
                                  _ptr(gi),
                                  _ptr(pix), 0 if pix is None else pix.shape[0],
                                  _ptr(out["mean2d"]), _ptr(out["conic"]), _ptr(out["opacity"]), _ptr(out["rgb"]))
    return out


def render_backward(arrays: dict, sh_degree: int, camera: dict, g_image, bg=(0.0, 0.0, 0.0), pixels=None,
                    tile_test: int = TILE_SQUARE) -> dict:
    """Gradient of sum(g_image * render(arrays)) for every Gaussian parameter.

    The lists (tile rectangles, visibility, depth order) come from the binary32
    projection of `preprocess`; compositing and all derivatives are binary64,
    with the per-pixel stop at T < 1e-4 found by the binary64 forward walk.
    Returns parameter gradients (mean, quat, log_scale, opacity, sh), the
    screen-space ones (screen_mean2d, screen_conic, screen_rgb) and the
    per-pixel blended counts (None when `pixels` restricts the cotangent to
    the listed flat pixel indices, y*W+x).
    """
    proj = preprocess(arrays, sh_degree, camera, tile_test=tile_test)
    order = depth_order(proj["depth"], proj["tile_count"])
    scr = project64(arrays, sh_degree, camera)
    scr["opacity"] = _f64(arrays["opacity"])
    cnt = None
    if pixels is None:
        _, _, cnt = composite_fixed(scr, proj["rect"], order, camera, bg=bg, proj32=proj)
    gs = composite_backward(scr, proj["rect"], order, camera, g_image, bg=bg, pixels=pixels, proj32=proj)
    gp = project_backward(arrays, sh_degree, camera, gs["mean2d"], gs["conic"], gs["rgb"])
    gp["opacity"] = gs["opacity"]
    gp.update(screen_mean2d=gs["mean2d"], screen_conic=gs["conic"], screen_rgb=gs["rgb"], screen_opacity=gs["opacity"],
              n_blend=cnt)
    return gp
