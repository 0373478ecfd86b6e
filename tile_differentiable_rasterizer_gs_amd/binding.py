"""ctypes binding of libgsrast.so (include/gsrast.h).

Argument marshalling only: every stage runs in the HIP library.  torch supplies
device memory and the current stream.  There is no CPU fallback: if the library
is missing or no GPU is present the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsrast.so")

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_OUT_OF_MEMORY, GS_ERR_CAPACITY, GS_ERR_DEVICE = range(5)
GS_SORT_DEPTH_FIRST, GS_SORT_KEY64 = 0, 1
(GS_OPT_SORT_MODE, GS_OPT_EMIT_KEYS, GS_OPT_MAX_DUPS, GS_OPT_MAX_WORKSPACE_BYTES, GS_OPT_PROFILE, GS_OPT_TILE_TEST,
 GS_OPT_BINNING, GS_OPT_DEPTH_ORDER) = range(8)
GS_TILE_SQUARE, GS_TILE_ELLIPSE = 0, 1
GS_BINNING_AUTO, GS_BINNING_SUPER_TILE, GS_BINNING_RADIX = 0, 1, 2
GS_DEPTH_ORDER_BUCKETS, GS_DEPTH_ORDER_RADIX = 0, 1
STAGES = ("preprocess", "depth_sort", "scan", "duplicate", "tile_sort", "ranges", "composite", "readback",
          "backward_composite", "backward_setup", "backward_gaussian")
SPLAT_STRIDE = 16
TILE = 16

# symbols declared in include/gsrast.h
EXPORTED = ("gs_context_create", "gs_context_destroy", "gs_context_set_option", "gs_check_arguments",
            "gs_preprocess", "gs_cache_covariance", "gs_bin_and_sort", "gs_composite", "gs_composite_ex", "gs_render",
            "gs_render_noalloc",
            "gs_backward", "gs_splat2d_forward", "gs_splat2d_backward", "gs_scale_activation", "gs_profile_read",
            "gs_status_string", "gs_last_error")


class GsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gsrast status {status}: {message}")
        self.status = status


class Gaussians(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("sh_degree", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("mean", ctypes.c_void_p), ("quat", ctypes.c_void_p), ("log_scale", ctypes.c_void_p),
                ("opacity", ctypes.c_void_p), ("sh", ctypes.c_void_p)]


class Camera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("t", ctypes.c_float * 3), ("fx", ctypes.c_float),
                ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float),
                ("znear", ctypes.c_float), ("width", ctypes.c_int32), ("height", ctypes.c_int32)]


class Projected(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("tiles_x", ctypes.c_int32), ("tiles_y", ctypes.c_int32),
                ("splat", ctypes.c_void_p), ("depth", ctypes.c_void_p), ("rect", ctypes.c_void_p),
                ("tile_count", ctypes.c_void_p)]


class Binning(ctypes.Structure):
    _fields_ = [("num_dups", ctypes.c_int64), ("tiles_x", ctypes.c_int32), ("tiles_y", ctypes.c_int32),
                ("keys", ctypes.c_void_p), ("values", ctypes.c_void_p), ("tile_ranges", ctypes.c_void_p),
                ("keys_unsorted", ctypes.c_void_p), ("values_unsorted", ctypes.c_void_p),
                ("super_entries", ctypes.c_int64), ("depth_buckets", ctypes.c_int64)]


class Profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(STAGES)), ("launches", ctypes.c_int64 * len(STAGES))]


GRAD_FIELDS = ("mean", "quat", "log_scale", "opacity", "sh", "mean2d", "conic", "rgb")


class Gradients(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in GRAD_FIELDS]


_lib = None
_hip = None


def load_library(path: str = LIB_PATH):
    """Loads libgsrast.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.gs_context_create.argtypes = [ctypes.POINTER(P), ctypes.c_int]
    lib.gs_context_destroy.argtypes = [P]
    lib.gs_context_destroy.restype = None
    lib.gs_context_set_option.argtypes = [P, ctypes.c_int, i64]
    lib.gs_check_arguments.argtypes = [ctypes.POINTER(Gaussians), ctypes.POINTER(Camera), ctypes.c_char_p,
                                       ctypes.c_size_t]
    lib.gs_preprocess.argtypes = [P, ctypes.POINTER(Gaussians), ctypes.POINTER(Camera), ctypes.POINTER(Projected), P]
    lib.gs_cache_covariance.argtypes = [P, ctypes.POINTER(Gaussians), P]
    lib.gs_bin_and_sort.argtypes = [P, ctypes.POINTER(Projected), ctypes.POINTER(Camera), ctypes.POINTER(Binning), P]
    lib.gs_composite.argtypes = [P, ctypes.POINTER(Projected), ctypes.POINTER(Binning), ctypes.POINTER(Camera),
                                 ctypes.POINTER(ctypes.c_float), P, P]
    lib.gs_composite_ex.argtypes = [P, ctypes.POINTER(Projected), ctypes.POINTER(Binning), ctypes.POINTER(Camera),
                                    ctypes.POINTER(ctypes.c_float), P, P, P, P, P]
    lib.gs_render.argtypes = [P, ctypes.POINTER(Gaussians), ctypes.POINTER(Camera), ctypes.POINTER(ctypes.c_float),
                              P, P]
    lib.gs_render_noalloc.argtypes = [P, ctypes.POINTER(Gaussians), ctypes.POINTER(Camera), ctypes.POINTER(ctypes.c_float),
                              P, P]
    lib.gs_backward.argtypes = [P, ctypes.POINTER(Gaussians), ctypes.POINTER(Camera), ctypes.POINTER(Projected),
                                ctypes.POINTER(Binning), ctypes.POINTER(ctypes.c_float), P, P, P,
                                ctypes.POINTER(Gradients), P]
    FP = ctypes.POINTER(ctypes.c_float)
    lib.gs_splat2d_forward.argtypes = [P, i64, P, P, P, P, P, i32, i32, FP, P, P]
    lib.gs_splat2d_backward.argtypes = [P, i64, P, P, P, P, P, i32, i32, FP, P, P, P, P, P, P]
    lib.gs_scale_activation.argtypes = [P, P, P, i64, P]
    lib.gs_profile_read.argtypes = [P, ctypes.POINTER(Profile)]
    lib.gs_status_string.argtypes = [ctypes.c_int]
    lib.gs_status_string.restype = ctypes.c_char_p
    lib.gs_last_error.argtypes = [P]
    lib.gs_last_error.restype = ctypes.c_char_p
    for name in ("gs_context_create", "gs_context_set_option", "gs_check_arguments", "gs_preprocess",
                 "gs_cache_covariance", "gs_bin_and_sort", "gs_composite", "gs_composite_ex", "gs_render",
                 "gs_backward",
                 "gs_splat2d_forward", "gs_splat2d_backward", "gs_profile_read"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _hip_runtime():
    """The HIP runtime torch already loaded (same SONAME), for device copies."""
    global _hip
    if _hip is None:
        torch.cuda.init()
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    return _hip


def _stream_handle(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def copy_device(ptr: int, shape, dtype: torch.dtype, device=None, stream=None) -> torch.Tensor:
    """Copies a library-owned device array into a new torch tensor (device-to-device)."""
    out = torch.empty(shape, dtype=dtype, device=device or torch.device("cuda", torch.cuda.current_device()))
    nbytes = out.numel() * out.element_size()
    if nbytes == 0:
        return out
    if not ptr:
        raise ValueError("NULL device pointer")
    err = _hip_runtime().hipMemcpyAsync(ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ptr), nbytes, 3,
                                        _stream_handle(stream))
    if err != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with {err}")
    return out


def make_camera(camera: dict) -> Camera:
    c = Camera()
    c.R[:] = [float(v) for v in np.asarray(camera["R"], np.float32).reshape(9)]
    c.t[:] = [float(v) for v in np.asarray(camera["t"], np.float32).reshape(3)]
    for k in ("fx", "fy", "cx", "cy", "znear"):
        setattr(c, k, float(np.float32(camera[k])))
    c.width, c.height = int(camera["width"]), int(camera["height"])
    return c


def gaussians_to_device(arrays: dict, device="cuda") -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device) for k, v in arrays.items()}


def make_gaussians(tensors: dict, sh_degree: int) -> Gaussians:
    K = (sh_degree + 1) ** 2
    n = int(tensors["opacity"].shape[0])
    want = dict(mean=(3, n), quat=(4, n), log_scale=(3, n), opacity=(n,), sh=(K * 3, n))
    g = Gaussians()
    g.n, g.sh_degree = n, sh_degree
    for k, shape in want.items():
        t = tensors[k]
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{k} must be a CUDA (HIP) tensor")
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{k} must be contiguous float32 of shape {shape}, got {t.dtype} {tuple(t.shape)}")
        setattr(g, k, t.data_ptr() if n else None)
    return g


class Rasterizer:
    """One library context on the current HIP device."""

    def __init__(self, device: int | None = None, sort_mode: int = GS_SORT_DEPTH_FIRST, emit_keys: bool = True,
                 tile_test: int = GS_TILE_SQUARE, binning: int = GS_BINNING_AUTO,
                 depth_order: int = GS_DEPTH_ORDER_BUCKETS):
        self.lib = load_library()
        self.device = torch.cuda.current_device() if device is None else device
        ctx = ctypes.c_void_p()
        st = self.lib.gs_context_create(ctypes.byref(ctx), self.device)
        if st != GS_OK:
            raise GsError(st, "gs_context_create failed")
        self.ctx = ctx
        self.set_option(GS_OPT_SORT_MODE, sort_mode)
        self.set_option(GS_OPT_EMIT_KEYS, 1 if emit_keys else 0)
        self.set_option(GS_OPT_TILE_TEST, tile_test)
        self.set_option(GS_OPT_BINNING, binning)
        self.set_option(GS_OPT_DEPTH_ORDER, depth_order)
        self._keep = []

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.gs_context_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int):
        if st != GS_OK:
            msg = self.lib.gs_last_error(self.ctx).decode(errors="replace")
            raise GsError(st, msg or self.lib.gs_status_string(st).decode())

    def set_option(self, option: int, value: int):
        self._check(self.lib.gs_context_set_option(self.ctx, option, int(value)))

    def preprocess(self, tensors: dict, sh_degree: int, camera: dict, stream=None) -> Projected:
        g = make_gaussians(tensors, sh_degree)
        cam = make_camera(camera)
        out = Projected()
        self._check(self.lib.gs_preprocess(self.ctx, ctypes.byref(g), ctypes.byref(cam), ctypes.byref(out),
                                           _stream_handle(stream)))
        return out

    def cache_covariance(self, tensors: dict | None, sh_degree: int = 0, stream=None):
        """gs_cache_covariance: Sigma of these Gaussians computed once and reused by later
        preprocess / render calls with the same quat and log_scale tensors (None drops it)."""
        if tensors is None:
            self._check(self.lib.gs_cache_covariance(self.ctx, None, _stream_handle(stream)))
            return
        g = make_gaussians(tensors, sh_degree)
        self._check(self.lib.gs_cache_covariance(self.ctx, ctypes.byref(g), _stream_handle(stream)))

    def bin_and_sort(self, projected: Projected, camera: dict, stream=None) -> Binning:
        cam = make_camera(camera)
        out = Binning()
        self._check(self.lib.gs_bin_and_sort(self.ctx, ctypes.byref(projected), ctypes.byref(cam),
                                             ctypes.byref(out), _stream_handle(stream)))
        return out

    def composite(self, projected: Projected, binning: Binning, camera: dict, bg=(0.0, 0.0, 0.0), out=None,
                  final_T=None, n_blend=None, blend_total=None, stream=None) -> torch.Tensor:
        cam = make_camera(camera)
        H, W = cam.height, cam.width
        if out is None:
            out = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
        self._check_image(out, (H, W, 3), torch.float32)
        bgv = (ctypes.c_float * 3)(*[float(v) for v in bg])
        ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        if final_T is not None:
            self._check_image(final_T, (H, W), torch.float32)
        if n_blend is not None:
            self._check_image(n_blend, (H, W), torch.int32)
        if blend_total is not None:
            self._check_image(blend_total, (1,), torch.int64)
        self._check(self.lib.gs_composite_ex(self.ctx, ctypes.byref(projected), ctypes.byref(binning),
                                             ctypes.byref(cam), bgv, ptr(out), ptr(final_T), ptr(n_blend),
                                             ptr(blend_total), _stream_handle(stream)))
        return out

    def render(self, tensors: dict, sh_degree: int, camera: dict, bg=(0.0, 0.0, 0.0), out=None,
               stream=None) -> torch.Tensor:
        g = make_gaussians(tensors, sh_degree)
        cam = make_camera(camera)
        if out is None:
            out = torch.empty((cam.height, cam.width, 3), dtype=torch.float32, device="cuda")
        self._check_image(out, (cam.height, cam.width, 3), torch.float32)
        bgv = (ctypes.c_float * 3)(*[float(v) for v in bg])
        self._check(self.lib.gs_render(self.ctx, ctypes.byref(g), ctypes.byref(cam), bgv,
                                       ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)))
        return out

    def render_noalloc(self, tensors: dict, sh_degree: int, camera: dict, bg=(0.0, 0.0, 0.0), out=None,
                       stream=None) -> torch.Tensor:
        """gs_render_noalloc: as render, with every intermediate buffer in the library's static scratch."""
        g = make_gaussians(tensors, sh_degree)
        cam = make_camera(camera)
        if out is None:
            out = torch.empty((cam.height, cam.width, 3), dtype=torch.float32, device="cuda")
        self._check_image(out, (cam.height, cam.width, 3), torch.float32)
        bgv = (ctypes.c_float * 3)(*[float(v) for v in bg])
        self._check(self.lib.gs_render_noalloc(self.ctx, ctypes.byref(g), ctypes.byref(cam), bgv,
                                               ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)))
        return out

    def backward(self, tensors: dict, sh_degree: int, camera: dict, projected: Projected, binning: Binning,
                 final_T: torch.Tensor, n_blend: torch.Tensor, grad_image: torch.Tensor, bg=(0.0, 0.0, 0.0),
                 screen: bool = False, out: dict | None = None, stream=None) -> dict:
        """Gradients of sum(grad_image * image) for the last forward on this context.

        final_T / n_blend: the per-pixel outputs of that forward's composite.  Returns
        parameter gradients (mean, quat, log_scale, opacity, sh) and, with screen=True,
        the screen-space ones (mean2d, conic, rgb).
        """
        g = make_gaussians(tensors, sh_degree)
        cam = make_camera(camera)
        H, W = cam.height, cam.width
        self._check_image(final_T, (H, W), torch.float32)
        self._check_image(n_blend, (H, W), torch.int32)
        self._check_image(grad_image, (H, W, 3), torch.float32)
        n = g.n
        K = (sh_degree + 1) ** 2
        shapes = dict(mean=(3, n), quat=(4, n), log_scale=(3, n), opacity=(n,), sh=(K * 3, n))
        if screen:
            shapes.update(mean2d=(2, n), conic=(3, n), rgb=(3, n))
        grads = dict(out or {})
        for k, shp in shapes.items():
            if k not in grads:
                grads[k] = torch.empty(shp, dtype=torch.float32, device="cuda")
            self._check_image(grads[k], shp, torch.float32)
        gr = Gradients(**{k: (grads[k].data_ptr() if k in grads and n else None) for k in GRAD_FIELDS})
        bgv = (ctypes.c_float * 3)(*[float(v) for v in bg])
        self._check(self.lib.gs_backward(self.ctx, ctypes.byref(g), ctypes.byref(cam), ctypes.byref(projected),
                                         ctypes.byref(binning), bgv, ctypes.c_void_p(final_T.data_ptr()),
                                         ctypes.c_void_p(n_blend.data_ptr()), ctypes.c_void_p(grad_image.data_ptr()),
                                         ctypes.byref(gr), _stream_handle(stream)))
        return grads

    # ---- the lesson's dense 2D splat rasteriser ----
    @staticmethod
    def _splat2d_tensors(means, covs, colours, opacities, depths):
        n = int(opacities.shape[0])
        want = dict(means=(n, 2), covs=(n, 2, 2), colours=(n, 3), opacities=(n,), depths=(n,))
        ts = dict(means=means, covs=covs, colours=colours, opacities=opacities, depths=depths)
        for k, shape in want.items():
            t = ts[k]
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or \
                    not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{k} must be a contiguous CUDA float32 tensor of shape {shape}")
        return n, [ctypes.c_void_p(ts[k].data_ptr()) if n else None for k in want]

    def scale_activation(self, log_scale, out=None, stream=None) -> torch.Tensor:
        """gs_scale_activation: (float)exp((double)x) elementwise on a contiguous fp32 device tensor."""
        if log_scale.dtype != torch.float32 or not log_scale.is_cuda or not log_scale.is_contiguous():
            raise ValueError("log_scale must be a contiguous float32 device tensor")
        if out is None:
            out = torch.empty_like(log_scale)
        if out.shape != log_scale.shape or out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor shaped like log_scale")
        self._check(self.lib.gs_scale_activation(self.ctx, ctypes.c_void_p(log_scale.data_ptr()),
                                                 ctypes.c_void_p(out.data_ptr()), log_scale.numel(),
                                                 _stream_handle(stream)))
        return out

    def splat2d_forward(self, means, covs, colours, opacities, depths, height: int, width: int, bg=None,
                        out=None, stream=None) -> torch.Tensor:
        n, ptrs = self._splat2d_tensors(means, covs, colours, opacities, depths)
        if out is None:
            out = torch.empty((height, width, 3), dtype=torch.float32, device="cuda")
        self._check_image(out, (height, width, 3), torch.float32)
        bgv = None if bg is None else (ctypes.c_float * 3)(*[float(v) for v in bg])
        self._check(self.lib.gs_splat2d_forward(self.ctx, n, *ptrs, int(height), int(width), bgv,
                                                ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)))
        return out

    def splat2d_backward(self, means, covs, colours, opacities, depths, height: int, width: int, grad_image,
                         bg=None, stream=None) -> dict:
        n, ptrs = self._splat2d_tensors(means, covs, colours, opacities, depths)
        self._check_image(grad_image, (height, width, 3), torch.float32)
        g = dict(means=torch.empty((n, 2), dtype=torch.float32, device="cuda"),
                 covs=torch.empty((n, 2, 2), dtype=torch.float32, device="cuda"),
                 colours=torch.empty((n, 3), dtype=torch.float32, device="cuda"),
                 opacities=torch.empty((n,), dtype=torch.float32, device="cuda"))
        bgv = None if bg is None else (ctypes.c_float * 3)(*[float(v) for v in bg])
        gp = [ctypes.c_void_p(g[k].data_ptr()) if n else None for k in ("means", "covs", "colours", "opacities")]
        self._check(self.lib.gs_splat2d_backward(self.ctx, n, *ptrs, int(height), int(width), bgv,
                                                 ctypes.c_void_p(grad_image.data_ptr()), *gp,
                                                 _stream_handle(stream)))
        return g

    def profile_read(self) -> dict:
        p = Profile()
        self._check(self.lib.gs_profile_read(self.ctx, ctypes.byref(p)))
        return {name: (p.ms[i], p.launches[i]) for i, name in enumerate(STAGES)}

    @staticmethod
    def _check_image(t, shape, dtype):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous() \
                or tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected a contiguous CUDA {dtype} tensor of shape {shape}")

    # ---- readers of library-owned views (device copies as torch tensors) ----
    @staticmethod
    def projected_tensors(pr: Projected, stream=None) -> dict:
        n = pr.n
        return dict(splat=copy_device(pr.splat, (n, SPLAT_STRIDE), torch.float32, stream=stream),
                    depth=copy_device(pr.depth, (n,), torch.float32, stream=stream),
                    rect=copy_device(pr.rect, (n, 4), torch.int16, stream=stream),
                    tile_count=copy_device(pr.tile_count, (n,), torch.int32, stream=stream))

    @staticmethod
    def binning_tensors(b: Binning, stream=None) -> dict:
        m, tiles = b.num_dups, b.tiles_x * b.tiles_y
        out = dict(num_dups=m,
                   ranges=copy_device(b.tile_ranges, (tiles, 2), torch.int32, stream=stream),
                   values=copy_device(b.values, (m,), torch.int32, stream=stream) if m else
                   torch.zeros(0, dtype=torch.int32, device="cuda"))
        for k in ("keys", "keys_unsorted"):
            p = getattr(b, k)
            out[k] = copy_device(p, (m,), torch.int64, stream=stream) if (p and m) else None
        p = b.values_unsorted
        out["values_unsorted"] = copy_device(p, (m,), torch.int32, stream=stream) if (p and m) else None
        return out


class RenderFunction(torch.autograd.Function):
    """Differentiable render through the HIP library (forward gs_preprocess + gs_bin_and_sort +
    gs_composite_ex, backward gs_backward).  The rasterizer's context holds the forward state
    until backward: do not render on the same Rasterizer in between."""

    @staticmethod
    def forward(ctx, mean, quat, log_scale, opacity, sh, rasterizer, sh_degree, camera, bg):
        tensors = dict(mean=mean.detach(), quat=quat.detach(), log_scale=log_scale.detach(),
                       opacity=opacity.detach(), sh=sh.detach())
        pr = rasterizer.preprocess(tensors, sh_degree, camera)
        bn = rasterizer.bin_and_sort(pr, camera)
        H, W = int(camera["height"]), int(camera["width"])
        final_T = torch.empty((H, W), dtype=torch.float32, device="cuda")
        n_blend = torch.empty((H, W), dtype=torch.int32, device="cuda")
        img = rasterizer.composite(pr, bn, camera, bg=bg, final_T=final_T, n_blend=n_blend)
        ctx.state = (rasterizer, tensors, sh_degree, camera, pr, bn, final_T, n_blend, bg)
        return img

    @staticmethod
    def backward(ctx, grad_image):
        rasterizer, tensors, sh_degree, camera, pr, bn, final_T, n_blend, bg = ctx.state
        g = rasterizer.backward(tensors, sh_degree, camera, pr, bn, final_T, n_blend,
                                grad_image.contiguous().float(), bg=bg)
        return g["mean"], g["quat"], g["log_scale"], g["opacity"], g["sh"], None, None, None, None


def render_differentiable(rasterizer: "Rasterizer", params: dict, sh_degree: int, camera: dict,
                          bg=(0.0, 0.0, 0.0)) -> torch.Tensor:
    """Image [H, W, 3] with autograd support for the five parameter tensors in `params`."""
    return RenderFunction.apply(params["mean"], params["quat"], params["log_scale"], params["opacity"],
                                params["sh"], rasterizer, sh_degree, camera, tuple(float(v) for v in bg))


class Splat2DFunction(torch.autograd.Function):
    """The lesson's dense 2D rasteriser through the HIP library, with autograd (depths only order
    the splats and get no gradient).  Forward state lives in the rasterizer's context until
    backward: do not run another 2D forward on the same Rasterizer in between."""

    @staticmethod
    def forward(ctx, means, covs, colours, opacities, depths, rasterizer, height, width, bg):
        args = [t.detach().contiguous().float() for t in (means, covs, colours, opacities, depths)]
        img = rasterizer.splat2d_forward(*args, height, width, bg=bg)
        ctx.state = (rasterizer, args, height, width, bg)
        return img

    @staticmethod
    def backward(ctx, grad_image):
        rasterizer, args, height, width, bg = ctx.state
        g = rasterizer.splat2d_backward(*args, height, width, grad_image.contiguous().float(), bg=bg)
        return g["means"], g["covs"], g["colours"], g["opacities"], None, None, None, None, None


def rasterise_2d(rasterizer: "Rasterizer", means, covs, colours, opacities, depths, image_size, bg=None):
    """Image [H, W, 3] of 2D splats (the lesson's rasteriser signature), differentiable."""
    H, W = image_size
    return Splat2DFunction.apply(means, covs, colours, opacities, depths, rasterizer, int(H), int(W), bg)
