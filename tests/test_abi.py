"""C-ABI checks that need no GPU: exports, struct layout, host-side argument checks."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsrast.h")


@pytest.fixture(scope="module")
def lib():
    from tile_differentiable_rasterizer_gs_amd import binding

    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gs_\w+)\s*\(", text, re.M)))


def test_header_declarations_are_exported(lib):
    from tile_differentiable_rasterizer_gs_amd import binding

    names = _declared_functions()
    assert len(names) == len(binding.EXPORTED) and set(names) == set(binding.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (gs_\w+)$", out, re.M))
    assert exported == set(names)


def test_struct_layout_matches_header(tmp_path):
    from tile_differentiable_rasterizer_gs_amd import binding as b

    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "gsrast.h"
#define P(T) printf(#T " %zu\\n", sizeof(T));
#define O(T, f) printf(#T "." #f " %zu\\n", offsetof(T, f));
int main(void) {
  P(gs_gaussians) O(gs_gaussians, sh_degree) O(gs_gaussians, mean) O(gs_gaussians, sh)
  P(gs_camera) O(gs_camera, t) O(gs_camera, fx) O(gs_camera, znear) O(gs_camera, width) O(gs_camera, height)
  P(gs_projected) O(gs_projected, tiles_x) O(gs_projected, splat) O(gs_projected, tile_count)
  P(gs_binning) O(gs_binning, keys) O(gs_binning, tile_ranges) O(gs_binning, values_unsorted)
  O(gs_binning, super_entries) O(gs_binning, depth_buckets)
  P(gs_profile) O(gs_profile, launches)
  P(gs_gradients) O(gs_gradients, sh) O(gs_gradients, mean2d) O(gs_gradients, rgb)
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include", "-o", str(exe), str(src)])
    got = dict(line.rsplit(" ", 1) for line in subprocess.check_output([str(exe)], text=True).splitlines())
    ct = {"gs_gaussians": b.Gaussians, "gs_camera": b.Camera, "gs_projected": b.Projected,
          "gs_binning": b.Binning, "gs_profile": b.Profile, "gs_gradients": b.Gradients}
    for key, val in got.items():
        if "." in key:
            t, f = key.split(".")
            assert getattr(ct[t], f).offset == int(val), key
        else:
            assert ctypes.sizeof(ct[key]) == int(val), key


def _good():
    from tile_differentiable_rasterizer_gs_amd import binding as b

    g = b.Gaussians()
    g.n, g.sh_degree = 10, 3
    for f in ("mean", "quat", "log_scale", "opacity", "sh"):
        setattr(g, f, 0x1000)
    cam = b.make_camera(dict(R=np.eye(3), t=np.zeros(3), fx=100.0, fy=100.0, cx=32.0, cy=32.0, znear=0.2,
                             width=64, height=64))
    return g, cam


def _check(lib, g, cam):
    buf = ctypes.create_string_buffer(256)
    st = lib.gs_check_arguments(ctypes.byref(g) if g is not None else None,
                                ctypes.byref(cam) if cam is not None else None, buf, 256)
    return st, buf.value.decode()


def test_check_arguments_accepts_valid(lib):
    g, cam = _good()
    assert _check(lib, g, cam) == (0, "")
    g.n = 0
    g.mean = None
    assert _check(lib, g, cam)[0] == 0      # empty scene: pointers may be NULL


@pytest.mark.parametrize("field,value,words", [
    ("n", -1, "count"), ("n", 1 << 31, "count"), ("sh_degree", 4, "sh_degree"), ("sh_degree", -1, "sh_degree"),
    ("mean", None, "NULL"), ("sh", None, "NULL"),
])
def test_check_arguments_rejects_gaussians(lib, field, value, words):
    g, cam = _good()
    setattr(g, field, value)
    st, msg = _check(lib, g, cam)
    assert st == 1 and words in msg


@pytest.mark.parametrize("field,value,words", [
    ("width", 0, "image size"), ("height", -3, "image size"), ("width", 40000, "image size"),
    ("fx", 0.0, "focal"), ("fy", -1.0, "focal"), ("znear", 0.0, "znear"), ("fx", float("nan"), "non-finite"),
    ("cx", float("inf"), "non-finite"),
])
def test_check_arguments_rejects_camera(lib, field, value, words):
    g, cam = _good()
    setattr(cam, field, value)
    st, msg = _check(lib, g, cam)
    assert st == 1 and words in msg


def test_check_arguments_rejects_nan_rotation(lib):
    g, cam = _good()
    cam.R[4] = float("nan")
    assert _check(lib, None, cam)[0] == 1


def test_null_context_is_invalid_argument(lib):
    from tile_differentiable_rasterizer_gs_amd import binding as b

    g, cam = _good()
    pr, bn, prof = b.Projected(), b.Binning(), b.Profile()
    bg = (ctypes.c_float * 3)(0, 0, 0)
    assert lib.gs_preprocess(None, ctypes.byref(g), ctypes.byref(cam), ctypes.byref(pr), None) == 1
    assert lib.gs_bin_and_sort(None, ctypes.byref(pr), ctypes.byref(cam), ctypes.byref(bn), None) == 1
    assert lib.gs_composite(None, ctypes.byref(pr), ctypes.byref(bn), ctypes.byref(cam), bg, None, None) == 1
    assert lib.gs_render(None, ctypes.byref(g), ctypes.byref(cam), bg, None, None) == 1
    gr = b.Gradients()
    assert lib.gs_backward(None, ctypes.byref(g), ctypes.byref(cam), ctypes.byref(pr), ctypes.byref(bn), bg,
                           None, None, None, ctypes.byref(gr), None) == 1
    assert lib.gs_context_set_option(None, 0, 0) == 1
    assert lib.gs_profile_read(None, ctypes.byref(prof)) == 1
    assert lib.gs_splat2d_forward(None, 0, None, None, None, None, None, 4, 4, bg, None, None) == 1
    assert lib.gs_splat2d_backward(None, 0, None, None, None, None, None, 4, 4, bg, None, None, None, None,
                                   None, None) == 1
    assert lib.gs_scale_activation(None, None, None, 0, None) == 1
    assert lib.gs_context_create(None, 0) == 1
    lib.gs_context_destroy(None)
    assert lib.gs_last_error(None) == b""


def test_status_strings(lib):
    assert lib.gs_status_string(0) == b"ok"
    assert b"invalid" in lib.gs_status_string(1)
    assert b"memory" in lib.gs_status_string(2)
    assert b"capacity" in lib.gs_status_string(3)
    assert b"HIP" in lib.gs_status_string(4)


def test_context_create_without_device(lib):
    import torch

    ctx = ctypes.c_void_p()
    st = lib.gs_context_create(ctypes.byref(ctx), 0)
    if torch.cuda.is_available():
        assert st == 0
        lib.gs_context_destroy(ctx)
    else:
        assert st == 4 and not ctx.value
    assert lib.gs_context_create(ctypes.byref(ctx), -1) == 4


def test_binding_rejects_bad_tensors():
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding as b

    t = {k: torch.zeros(s) for k, s in dict(mean=(3, 4), quat=(4, 4), log_scale=(3, 4), opacity=(4,),
                                             sh=(3, 4)).items()}
    with pytest.raises(ValueError):
        b.make_gaussians(t, 0)          # CPU tensors are refused: no CPU fallback
