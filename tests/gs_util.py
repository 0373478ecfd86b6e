"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on one input."""
from __future__ import annotations

import sys

import numpy as np

import oracle

IMAGE_TOL = 2e-4      # max abs error per pixel channel, fp32 GPU vs fp64 oracle
RGB_TOL = 2e-5        # SH colour: fp32 GPU vs fp64 oracle


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(arrays: dict, sh_degree: int, camera: dict, bg=(0.0, 0.0, 0.0), sort_mode: int = 0,
            emit_keys: bool = True, aux: bool = True, rast=None, tile_test: int = 0):
    """Preprocess + bin + composite through the C ABI; returns numpy copies."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = rast or binding.Rasterizer(sort_mode=sort_mode, emit_keys=emit_keys, tile_test=tile_test)
    dev = binding.gaussians_to_device(arrays)
    pr = r.preprocess(dev, sh_degree, camera)
    bn = r.bin_and_sort(pr, camera)
    H, W = camera["height"], camera["width"]
    T = torch.empty((H, W), dtype=torch.float32, device="cuda") if aux else None
    nb = torch.empty((H, W), dtype=torch.int32, device="cuda") if aux else None
    tot = torch.zeros(1, dtype=torch.int64, device="cuda") if aux else None
    img = r.composite(pr, bn, camera, bg=bg, final_T=T, n_blend=nb, blend_total=tot)
    pt = r.projected_tensors(pr)
    bt = r.binning_tensors(bn)
    torch.cuda.synchronize()
    out = dict(
        splat=pt["splat"].cpu().numpy(),
        depth=pt["depth"].cpu().numpy(),
        rect=pt["rect"].cpu().numpy().view(np.uint16).astype(np.int32),
        tile_count=pt["tile_count"].cpu().numpy().view(np.uint32),
        num_dups=bt["num_dups"],
        depth_buckets=int(bn.depth_buckets),
        values=bt["values"].cpu().numpy().view(np.uint32),
        ranges=bt["ranges"].cpu().numpy().view(np.uint32),
        keys=None if bt["keys"] is None else bt["keys"].cpu().numpy().view(np.uint64),
        keys_unsorted=None if bt["keys_unsorted"] is None else bt["keys_unsorted"].cpu().numpy().view(np.uint64),
        values_unsorted=None if bt["values_unsorted"] is None else bt["values_unsorted"].cpu().numpy().view(np.uint32),
        image=img.cpu().numpy(),
    )
    if aux:
        out["T"] = T.cpu().numpy()
        out["n_blend"] = nb.cpu().numpy()
        out["blend_total"] = int(tot.item())
    if rast is None:
        r.close()
    return out


def check_preprocess(g: dict, o: dict):
    """Integer and fp32 projection fields must match the oracle bit for bit."""
    assert np.array_equal(g["tile_count"], o["tile_count"]), "tile_count"
    vis = o["tile_count"] > 0
    assert np.array_equal(g["depth"].view(np.uint32), o["depth"].view(np.uint32)), "depth bits"
    assert np.array_equal(g["rect"].T[:, vis], o["rect"][:, vis]), "rect"
    sp = g["splat"]
    assert np.array_equal(sp[vis, 0].view(np.uint32), o["mean2d"][0, vis].view(np.uint32)), "u"
    assert np.array_equal(sp[vis, 1].view(np.uint32), o["mean2d"][1, vis].view(np.uint32)), "v"
    for k in range(3):
        assert np.array_equal(sp[vis, 10 + k].view(np.uint32), o["conic"][k, vis].view(np.uint32)), f"conic {k}"
    assert np.array_equal(sp[vis, 2], o["opacity"][vis]), "opacity"
    assert np.array_equal(sp[vis, 13].view(np.uint32), o["depth"][vis].view(np.uint32)), "record depth"
    assert np.array_equal(sp[vis, 9], o["radius"][vis]), "radius"
    if vis.any():
        err = np.abs(sp[vis, 6:9].astype(np.float64) - o["rgb"][:, vis].T).max()
        assert err <= RGB_TOL, f"rgb err {err}"


def check_binning(g: dict, ob: dict, check_keys: bool = True):
    assert g["num_dups"] == ob["num_dups"], f"num_dups {g['num_dups']} vs {ob['num_dups']}"
    assert np.array_equal(g["values"], ob["values"]), "sorted values"
    assert np.array_equal(g["ranges"], ob["ranges"]), "tile ranges"
    if check_keys:
        assert g["keys"] is not None and np.array_equal(g["keys"], ob["keys"]), "sorted keys"


def image_error(g_img, o_img):
    return float(np.abs(g_img.astype(np.float64) - o_img).max()) if g_img.size else 0.0


def tile_pixels(cam: dict, tiles) -> np.ndarray:
    """Flat indices y*W+x of every image pixel of the given 16x16 tiles (partial tiles clipped)."""
    W, H = cam["width"], cam["height"]
    tx_n = (W + 15) // 16
    out = []
    for t in tiles:
        tx, ty = int(t) % tx_n, int(t) // tx_n
        ys = np.arange(16 * ty, min(16 * ty + 16, H))
        xs = np.arange(16 * tx, min(16 * tx + 16, W))
        out.append((ys[:, None] * W + xs[None, :]).ravel())
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def bottom_tile_row_pixels(cam: dict) -> np.ndarray:
    """Every pixel of the last tile row (partial when the height is not a multiple of 16)."""
    W, H = cam["width"], cam["height"]
    y0 = 16 * ((H - 1) // 16)
    return np.arange(y0 * W, H * W, dtype=np.int64)


def per_tile_counts(o: dict) -> np.ndarray:
    """Pairs per tile under the square rule, counted independently of the binning: every
    visible Gaussian adds one to each tile of its rectangle (2D difference array)."""
    tx, ty = o["tiles"]
    vis = o["tile_count"] > 0
    x0, x1, y0, y1 = (o["rect"][i][vis].astype(np.int64) for i in range(4))
    D = np.zeros((ty + 1, tx + 1), np.int64)
    np.add.at(D, (y0, x0), 1)
    np.add.at(D, (y0, x1), -1)
    np.add.at(D, (y1, x0), -1)
    np.add.at(D, (y1, x1), 1)
    return D.cumsum(0).cumsum(1)[:ty, :tx].reshape(-1)


def ranges_from_counts(per_tile: np.ndarray) -> np.ndarray:
    """[tiles][2] half-open ranges of a list sorted by tile: (0, 0) for empty tiles."""
    end = np.cumsum(per_tile)
    start = end - per_tile
    return np.where(per_tile[:, None] > 0, np.stack([start, end], 1), 0).astype(np.int64)


def plane_scene(seed: int, n: int, depths, w: int = 320, h: int = 240, sh_degree: int = 0):
    """Means spread over x, y in front of a camera at the origin looking down +z (R = I, t = 0,
    so each camera-space depth is exactly the mean's z), z drawn from `depths`: a scene whose
    depths crowd into a few values, as a flat wall facing the camera gives."""
    rng = np.random.default_rng(seed)
    z = rng.choice(np.asarray(depths, np.float32), n)
    mean = np.stack([rng.uniform(-2.0, 2.0, n) * z / 5.0, rng.uniform(-1.5, 1.5, n) * z / 5.0, z]).astype(np.float32)
    k = 3 * (sh_degree + 1) ** 2
    arrays = dict(mean=np.ascontiguousarray(mean), quat=rng.normal(size=(4, n)).astype(np.float32),
                  log_scale=rng.uniform(-4.5, -3.0, (3, n)).astype(np.float32),
                  opacity=rng.uniform(-1.0, 2.0, n).astype(np.float32),
                  sh=rng.normal(0.0, 0.3, (k, n)).astype(np.float32))
    cam = dict(R=[1.0, 0.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 1.0], t=[0.0, 0.0, 0.0], fx=250.0, fy=250.0,
               cx=w / 2.0, cy=h / 2.0, znear=0.2, width=w, height=h)
    return arrays, cam
