"""Benchmark: frames/s of the forward rasterizer on the 1M-Gaussian SH3 1920x1080 scene.

One step = one full frame through gs_render (preprocess, depth sort, prefix sum,
pair listing, tile sort, ranges, composite) with the scene already resident in
HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sort-mode 0|1]
                  [--no-cpu-baseline] [--no-backward] [--calibration-copy]

A workload with several cameras (the 32-view orbit) renders its views round-robin.
The JSON line also carries the backward pass (gs_backward for a fixed random
image cotangent) timed on its own and as part of a forward + backward step, and
the lesson's 2D splat-fitting workload (64 splats, 64x64, 200 Adam steps), and the
same frames under the exact-footprint tile rule (GS_TILE_ELLIPSE), and (field
`workloads`) the other four scenes: 10 k SH0 256x256, 100 k SH3 800x800, 5 M SH3
1080p with 2 % large Gaussians, and the 3 M SH3 1080p 32-view orbit (one stream and
three views in flight), each with its stage split and stage rooflines.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
# LDS read path: 256 bytes per clock per CU (gfx950 doubles the previous generation's 128),
# x 256 CUs x 2.4 GHz, in GB/s
LDS_PEAK_GBS = 256 * 256 * 2.4
EXTRA_WORKLOADS = ("c1_10k_sh0_256", "c2_100k_sh3_800", "c4_5m_sh3_1080p_large", "c5_3m_sh3_1080p_orbit32")
# VALU issue peak: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz, one lane-op per lane per clock
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4
# lane-ops per blended (pixel, Gaussian) pair in the composite inner loop, counting a
# multiply-add as one: dx (1); exponent (A' dx + B' dy) dx + (C' dy^2 + log2(o / 0.99)) as
# two multiply-adds on the row terms (2); exp2 with its clamp to 1 (1); stop test and
# masked T (2); T*alpha (1); three colour multiply-adds (3); transmittance update (1);
# plus the row terms dy, B' dy, C' dy^2 + log2(o / 0.99) (4), computed once per (splat,
# pixel row of 16): 0.25
COMPOSITE_OPS_PER_PAIR = 11.25
# lane-ops per blended pair in the backward walk: alpha as in the forward (dx, dy, exponent
# 4, exp2, clamp: 7); 1 - alpha and its reciprocal (2); T recovery (1); dL/dalpha from
# c . dL/dC, the carried (colour behind) . dL/dC and the background (7); the update of that
# carried product (1); colour gradient weights (4); clamp test and opacity gradient (3);
# dL/dQ (2); the moments dy S0, dy S1, dy^2 S0 that the u, v, A, B, C gradients are linear in (3;
# the conic is applied per Gaussian, after the sum over its records)
BACKWARD_OPS_PER_PAIR = 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def stage_bytes(n, sh_degree, m, n_visible, supers, tiles, buckets):
    """Algorithmic HBM bytes per frame for each stage (depth-first mode).  m pairs; supers > 0:
    the per-tile lists came from super-tile binning over `supers` super-list entries, else from
    the radix sort of the pairs on the tile id; buckets > 0: the depth order came from that many
    depth buckets, else from the radix sort of the depth bits."""
    K = (sh_degree + 1) ** 2
    pre = n * ((3 + 4 + 3 + 1 + 3 * K) * 4 + 12 * 4 + 4 + 8 + 4 + 8)
    if buckets:
        # count and scatter read the key (4 + 4), the scatter reads the rectangle (8) and writes
        # a 16-byte entry (index, depth bits, rectangle), the bucket sort reads it and writes
        # rank -> Gaussian, the count and the rectangle in rank order (4 + 4 + 8)
        depth_sort = n * (4 + 4 + 8 + 16 + 16 + 16)
    else:
        depth_sort = 4 * n * 16 + n * 8    # 4 passes x (read key+value, write key+value); the last gathers
    scan = n * (4 + 4 + 4)             # gathered count + order read, offset write
    if supers:
        # listing: offset, rank and rectangle per visible Gaussian, one (key, Gaussian) per entry
        dup = n_visible * (4 + 4 + 8) + supers * 8
        # one 8-bit pass over the super list (count reads the key; scatter reads and writes key and
        # value), the count and place kernels read it again, each tile entry written once (4 B),
        # the per-segment tile counts written, read and rewritten by the column scan, read by place
        # (+ the tile totals read and the heaviest-first launch order written by the place kernel)
        segs = supers // 64 + 257
        tile_sort = supers * (4 + 16) + supers * (4 + 8) + m * 4 + segs * 64 * 4 * 4 + tiles * 12 + tiles * 8
        ranges = None
    else:
        kb = 2 if tiles <= 1 << 16 else 4   # tile-id key bytes
        passes = max(1, (max(tiles - 1, 1).bit_length() + 7) // 8)
        dup = n_visible * (4 + 4 + 8) + m * (kb + 4)
        tile_sort = passes * m * (kb + 2 * (kb + 4))   # count reads the key; scatter reads and writes both
        ranges = m * kb + tiles * 12
    out = dict(preprocess=pre, depth_sort=depth_sort, scan=scan, duplicate=dup, tile_sort=tile_sort, ranges=ranges)
    return {k: v for k, v in out.items() if v is not None}


def _profile_summary(path):
    """key: value lines of a committed rocprofv3 summary, or None when it is missing or was
    taken on another composite kernel source."""
    import hashlib

    src = os.path.join(ROOT, "tile_differentiable_rasterizer_gs_amd", "csrc", "composite.hip")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("composite_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return kv


def measured_traffic(workload):
    """HBM bytes per composite launch from the committed rocprofv3 summary (None if stale)."""
    kv = _profile_summary(os.path.join(ROOT, "profiles", f"traffic_{workload}.txt"))
    return None if kv is None else int(float(kv["composite_traffic_bytes"]))


def composite_lds(workload, comp_ms):
    """LDS roofline of the composite: bytes its LDS instructions deliver per launch (rocprofv3
    SQ_INSTS_LDS_LOAD_BANDWIDTH + SQ_INSTS_LDS_STORE_BANDWIDTH, 64-byte units, from the
    committed summary) over the launch time measured here, against LDS_PEAK_GBS; and the LDS
    pipe's busy fraction (SQ_LDS_IDX_ACTIVE over the kernel's cycles x CUs).  None if stale."""
    kv = _profile_summary(os.path.join(ROOT, "profiles", f"lds_{workload}.txt"))
    if kv is None or not comp_ms:
        return None
    nbytes = float(kv["composite_lds_bytes"])
    gbs = nbytes / (comp_ms * 1e-3) / 1e9
    return dict(bound="lds", achieved=round(gbs, 1), peak=round(LDS_PEAK_GBS, 1), unit="GB/s",
                frac=round(gbs / LDS_PEAK_GBS, 4), bytes=nbytes,
                pipe_busy_frac=round(float(kv["composite_lds_busy_frac"]), 4),
                source="profiles/lds_%s.txt" % workload)


def _host_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n):
    """Thread count of the oracle's OpenMP regions started from this thread (libgomp)."""
    import ctypes

    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def oracle_frame(scene, cam, pixels_target, binning=True, seed=0):
    """The oracle on one frame: projection and binning (single thread) in full, the per-pixel
    composite (OpenMP) on `pixels_target` sampled pixels scaled to the whole image (or every
    pixel when the image has fewer).  Returns seconds per frame and what was sampled."""
    import numpy as np

    import oracle

    t0 = time.perf_counter()
    p = oracle.preprocess(scene.arrays(), scene.sh_degree, cam)
    t1 = time.perf_counter()
    if binning:
        oracle.bin_pairs(p, want_unsorted=False)
    t2 = time.perf_counter()
    npx = cam["width"] * cam["height"]
    pix = None
    if pixels_target < npx:
        pix = np.random.default_rng(seed).choice(npx, pixels_target, replace=False)
    oracle.composite(p, cam, pixels=pix)
    t3 = time.perf_counter()
    done = npx if pix is None else len(pix)
    frame_s = (t1 - t0) + (t2 - t1) + (t3 - t2) * npx / done
    what = (f"projection {t1 - t0:.2f}s" + (f", binning {t2 - t1:.2f}s" if binning else ", binning not run") +
            f" (1 thread), composite of {done} of {npx} pixels {t3 - t2:.2f}s")
    return frame_s, what


def cpu_baseline(scene, cam, pixels_target=262144):
    """The oracle on a bounded sample of the timed workload (about 10 s of host work at 1080p
    on 16 threads): full projection + binning, composite on 262144 sampled pixels (12.6 % of
    the frame)."""
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    _omp_threads(threads)
    frame_s, what = oracle_frame(scene, cam, pixels_target)
    return dict(value=1.0 / frame_s, unit="frames/s", cores=threads, kind="oracle", host_cpu=_host_model(),
                sample=f"{scene.n}-Gaussian scene: {what}, {threads} threads, scaled to the full image")


def cpu_baseline_workloads(scenes_by_name):
    """One oracle frame of every other workload (sampled where the full frame would take minutes)
    and the 10 k frame on one thread.  The 5 M scene's binning (4e8 pairs through a host qsort)
    is not run; its per-pixel composite needs no binning."""
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    plan = {"c1_10k_sh0_256": (1 << 20, True), "c2_100k_sh3_800": (65536, True),
            "c4_5m_sh3_1080p_large": (4096, False), "c5_3m_sh3_1080p_orbit32": (16384, True)}
    out = {}
    for name, (px, binning) in plan.items():
        sc = scenes_by_name.get(name)
        if sc is None:
            continue
        _omp_threads(threads)
        frame_s, what = oracle_frame(sc, sc.cameras[0], px, binning=binning)
        out[name] = dict(value=round(1.0 / frame_s, 5), unit="frames/s", cores=threads,
                         sample=what + ("; view 0 of 32" if len(sc.cameras) > 1 else ""))
        log(f"oracle {name}: {frame_s:.2f} s/frame ({what})")
    sc = scenes_by_name.get("c1_10k_sh0_256")
    if sc is not None:
        _omp_threads(1)
        frame_s, what = oracle_frame(sc, sc.cameras[0], 1 << 20)
        out["c1_10k_sh0_256_single_thread"] = dict(value=round(1.0 / frame_s, 5), unit="frames/s", cores=1,
                                                   sample=what)
        log(f"oracle c1 on 1 thread: {frame_s:.2f} s/frame")
        _omp_threads(threads)
    return out


def time_backward(r, dev, scene, cams, img, bg, steps, blends):
    """Backward pass (gs_backward) for a fixed random cotangent dL/dimage, timed alone on one
    view's forward state, and as part of forward (with per-pixel state) + backward steps."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    H, W = cams[0]["height"], cams[0]["width"]
    deg = scene.sh_degree
    T = torch.empty((H, W), dtype=torch.float32, device="cuda")
    nb = torch.empty((H, W), dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(0)
    gimg = torch.randn((H, W, 3), generator=gen, device="cuda", dtype=torch.float32)
    K = (deg + 1) ** 2
    n = scene.n
    grads = {k: torch.empty(shp, dtype=torch.float32, device="cuda")
             for k, shp in dict(mean=(3, n), quat=(4, n), log_scale=(3, n), opacity=(n,), sh=(K * 3, n)).items()}

    def forward(c):
        pr = r.preprocess(dev, deg, c)
        bn = r.bin_and_sort(pr, c)
        r.composite(pr, bn, c, bg=bg, out=img, final_T=T, n_blend=nb)
        return pr, bn

    def backward(c, pr, bn):
        r.backward(dev, deg, c, pr, bn, T, nb, gimg, bg=bg, out=grads)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(3):
        backward(cams[i % len(cams)], *forward(cams[i % len(cams)]))
    torch.cuda.synchronize()
    # forward + backward steps
    start.record()
    for i in range(steps):
        c = cams[i % len(cams)]
        backward(c, *forward(c))
    stop.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(stop) / steps
    # backward alone, repeated on the first view's forward state
    pr, bn = forward(cams[0])
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        backward(cams[0], pr, bn)
    stop.record()
    torch.cuda.synchronize()
    bwd_ms = start.elapsed_time(stop) / steps
    # per-stage split of the backward
    r.set_option(binding.GS_OPT_PROFILE, 1)
    r.profile_read()
    for _ in range(steps):
        backward(cams[0], pr, bn)
    prof = r.profile_read()
    r.set_option(binding.GS_OPT_PROFILE, 0)
    stage = {k: ms / steps for k, (ms, cnt) in prof.items() if cnt and k.startswith("backward")}
    comp = stage.get("backward_composite", 0.0)
    ops = blends * BACKWARD_OPS_PER_PAIR
    gops = ops / (comp * 1e-3) / 1e9 if comp else 0.0
    log(f"backward: {bwd_ms:.4f} ms alone, forward+backward step {step_ms:.4f} ms; stages " +
        ", ".join(f"{k}={v:.4f}" for k, v in stage.items()))
    return dict(ms=round(bwd_ms, 5), train_step_ms=round(step_ms, 5),
                train_steps_per_s=round(1000.0 / step_ms, 2),
                stage_ms={k: round(v, 5) for k, v in stage.items()},
                composite_roofline=dict(bound="alu", achieved=round(gops / 1e3, 3),
                                        peak=round(VALU_PEAK_GOPS / 1e3, 3), unit="Tlane-op/s",
                                        frac=round(gops / VALU_PEAK_GOPS, 4), ops=ops),
                cotangent="standard normal per pixel channel, seed 0")


def copy_bandwidth(reps: int = 20) -> float:
    """Device-to-device copy of 1 GiB (read 1 GiB + write 1 GiB), best of `reps`: GB/s moved."""
    import torch

    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        start.record()
        dst.copy_(src)
        stop.record()
        stop.synchronize()
        best = min(best, start.elapsed_time(stop))
    nbytes = 2 * src.numel() * 4
    del src, dst
    return nbytes / (best * 1e-3) / 1e9


def frame_distribution(r, dev, scene, cams, bg, img, steps):
    """Per-frame times from a HIP event pair around each frame: median, p10, p90 (ms)."""
    import numpy as np
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return dict(median=round(float(np.median(t)), 5), p10=round(float(np.percentile(t, 10)), 5),
                p90=round(float(np.percentile(t, 90)), 5))


def time_ellipse_rule(dev, scene, cams, bg, steps, sort_mode):
    """The same frames under the exact-footprint tile rule (GS_TILE_ELLIPSE): fewer pairs, an
    image that drops contributions below o exp(-9/2) per pixel.  Forward frame time, stage
    split, pairs, and the backward."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    r = binding.Rasterizer(sort_mode=sort_mode, emit_keys=False, tile_test=binding.GS_TILE_ELLIPSE)
    H, W = cams[0]["height"], cams[0]["width"]
    img = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
    pr = r.preprocess(dev, scene.sh_degree, cams[0])
    bn = r.bin_and_sort(pr, cams[0])
    pairs = int(bn.num_dups)
    for i in range(10):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    r.set_option(binding.GS_OPT_PROFILE, 1)
    r.profile_read()
    for i in range(steps):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    prof = r.profile_read()
    r.set_option(binding.GS_OPT_PROFILE, 0)
    stage = {k: round(v / steps, 5) for k, (v, c) in prof.items() if c}
    bwd = time_backward(r, dev, scene, cams[:1], img, bg, max(10, steps // 4), 0)
    r.close()
    log(f"ellipse rule: {ms:.4f} ms/frame, {pairs} pairs; stages {stage}; backward {bwd['ms']} ms")
    return dict(ms_per_step=round(ms, 5), frames_per_s=round(1000.0 / ms, 2), pairs_per_frame=pairs,
                stage_ms=stage, backward_ms=bwd["ms"], train_step_ms=bwd["train_step_ms"],
                note="GS_TILE_ELLIPSE: tiles of the square whose pixel-centre box meets the 3-sigma ellipse")


def time_splat2d_fit():
    """The lesson's 2D splat-fitting workload (64 splats, 64x64 target, Adam 0.05, 200 steps) on the
    HIP 2D rasteriser: whole-fit wall time and the rasteriser's forward + backward kernel time."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding, splat2d

    r = binding.Rasterizer(emit_keys=False)
    splat2d.fit(r, steps=10)                     # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = splat2d.fit(r, steps=200, record_every=200)
    torch.cuda.synchronize()
    fit_s = time.perf_counter() - t0
    # the rasteriser alone on the fitted splats, forward + backward
    p = res["params"]
    args = [t.detach().contiguous() for t in splat2d.splat_arrays(p)]
    g = torch.ones((64, 64, 3), dtype=torch.float32, device="cuda")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(5):
        r.splat2d_forward(*args, 64, 64)
        r.splat2d_backward(*args, 64, 64, g)
    start.record()
    for _ in range(100):
        r.splat2d_forward(*args, 64, 64)
        r.splat2d_backward(*args, 64, 64, g)
    stop.record()
    torch.cuda.synchronize()
    r.close()
    losses = dict(res["losses"])
    return dict(steps=200, fit_ms_per_step=round(fit_s * 1e3 / 200, 4), fit_steps_per_s=round(200 / fit_s, 1),
                rasteriser_fwd_bwd_ms=round(start.elapsed_time(stop) / 100, 5),
                mse_first=round(losses[0], 6), mse_final=round(res["final_loss"], 6),
                note="step = forward + backward through gs_splat2d_* plus torch activations, loss and Adam")


def frame_stats(r, dev, scene, cams, img, bg):
    """Pairs, blended (pixel, Gaussian) pairs, visible Gaussians, super-tile list entries (0
    when the radix binning ran) and depth buckets (0 when the radix sort ordered the depths) per
    frame, averaged over the views (outside any timed region)."""
    import torch

    pairs = blends = n_visible = supers = buckets = 0
    for c in cams:
        pr = r.preprocess(dev, scene.sh_degree, c)
        bn = r.bin_and_sort(pr, c)
        tot = torch.zeros(1, dtype=torch.int64, device="cuda")
        r.composite(pr, bn, c, bg=bg, out=img, blend_total=tot)
        tc = r.projected_tensors(pr)["tile_count"]
        torch.cuda.synchronize()
        pairs += int(bn.num_dups)
        supers += int(bn.super_entries)
        buckets += int(bn.depth_buckets)
        blends += int(tot.item())
        n_visible += int((tc > 0).sum().item())
    return tuple(v / len(cams) for v in (pairs, blends, n_visible, supers, buckets))


def settle_clock(r, dev, scene, cams, img, bg, seconds=0.3):
    """Untimed frames for about `seconds`, so that the shader clock has left its idle state
    before the warm-up and timed frames (a 20-frame timed region lasts ~12 ms).  Returns the
    number of frames rendered."""
    import torch

    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for i in range(10):
            r.render(dev, scene.sh_degree, cams[(n + i) % len(cams)], bg=bg, out=img)
        n += 10
        torch.cuda.synchronize()
    return n


def timed_frames(r, dev, scene, cams, img, bg, steps, S, sort_mode):
    """`steps` frames back to back on one stream, or with S > 1 view i on context i mod S with
    its own stream, so that one view's compositing overlaps the next view's front end.
    Returns (ms per frame from HIP events, wall seconds)."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    lanes = [(r, torch.cuda.current_stream(), img)]
    for _ in range(S - 1):
        lanes.append((binding.Rasterizer(sort_mode=sort_mode, emit_keys=False), torch.cuda.Stream(),
                      torch.empty_like(img)))
    for i in range(S):   # warm every context (workspace sized before timing)
        lr, ls, li = lanes[i]
        for c in cams[:2]:
            lr.render(dev, scene.sh_degree, c, bg=bg, out=li, stream=ls)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for ls in (l[1] for l in lanes[1:]):
        ls.wait_event(start)
    for i in range(steps):
        lr, ls, li = lanes[i % S]
        lr.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=li, stream=ls)
    main = torch.cuda.current_stream()
    for ls in (l[1] for l in lanes[1:]):
        main.wait_stream(ls)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for extra in lanes[1:]:
        extra[0].close()
    return start.elapsed_time(stop) / steps, wall


def stage_split(r, dev, scene, cams, img, bg, steps):
    """The same frames with HIP events around every stage (GS_OPT_PROFILE, on the render
    stream): (ms per stage per frame, ms per frame with the events)."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r.set_option(binding.GS_OPT_PROFILE, 1)
    r.profile_read()
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    stop.record()
    torch.cuda.synchronize()
    prof_ms = start.elapsed_time(stop) / steps
    prof = r.profile_read()
    r.set_option(binding.GS_OPT_PROFILE, 0)
    return {k: (ms / steps) for k, (ms, cnt) in prof.items() if cnt}, prof_ms


def stage_rooflines(scene, pairs, n_visible, supers, buckets, blends, stage_ms, copy_gbs):
    cam = scene.cameras[0]
    tiles = ((cam["width"] + 15) // 16) * ((cam["height"] + 15) // 16)
    nbytes = stage_bytes(scene.n, scene.sh_degree, round(pairs), round(n_visible), round(supers), tiles,
                         round(buckets))
    out = {}
    for st, b in nbytes.items():
        if st in stage_ms and stage_ms[st] > 0:
            gbs = b / (stage_ms[st] * 1e-3) / 1e9
            out[st] = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                           frac=round(gbs / HBM_PEAK_GBS, 4), frac_of_copy=round(gbs / copy_gbs, 4), bytes=b)
    comp_ms = stage_ms.get("composite", 0.0)
    comp_gops = blends * COMPOSITE_OPS_PER_PAIR / (comp_ms * 1e-3) / 1e9 if comp_ms else 0.0
    out["composite"] = dict(bound="alu", achieved=round(comp_gops / 1e3, 3), peak=round(VALU_PEAK_GOPS / 1e3, 3),
                            unit="Tlane-op/s", frac=round(comp_gops / VALU_PEAK_GOPS, 4),
                            ops=blends * COMPOSITE_OPS_PER_PAIR)
    return out


def measure_workload(name, scene, steps, warmup, sort_mode, copy_gbs, bg=(0.0, 0.0, 0.0)):
    """Frame time (one stream; multi-view scenes also three views in flight), stage split and
    stage rooflines of one workload, on a context of its own."""
    import torch

    from tile_differentiable_rasterizer_gs_amd import binding

    cams = scene.cameras
    dev = binding.gaussians_to_device(scene.arrays())
    r = binding.Rasterizer(sort_mode=sort_mode, emit_keys=False)
    img = torch.empty((cams[0]["height"], cams[0]["width"], 3), dtype=torch.float32, device="cuda")
    pairs, blends, n_visible, supers, buckets = frame_stats(r, dev, scene, cams, img, bg)
    for i in range(warmup):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    ms, _ = timed_frames(r, dev, scene, cams, img, bg, steps, 1, sort_mode)
    res = dict(n_gaussians=scene.n, sh_degree=scene.sh_degree, width=cams[0]["width"], height=cams[0]["height"],
               views=len(cams), steps=steps, ms_per_frame=round(ms, 5), frames_per_s=round(1000.0 / ms, 2),
               blends_per_s=round(blends * 1000.0 / ms, 1), pairs_per_frame=round(pairs),
               blended_pairs_per_frame=round(blends), visible_per_frame=round(n_visible),
               super_entries_per_frame=round(supers), depth_buckets=round(buckets))
    if len(cams) > 1:
        p_ms, _ = timed_frames(r, dev, scene, cams, img, bg, steps, 3, sort_mode)
        res["pipelined"] = {"views_in_flight": 3, "ms_per_frame": round(p_ms, 5),
                            "frames_per_s": round(1000.0 / p_ms, 2)}
    stage_ms, _ = stage_split(r, dev, scene, cams, img, bg, steps)
    res["stage_ms"] = {k: round(v, 5) for k, v in stage_ms.items()}
    if len(cams) > 1:   # several views of one scene: the 3D covariances computed once (row f3)
        r.cache_covariance(dev, scene.sh_degree)
        c_ms, _ = timed_frames(r, dev, scene, cams, img, bg, steps, 1, sort_mode)
        c_stage, _ = stage_split(r, dev, scene, cams, img, bg, steps)
        r.cache_covariance(None)
        res["covariance_cache"] = {"ms_per_frame": round(c_ms, 5), "preprocess_ms": round(c_stage["preprocess"], 5),
                                   "note": "gs_cache_covariance once, then every view reads Sigma"}
    res["stage_rooflines"] = stage_rooflines(scene, pairs, n_visible, supers, buckets, blends, stage_ms, copy_gbs)
    r.close()
    del dev, img
    torch.cuda.empty_cache()
    log(f"{name}: {ms:.4f} ms/frame" + (f", {res['pipelined']['ms_per_frame']:.4f} with 3 in flight"
                                         if "pipelined" in res else "") +
        f"; pairs {pairs:.0f}; stages " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--sort-mode", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-splat2d", action="store_true", help="skip the 2D splat-fitting timing")
    ap.add_argument("--no-ellipse", action="store_true", help="skip the exact-footprint tile rule timing")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other four workloads")
    ap.add_argument("--streams", type=int, default=0,
                    help="views in flight (contexts on their own streams) for the timed frames; default 1 "
                         "(multi-view workloads also report three in flight as `pipelined`)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run one 1 GiB read + 1 GiB write elementwise kernel first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this rasterizer has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from tile_differentiable_rasterizer_gs_amd import binding, scenes

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibration_copy:
        # a plain elementwise kernel that reads 1 GiB and writes 1 GiB (larger than the caches)
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    name = args.workload or scenes.HEADLINE
    t = time.perf_counter()
    scene = scenes.make_scene(name)
    cams = scene.cameras          # several views: rendered round-robin, back to back on one stream
    cam = cams[0]
    log(f"scene {name}: n={scene.n} generated in {time.perf_counter() - t:.1f}s")
    dev = binding.gaussians_to_device(scene.arrays())
    r = binding.Rasterizer(sort_mode=args.sort_mode, emit_keys=False)
    H, W = cam["height"], cam["width"]
    img = torch.empty((H, W, 3), dtype=torch.float32, device="cuda")
    bg = (0.0, 0.0, 0.0)

    pairs, blends, n_visible, supers, buckets = frame_stats(r, dev, scene, cams, img, bg)
    log(f"per frame: pairs={pairs:.0f} visible={n_visible:.0f} super-list entries={supers:.0f} "
        f"depth buckets={buckets:.0f} "
        f"blended pairs={blends:.0f} ({len(cams)} view(s))")
    settle = settle_clock(r, dev, scene, cams, img, bg)
    for i in range(args.warmup):
        r.render(dev, scene.sh_degree, cams[i % len(cams)], bg=bg, out=img)
    torch.cuda.synchronize()

    # timed region: plain frames (`value`)
    S = max(1, args.streams)
    ms_per_step, wall = timed_frames(r, dev, scene, cams, img, bg, args.steps, S, args.sort_mode)
    log(f"timed: {ms_per_step:.4f} ms/frame (wall {wall / args.steps * 1e3:.4f} ms, {S} view(s) in flight)")
    pipelined = None
    if len(cams) > 1 and args.streams == 0:
        p_ms, p_wall = timed_frames(r, dev, scene, cams, img, bg, args.steps, 3, args.sort_mode)
        pipelined = {"views_in_flight": 3, "ms_per_frame": round(p_ms, 5), "frames_per_s": round(1000.0 / p_ms, 2)}
        log(f"three views in flight: {p_ms:.4f} ms/frame (wall {p_wall / args.steps * 1e3:.4f} ms)")

    # same frames with HIP events around every stage (on the render stream)
    stage_ms, prof_ms_per_step = stage_split(r, dev, scene, cams, img, bg, args.steps)
    log("stages (ms/frame): " + ", ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))

    # per-frame distribution (one event pair per frame) and the device's copy bandwidth
    dist = frame_distribution(r, dev, scene, cams, bg, img, args.steps)
    copy_gbs = copy_bandwidth()
    log(f"frame ms median {dist['median']} p10 {dist['p10']} p90 {dist['p90']}; 1 GiB copy {copy_gbs:.0f} GB/s")

    rooflines = stage_rooflines(scene, pairs, n_visible, supers, buckets, blends, stage_ms, copy_gbs)
    lds = composite_lds(name, stage_ms.get("composite", 0.0))
    if lds:
        rooflines["composite_lds"] = lds
    dominant = max(stage_ms, key=stage_ms.get)
    dom = dict(rooflines.get(dominant, {}))
    dom["kernel"] = dominant
    dom["traffic"] = measured_traffic(name) if dominant == "composite" else None

    out = {
        "metric": "frames/s and Gaussian-pixel blends/s, 1M Gaussians SH3 @1920x1080, 1 GPU",
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "frames/s",
        "blends_per_s": round(blends * 1000.0 / ms_per_step, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_frames": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "n_gaussians": scene.n, "sh_degree": scene.sh_degree, "width": W,
                   "height": H, "views": len(cams), "views_in_flight": S,
                   "sort_mode": "depth_first" if args.sort_mode == 0 else "key64",
                   "pairs_per_frame": round(pairs), "blended_pairs_per_frame": round(blends)},
        "roofline": dom,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_rooflines": rooflines,
        "profiled_ms_per_step": round(prof_ms_per_step, 5),
        "frame_ms_distribution": dist,
        "copy_gbs": round(copy_gbs, 1),
        "context": "pages: '100+ FPS at 1080p' for a trained scene on an unnamed GPU; 147 fps for 6M splats on an "
                   "RTX 3080 Ti (resolution not stated)",
    }
    if pipelined:
        out["pipelined"] = pipelined
    if not args.no_ellipse:
        out["tile_test_ellipse"] = time_ellipse_rule(dev, scene, cams, bg, args.steps, args.sort_mode)
    if not args.no_backward:
        out["backward"] = time_backward(r, dev, scene, cams, img, bg, args.steps, blends)
    if not args.no_splat2d:
        log("2D splat fit ...")
        out["splat2d_fit"] = time_splat2d_fit()
        log(f"2D splat fit: {out['splat2d_fit']}")
    r.close()
    del dev, img
    torch.cuda.empty_cache()
    others = {}
    if not args.no_workloads:
        out["workloads"] = {}
        for wname in EXTRA_WORKLOADS:
            if wname == name:
                continue
            t = time.perf_counter()
            others[wname] = scenes.make_scene(wname)
            log(f"scene {wname}: n={others[wname].n} generated in {time.perf_counter() - t:.1f}s")
            many = len(others[wname].cameras) > 1 or others[wname].n >= 5_000_000
            steps = 64 if len(others[wname].cameras) > 1 else (20 if many else args.steps)
            warmup = 8 if many else args.warmup
            out["workloads"][wname] = measure_workload(wname, others[wname], steps, warmup, args.sort_mode, copy_gbs)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(scene, cam)
        if others:
            out["cpu_baseline"]["workloads"] = cpu_baseline_workloads(others)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
