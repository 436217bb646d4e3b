#!/usr/bin/env python3
"""Benchmark of the spatial-transformer grid generator + sampler on one MI355X.

One step = the whole hot path over one batch of the 2D STN workload:
theta (64,2,3) -> gs_affine_grid -> grid (64,128,128,2) -> gs_grid_sample_2d
(bilinear, zeros, align_corners=0) on X (64,64,128,128) fp32 -> Y.

Prints ONE JSON line.  `value` is output elements per second of the whole step
(inputs resident in HBM, K back-to-back steps between two synchronisations).
`roofline` describes the dominant kernel (the sampler): algorithmic bytes per
launch (distinct X elements the launch reads with non-zero weight, the grid,
and Y) divided by its mean duration, measured with events on the launch stream
inside the timed region.  `traffic` is the HBM byte count from rocprofv3
counters (profiles/sampler_traffic.json) when those were taken on the current
kernel source, else null.  `cpu_baseline` times the plain CPU oracle on the
same workload.  `paths` reports the other workload shapes, Resize included
(kernel time only).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "GridSample output elem/s + achieved HBM GB/s (% of MI355X peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sampler_traffic.json")
KERNEL_SOURCES = ["gs_kernels.hip", "gs_device.hpp", "gs_launch.hpp", "gs_api.cpp"]


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "spatial_transformer_grid_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------- accounting
# Distinct X elements a launch reads with a non-zero weight (its compulsory
# X traffic).  Host-side bookkeeping for the byte count only.

def _pixel(g, n, ac):
    g = g.astype(np.float64)
    return (g + 1) / 2 * (n - 1) if ac else ((g + 1) * n - 1) / 2


def _reflect_index(i, n, ac):
    if ac:
        if n == 1:
            return np.zeros_like(i)
        m = np.abs(i) % (2 * (n - 1))
        return np.where(m <= n - 1, m, 2 * (n - 1) - m)
    m = np.mod(i, 2 * n)
    return np.where(m < n, m, 2 * n - 1 - m)


def _reflect_coord(p, n, ac):
    lo, hi = (0.0, n - 1.0) if ac else (-0.5, n - 0.5)
    span = hi - lo
    if span <= 0:
        return np.zeros_like(p)
    d = np.abs(p - lo)
    f = np.floor(d / span)
    e = d - f * span
    r = np.where(np.mod(f, 2) == 0, lo + e, hi - e)
    return np.clip(r, 0, n - 1)


def _axis_taps(g, n, ac, mode, pad):
    """(index, usable) per tap along one axis; usable = in range, weight != 0."""
    p = _pixel(g, n, ac)
    if mode == "cubic":
        i0 = np.floor(p)
        idx = i0[..., None] + np.array([-1, 0, 1, 2])
        t = (p - i0)[..., None]
        # the cubic kernel vanishes only at integer distances 1 and 2: with
        # t = 0 just the centre tap carries weight
        use = (t != 0) | (np.array([-1, 0, 1, 2]) == 0)
        if pad == "zeros":
            use = use & (idx >= 0) & (idx < n)
        elif pad == "border":
            idx = np.clip(idx, 0, n - 1)
        else:
            idx = _reflect_index(idx.astype(np.int64), n, ac)
        return idx.astype(np.int64), use
    if pad == "border":
        p = np.clip(p, 0, n - 1)
    elif pad == "reflection":
        p = _reflect_coord(p, n, ac)
    if mode == "nearest":
        idx = np.rint(p)[..., None]
        return idx.astype(np.int64), (idx >= 0) & (idx < n)
    i0 = np.floor(p)
    t = p - i0
    idx = i0[..., None] + np.array([0, 1])
    w = np.stack([1 - t, t], -1)
    return idx.astype(np.int64), (w != 0) & (idx >= 0) & (idx < n)


def footprint_elements(grid: np.ndarray, in_sp, mode, pad, ac) -> int:
    """Sum over images of the number of distinct input pixels touched."""
    r = len(in_sp)
    total = 0
    for b in range(grid.shape[0]):
        g = grid[b].reshape(-1, r)
        L = g.shape[0]
        flat = np.zeros((L, 1), np.int64)
        use = np.ones((L, 1), bool)
        for a in range(r):
            idx, ok = _axis_taps(g[:, r - 1 - a], in_sp[a], ac, mode, pad)   # (L, taps)
            flat = (flat[:, :, None] * in_sp[a] + idx[:, None, :]).reshape(L, -1)
            use = (use[:, :, None] & ok[:, None, :]).reshape(L, -1)
        total += np.unique(flat[use]).size
    return int(total)


# ------------------------------------------------------------------- timing

def elapsed_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def time_kernel(torch, fn, reps, flush=None):
    """Median and mean duration (us) of fn(), events on the current stream."""
    ev = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = elapsed_ms(ev)
    return statistics.median(ms) * 1e3, statistics.mean(ms) * 1e3


def copy_bandwidth(torch, mib=512, reps=10):
    n = mib * 1024 * 1024 // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    med, _ = time_kernel(torch, lambda: dst.copy_(src), reps)
    del src, dst
    return 2 * mib * 1024 * 1024 / (med * 1e-6) / 1e9


# ------------------------------------------------------------------ paths

def run_paths(torch, gsa, flush_buf):
    """Kernel-only measurements of every workload shape (median of events)."""
    out = []

    # a read-only pass over 512 MiB evicts the Infinity Cache without leaving
    # dirty lines whose write-back would land in the next timed launch
    sink = torch.empty((), device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=sink)

    def record(name, workload, kernel, us, outputs, x_bytes_full, x_bytes_fp, other_bytes, warm_us=None):
        comp = x_bytes_fp + other_bytes
        rec = {"path": name, "workload": workload, "kernel": kernel, "kernel_us": round(us, 2),
               "out_elems_per_s": outputs / (us * 1e-6),
               "compulsory_bytes": comp, "compulsory_bytes_full_x": x_bytes_full + other_bytes,
               "GBps": comp / (us * 1e-6) / 1e9,
               "frac_hbm_peak": comp / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        if warm_us is not None:
            rec["warm_kernel_us"] = round(warm_us, 2)
            rec["warm_GBps"] = comp / (warm_us * 1e-6) / 1e9
        out.append(rec)
        log("%-28s %8.1f us  %7.0f GB/s  %.3f of peak" % (name, us, rec["GBps"], rec["frac_hbm_peak"]))

    # 2D STN batch: nearest + border and fused bilinear
    w = W.WORKLOADS["stn2d_batch"]
    inp = W.make_inputs(w)
    n, c, h, wd = w.x_shape
    X = torch.from_numpy(inp["X"]).cuda()
    th = torch.from_numpy(inp["theta"]).cuda()
    size = (n, c) + w.out_spatial
    grid = gsa.affine_grid(th, size, 0)
    Y = torch.empty((n, c) + w.out_spatial, device="cuda")
    g_host = grid.cpu().numpy()
    outputs = w.outputs
    gbytes = grid.numel() * 4
    for mode, pad in (("linear", "zeros"), ("nearest", "border")):
        fp = footprint_elements(g_host, (h, wd), mode, pad, 0) * c * 4
        us, _ = time_kernel(torch, lambda: gsa.grid_sample(X, grid, mode, pad, 0, out=Y), 30)
        record("stn2d_batch/%s-%s" % (mode, pad), w.name, "gs_grid_sample_2d", us, outputs,
               X.numel() * 4, fp, gbytes + outputs * 4)
    # the same call with a workspace: the probe keeps the staged sampler (the
    # difference is the probe and two launches that return at once)
    ws = torch.empty(gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(grid.shape), 0),
                     dtype=torch.uint8, device="cuda")
    fp = footprint_elements(g_host, (h, wd), "linear", "zeros", 0) * c * 4
    us, _ = time_kernel(torch, lambda: gsa.grid_sample(X, grid, "linear", "zeros", 0, out=Y,
                                                       workspace=ws), 30)
    record("stn2d_batch/linear-zeros-workspace", w.name, "gs_grid_sample_2d_ws (staged chosen)", us,
           outputs, X.numel() * 4, fp, gbytes + outputs * 4)
    del ws
    fp = footprint_elements(g_host, (h, wd), "linear", "zeros", 0) * c * 4
    us, _ = time_kernel(torch, lambda: gsa.affine_grid_sample_fused(th, X, w.out_spatial, "linear",
                                                                      "zeros", 0, out=Y), 30)
    record("stn2d_batch/fused-linear-zeros", w.name, "gs_affine_grid_sample_fused", us, outputs,
           X.numel() * 4, fp, th.numel() * 4 + outputs * 4)
    del X, Y, grid

    # 2D random flow, bicubic + reflection
    w = W.WORKLOADS["flow2d_bicubic"]
    inp = W.make_inputs(w)
    n, c, h, wd = w.x_shape
    X = torch.from_numpy(inp["X"]).cuda()
    G = torch.from_numpy(inp["grid"]).cuda()
    Y = torch.empty((n, c) + w.out_spatial, device="cuda")
    fp = footprint_elements(inp["grid"], (h, wd), "cubic", "reflection", 1) * c * 4
    us, _ = time_kernel(torch, lambda: gsa.grid_sample(X, G, "cubic", "reflection", 1, out=Y), 20)
    record("flow2d_bicubic/cubic-reflection", w.name, "gs_grid_sample_2d", us, w.outputs,
           X.numel() * 4, fp, G.numel() * 4 + w.outputs * 4)
    # with a workspace: probe, sliced channels-last copy of X, gather (the
    # whole call is timed, the copy included)
    ws = torch.empty(gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(G.shape), 0),
                     dtype=torch.uint8, device="cuda")
    us, _ = time_kernel(torch, lambda: gsa.grid_sample(X, G, "cubic", "reflection", 1, out=Y,
                                                       workspace=ws), 20)
    record("flow2d_bicubic/cubic-reflection-workspace", w.name,
           "gs_grid_sample_2d_ws (gather path)", us, w.outputs, X.numel() * 4, fp,
           G.numel() * 4 + w.outputs * 4)
    del X, Y, G, inp, ws

    # 3D volumetric, fused trilinear + border (working set fits the MALL:
    # report the flushed time as the figure and the warm one beside it)
    w = W.WORKLOADS["vol3d"]
    inp = W.make_inputs(w)
    n, c = w.x_shape[:2]
    X = torch.from_numpy(inp["X"]).cuda()
    th = torch.from_numpy(inp["theta"]).cuda()
    Y = torch.empty((n, c) + w.out_spatial, device="cuda")
    grid = gsa.affine_grid(th, (n, c) + w.out_spatial, 0)
    fp = footprint_elements(grid.cpu().numpy(), w.x_shape[2:], "linear", "border", 0) * c * 4
    fn = lambda: gsa.affine_grid_sample_fused(th, X, w.out_spatial, "linear", "border", 0, out=Y)
    us, _ = time_kernel(torch, fn, 20, flush)
    warm, _ = time_kernel(torch, fn, 20)
    record("vol3d/fused-linear-border", w.name, "gs_affine_grid_sample_fused", us, w.outputs,
           X.numel() * 4, fp, th.numel() * 4 + w.outputs * 4, warm)
    fn = lambda: gsa.grid_sample(X, grid, "linear", "border", 0, out=Y)
    us, _ = time_kernel(torch, fn, 20, flush)
    warm, _ = time_kernel(torch, fn, 20)
    record("vol3d/unfused-linear-border", w.name, "gs_grid_sample_3d", us, w.outputs,
           X.numel() * 4, fp, grid.numel() * 4 + w.outputs * 4, warm)
    del X, Y, grid

    # 2D large half precision, smooth flow
    w = W.WORKLOADS["flow2d_half"]
    inp = W.make_inputs(w)
    n, c, h, wd = w.x_shape
    G = torch.from_numpy(inp["grid"]).cuda()
    fp = footprint_elements(inp["grid"], (h, wd), "linear", "zeros", 0) * c * 2
    for kind, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        X = torch.from_numpy(inp["X_bits"][kind].view(np.int16)).cuda().view(tdt)
        Y = torch.empty((n, c) + w.out_spatial, device="cuda", dtype=tdt)
        us, _ = time_kernel(torch, lambda: gsa.grid_sample(X, G, "linear", "zeros", 0, out=Y), 20)
        record("flow2d_half/%s-linear-zeros" % kind, w.name, "gs_grid_sample_2d", us, w.outputs,
               X.numel() * 2, fp, G.numel() * 4 + w.outputs * 2)
        del X, Y

    # other ranks and element types (the any-rank kernel)
    for name, tw in W.TYPE_WORKLOADS.items():
        inp = W.make_type_inputs(tw)
        n, c = tw.x_shape[:2]
        X = torch.from_numpy(inp["X"]).cuda()
        if inp["theta"] is not None:
            th = torch.from_numpy(inp["theta"]).cuda()
            G = gsa.affine_grid(th, (n, c) + tw.out_spatial, tw.align_corners)
        else:
            G = torch.from_numpy(inp["grid"]).cuda()
        Y = torch.empty((n, c) + tw.out_spatial, dtype=X.dtype, device="cuda")
        es = X.element_size()
        fp = footprint_elements(G.cpu().numpy(), tw.x_shape[2:], tw.mode, tw.padding,
                                tw.align_corners) * c * es
        fn = lambda: gsa.grid_sample(X, G, tw.mode, tw.padding, tw.align_corners, out=Y)
        fn()
        us, _ = time_kernel(torch, fn, 20, flush)
        warm, _ = time_kernel(torch, fn, 20)
        record("%s/%s-%s" % (name, tw.mode, tw.padding), name, "gs_grid_sample (any-rank kernel)",
               us, tw.outputs, X.numel() * es, fp, G.numel() * G.element_size() + tw.outputs * es,
               warm)
        del X, Y, G, inp

    # DeformConv layers: matrix-core throughput (flops of the convolution)
    for name, dw in W.DEFORM_WORKLOADS.items():
        inp = W.make_deform_inputs(dw)
        for kind in dw.dtypes:
            tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[kind]
            d = {k: torch.from_numpy(v).cuda().to(tdt) for k, v in inp.items()}
            Y = torch.empty(dw.out_shape(), dtype=tdt, device="cuda")
            ws = torch.empty(gsa.deform_conv_workspace_size(
                dw.x_shape, dw.w_shape, gsa.dtype_code(d["X"]), None, list(dw.pads), None,
                dw.group, dw.offset_group), dtype=torch.uint8, device="cuda")
            fn = lambda: gsa.deform_conv(d["X"], d["W"], d["offset"], d["B"], d["mask"],
                                         pads=list(dw.pads), group=dw.group,
                                         offset_group=dw.offset_group, out=Y, workspace=ws)
            fn()
            us, _ = time_kernel(torch, fn, 20, flush)
            peak = 157.3 if kind == "f32" else 2500.0
            tflops = dw.flops / (us * 1e-6) / 1e12
            es = 4 if kind == "f32" else 2
            io = (inp["X"].size + inp["W"].size + inp["offset"].size + inp["mask"].size
                  + inp["B"].size + Y.numel()) * es
            out.append({"path": "%s/%s" % (name, kind), "workload": name,
                        "kernel": "gs_deform_conv (implicit GEMM, MFMA)", "kernel_us": round(us, 2),
                        "bound": "mfma", "TFLOPs": tflops, "peak_TFLOPs": peak,
                        "frac_mfma_peak": tflops / peak, "flops": dw.flops, "io_bytes": io,
                        "GBps_io": io / (us * 1e-6) / 1e9})
            log("%-28s %8.1f us  %7.1f TFLOP/s  %.3f of the %s MFMA peak" % (
                "%s/%s" % (name, kind), us, tflops, tflops / peak, kind))
            del d, Y

    # Resize workloads (fp32): at their scales every input element has a
    # non-zero weight, so all of X is compulsory
    for name, rw in W.RESIZE_WORKLOADS.items():
        X = torch.from_numpy(W.make_resize_input(rw)).cuda()
        rank = X.dim()
        axes = list(range(rank - len(rw.scales), rank))
        shape = gsa.resize_output_shape(X.shape, list(rw.scales), None, axes)
        Y = torch.empty(shape, device="cuda")
        scales = rw.full_scales()
        fn = lambda: gsa.resize_to(X, shape, scales, rw.mode, rw.coordinate_transformation_mode,
                                   out=Y)
        fn()
        us, _ = time_kernel(torch, fn, 20, flush)
        warm, _ = time_kernel(torch, fn, 20)
        record(name, name, "gs_resize", us, Y.numel(), X.numel() * 4, X.numel() * 4,
               Y.numel() * 4, warm)
        del X, Y
    return out


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-paths", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 512 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the sampler has no multi-GPU path in this "
              "build (it would shard over images or channels with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import spatial_transformer_grid_amd as gsa

    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    gsa.lib()

    if args.copy_calibration:
        gbps = copy_bandwidth(torch)
        log("copy 512 MiB: %.0f GB/s" % gbps)
        return

    w = W.WORKLOADS["stn2d_batch"]
    log("generating %s inputs" % w.name)
    inp = W.make_inputs(w)
    n, c, h, wd = w.x_shape
    size = (n, c) + w.out_spatial
    X = torch.from_numpy(inp["X"]).cuda()
    theta = torch.from_numpy(inp["theta"]).cuda()
    grid = torch.empty((n,) + w.out_spatial + (2,), device="cuda")
    Y = torch.empty(size, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gsa.affine_grid(theta, size, 0, out=grid)
        if ev is not None:
            ev[1].record()
        gsa.grid_sample(X, grid, "linear", "zeros", 0, out=Y)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    sampler_ms = [e[1].elapsed_time(e[2]) for e in events]
    affine_ms = [e[0].elapsed_time(e[1]) for e in events]
    sampler_us = statistics.mean(sampler_ms) * 1e3
    outputs = w.outputs
    value = args.steps * outputs / elapsed

    g_host = grid.cpu().numpy()
    fp_elems = footprint_elements(g_host, (h, wd), "linear", "zeros", 0)
    x_fp_bytes = fp_elems * c * 4
    algo_bytes = x_fp_bytes + grid.numel() * 4 + outputs * 4
    achieved = algo_bytes / (sampler_us * 1e-6) / 1e9
    traffic = None
    digest = kernel_source_digest()
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_digest") == digest:
            traffic = tr.get("hbm_bytes_per_launch")
    log("step %.1f us (affine %.1f us, sampler %.1f us); sampler %.0f GB/s on %.1f MB" % (
        elapsed / args.steps * 1e6, statistics.mean(affine_ms) * 1e3, sampler_us, achieved,
        algo_bytes / 1e6))

    copy_gbps = copy_bandwidth(torch)
    log("device copy: %.0f GB/s" % copy_gbps)

    paths = None
    if not args.no_paths:
        flush_buf = torch.ones(512 * 1024 * 1024 // 4, device="cuda")
        paths = run_paths(torch, gsa, flush_buf)
        del flush_buf

    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # the CPU-baseline leg is the one place the benchmark runs the oracle

        oracle.build(force=False)
        th_np = inp["theta"]
        times = []
        for rep in range(3):
            a = time.perf_counter()
            G = oracle.affine_grid(th_np, size, 0)
            oracle.grid_sample(inp["X"], G, "linear", "zeros", 0)
            times.append(time.perf_counter() - a)
            log("cpu oracle rep %d: %.2f s" % (rep, times[-1]))
        cpu = {"value": outputs / statistics.median(times), "unit": "output elem/s", "cores": 1,
               "kind": "oracle",
               "sample": "the full stn2d_batch step (AffineGrid + bilinear/zeros GridSample, "
                         "67,108,864 outputs), median of 3 runs, one thread"}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "output elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: X U(-1,1), theta = I + N(0, 0.1^2))",
        "config": {"workload": "stn2d_batch: AffineGrid theta (64,2,3) -> grid (64,128,128,2) -> "
                               "GridSample bilinear, zeros, align_corners=0, X (64,64,128,128) fp32",
                   "global_batch": n, "channels": c, "in_hw": [h, wd],
                   "out_hw": list(w.out_spatial), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gs_grid_sample_2d (bilinear, zeros, fp32)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "x_footprint_fraction": fp_elems / (n * h * wd),
                     "kernel_us": sampler_us,
                     "affine_grid_us": statistics.mean(affine_ms) * 1e3,
                     "copy_GBps": copy_gbps, "kernel_source_digest": digest},
        "cpu_baseline": cpu,
        "paths": paths,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
