#!/usr/bin/env python3
"""Benchmark of the spatial-transformer grid generator + sampler on one MI355X.

One step = the whole hot path over one batch of the 2D STN workload:
theta (64,2,3) -> gs_affine_grid -> grid (64,128,128,2) -> gs_grid_sample_2d
(bilinear, zeros, align_corners=0) on X (64,64,128,128) fp32 -> Y.

Prints ONE JSON line.

* `value`: output elements per second of the whole step (inputs resident in
  HBM, K back-to-back steps between two synchronisations, no event records
  among them; before the W warm-up steps the step runs 400 times untimed,
  about 43 ms, so that the GPU is at its working clock).
* `roofline`: the dominant kernel (the sampler).  Algorithmic bytes per launch
  (distinct X elements the launch reads with a non-zero weight, the grid, and
  Y) divided by its median duration over launches that each follow a pass
  over 512 MiB, which evicts the 256 MB Infinity Cache (events on the launch
  stream); the mean duration of the launches in a second run of the same
  loop with events around each kernel is kept beside it
  (`achieved_in_loop`, `frac_in_loop`).  `traffic` is the HBM byte
  count from rocprofv3 counters (profiles/counters_bench_paths.json) when they
  were taken on the current kernel sources, else null.
* `cpu_baseline`: the oracle (its OpenMP build, every host core) timed on the
  same step; the same leg compares every bench path's output with the oracle
  (`paths[i].max_err`).
* `paths`: the other workload shapes, Resize, the other element types and the
  DeformConv layer (kernel time only, cold and warm), each with the L2 hit
  rate and HBM traffic of its kernel from the stored counters.

`python bench.py --summarize-counters DIR...` turns rocprofv3 output (CSV)
into profiles/counters_bench_paths.json and its Markdown summaries.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "GridSample output elem/s + achieved HBM GB/s (% of MI355X peak), 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")
COUNTER_FILE = os.path.join(PROFILES, "counters_bench_paths.json")
CSRC = os.path.join(ROOT, "spatial_transformer_grid_amd", "csrc")
KERNEL_SOURCES = ["gs_kernels.hip", "gs_gather.hip", "gs_resize.hip", "gs_nd.hip", "gs_deform.hip",
                  "gs_device.hpp", "gs_launch.hpp", "gs_layout.hpp", "gs_api.cpp"]
FLUSH_MIB = 512

# The kernel (as the profiler names it) that dominates each path, and its
# launch size in threads where one kernel runs at two sizes.
HEADLINE_KERNEL = ("gs::grid_sample_kernel<2, 0, 0, gs::F32, false, true>", None)
PATH_KERNELS = {
    "stn2d_batch/linear-zeros": HEADLINE_KERNEL,
    "stn2d_batch/nearest-border": ("gs::grid_sample_kernel<2, 1, 1, gs::F32, false, true>", None),
    "stn2d_batch/linear-zeros-workspace": HEADLINE_KERNEL,
    "stn2d_batch/fused-linear-zeros": ("gs::grid_sample_kernel<2, 0, 0, gs::F32, true, true>", None),
    "flow2d_bicubic/cubic-reflection": ("gs::grid_sample_kernel<2, 2, 2, gs::F32, false, true>",
                                        None),
    "flow2d_bicubic/cubic-reflection-workspace": ("gs::grid_sample_gather<2, 2, gs::F32, 64>",
                                                  None),
    "vol3d/fused-linear-border": ("gs::grid_sample_kernel<3, 0, 1, gs::F32, true, true>", None),
    "vol3d/unfused-linear-border": ("gs::grid_sample_kernel<3, 0, 1, gs::F32, false, true>", None),
    "flow2d_half/bf16-linear-zeros": ("gs::grid_sample_kernel<2, 0, 0, gs::BF16, false, true>",
                                      None),
    "flow2d_half/f16-linear-zeros": ("gs::grid_sample_kernel<2, 0, 0, gs::F16, false, true>", None),
    "stn2d_u8/linear-zeros": ("gs::grid_sample_nd_kernel<2, 0, float, 2>", None),
    "signal1d_f32/linear-zeros": ("gs::grid_sample_nd_kernel<1, 0, float, 4>", None),
    "vol3d_f64/linear-border": ("gs::grid_sample_nd_kernel<3, 0, double, 1>", None),
    "dcn2d_resnet/bf16": ("gs::deform_conv2d_cl<gs::BF16, 1, true, 8>", None),
    "dcn2d_resnet/f32": ("gs::deform_conv2d_cl<gs::F32, 2, true, 4>", None),
    "resize2d_up2_linear": ("gs::resize_kernel<1, gs::F32, true, false>", 1048576),
    "resize2d_up2_nearest": ("gs::resize_kernel<0, gs::F32, true, false>", None),
    "resize2d_up2_cubic": ("gs::resize_kernel<2, gs::F32, true, false>", None),
    "resize2d_down2_linear": ("gs::resize_kernel<1, gs::F32, true, false>", 524288),
    "resize3d_up2_linear": ("gs::resize_kernel<1, gs::F32, true, true>", None),
}


CLOCK_WARMUP_STEPS = 400  # untimed steps before the warm-up steps (clock ramp)


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
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


# ------------------------------------------------------------------ counters

def load_counters():
    """Stored per-kernel counters when they were taken on the current kernel
    sources, else None."""
    if not os.path.exists(COUNTER_FILE):
        return None
    with open(COUNTER_FILE) as f:
        data = json.load(f)
    if data.get("kernel_source_digest") != kernel_source_digest():
        return None
    return data


def counter_row(counters, kernel, grid=None):
    """The stored row of `kernel` (at launch size `grid` when given)."""
    if counters is None:
        return None
    rows = [r for r in counters["kernels"] if r["kernel"] == kernel
            and (grid is None or r["grid"] == grid)]
    if len(rows) != 1:
        return None
    return rows[0]


# ------------------------------------------------------------------- timing

def time_kernel(torch, fn, reps, flush=None, warmup=5):
    """Median and mean duration (us) of fn(), events on the current stream,
    after `warmup` untimed calls (the first calls after host-side work run
    while the GPU's clocks are still ramping up)."""
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
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
    ms = [a.elapsed_time(b) for a, b in ev]
    return statistics.median(ms) * 1e3, statistics.mean(ms) * 1e3


def make_flush(torch):
    """A read-only pass over 512 MiB: evicts the Infinity Cache without
    leaving dirty lines whose write-back would land in the next timed launch."""
    buf = torch.ones(FLUSH_MIB * 1024 * 1024 // 4, device="cuda")
    sink = torch.empty((), device="cuda")

    def flush():
        torch.sum(buf, dim=0, out=sink)

    return flush, buf


def copy_bandwidth(torch, mib=512, reps=10):
    n = mib * 1024 * 1024 // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    med, _ = time_kernel(torch, lambda: dst.copy_(src), reps, warmup=0)
    del src, dst
    return 2 * mib * 1024 * 1024 / (med * 1e-6) / 1e9


# ------------------------------------------------------------------ paths

# Groups of bench paths, one per workload family (bench.py --paths).
PATH_GROUPS = ("stn2d_batch", "flow2d_bicubic", "vol3d", "flow2d_half", "types", "deform",
               "resize")

class ErrJob:
    """A bench path's output kept on the host for the oracle comparison of the
    CPU-baseline leg.  `ref(lib, b)` gives the oracle's float64 values of
    image (or leading slice) b; `images` are the slices compared."""

    def __init__(self, path, got, ref, images, mode, kind, xmax, exact=False):
        self.path, self.got, self.ref, self.images = path, got, ref, images
        self.mode, self.kind, self.xmax, self.exact = mode, kind, xmax, exact


def host_values(torch, Y):
    """Y on the host as float64-convertible values (half types widened)."""
    torch.cuda.synchronize()
    if Y.dtype in (torch.float16, torch.bfloat16):
        return Y.float().cpu().numpy()
    return Y.cpu().numpy()


def run_paths(torch, gsa, flush, counters, only=None):
    """Kernel-only measurements of every workload shape (median of events),
    and the outputs for the oracle comparison.  `only`: the path groups to
    run (PATH_GROUPS), all when None."""
    out, jobs = [], []

    def want(group):
        return only is None or group in only

    def record(name, workload, kernel, us, outputs, x_bytes_full, x_bytes_fp, other_bytes,
               warm_us=None):
        comp = x_bytes_fp + other_bytes
        rec = {"path": name, "workload": workload, "kernel": kernel, "kernel_us": round(us, 2),
               "out_elems_per_s": outputs / (us * 1e-6),
               "compulsory_bytes": comp, "compulsory_bytes_full_x": x_bytes_full + other_bytes,
               "GBps": comp / (us * 1e-6) / 1e9,
               "frac_hbm_peak": comp / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        if warm_us is not None:
            rec["warm_kernel_us"] = round(warm_us, 2)
            rec["warm_GBps"] = comp / (warm_us * 1e-6) / 1e9
        attach_counters(rec, counters)
        out.append(rec)
        log("%-36s %8.1f us  %7.0f GB/s  %.3f of peak" % (name, us, rec["GBps"],
                                                          rec["frac_hbm_peak"]))

    if want("stn2d_batch"):
        # 2D STN batch: bilinear + zeros, nearest + border, fused bilinear
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
        xmax = float(np.abs(inp["X"]).max())
        stn_ref = {}

        def stn_ref_fn(mode, pad, inp=inp, size=size):
            def ref(lib, b):
                import oracle
                key = ("grid", id(lib))
                if key not in stn_ref:
                    stn_ref[key] = oracle.affine_grid(inp["theta"], size, 0, lib=lib)
                return oracle.grid_sample(inp["X"][b:b + 1], stn_ref[key][b:b + 1], mode, pad, 0,
                                          lib=lib)
            return ref

        for mode, pad in (("linear", "zeros"), ("nearest", "border")):
            fp = footprint_elements(g_host, (h, wd), mode, pad, 0) * c * 4
            fn = lambda: gsa.grid_sample(X, grid, mode, pad, 0, out=Y)
            us, _ = time_kernel(torch, fn, 30, flush)
            warm, _ = time_kernel(torch, fn, 30)
            name = "stn2d_batch/%s-%s" % (mode, pad)
            record(name, w.name, "gs_grid_sample_2d", us, outputs, X.numel() * 4, fp,
                   gbytes + outputs * 4, warm)
            fn()
            jobs.append(ErrJob(name, host_values(torch, Y), stn_ref_fn(mode, pad), range(n), mode,
                               "f32", xmax))
        # the same call with a workspace: the probe keeps the staged sampler (the
        # difference is the probe and two launches that return at once)
        ws = torch.empty(gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(grid.shape), 0),
                         dtype=torch.uint8, device="cuda")
        fp = footprint_elements(g_host, (h, wd), "linear", "zeros", 0) * c * 4
        fn = lambda: gsa.grid_sample(X, grid, "linear", "zeros", 0, out=Y, workspace=ws)
        us, _ = time_kernel(torch, fn, 30, flush)
        warm, _ = time_kernel(torch, fn, 30)
        record("stn2d_batch/linear-zeros-workspace", w.name, "gs_grid_sample_2d_ws (staged chosen)",
               us, outputs, X.numel() * 4, fp, gbytes + outputs * 4, warm)
        fn()
        jobs.append(ErrJob("stn2d_batch/linear-zeros-workspace", host_values(torch, Y),
                           stn_ref_fn("linear", "zeros"), range(n), "linear", "f32", xmax))
        del ws
        fn = lambda: gsa.affine_grid_sample_fused(th, X, w.out_spatial, "linear", "zeros", 0, out=Y)
        us, _ = time_kernel(torch, fn, 30, flush)
        warm, _ = time_kernel(torch, fn, 30)
        record("stn2d_batch/fused-linear-zeros", w.name, "gs_affine_grid_sample_fused", us, outputs,
               X.numel() * 4, fp, th.numel() * 4 + outputs * 4, warm)
        fn()
        jobs.append(ErrJob("stn2d_batch/fused-linear-zeros", host_values(torch, Y),
                           stn_ref_fn("linear", "zeros"), range(n), "linear", "f32", xmax))
        del X, Y, grid

    if want("flow2d_bicubic"):
        # 2D random flow, bicubic + reflection
        w = W.WORKLOADS["flow2d_bicubic"]
        inp3 = W.make_inputs(w)
        n, c, h, wd = w.x_shape
        X = torch.from_numpy(inp3["X"]).cuda()
        G = torch.from_numpy(inp3["grid"]).cuda()
        Y = torch.empty((n, c) + w.out_spatial, device="cuda")
        fp = footprint_elements(inp3["grid"], (h, wd), "cubic", "reflection", 1) * c * 4
        fn = lambda: gsa.grid_sample(X, G, "cubic", "reflection", 1, out=Y)
        us, _ = time_kernel(torch, fn, 10, flush)
        record("flow2d_bicubic/cubic-reflection", w.name, "gs_grid_sample_2d", us, w.outputs,
               X.numel() * 4, fp, G.numel() * 4 + w.outputs * 4)

        def flow_ref(lib, b):
            import oracle
            return oracle.grid_sample(inp3["X"][b:b + 1], inp3["grid"][b:b + 1], "cubic",
                                      "reflection", 1, lib=lib)

        fn()
        Yplain = Y.clone()
        jobs.append(ErrJob("flow2d_bicubic/cubic-reflection", host_values(torch, Y), flow_ref,
                           range(n), "cubic", "f32", float(np.abs(inp3["X"]).max())))
        # with a workspace: probe, sliced channels-last copy of X, gather (the
        # whole call is timed, the copy included); same outputs bit for bit
        ws = torch.empty(gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(G.shape), 0),
                         dtype=torch.uint8, device="cuda")
        fn = lambda: gsa.grid_sample(X, G, "cubic", "reflection", 1, out=Y, workspace=ws)
        us, _ = time_kernel(torch, fn, 20, flush)
        record("flow2d_bicubic/cubic-reflection-workspace", w.name,
               "gs_grid_sample_2d_ws (gather path)", us, w.outputs, X.numel() * 4, fp,
               G.numel() * 4 + w.outputs * 4)
        fn()
        torch.cuda.synchronize()
        out[-1]["identical_to_plain_sampler"] = bool(torch.equal(Y, Yplain))
        jobs.append(ErrJob("flow2d_bicubic/cubic-reflection-workspace", host_values(torch, Y),
                           flow_ref, range(n), "cubic", "f32", float(np.abs(inp3["X"]).max())))
        del X, Y, G, ws, Yplain

    if want("vol3d"):
        # 3D volumetric, fused trilinear + border (working set fits the MALL:
        # report the flushed time as the figure and the warm one beside it)
        w = W.WORKLOADS["vol3d"]
        inp4 = W.make_inputs(w)
        n, c = w.x_shape[:2]
        X = torch.from_numpy(inp4["X"]).cuda()
        th = torch.from_numpy(inp4["theta"]).cuda()
        Y = torch.empty((n, c) + w.out_spatial, device="cuda")
        grid = gsa.affine_grid(th, (n, c) + w.out_spatial, 0)
        fp = footprint_elements(grid.cpu().numpy(), w.x_shape[2:], "linear", "border", 0) * c * 4
        vol_size = (n, c) + w.out_spatial

        def vol_ref(lib, b, c=c, out_spatial=w.out_spatial):
            import oracle
            G4 = oracle.affine_grid(inp4["theta"][b:b + 1], (1, c) + out_spatial, 0, lib=lib)
            return oracle.grid_sample(inp4["X"][b:b + 1], G4, "linear", "border", 0, lib=lib)

        xmax = float(np.abs(inp4["X"]).max())
        fn = lambda: gsa.affine_grid_sample_fused(th, X, w.out_spatial, "linear", "border", 0, out=Y)
        us, _ = time_kernel(torch, fn, 20, flush)
        warm, _ = time_kernel(torch, fn, 20)
        record("vol3d/fused-linear-border", w.name, "gs_affine_grid_sample_fused", us, w.outputs,
               X.numel() * 4, fp, th.numel() * 4 + w.outputs * 4, warm)
        fn()
        jobs.append(ErrJob("vol3d/fused-linear-border", host_values(torch, Y), vol_ref, range(n),
                           "linear", "f32", xmax))
        fn = lambda: gsa.grid_sample(X, grid, "linear", "border", 0, out=Y)
        us, _ = time_kernel(torch, fn, 20, flush)
        warm, _ = time_kernel(torch, fn, 20)
        record("vol3d/unfused-linear-border", w.name, "gs_grid_sample_3d", us, w.outputs,
               X.numel() * 4, fp, grid.numel() * 4 + w.outputs * 4, warm)
        fn()
        jobs.append(ErrJob("vol3d/unfused-linear-border", host_values(torch, Y), vol_ref, range(n),
                           "linear", "f32", xmax))
        del X, Y, grid, vol_size

    if want("flow2d_half"):
        # 2D large half precision, smooth flow
        w = W.WORKLOADS["flow2d_half"]
        inp5 = W.make_inputs(w)
        n, c, h, wd = w.x_shape
        G = torch.from_numpy(inp5["grid"]).cuda()
        fp = footprint_elements(inp5["grid"], (h, wd), "linear", "zeros", 0) * c * 2
        for kind, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
            X = torch.from_numpy(inp5["X_bits"][kind].view(np.int16)).cuda().view(tdt)
            Y = torch.empty((n, c) + w.out_spatial, device="cuda", dtype=tdt)
            fn = lambda: gsa.grid_sample(X, G, "linear", "zeros", 0, out=Y)
            us, _ = time_kernel(torch, fn, 20, flush)
            warm, _ = time_kernel(torch, fn, 20)
            name = "flow2d_half/%s-linear-zeros" % kind
            record(name, w.name, "gs_grid_sample_2d", us, w.outputs, X.numel() * 2, fp,
                   G.numel() * 4 + w.outputs * 2, warm)
            fn()
            xh = inp5["X_half_as_f32"][kind]

            def half_ref(lib, b, xh=xh):
                import oracle
                return oracle.grid_sample(xh[b:b + 1], inp5["grid"][b:b + 1], "linear", "zeros", 0,
                                          lib=lib)

            jobs.append(ErrJob(name, host_values(torch, Y), half_ref, range(n), "linear", kind,
                               float(np.abs(xh).max())))
            del X, Y
        del G

    if want("types"):
        # other ranks and element types (the any-rank kernel; bit-exact)
        for name, tw in W.TYPE_WORKLOADS.items():
            inpt = W.make_type_inputs(tw)
            n, c = tw.x_shape[:2]
            X = torch.from_numpy(inpt["X"]).cuda()
            if inpt["theta"] is not None:
                th = torch.from_numpy(inpt["theta"]).cuda()
                G = gsa.affine_grid(th, (n, c) + tw.out_spatial, tw.align_corners)
            else:
                G = torch.from_numpy(inpt["grid"]).cuda()
            Y = torch.empty((n, c) + tw.out_spatial, dtype=X.dtype, device="cuda")
            es = X.element_size()
            fp = footprint_elements(G.cpu().numpy(), tw.x_shape[2:], tw.mode, tw.padding,
                                    tw.align_corners) * c * es
            fn = lambda: gsa.grid_sample(X, G, tw.mode, tw.padding, tw.align_corners, out=Y)
            fn()
            us, _ = time_kernel(torch, fn, 20, flush)
            warm, _ = time_kernel(torch, fn, 20)
            pname = "%s/%s-%s" % (name, tw.mode, tw.padding)
            record(pname, name, "gs_grid_sample (any-rank kernel)", us, tw.outputs, X.numel() * es,
                   fp, G.numel() * G.element_size() + tw.outputs * es, warm)
            fn()

            def type_ref(lib, b, tw=tw, inpt=inpt):
                import oracle
                n_, c_ = inpt["x_shape"][:2]
                if inpt["theta"] is not None:
                    Gr = oracle.affine_grid(inpt["theta"][b:b + 1], (1, c_) + tuple(tw.out_spatial),
                                            tw.align_corners, lib=lib)
                else:
                    Gr = inpt["grid"][b:b + 1]
                v = oracle.grid_sample(inpt["X"][b:b + 1], Gr, tw.mode, tw.padding, tw.align_corners,
                                       lib=lib)
                if inpt["X"].dtype == np.uint8:
                    return oracle.to_integer(v, np.uint8).astype(np.float64)
                if inpt["X"].dtype == np.float32:
                    return v.astype(np.float32).astype(np.float64)
                return v

            jobs.append(ErrJob(pname, host_values(torch, Y), type_ref, range(n), tw.mode, "exact",
                               float(np.abs(inpt["X"].astype(np.float64)).max()), exact=True))
            del X, Y, G, inpt

    if want("deform"):
        # DeformConv layers: matrix-core throughput (flops of the convolution)
        for name, dw in W.DEFORM_WORKLOADS.items():
            inpd = W.make_deform_inputs(dw)
            for kind in dw.dtypes:
                tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[kind]
                d = {k: torch.from_numpy(v).cuda().to(tdt) for k, v in inpd.items()}
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
                io = (inpd["X"].size + inpd["W"].size + inpd["offset"].size + inpd["mask"].size
                      + inpd["B"].size + Y.numel()) * es
                pname = "%s/%s" % (name, kind)
                rec = {"path": pname, "workload": name,
                       "kernel": "gs_deform_conv (implicit GEMM, MFMA)", "kernel_us": round(us, 2),
                       "bound": "mfma", "TFLOPs": tflops, "peak_TFLOPs": peak,
                       "frac_mfma_peak": tflops / peak, "flops": dw.flops, "io_bytes": io,
                       "GBps_io": io / (us * 1e-6) / 1e9}
                attach_counters(rec, counters)
                out.append(rec)
                log("%-36s %8.1f us  %7.1f TFLOP/s  %.3f of the %s MFMA peak" % (
                    pname, us, tflops, tflops / peak, kind))
                fn()
                exact = {k: (v.float().cpu().numpy() if kind != "f32" else inpd[k])
                         for k, v in d.items()}
                jobs.append(deform_job(pname, host_values(torch, Y), exact, dw, kind))
                del d, Y, ws

    if want("resize"):
        # Resize workloads (fp32): at their scales every input element has a
        # non-zero weight, so all of X is compulsory
        for name, rw in W.RESIZE_WORKLOADS.items():
            Xh = W.make_resize_input(rw)
            X = torch.from_numpy(Xh).cuda()
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
            fn()

            def resize_ref(lib, b, Xh=Xh, shape=tuple(shape), rw=rw, scales=scales):
                import oracle
                return oracle.resize(Xh[b:b + 1], (1,) + shape[1:], scales, rw.mode,
                                     rw.coordinate_transformation_mode, lib=lib)

            jobs.append(ErrJob(name, host_values(torch, Y), resize_ref, range(shape[0]), rw.mode,
                               "f32", float(np.abs(Xh).max())))
            del X, Y

    return out, jobs


def deform_job(pname, got, exact, dw, kind):
    """Oracle comparison of a DeformConv path on 32,768 random outputs."""
    n, oc, oh, ow = dw.out_shape()
    idx = np.unique(np.random.default_rng(dw.seed).integers(0, n * oc * oh * ow, 32768))
    flat = got.reshape(-1)[idx][None]

    def ref(lib, b):
        import oracle
        return oracle.deform_conv(exact["X"], exact["W"], exact["offset"], exact["B"],
                                  exact["mask"], pads=list(dw.pads), group=dw.group,
                                  offset_group=dw.offset_group, flat_index=idx, lib=lib)[None]

    def scale(lib):
        # S of each sampled output: the same sum over |X|, |W|, |mask|, plus |B|
        import oracle
        absn = lambda a: None if a is None else np.abs(a)
        s = oracle.deform_conv(absn(exact["X"]), absn(exact["W"]), exact["offset"], None,
                               absn(exact["mask"]), pads=list(dw.pads), group=dw.group,
                               offset_group=dw.offset_group, flat_index=idx, lib=lib)
        if exact["B"] is not None:
            s = s + np.abs(np.asarray(exact["B"], np.float64))[(idx // (oh * ow)) % oc]
        return s[None]

    job = ErrJob(pname, flat, ref, [0], "linear", "deform-" + kind, 1.0)
    job.sample = "32,768 random outputs"
    job.scale = scale
    job.k_terms = int(np.prod(dw.w_shape[1:]))
    return job


def deform_tolerance(kind, k_terms):
    """Bound on |gpu - oracle| of one DeformConv output, as the factors of S
    (the sum of the absolute values of its products and bias) and of |ref|,
    and an absolute floor: each sampled column value is rounded once to the
    element type (half an ulp: 2^-8 relative for bf16, 2^-11 for fp16) before
    the matrix product, K products are accumulated in fp32, and the output
    itself is rounded to the element type; below the smallest normal value
    the spacing is fixed (2^-24 for fp16, 2^-133 for bf16), one spacing of
    which the floor allows for the output (the sampled values' share,
    half a spacing times |W|, is far below it on the bench's layer)."""
    if kind == "f32":
        return 2e-5, 0.0, 0.0
    u = 2.0 ** -11 if kind == "f16" else 2.0 ** -8
    ulp = 2.0 ** -10 if kind == "f16" else 2.0 ** -7
    sub = 2.0 ** -24 if kind == "f16" else 2.0 ** -133
    return u + (k_terms + 8) * 2.0 ** -24, ulp, sub


def attach_counters(rec, counters):
    """L2 hit rate and HBM traffic of the path's kernel from the stored
    counters (null when they were taken on other kernel sources)."""
    key = PATH_KERNELS.get(rec["path"])
    row = counter_row(counters, *key) if key else None
    rec["profiled_kernel"] = key[0] if key else None
    rec["l2_hit_rate"] = row.get("l2_hit_rate") if row else None
    rec["hbm_read_bytes"] = row.get("hbm_read_bytes") if row else None
    rec["hbm_write_bytes"] = row.get("hbm_write_bytes") if row else None


# ----------------------------------------------------- CPU-baseline leg
# The one place the benchmark runs the oracle: it times the oracle on the
# step's workload and compares every path's output with it.

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def tolerance_ok(err, ref, job):
    if job.exact:
        return bool(np.all(err == 0))
    if job.mode == "nearest":
        return bool(np.all(err == 0))
    if job.kind == "f32":
        return bool(err.max(initial=0.0) <= (1e-5 if job.mode == "linear" else 1e-4) * job.xmax)
    return bool(np.all(err <= 2e-2 * np.maximum(np.abs(ref), 1e-3 * job.xmax)))


def cpu_baseline_leg(inp, size, jobs, paths):
    import oracle

    oracle.build(force=False)
    par = oracle.parallel()
    threads = oracle.threads(par)
    times = []
    for rep in range(3):
        a = time.perf_counter()
        G = oracle.affine_grid(inp["theta"], size, 0, lib=par)
        oracle.grid_sample(inp["X"], G, "linear", "zeros", 0, lib=par)
        times.append(time.perf_counter() - a)
        log("cpu oracle (%d threads) rep %d: %.2f s" % (threads, rep, times[-1]))
    outputs = int(np.prod(size))
    # one thread, on the first 8 images (a bounded sample of the same step)
    a = time.perf_counter()
    G8 = oracle.affine_grid(inp["theta"][:8], (8,) + tuple(size[1:]), 0)
    oracle.grid_sample(inp["X"][:8], G8, "linear", "zeros", 0)
    single = 8 * int(np.prod(size[1:])) / (time.perf_counter() - a)
    cpu = {"value": outputs / statistics.median(times), "unit": "output elem/s",
           "cores": threads, "kind": "oracle",
           "sample": "the full stn2d_batch step (AffineGrid + bilinear/zeros GridSample, "
                     "67,108,864 outputs) on the oracle's OpenMP build, median of 3 runs",
           "threads": threads, "host_cpus": len(os.sched_getaffinity(0)),
           "cpu_model": cpu_model(), "single_thread_value": single,
           "single_thread_sample": "the first 8 images of the same step, serial build"}

    by_path = {p["path"]: p for p in paths}
    for job in jobs:
        t0 = time.perf_counter()
        worst, worst_rel, ok = 0.0, 0.0, True
        for b in job.images:
            ref = job.ref(par, b)
            got = np.asarray(job.got[b:b + 1], dtype=np.float64).reshape(ref.shape)
            err = np.abs(got - ref)
            worst = max(worst, float(err.max(initial=0.0)))
            if job.kind in ("f16", "bf16"):
                rel = err / np.maximum(np.abs(ref), 1e-3 * job.xmax)
                worst_rel = max(worst_rel, float(rel.max(initial=0.0)))
            if job.kind.startswith("deform"):
                rel_s, ulp, sub = deform_tolerance(job.kind[len("deform-"):], job.k_terms)
                S = job.scale(par).reshape(ref.shape)
                r = bool(np.all(err <= rel_s * S + ulp * np.abs(ref) + sub + 1e-30))
            else:
                r = tolerance_ok(err, ref, job)
            ok = ok and (r is None or r)
        rec = by_path.get(job.path)
        if rec is not None:
            rec["max_err"] = {"max_abs_err": worst, "max_abs_err_over_max_abs_x":
                              worst / max(job.xmax, 1e-30),
                              "within_tolerance": ok,
                              "compared": getattr(job, "sample", "every output")}
            if job.kind in ("f16", "bf16"):
                rec["max_err"]["max_rel_err"] = worst_rel
        log("oracle check %-36s max err %.3g (%.1f s)" % (job.path, worst,
                                                         time.perf_counter() - t0))
        job.got = None
    return cpu


# ----------------------------------------------------- counter summaries

def _read_csvs(dirs, suffix):
    rows = []
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
            with open(path, newline="") as f:
                rows.extend(csv.DictReader(f))
    return rows


def _short_name(name: str) -> str:
    """Kernel name without 'void ' and its argument list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def _dispatch_counters(rows):
    """{dispatch id: (kernel, grid, {counter: value})} from rocprofv3's
    counter-collection rows."""
    out = {}
    for r in rows:
        key = (r.get("Process_Id", ""), r["Dispatch_Id"])
        if key not in out:
            out[key] = (_short_name(r["Kernel_Name"]), int(r["Grid_Size"]), {})
        name = r["Counter_Name"]
        out[key][2][name] = out[key][2].get(name, 0.0) + float(r["Counter_Value"])
    return out


def summarize_counters(run_dirs, copy_dirs, command, copy_command):
    """Write profiles/counters_bench_paths.json (and .md): per kernel and
    launch size, the median per dispatch of FETCH_SIZE, WRITE_SIZE (KiB),
    TCC_HIT and TCC_MISS; FETCH/WRITE scaled by the factors that make the same
    counters read 512 MiB for a plain 512 MiB device copy."""
    copy = _dispatch_counters(_read_csvs(copy_dirs, "counter_collection.csv"))
    # the 512 MiB copies are the largest copy dispatches of those runs
    big = max((v[1] for v in copy.values() if "copy" in v[0].lower()), default=0)
    sel = [v[2] for v in copy.values() if "copy" in v[0].lower() and v[1] == big]
    cf = [d["FETCH_SIZE"] for d in sel if "FETCH_SIZE" in d]
    cw = [d["WRITE_SIZE"] for d in sel if "WRITE_SIZE" in d]
    copy_kib = 512 * 1024
    fetch_scale = copy_kib / statistics.median(cf) if cf else None
    write_scale = copy_kib / statistics.median(cw) if cw else None
    # the bench launches the same kernels in the same order in every run, so
    # a dispatch id names the same launch in each counter run: join them
    merged = {}
    for d in run_dirs:
        for (_, did), (kernel, grid, vals) in _dispatch_counters(
                _read_csvs([d], "counter_collection.csv")).items():
            k0, g0, v0 = merged.setdefault(did, (kernel, grid, {}))
            if (k0, g0) != (kernel, grid):
                raise ValueError("dispatch %s is %s in one run and %s in another: the runs "
                                 "did not launch the same sequence" % (did, k0, kernel))
            v0.update(vals)
    groups = {}
    for kernel, grid, vals in merged.values():
        if not kernel.startswith("gs::"):
            continue
        groups.setdefault((kernel, grid), []).append(vals)
    # launches that return at once because the device chose the other 2-D
    # path (staged sampler or gather) move almost nothing: left out
    for key, lst in groups.items():
        moved = [d.get("FETCH_SIZE", 0.0) + d.get("WRITE_SIZE", 0.0) for d in lst]
        top = max(moved) if moved else 0.0
        active = [d for d, m in zip(lst, moved) if m >= 0.01 * top]
        groups[key] = active if active else lst
    kernels = []
    for (kernel, grid), lst in sorted(groups.items()):
        row = {"kernel": kernel, "grid": grid}
        for cname in ("FETCH_SIZE", "WRITE_SIZE", "TCC_HIT_sum", "TCC_MISS_sum"):
            v = [d[cname] for d in lst if cname in d]
            if v:
                row[cname] = statistics.median(v)
                row["dispatches_" + cname] = len(v)
        if "FETCH_SIZE" in row and fetch_scale:
            row["hbm_read_bytes"] = row["FETCH_SIZE"] * 1024 * fetch_scale
        if "WRITE_SIZE" in row and write_scale:
            row["hbm_write_bytes"] = row["WRITE_SIZE"] * 1024 * write_scale
        if "TCC_HIT_sum" in row and "TCC_MISS_sum" in row:
            tot = row["TCC_HIT_sum"] + row["TCC_MISS_sum"]
            row["l2_hit_rate"] = row["TCC_HIT_sum"] / tot if tot else None
        kernels.append(row)
    data = {"kernel_source_digest": kernel_source_digest(), "command": command,
            "copy_command": copy_command, "copy_kib": copy_kib,
            "copy_fetch_size_kib": statistics.median(cf) if cf else None,
            "copy_write_size_kib": statistics.median(cw) if cw else None,
            "fetch_scale": fetch_scale, "write_scale": write_scale, "kernels": kernels}
    with open(COUNTER_FILE, "w") as f:
        json.dump(data, f, indent=1)
    lines = ["# HBM traffic and L2 hit rate per dispatch of every bench kernel", "",
             "Commands (repository root, MI355X), one counter set per run:", ""]
    for c in command:
        lines.append("    " + c)
    for c in copy_command:
        lines.append("    " + c)
    lines += ["",
              "Median per dispatch of each (kernel, launch size in threads).  FETCH_SIZE is "
              "scaled by %.3f and WRITE_SIZE by %.3f, the factors that make each read 512 MiB "
              "for a plain 512 MiB device copy.  L2 hit rate = TCC_HIT / (TCC_HIT + TCC_MISS).  "
              "Kernel source digest %s." % (fetch_scale or float("nan"), write_scale or
                                           float("nan"), data["kernel_source_digest"]), "",
              "| kernel | grid (threads) | dispatches | HBM read MB | HBM write MB | L2 hit rate |",
              "|---|---|---|---|---|---|"]
    for r in sorted(kernels, key=lambda r: -(r.get("hbm_read_bytes") or 0)):
        lines.append("| `%s` | %d | %d | %s | %s | %s |" % (
            r["kernel"], r["grid"], max(v for k, v in r.items() if k.startswith("dispatches_")),
            "%.1f" % (r["hbm_read_bytes"] / 1e6) if "hbm_read_bytes" in r else "-",
            "%.1f" % (r["hbm_write_bytes"] / 1e6) if "hbm_write_bytes" in r else "-",
            "%.3f" % r["l2_hit_rate"] if r.get("l2_hit_rate") is not None else "-"))
    with open(os.path.join(PROFILES, "counters_bench_paths.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote %s (%d kernels)" % (COUNTER_FILE, len(kernels)))


def summarize_stats(stats_dirs, command, out_name):
    """Markdown table of rocprofv3 --kernel-trace --stats output."""
    rows = _read_csvs(stats_dirs, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel statistics", "", "Command (repository root, MI355X):", "",
             "    " + command, "", "Kernel source digest %s." % kernel_source_digest(), "",
             "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    rows = sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        lines.append("| `%s` | %s | %.1f | %.1f | %.1f |" % (
            _short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote profiles/%s (%d kernels)" % (out_name, len(rows)))


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-paths", action="store_true", help="skip the other workload shapes")
    ap.add_argument("--paths", nargs="+", choices=PATH_GROUPS, metavar="GROUP",
                    help="run only these path groups (%s)" % ", ".join(PATH_GROUPS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 512 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="rocprofv3 --pmc output directories of bench runs: write "
                         "profiles/counters_bench_paths.json (no GPU needed)")
    ap.add_argument("--copy-dirs", nargs="+", default=[], metavar="DIR",
                    help="with --summarize-counters: the copy-calibration runs")
    ap.add_argument("--commands", nargs="+", default=[], help="commands to cite in summaries")
    ap.add_argument("--summarize-stats", nargs="+", metavar="DIR",
                    help="rocprofv3 --kernel-trace --stats output directories")
    ap.add_argument("--stats-name", default="kernel_stats_bench.md")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.copy_dirs,
                           [c for c in args.commands if "copy-calibration" not in c],
                           [c for c in args.commands if "copy-calibration" in c])
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, " ".join(args.commands), args.stats_name)
        return

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

    # the GPU settles at its working clock only after some tens of
    # milliseconds of work (a loop started from idle ran 113-115 us per step,
    # 106-107 after 20 ms of steps): run 400 steps (about 43 ms) first,
    # untimed; a fixed count keeps the launch sequence the same from run to
    # run, which the counter summaries rely on
    for _ in range(CLOCK_WARMUP_STEPS):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    # the timed steps carry no event records: a record between two launches
    # holds the second back by a few microseconds (118-128 against 107-108
    # us per step measured on stn2d_batch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    # the same loop again with events around each kernel: the in-loop
    # duration of each (event overhead included)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    sampler_ms = [e[1].elapsed_time(e[2]) for e in events]
    affine_ms = [e[0].elapsed_time(e[1]) for e in events]
    in_loop_us = statistics.mean(sampler_ms) * 1e3
    outputs = w.outputs
    value = args.steps * outputs / elapsed

    # the sampler alone, each launch after a pass that evicts the Infinity
    # Cache: the median is the roofline figure
    flush, flush_buf = make_flush(torch)
    sample = lambda: gsa.grid_sample(X, grid, "linear", "zeros", 0, out=Y)
    flushed_us, _ = time_kernel(torch, sample, 30, flush)

    g_host = grid.cpu().numpy()
    fp_elems = footprint_elements(g_host, (h, wd), "linear", "zeros", 0)
    x_fp_bytes = fp_elems * c * 4
    algo_bytes = x_fp_bytes + grid.numel() * 4 + outputs * 4
    achieved = algo_bytes / (flushed_us * 1e-6) / 1e9
    achieved_in_loop = algo_bytes / (in_loop_us * 1e-6) / 1e9
    counters = load_counters()
    row = counter_row(counters, *HEADLINE_KERNEL)
    traffic = None
    if row and "hbm_read_bytes" in row and "hbm_write_bytes" in row:
        traffic = row["hbm_read_bytes"] + row["hbm_write_bytes"]
    log("step %.1f us (affine %.1f us, sampler %.1f us in the loop, %.1f us flushed median); "
        "%.0f GB/s on %.1f MB" % (elapsed / args.steps * 1e6, statistics.mean(affine_ms) * 1e3,
                                  in_loop_us, flushed_us, achieved, algo_bytes / 1e6))

    copy_gbps = copy_bandwidth(torch)
    log("device copy: %.0f GB/s" % copy_gbps)

    paths, jobs = None, []
    if not args.no_paths:
        paths, jobs = run_paths(torch, gsa, flush, counters, args.paths)
    del flush_buf

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_leg(inp, size, jobs, paths or [])

    digest = kernel_source_digest()
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
                     "timing": "median of 30 launches after 5 warm-up launches, each after a "
                               "read pass over 512 MiB (Infinity Cache evicted); events on the "
                               "launch stream",
                     "kernel_us": flushed_us,
                     "achieved_in_loop": achieved_in_loop,
                     "frac_in_loop": achieved_in_loop / HBM_PEAK_GBPS,
                     "kernel_us_in_loop": in_loop_us,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "x_footprint_fraction": fp_elems / (n * h * wd),
                     "l2_hit_rate": row.get("l2_hit_rate") if row else None,
                     "affine_grid_us": statistics.mean(affine_ms) * 1e3,
                     "copy_GBps": copy_gbps, "kernel_source_digest": digest},
        "cpu_baseline": cpu,
        "paths": paths,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
