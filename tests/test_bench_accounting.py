"""The benchmark's compulsory-byte accounting counts exactly the input pixels a
launch reads with non-zero weight: checked against the oracle fed one-hot
channels (a pixel is touched iff its one-hot channel gives a non-zero
output somewhere)."""

import itertools
import json
import subprocess
import sys

import numpy as np
import pytest

import bench
from conftest import ROOT

COMBOS = list(itertools.product(["nearest", "linear", "cubic"], ["zeros", "border", "reflection"],
                                [0, 1]))


@pytest.mark.parametrize("mode,pad,ac", COMBOS)
def test_footprint_matches_one_hot_oracle(oracle_mod, mode, pad, ac):
    rng = np.random.default_rng(3 + ac)
    g = rng.uniform(-1.3, 1.3, (2, 7, 9, 2)).astype(np.float32)
    counted = bench.footprint_elements(g, (6, 8), mode, pad, ac)
    touched = 0
    X = np.eye(48, dtype=np.float32).reshape(1, 48, 6, 8)
    for b in range(2):
        Y = oracle_mod.grid_sample(X, g[b:b + 1], mode, pad, ac)
        touched += int((np.abs(Y).reshape(48, -1).max(1) > 0).sum())
    assert counted == touched


def test_footprint_3d(oracle_mod):
    rng = np.random.default_rng(4)
    g = rng.uniform(-1.2, 1.2, (1, 3, 4, 5, 3)).astype(np.float32)
    X = np.eye(120, dtype=np.float32).reshape(1, 120, 4, 5, 6)
    for mode, pad in [("linear", "border"), ("linear", "zeros"), ("nearest", "zeros")]:
        Y = oracle_mod.grid_sample(X, g, mode, pad, 0)
        touched = int((np.abs(Y).reshape(120, -1).max(1) > 0).sum())
        assert bench.footprint_elements(g, (4, 5, 6), mode, pad, 0) == touched


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name", list(__import__("workloads").RESIZE_WORKLOADS))
def test_resize_workloads_read_every_input_element(oracle_mod, name):
    """The benchmark counts all of X as compulsory for the Resize workloads:
    at their scales every input element gets a non-zero weight (checked with
    one-hot inputs on a reduced extent with the same scales)."""
    import workloads as W

    w = W.RESIZE_WORKLOADS[name]
    r = len(w.scales)
    ext = (6,) * r if r == 3 else (10, 12)
    count = int(np.prod(ext))
    X = np.eye(count, dtype=np.float32).reshape((count,) + ext)
    shape = oracle_mod.resize_output_shape((count,) + ext, scales=list(w.scales),
                                           axes=list(range(1, r + 1)))
    Y = oracle_mod.resize(X, shape, [1.0] + list(w.scales), w.mode,
                          w.coordinate_transformation_mode)
    assert (np.abs(Y).reshape(count, -1).max(1) > 0).all()


HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
          '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size",'
          '"VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value",'
          '"Start_Timestamp","End_Timestamp"')


def _write_run(path, pid, rows):
    path.mkdir()
    lines = [HEADER]
    for did, kernel, grid, counter, value in rows:
        lines.append('%d,%d,"Agent 1",1,%d,%d,%d,1,"%s",256,0,0,8,0,32,"%s",%f,1,2' % (
            did, did, pid, pid, grid, kernel, counter, value))
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_counter_summary_joins_runs_and_drops_skipped_launches(tmp_path, monkeypatch):
    """The summary joins the counter runs by dispatch id, scales FETCH_SIZE /
    WRITE_SIZE by the copy calibration, and leaves out launches that moved
    almost nothing (the device chose the other 2-D path)."""
    k = "void gs::grid_sample_kernel<2, 0, 0, gs::F32, false, true>(gs::SampleParams)"
    copy = "__amd_rocclr_copyBuffer"
    _write_run(tmp_path / "f", 1, [(1, k, 1024, "FETCH_SIZE", 100.0), (2, k, 1024, "FETCH_SIZE", 0.01),
                                   (3, k, 1024, "FETCH_SIZE", 120.0)])
    _write_run(tmp_path / "w", 2, [(1, k, 1024, "WRITE_SIZE", 50.0), (2, k, 1024, "WRITE_SIZE", 0.0),
                                   (3, k, 1024, "WRITE_SIZE", 50.0)])
    _write_run(tmp_path / "t", 3, [(d, k, 1024, c, v) for d, c, v in
                                   [(1, "TCC_HIT_sum", 30), (1, "TCC_MISS_sum", 70),
                                    (2, "TCC_HIT_sum", 1), (2, "TCC_MISS_sum", 1),
                                    (3, "TCC_HIT_sum", 50), (3, "TCC_MISS_sum", 50)]])
    _write_run(tmp_path / "cf", 4, [(1, copy, 512, "FETCH_SIZE", 3.0),
                                    (2, copy, 1 << 20, "FETCH_SIZE", 262144.0)])
    _write_run(tmp_path / "cw", 5, [(1, copy, 1 << 20, "WRITE_SIZE", 524288.0)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "COUNTER_FILE", str(tmp_path / "c.json"))
    bench.summarize_counters([str(tmp_path / d) for d in "fwt"],
                             [str(tmp_path / "cf"), str(tmp_path / "cw")], ["cmd"], ["copy cmd"])
    data = json.load(open(tmp_path / "c.json"))
    assert data["fetch_scale"] == 2.0 and data["write_scale"] == 1.0
    (row,) = data["kernels"]
    assert row["kernel"] == "gs::grid_sample_kernel<2, 0, 0, gs::F32, false, true>"
    assert row["dispatches_FETCH_SIZE"] == 2                 # dispatch 2 was skipped
    assert row["hbm_read_bytes"] == 110.0 * 1024 * 2
    assert row["hbm_write_bytes"] == 50.0 * 1024
    assert row["l2_hit_rate"] == 40.0 / 100.0               # medians 40 hits, 60 misses
    assert bench.counter_row(data, row["kernel"]) == row


@pytest.mark.parametrize("kind", ["bf16", "f16"])
def test_deform_bound_accepts_rounding_and_rejects_a_dropped_term(oracle_mod, kind):
    """The bench's DeformConv bound (factors of S and of |ref|): the oracle's
    own output rounded to the element type passes; the output with one input
    channel's nine products dropped fails on most outputs (a single product
    of the 144 is below bf16's resolution of S)."""
    import workloads as W

    dw = W.DEFORM_WORKLOADS["dcn2d_resnet"]
    inp = W.make_deform_inputs(dw, x_shape=(1, 16, 6, 7), w_shape=(8, 16, 3, 3))
    Y = oracle_mod.deform_conv(inp["X"], inp["W"], inp["offset"], inp["B"], inp["mask"],
                               pads=list(dw.pads))
    n, oc, oh, ow = Y.shape
    idx = np.arange(Y.size)
    ref = Y.reshape(-1)
    absn = lambda a: None if a is None else np.abs(a)
    S = oracle_mod.deform_conv(absn(inp["X"]), absn(inp["W"]), inp["offset"], None,
                               absn(inp["mask"]), pads=list(dw.pads)).reshape(-1)
    S = S + np.abs(inp["B"].astype(np.float64))[(idx // (oh * ow)) % oc]
    rel_s, ulp, sub = bench.deform_tolerance(kind, 16 * 9)
    got = W.half_bits_to_f32(W.to_half_bits(ref.astype(np.float32), kind), kind).astype(np.float64)
    assert np.all(np.abs(got - ref) <= rel_s * S + ulp * np.abs(ref) + sub + 1e-30)
    W0 = inp["W"].copy()
    W0[:, 0] = 0  # every tap of input channel 0
    Yd = oracle_mod.deform_conv(inp["X"], W0, inp["offset"], inp["B"], inp["mask"],
                                pads=list(dw.pads)).reshape(-1)
    moved = np.abs(Yd - ref) > rel_s * S + ulp * np.abs(ref) + sub
    assert moved.mean() > 0.75


def test_deform_job_scale_bounds_the_outputs(oracle_mod):
    """S of the bench's DeformConv check (sum of |X|, |W|, |mask| products
    plus |B|) bounds |Y| at every sampled output of the full workload."""
    import workloads as W

    dw = W.DEFORM_WORKLOADS["dcn2d_resnet"]
    inp = W.make_deform_inputs(dw)
    job = bench.deform_job("t", np.zeros(dw.out_shape(), np.float32), dict(inp), dw, "bf16")
    ref = job.ref(None, 0).reshape(-1)
    S = job.scale(None).reshape(-1)
    assert job.k_terms == 256 * 9
    assert np.all(S > 0) and np.all(np.abs(ref) <= S * (1 + 1e-12))
    assert np.median(np.abs(ref) / S) < 0.5


def test_every_bench_path_names_a_profiled_kernel():
    """Each bench path's kernel (and launch size, where given) has a row in
    the stored counter summary, so the bench can attach its traffic and L2
    hit rate (a kernel renamed without re-collecting the counters fails;
    whether the counters match the current sources is the bench's check)."""
    with open(bench.COUNTER_FILE) as f:
        rows = json.load(f)   # names only: the digest of the sources is not checked here
    missing = [p for p, k in bench.PATH_KERNELS.items() if k and not bench.counter_row(rows, *k)]
    assert not missing, missing
    assert bench.counter_row(rows, *bench.HEADLINE_KERNEL)
