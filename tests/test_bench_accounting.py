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
