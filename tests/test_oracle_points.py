"""The oracle's point-wise entry points and its OpenMP build, against the
full serial oracle.

The full-size GPU checks compare outputs with ``grid_sample_points``,
``resize_points`` and ``deform_conv(..., flat_index=...)``, and the large
ones run on the OpenMP build of the same sources.  Those entry points share
the tap arithmetic of the full functions (pinned by the page examples, the
brute force and the closed forms in the other oracle tests); what is theirs
alone is the flat index -> (image, channel, location) decomposition and, for
the OpenMP build, the split of the output loop over threads.  Both are checked
here on every flat index, on a shuffled subset with repeats, and for a
rejected index:

* every mode x padding x align_corners, ranks 1-4, fp32 and float64 grids,
  fp32 and float64 X (GridSample);
* every mode x coordinate transformation, 1-3 resized axes, scales and sizes
  (Resize);
* ranks 1-3, conv groups, offset groups, mask and bias (DeformConv);
* the OpenMP build bit-identical to the serial build on all of them.
"""

import itertools
import os

import numpy as np
import pytest

from conftest import ROOT

MODES = ["linear", "nearest", "cubic"]
PADS = ["zeros", "border", "reflection"]

SAMPLE_SHAPES = {
    1: ((2, 3, 9), (2, 11, 1)),
    2: ((2, 3, 6, 7), (2, 5, 4, 2)),
    3: ((2, 2, 4, 5, 3), (2, 3, 2, 4, 3)),
    4: ((1, 2, 3, 4, 3, 2), (1, 2, 3, 2, 2, 4)),
}


def same(a, b):
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def index_sets(total, seed):
    rng = np.random.default_rng(seed)
    every = np.arange(total, dtype=np.int64)
    shuffled = rng.permutation(total)[: max(1, total // 3)]
    repeats = rng.integers(0, total, size=max(4, total // 5))
    return [every, np.concatenate([shuffled, repeats]).astype(np.int64)]


def sample_inputs(rank, seed, x64, g64):
    rng = np.random.default_rng(seed)
    xs, gs = SAMPLE_SHAPES[rank]
    X = rng.uniform(-1, 1, xs)
    G = rng.uniform(-1.3, 1.3, gs)
    # exact border hits and a non-finite location exercise the special paths
    G.reshape(-1, rank)[0] = 1.0
    G.reshape(-1, rank)[1] = -1.0
    if rank >= 2:
        G.reshape(-1, rank)[2, 0] = np.nan
    return (X if x64 else X.astype(np.float32)), (G if g64 else G.astype(np.float32))


@pytest.mark.parametrize("rank,mode,pad,ac", list(itertools.product(
    [1, 2, 3, 4], MODES, PADS, [0, 1])))
def test_grid_sample_points_match_full(oracle_mod, rank, mode, pad, ac):
    for x64, g64 in ((False, False), (False, True), (True, False), (True, True)):
        X, G = sample_inputs(rank, 7 * rank + ac, x64, g64)
        full = oracle_mod.grid_sample(X, G, mode, pad, ac).reshape(-1)
        for idx in index_sets(full.size, rank + 100 * ac):
            pts = oracle_mod.grid_sample_points(X, G, idx, mode, pad, ac)
            assert same(pts, full[idx]), (rank, mode, pad, ac, x64, g64)


def test_grid_sample_points_reject_bad_index(oracle_mod):
    X, G = sample_inputs(2, 1, False, False)
    total = X.shape[0] * X.shape[1] * G.shape[1] * G.shape[2]
    for bad in (-1, total):
        with pytest.raises(ValueError):
            oracle_mod.grid_sample_points(X, G, np.array([0, bad]), "linear", "zeros", 0)


RESIZE_CASES = [
    # (x shape, output shape, scales or None)
    ((2, 3, 11), (2, 3, 17), (1.0, 1.0, 17 / 11)),
    ((2, 3, 11), (2, 3, 5), None),
    ((2, 7, 9), (2, 14, 18), (1.0, 2.0, 2.0)),
    ((3, 12, 10), (3, 5, 7), None),
    ((1, 5, 4, 6), (1, 9, 7, 11), (1.0, 1.8, 1.75, 1.85)),
    ((2, 6, 5, 4), (2, 3, 3, 2), (1.0, 0.5, 0.6, 0.5)),
]


@pytest.mark.parametrize("case,mode,ct", list(itertools.product(
    range(len(RESIZE_CASES)), ["nearest", "linear", "cubic"],
    ["half_pixel", "pytorch_half_pixel", "align_corners", "asymmetric"])))
def test_resize_points_match_full(oracle_mod, case, mode, ct):
    xs, ys, scales = RESIZE_CASES[case]
    X = np.random.default_rng(case).uniform(-1, 1, xs).astype(np.float32)
    kw = dict(scales=scales, mode=mode, coordinate_transformation_mode=ct)
    for extra in (dict(), dict(nearest_mode="ceil", cubic_coeff_a=-0.5, exclude_outside=1)):
        full = oracle_mod.resize(X, ys, **kw, **extra).reshape(-1)
        for idx in index_sets(full.size, case):
            pts = oracle_mod.resize_points(X, ys, idx, **kw, **extra)
            assert same(pts, full[idx]), (case, mode, ct, extra)
    with pytest.raises(ValueError):
        oracle_mod.resize_points(X, ys, np.array([full.size]), **kw)


DEFORM_CASES = [
    # (x shape, w shape, group, offset group, strides, pads, dilations, mask, bias)
    ((2, 4, 9), (6, 2, 3), 2, 2, [2], [1, 0], [1], True, True),
    ((2, 4, 6, 7), (4, 4, 3, 3), 1, 2, [1, 1], [1, 1, 1, 1], [1, 1], True, False),
    ((1, 6, 7, 5), (9, 2, 2, 3), 3, 1, [2, 1], [0, 1, 1, 0], [1, 2], False, True),
    ((1, 2, 4, 5, 4), (3, 2, 2, 2, 2), 1, 2, [1, 1, 1], [0, 0, 0, 1, 1, 1], [1, 1, 1], True,
     True),
]


def deform_inputs(case, seed):
    xs, ws, group, og, st, pd, dl, has_mask, has_bias = DEFORM_CASES[case]
    r = len(xs) - 2
    rng = np.random.default_rng(seed)
    out_sp = tuple((xs[2 + a] + pd[a] + pd[r + a] - (dl[a] * (ws[2 + a] - 1) + 1)) // st[a] + 1
                   for a in range(r))
    K = int(np.prod(ws[2:]))
    X = rng.uniform(-1, 1, xs)
    W = rng.uniform(-1, 1, ws)
    off = rng.normal(0, 1.5, (xs[0], og * K * r) + out_sp)
    mask = rng.uniform(0, 1, (xs[0], og * K) + out_sp) if has_mask else None
    B = rng.uniform(-1, 1, ws[0]) if has_bias else None
    attrs = dict(strides=st, pads=pd, dilations=dl, group=group, offset_group=og)
    return X, W, off, B, mask, attrs


@pytest.mark.parametrize("case,f32", list(itertools.product(range(len(DEFORM_CASES)),
                                                            [False, True])))
def test_deform_conv_points_match_full(oracle_mod, case, f32):
    X, W, off, B, mask, attrs = deform_inputs(case, case)
    if f32:  # locations in fp32
        X, W, off = (a.astype(np.float32) for a in (X, W, off))
    full = oracle_mod.deform_conv(X, W, off, B, mask, **attrs).reshape(-1)
    for idx in index_sets(full.size, case):
        pts = oracle_mod.deform_conv(X, W, off, B, mask, flat_index=idx, **attrs)
        assert same(pts, full[idx]), (case, f32)
    with pytest.raises(ValueError):
        oracle_mod.deform_conv(X, W, off, B, mask, flat_index=np.array([full.size]), **attrs)


# ------------------------------------------------------- the OpenMP build

def test_parallel_build_uses_threads(oracle_mod):
    assert oracle_mod.threads() == 1
    assert oracle_mod.threads(oracle_mod.parallel()) >= 1


@pytest.mark.parametrize("mode,pad,ac", list(itertools.product(MODES, PADS, [0, 1])))
def test_parallel_grid_sample_identical(oracle_mod, mode, pad, ac):
    par = oracle_mod.parallel()
    rng = np.random.default_rng(3)
    X = rng.uniform(-1, 1, (3, 5, 31, 37)).astype(np.float32)
    G = rng.uniform(-1.2, 1.2, (3, 29, 33, 2)).astype(np.float32)
    ref = oracle_mod.grid_sample(X, G, mode, pad, ac)
    assert same(oracle_mod.grid_sample(X, G, mode, pad, ac, lib=par), ref)
    idx = rng.integers(0, ref.size, 5000)
    assert same(oracle_mod.grid_sample_points(X, G, idx, mode, pad, ac, lib=par),
                ref.reshape(-1)[idx])
    X3 = rng.normal(0, 1, (2, 3, 9, 10, 11))
    G3 = rng.uniform(-1.2, 1.2, (2, 7, 8, 9, 3))
    assert same(oracle_mod.grid_sample(X3, G3, mode, pad, ac, lib=par),
                oracle_mod.grid_sample(X3, G3, mode, pad, ac))


@pytest.mark.parametrize("ac", [0, 1])
def test_parallel_affine_grid_identical(oracle_mod, ac):
    par = oracle_mod.parallel()
    rng = np.random.default_rng(4)
    th2 = rng.normal(0, 1, (5, 2, 3)).astype(np.float32)
    th3 = rng.normal(0, 1, (3, 3, 4))
    for th, size in ((th2, (5, 1, 67, 71)), (th3, (3, 1, 17, 19, 23)),
                     (th3.astype(np.float32), (3, 1, 17, 19, 23))):
        assert same(oracle_mod.affine_grid(th, size, ac, lib=par),
                    oracle_mod.affine_grid(th, size, ac))


@pytest.mark.parametrize("mode", ["nearest", "linear", "cubic"])
def test_parallel_resize_identical(oracle_mod, mode):
    par = oracle_mod.parallel()
    X = np.random.default_rng(5).uniform(-1, 1, (4, 6, 33, 35)).astype(np.float32)
    ys = (4, 6, 66, 70)
    sc = (1.0, 1.0, 2.0, 2.0)
    ref = oracle_mod.resize(X, ys, sc, mode)
    assert same(oracle_mod.resize(X, ys, sc, mode, lib=par), ref)
    idx = np.random.default_rng(6).integers(0, ref.size, 4000)
    assert same(oracle_mod.resize_points(X, ys, idx, sc, mode, lib=par), ref.reshape(-1)[idx])


@pytest.mark.parametrize("case", range(len(DEFORM_CASES)))
def test_parallel_deform_conv_identical(oracle_mod, case):
    par = oracle_mod.parallel()
    X, W, off, B, mask, attrs = deform_inputs(case, 10 + case)
    ref = oracle_mod.deform_conv(X, W, off, B, mask, **attrs)
    assert same(oracle_mod.deform_conv(X, W, off, B, mask, lib=par, **attrs), ref)
    idx = np.arange(ref.size)[::-1].copy()
    assert same(oracle_mod.deform_conv(X, W, off, B, mask, lib=par, flat_index=idx, **attrs),
                ref.reshape(-1)[idx])


# ------------------------------------------- planted mistakes in the indexing

ORACLE_DIR = os.path.join(ROOT, "oracle")

# (file, description, original line, mutated line); every mutant stays inside
# its arrays
POINT_MUTANTS = [
    ("oracle.c", "points: location index shifted by one",
     "int64_t o = f % P.out_count;", "int64_t o = (f + 1) % P.out_count;"),
    ("oracle.c", "points: neighbouring channel",
     "int64_t c = nc % C;", "int64_t c = (nc + 1) % C;"),
    ("resize.c", "points: neighbouring output",
     "Y[i] = rz_value(&P, flat[i]);", "Y[i] = rz_value(&P, (flat[i] + 1) % P.out_count);"),
    ("deform_conv.c", "points: neighbouring output channel",
     "const int64_t oc = (f / P.out_count) % OC;\n        const int64_t n = f / (P.out_count * OC);\n        Y[i]",
     "const int64_t oc = (f / P.out_count + 1) % OC;\n        const int64_t n = f / (P.out_count * OC);\n        Y[i]"),
]


def points_battery(om, lib):
    """Name of the first point-wise check the library fails, or None."""
    for rank, mode in itertools.product([2, 3], ["linear", "nearest"]):
        X, G = sample_inputs(rank, 5, False, False)
        full = om.grid_sample(X, G, mode, "zeros", 0).reshape(-1)
        idx = np.arange(full.size)
        if not same(om.grid_sample_points(X, G, idx, mode, "zeros", 0, lib=lib), full[idx]):
            return "grid_sample_points rank %d %s" % (rank, mode)
    xs, ys, sc = RESIZE_CASES[4]
    X = np.random.default_rng(1).uniform(-1, 1, xs).astype(np.float32)
    full = om.resize(X, ys, sc, "linear").reshape(-1)
    if not same(om.resize_points(X, ys, np.arange(full.size), sc, "linear", lib=lib), full):
        return "resize_points"
    X, W, off, B, mask, attrs = deform_inputs(1, 2)
    full = om.deform_conv(X, W, off, B, mask, **attrs).reshape(-1)
    pts = om.deform_conv(X, W, off, B, mask, flat_index=np.arange(full.size), lib=lib, **attrs)
    if not same(pts, full):
        return "deform_conv points"
    return None


def test_unmodified_oracle_passes_points_battery(oracle_mod):
    assert points_battery(oracle_mod, None) is None


@pytest.mark.parametrize("fname,desc,old,new", POINT_MUTANTS, ids=[m[1] for m in POINT_MUTANTS])
def test_planted_index_mistake_is_caught(oracle_mod, tmp_path, fname, desc, old, new):
    srcs = {f: open(os.path.join(ORACLE_DIR, f)).read()
            for f in ("oracle.c", "resize.c", "deform_conv.c")}
    assert srcs[fname].count(old) == 1, "mutation site not unique: " + old
    srcs[fname] = srcs[fname].replace(old, new)
    paths = {}
    for f, text in srcs.items():
        paths[f] = tmp_path / f
        paths[f].write_text(text)
    so = oracle_mod.build(src=str(paths["oracle.c"]), resize_src=str(paths["resize.c"]),
                          deform_src=str(paths["deform_conv.c"]), out=str(tmp_path / "libm.so"))
    caught = points_battery(oracle_mod, oracle_mod.load_library(so))
    assert caught is not None, "no check rejects the mutant: " + desc
