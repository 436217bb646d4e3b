"""The oracle's pins catch plausible mistakes planted in a copy of the oracle.

Each mutant is a one-line edit of oracle/oracle.c (an index off by one, a
dropped term, a swapped sign or operand, a wrong constant or rounding rule),
compiled on the CPU into a temporary library.  Where the same line appears in
the fp32-coordinate and the float64-coordinate paths, the first one (fp32) is
mutated; the DOUBLE_MUTANTS hit the float64 path, which the battery also
exercises with double grids.  The pin battery below — the
pages' printed examples, the Resize cross-checks, the dense-lattice brute
force and the reflection symmetry — must reject every mutant while accepting
the unmodified oracle.  Mutants are chosen so that none reads outside its
input arrays.
"""

import itertools
import os

import numpy as np
import pytest

from conftest import ROOT, load_golden
from test_oracle_bruteforce import brute_force
from test_oracle_pages import RESIZE_SAMPLING, resize_as_sampling_grid

SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("pixel-centre position off by half a pixel",
     "return (float)(2 * i + 1) / (float)m - 1.0f;", "return (float)(2 * i) / (float)m - 1.0f;"),
    ("corner-aligned spacing uses m instead of m-1",
     "return (float)(2 * i) / (float)(m - 1) - 1.0f;", "return (float)(2 * i) / (float)m - 1.0f;"),
    ("translation column dropped", "s = s + row[r];", "s = s + 0.0f * row[r];"),
    ("position vector in outermost-first order", "float prod = row[j] * b[j];",
     "float prod = row[j] * b[r - 1 - j];"),
    ("align_corners=1 scale uses n", "return u * (float)(n - 1);", "return u * (float)n;"),
    ("align_corners=0 shift has wrong sign", "return (v - 1.0f) / 2.0f;", "return (v + 1.0f) / 2.0f;"),
    ("reflection branches swapped", "return odd ? hi - e : lo + e;", "return odd ? lo + e : hi - e;"),
    ("reflection bound at the pixel centre for align_corners=0", "*lo = -0.5f;", "*lo = 0.0f;"),
    ("nearest rounds half away from zero", "return (int64_t)rintf(p);", "return (int64_t)roundf(p);"),
    ("linear second tap repeats the first", "t->index[1] = i0 + 1;", "t->index[1] = i0;"),
    ("linear weights swapped", "t->weight[0] = 1.0 - frac;", "t->weight[0] = frac;"),
    ("cubic coefficient -0.5", "#define OR_CUBIC_A (-0.75)", "#define OR_CUBIC_A (-0.5)"),
    ("cubic outer weight evaluated at the wrong distance",
     "t->weight[3] = keys_kernel(2.0 - frac, OR_CUBIC_A);",
     "t->weight[3] = keys_kernel(1.0 + frac, OR_CUBIC_A);"),
    ("Keys inner piece with a+2 for a+3", "((a + 2.0) * x - (a + 3.0)) * x * x + 1.0",
     "((a + 2.0) * x - (a + 2.0)) * x * x + 1.0"),
    ("cubic zeros padding drops the first pixel", "t->valid[j] = (i >= 0 && i < n);",
     "t->valid[j] = (i > 0 && i < n);"),
    ("cubic border clamps to n-2", "t->index[j] = i < 0 ? 0 : (i > n - 1 ? n - 1 : i);",
     "t->index[j] = i < 0 ? 0 : (i > n - 2 ? (n > 1 ? n - 2 : 0) : i);"),
    ("location vector read outermost first", "(n * P->out_count + o) * P->r + (P->r - 1 - a);",
     "(n * P->out_count + o) * P->r + a;"),
    ("reflection result not clamped back into the image",
     "return clampf(reflect(p, lo, hi), 0.0f, (float)(n - 1));", "return reflect(p, lo, hi);"),
    ("border clamp at n instead of n-1", "return clampf(p, 0.0f, (float)(n - 1));",
     "return clampf(p, 0.0f, (float)n - 0.5f);"),
]


DOUBLE_MUTANTS = [
    ("double theta: pixel-centre position off by half a pixel",
     "return (double)(2 * i + 1) / (double)m - 1.0;", "return (double)(2 * i) / (double)m - 1.0;"),
    ("double theta: translation column dropped", "s = s + row[r];", "s = s + 0.0 * row[r];"),
    ("double grid: align_corners=0 shift with the wrong sign", "return (v - 1.0) / 2.0;",
     "return (v + 1.0) / 2.0;"),
    ("double grid: reflection bound at the pixel centre", "*lo = -0.5;", "*lo = 0.0;"),
    ("double grid: nearest rounds half away from zero", "int64_t i = (int64_t)rint(q);",
     "int64_t i = (int64_t)round(q);"),
    ("double grid: linear second tap repeats the first", "t->index[1] = i0 + 1;",
     "t->index[1] = i0;"),
    ("double grid: cubic outer weight at the wrong distance",
     "t->weight[3] = keys_kernel(2.0 - frac, OR_CUBIC_A);",
     "t->weight[3] = keys_kernel(1.0 + frac, OR_CUBIC_A);"),
    ("double grid: border clamp at n", "return clamp_d(p, 0.0, (double)(n - 1));",
     "return clamp_d(p, 0.0, (double)n - 0.5);"),
]


def pin_battery(om, lib):
    """Return the name of the first pin that fails, or None."""
    for ex in load_golden("affine_grid_examples.json"):
        th = np.array(ex["theta"], np.float32).reshape(ex["theta_shape"])
        g = om.affine_grid(th, ex["size"], ex["align_corners"], lib=lib)
        ref = np.array(ex["grid"]).reshape(ex["grid_shape"])
        if (np.abs(g - ref) / np.maximum(1, np.abs(ref))).max() > 2e-6:
            return ex["name"]
    for ex in load_golden("grid_sample_examples.json"):
        X = np.array(ex["X"], np.float32).reshape(ex["X_shape"])
        G = np.array(ex["grid"], np.float32).reshape(ex["grid_shape"])
        Y = om.grid_sample(X, G, ex["mode"] or "linear", ex["padding_mode"] or "zeros",
                           ex["align_corners"] or 0, lib=lib)
        ref = np.array(ex["Y"]).reshape(ex["Y_shape"])
        if (np.abs(Y - ref) / np.maximum(1, np.abs(ref))).max() > 2e-6:
            return ex["name"]
    for ex in RESIZE_SAMPLING:
        data, G = resize_as_sampling_grid(ex)
        Y = om.grid_sample(data, G, ex["mode"], "border", 0, lib=lib)
        ref = np.array(ex["expected"]).reshape(Y.shape)
        if (np.abs(Y - ref) / np.maximum(1, np.abs(ref))).max() > 2e-6:
            return ex["name"]
    for ex in load_golden("affine_grid_examples.json"):
        th = np.array(ex["theta"], np.float64).reshape(ex["theta_shape"])
        g = om.affine_grid(th, ex["size"], ex["align_corners"], lib=lib)
        ref = np.array(ex["grid"]).reshape(ex["grid_shape"])
        if (np.abs(g - ref) / np.maximum(1, np.abs(ref))).max() > 2e-6:
            return ex["name"] + " (double)"
    for ex in load_golden("grid_sample_examples.json"):
        X = np.array(ex["X"], np.float64).reshape(ex["X_shape"])
        G = np.array(ex["grid"], np.float64).reshape(ex["grid_shape"])
        Y = om.grid_sample(X, G, ex["mode"] or "linear", ex["padding_mode"] or "zeros",
                           ex["align_corners"] or 0, lib=lib)
        ref = np.array(ex["Y"]).reshape(ex["Y_shape"])
        if (np.abs(Y - ref) / np.maximum(1, np.abs(ref))).max() > 2e-6:
            return ex["name"] + " (double)"
    rng = np.random.default_rng(2024)
    for mode, pad, ac in itertools.product(["nearest", "linear", "cubic"],
                                           ["zeros", "border", "reflection"], [0, 1]):
        for rank, dt in ((2, np.float32), (3, np.float32), (1, np.float64), (2, np.float64)):
            in_sp = tuple(int(v) for v in rng.integers(1, 6, size=rank))
            out_sp = (3,) * rank
            X = rng.uniform(-1, 1, (1, 2) + in_sp).astype(dt)
            G = rng.uniform(-1.7, 1.7, (1,) + out_sp + (rank,)).astype(dt)
            if dt == np.float64 and mode == "nearest":
                # exact ties, so the rounding rule matters on the float64 path too
                G[..., 0] = rng.integers(-6, 7, size=G.shape[:-1]) / 4.0
            Y = om.grid_sample(X, G, mode, pad, ac, lib=lib)
            if np.abs(Y - brute_force(X, G, mode, pad, ac)).max() > 1e-12:
                return "brute force %s/%s/%d/%dD %s %s" % (mode, pad, ac, rank, in_sp,
                                                          np.dtype(dt).name)
    for mode, ac in itertools.product(["linear", "cubic"], [0, 1]):
        X = rng.uniform(-1, 1, (1, 1, 5, 7)).astype(np.float32)
        G = (rng.integers(-3072, 3072, (1, 6, 6, 2)) / 1024.0).astype(np.float32)
        Y = om.grid_sample(X, G, mode, "reflection", ac, lib=lib)
        Ym = om.grid_sample(X, (2.0 - G).astype(np.float32), mode, "reflection", ac, lib=lib)
        if np.abs(Y - Ym).max() > 4e-5:
            return "reflection symmetry %s/%d" % (mode, ac)
    return None


def test_unmodified_oracle_passes_battery(oracle_mod):
    assert pin_battery(oracle_mod, None) is None


def mutate(src, old, new, last):
    """Replace the first (fp32 path) or the last (float64 path) occurrence."""
    i = src.rfind(old) if last else src.find(old)
    assert i >= 0, "mutation site not found: " + old
    return src[:i] + new + src[i + len(old):]


@pytest.mark.parametrize("desc,old,new,last",
                         [m + (False,) for m in MUTANTS] + [m + (True,) for m in DOUBLE_MUTANTS],
                         ids=[m[0] for m in MUTANTS + DOUBLE_MUTANTS])
def test_planted_mistake_is_caught(oracle_mod, tmp_path, desc, old, new, last):
    src = open(SRC).read()
    mutant = tmp_path / "mutant.c"
    mutant.write_text(mutate(src, old, new, last))
    so = oracle_mod.build(src=str(mutant), out=str(tmp_path / "libmutant.so"))
    lib = oracle_mod.load_library(so)
    caught = pin_battery(oracle_mod, lib)
    assert caught is not None, "no pin rejects the mutant: " + desc
