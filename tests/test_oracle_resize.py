"""Resize oracle pinned to what the Resize (version 18) page and mathematics fix.

* Resize page, Examples: every printed output except the antialias and
  tf_crop_and_resize ones -- 29 examples covering nearest with its four
  rounding rules, linear, cubic (a = -0.75, and a = -0.5 with
  exclude_outside), the half_pixel, pytorch_half_pixel, align_corners and
  asymmetric coordinate modes, `axes`, and the keep_aspect_ratio_policy
  output extents.
* Closed forms: a resize with every scale 1 is the identity; a constant input
  stays constant; linear interpolation reproduces affine ramps and the cubic
  convolution kernel with a = -0.5 reproduces affine ramps and quadratics
  (Keys 1981, the paper the page cites for cubic_coeff_a); the four
  nearest rounding rules on locations with fractions 0, 1/4, 1/2, 3/4,
  tabulated by hand from their definitions.
* Separability: the N-linear and N-cubic modes are applied axis by axis, so a
  2-D resize equals a resize of H followed by a resize of W.
* torch CPU `interpolate` where it is the same operation (bilinear, bicubic
  a = -0.75, trilinear, half_pixel and align_corners; nearest-exact for
  half_pixel with round_prefer_ceil at integer scales).
* Planted mistakes: one-line edits of oracle/resize.c that the battery above
  must reject.
"""

import itertools
import os

import numpy as np
import pytest

from conftest import ROOT, load_golden

RESIZE = load_golden("resize_examples.json")
PRINT_TOL = 2e-6
SRC = os.path.join(ROOT, "oracle", "resize.c")


def full_scales(ex):
    """Per-axis scales of an example that gives scales (unlisted axes keep 1)."""
    rank = len(ex["data_shape"])
    if ex["scales"] is None:
        return None
    if ex["axes"] is None:
        return list(ex["scales"])
    s = [1.0] * rank
    for a, v in zip(ex["axes"], ex["scales"]):
        s[a] = v
    return s


def example_output(om, ex, lib=None):
    X = np.array(ex["data"], np.float32).reshape(ex["data_shape"])
    shape = om.resize_output_shape(ex["data_shape"], scales=ex["scales"], sizes=ex["sizes"],
                                   axes=ex["axes"],
                                   keep_aspect_ratio_policy=ex["keep_aspect_ratio_policy"]
                                   or "stretch", lib=lib)
    Y = om.resize(X, shape, full_scales(ex), ex["mode"],
                  ex["coordinate_transformation_mode"] or "half_pixel",
                  ex["nearest_mode"] or "round_prefer_floor",
                  ex["cubic_coeff_a"] if ex["cubic_coeff_a"] is not None else -0.75,
                  ex["exclude_outside"], lib=lib)
    return shape, Y


def check_example(om, ex, lib=None):
    """None if the oracle reproduces the example, else a message."""
    shape, Y = example_output(om, ex, lib)
    if ex["results_in"] and tuple(shape[2:]) != tuple(ex["results_in"]):
        return "%s: extents %s, page states %s" % (ex["name"], shape, ex["results_in"])
    ref = np.array(ex["expected"]).reshape(ex["expected_shape"])
    if tuple(shape) != tuple(ref.shape):
        # The upsample not_smaller listing states 8x8 but prints 7 of the 8
        # (identical) rows; compare the rows it prints.
        if ex["name"] != "test_resize_upsample_sizes_nearest_not_smaller":
            return "%s: shape %s, page prints %s" % (ex["name"], shape, ref.shape)
        if shape[3] != ref.shape[3] or shape[2] < ref.shape[2]:
            return "%s: shape %s" % (ex["name"], shape)
        Y = Y[:, :, :ref.shape[2], :]
    err = np.abs(Y - ref) / np.maximum(1.0, np.abs(ref))
    if err.max() > PRINT_TOL:
        return "%s: error %.3g" % (ex["name"], err.max())
    return None


@pytest.mark.parametrize("ex", RESIZE, ids=[e["name"] for e in RESIZE])
def test_resize_page_examples(oracle_mod, ex):
    assert check_example(oracle_mod, ex) is None, ex["citation"]


def test_page_examples_cover_the_attributes():
    got = {(e["mode"], e["coordinate_transformation_mode"] or "half_pixel") for e in RESIZE}
    assert {m for m, _ in got} == {"nearest", "linear", "cubic"}
    assert {c for _, c in got} == {"half_pixel", "pytorch_half_pixel", "align_corners",
                                   "asymmetric"}
    assert {e["nearest_mode"] for e in RESIZE} >= {"floor", "ceil", "round_prefer_ceil"}
    assert {e["keep_aspect_ratio_policy"] for e in RESIZE} >= {"not_larger", "not_smaller"}
    assert any(e["exclude_outside"] for e in RESIZE)
    assert len(RESIZE) == 29


MODES = ["nearest", "linear", "cubic"]
CTMS = ["half_pixel", "pytorch_half_pixel", "align_corners", "asymmetric"]
NEAREST = ["round_prefer_floor", "round_prefer_ceil", "floor", "ceil"]


def identity_ok(om, lib=None):
    rng = np.random.default_rng(11)
    X = rng.uniform(-1, 1, (2, 3, 5, 7)).astype(np.float32)
    for mode, ctm, nm, ex in itertools.product(MODES, CTMS, NEAREST, [0, 1]):
        for scales in ([1.0, 1.0, 1.0, 1.0], None):
            Y = om.resize(X, X.shape, scales, mode, ctm, nm, -0.75, ex, lib=lib)
            if not np.array_equal(Y, X.astype(np.float64)):
                return "identity %s/%s/%s/%d" % (mode, ctm, nm, ex)
    return None


def test_identity(oracle_mod):
    assert identity_ok(oracle_mod) is None


def constant_ok(om, lib=None):
    rng = np.random.default_rng(12)
    X = np.full((1, 2, 6, 5), 0.7, np.float32)
    for mode, ctm, ex in itertools.product(MODES, CTMS, [0, 1]):
        sh, sw = (float(np.float32(v)) for v in rng.uniform(0.3, 3.1, 2))
        shape = (1, 2, int(np.floor(6 * sh)), int(np.floor(5 * sw)))
        Y = om.resize(X, shape, [1.0, 1.0, sh, sw], mode, ctm, "round_prefer_floor", -0.75, ex,
                      lib=lib)
        if Y.size and np.abs(Y - np.float64(np.float32(0.7))).max() > 1e-12:
            return "constant %s/%s/%d" % (mode, ctm, ex)
    return None


def test_constant_input(oracle_mod):
    assert constant_ok(oracle_mod) is None


def asymmetric_positions(n_out, scale):
    # asymmetric: x_original = x_resized / scale (fp32)
    return np.arange(n_out, dtype=np.float32) / np.float32(scale)


def ramps_ok(om, lib=None):
    """Affine ramps through linear; affine ramps and quadratics through cubic
    with a = -0.5 (other values of a reproduce only constants)."""
    n = 12
    j = np.arange(n, dtype=np.float64)
    for scale in (2.5, 0.75, 1.6):
        m = int(np.floor(n * np.float32(scale)))
        p = asymmetric_positions(m, scale).astype(np.float64)
        cases = [("linear", -0.75, 0.5 * j - 1.0, lambda q: 0.5 * q - 1.0, 0.0, n - 1.0),
                 ("cubic", -0.5, 0.25 * j + 2.0, lambda q: 0.25 * q + 2.0, 1.0, n - 2.0),
                 ("cubic", -0.5, (j - 3.0) ** 2, lambda q: (q - 3.0) ** 2, 1.0, n - 2.0)]
        for mode, a, xs, f, lo, hi in cases:
            X = xs.astype(np.float32).reshape(1, 1, 1, n)
            Y = om.resize(X, (1, 1, 1, m), [1.0, 1.0, 1.0, scale], mode, "asymmetric",
                          "round_prefer_floor", a, 0, lib=lib)[0, 0, 0]
            inner = (p >= lo) & (p < hi)
            if np.abs(Y[inner] - f(p[inner])).max() > 1e-9:
                return "ramp %s a=%g scale=%g" % (mode, a, scale)
    return None


def test_ramps_and_quadratics(oracle_mod):
    assert ramps_ok(oracle_mod) is None


# Input index chosen for locations 0, 1/4, ..., 11/4 over 3 input elements
# (asymmetric, scale 4), written out from the rule names: halfway cases go
# down / up; floor; ceil; then clamped to the last element.
NEAREST_TABLE = {
    "round_prefer_floor": [0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 2],
    "round_prefer_ceil": [0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 2, 2],
    "floor": [0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2],
    "ceil": [0, 1, 1, 1, 1, 2, 2, 2, 2, 2, 2, 2],
}


def nearest_ok(om, lib=None):
    X = np.array([10.0, 20.0, 30.0], np.float32).reshape(1, 1, 1, 3)
    for nm, idx in NEAREST_TABLE.items():
        Y = om.resize(X, (1, 1, 1, 12), None, "nearest", "asymmetric", nm, lib=lib)[0, 0, 0]
        if not np.array_equal(Y, X[0, 0, 0, idx].astype(np.float64)):
            return "nearest table " + nm
    return None


def test_nearest_rounding_rules(oracle_mod):
    assert nearest_ok(oracle_mod) is None


def separable_ok(om, lib=None):
    rng = np.random.default_rng(13)
    X = rng.uniform(-1, 1, (1, 2, 5, 6)).astype(np.float32)
    for mode, ctm in itertools.product(MODES, CTMS):
        sh, sw = 1.75, 0.625
        Ho, Wo = int(np.floor(5 * sh)), int(np.floor(6 * sw))
        full = om.resize(X, (1, 2, Ho, Wo), [1, 1, sh, sw], mode, ctm, lib=lib)
        half = om.resize(X, (1, 2, Ho, 6), [1, 1, sh, 1], mode, ctm, lib=lib)
        two = om.resize(half.astype(np.float32), (1, 2, Ho, Wo), [1, 1, 1, sw], mode, ctm, lib=lib)
        if np.abs(full - two).max() > 1e-6:
            return "separability %s/%s" % (mode, ctm)
    return None


def test_separable(oracle_mod):
    assert separable_ok(oracle_mod) is None


def torch_ok(om, lib=None):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(14)
    X = rng.uniform(-1, 1, (2, 3, 7, 9)).astype(np.float32)
    Xt = torch.from_numpy(X).double()
    for (Ho, Wo), (tmode, mode, ac, ctm) in itertools.product(
            [(14, 18), (5, 4), (11, 23)],
            [("bilinear", "linear", False, "half_pixel"), ("bilinear", "linear", True, "align_corners"),
             ("bicubic", "cubic", False, "half_pixel"), ("bicubic", "cubic", True, "align_corners")]):
        ref = F.interpolate(Xt, size=(Ho, Wo), mode=tmode, align_corners=ac).numpy()
        Y = om.resize(X, (2, 3, Ho, Wo), None, mode, ctm, lib=lib)
        if np.abs(Y - ref).max() > 1e-5:
            return "torch %s ac=%s %dx%d" % (tmode, ac, Ho, Wo)
    ref = F.interpolate(Xt, size=(21, 27), mode="nearest-exact").numpy()
    Y = om.resize(X, (2, 3, 21, 27), None, "nearest", "half_pixel", "round_prefer_ceil", lib=lib)
    if not np.array_equal(Y, ref):
        return "torch nearest-exact"
    X3 = rng.uniform(-1, 1, (1, 2, 4, 5, 6)).astype(np.float32)
    for ac, ctm in ((False, "half_pixel"), (True, "align_corners")):
        ref = F.interpolate(torch.from_numpy(X3).double(), size=(7, 3, 9), mode="trilinear",
                            align_corners=ac).numpy()
        Y = om.resize(X3, (1, 2, 7, 3, 9), None, "linear", ctm, lib=lib)
        if np.abs(Y - ref).max() > 1e-5:
            return "torch trilinear ac=%s" % ac
    return None


def test_torch_interpolate_special_cases(oracle_mod):
    assert torch_ok(oracle_mod) is None


def shape_ok(om, lib=None):
    """Output extents written out from the Summary's floor(extent * scale)."""
    f = om.resize_output_shape
    if f((1, 1, 6, 3), scales=[1, 1, 0.75, 1.5], lib=lib) != (1, 1, 4, 4):
        return "output extent floor(4.5)"
    if f((2, 3, 5, 7), scales=[2.0, 0.5], axes=[-1, 2], lib=lib) != (2, 3, 2, 14):
        return "output extent with axes"
    return None


def test_output_shape_rules(oracle_mod):
    assert shape_ok(oracle_mod) is None
    f = oracle_mod.resize_output_shape
    assert f((1, 1, 4, 4), scales=[1, 1, 0.6, 0.6]) == (1, 1, 2, 2)
    assert f((2, 3, 5, 7), scales=[2.0, 0.5], axes=[-1, 2]) == (2, 3, 2, 14)
    assert f((1, 1, 2, 2), sizes=[7, 8], axes=[2, 3], keep_aspect_ratio_policy="not_larger") == \
        (1, 1, 7, 7)
    # round half up: 2 * 0.75 = 1.5 -> 2
    assert f((1, 1, 2, 4), sizes=[1, 3], axes=[2, 3], keep_aspect_ratio_policy="not_smaller") == \
        (1, 1, 2, 3)
    with pytest.raises(ValueError):
        f((1, 1, 2, 2), scales=[1.0, 1.0], axes=[2, 2])
    with pytest.raises(ValueError):
        f((1, 1, 2, 2), scales=[1.0, 0.0], axes=[2, 3])


def resize_pin_battery(om, lib):
    for ex in RESIZE:
        msg = check_example(om, ex, lib)
        if msg:
            return msg
    for check in (shape_ok, identity_ok, constant_ok, ramps_ok, nearest_ok, separable_ok,
                  torch_ok):
        msg = check(om, lib)
        if msg:
            return msg
    return None


RESIZE_MUTANTS = [
    ("half_pixel shift with the wrong sign", "return (xf + 0.5f) / scale - 0.5f;",
     "return (xf + 0.5f) / scale + 0.5f;"),
    ("pytorch_half_pixel without its guard",
     "return length_resized > 1.0f ? (xf + 0.5f) / scale - 0.5f : 0.0f;",
     "return (xf + 0.5f) / scale - 0.5f;"),
    ("align_corners divides by length_resized",
     "xf * (float)(n - 1) / (length_resized - 1.0f)", "xf * (float)(n - 1) / length_resized"),
    ("asymmetric multiplies by the scale", "return xf / scale;", "return xf * scale;"),
    ("length_resized floored", "P->length_resized[a] = (float)in_shape[a] * P->scale[a];",
     "P->length_resized[a] = floorf((float)in_shape[a] * P->scale[a]);"),
    ("scale from sizes inverted",
     "scale[a] = in_shape[a] > 0 ? (float)out_shape[a] / (float)in_shape[a] : 1.0f;",
     "scale[a] = out_shape[a] > 0 ? (float)in_shape[a] / (float)out_shape[a] : 1.0f;"),
    ("round_prefer_floor rounds halfway up", "q = ceilf(p - 0.5f);", "q = floorf(p + 0.5f);"),
    ("round_prefer_ceil rounds halfway down", "q = floorf(p + 0.5f);", "q = ceilf(p - 0.5f);"),
    ("floor mode takes the ceiling", "q = floorf(p);", "q = ceilf(p);"),
    ("edge clamp sends the high side to 0", "return i < 0 ? 0 : (i > n - 1 ? n - 1 : i);",
     "return i < 0 ? 0 : (i > n - 1 ? 0 : i);"),
    ("linear weights swapped", "t->weight[0] = 1.0 - frac;", "t->weight[0] = frac;"),
    ("cubic outer weight at the wrong distance", "t->weight[3] = cubic_kernel(2.0 - frac, a);",
     "t->weight[3] = cubic_kernel(1.0 + frac, a);"),
    ("Keys inner piece with a+2 for a+3", "((a + 2.0) * x - (a + 3.0)) * x * x + 1.0",
     "((a + 2.0) * x - (a + 2.0)) * x * x + 1.0"),
    ("exclude_outside ignored", "if (exclude_outside && (i < 0 || i >= n))",
     "if (0 && (i < 0 || i >= n))"),
    ("exclude_outside not renormalised",
     "t->weight[j] = kept != 0.0 ? t->weight[j] / kept : 0.0;",
     "t->weight[j] = kept != 0.0 ? t->weight[j] : 0.0;"),
    ("output extent rounded instead of floored",
     "out_shape[d] = (int64_t)floor((double)in_shape[d] * (double)scales[i]);",
     "out_shape[d] = (int64_t)floor((double)in_shape[d] * (double)scales[i] + 0.5);"),
    ("aspect-ratio policies swapped", "(policy == RZ_POLICY_NOT_LARGER ? r < s : r > s)",
     "(policy == RZ_POLICY_NOT_LARGER ? r > s : r < s)"),
]


def test_unmodified_oracle_passes_resize_battery(oracle_mod):
    assert resize_pin_battery(oracle_mod, None) is None


@pytest.mark.parametrize("desc,old,new", RESIZE_MUTANTS, ids=[m[0] for m in RESIZE_MUTANTS])
def test_planted_resize_mistake_is_caught(oracle_mod, tmp_path, desc, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + desc
    mutant = tmp_path / "resize_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = oracle_mod.build(resize_src=str(mutant), out=str(tmp_path / "libmutant.so"))
    lib = oracle_mod.load_library(so)
    assert resize_pin_battery(oracle_mod, lib) is not None, "no pin rejects the mutant: " + desc
