"""Oracle pinned to the values the operator pages print.

* AffineGrid page, Examples: the four worked grids (2D and 3D,
  align_corners 0 and 1).
* "GridSample - version 20" page, Examples: all eighteen worked outputs.
* Resize (version 18) page, Examples: the cubic and linear upsample and
  downsample outputs, re-expressed as sampling with padding_mode "border".
  They are the only printed values that fix how cubic treats taps beyond the
  image (each tap is clamped on its own), and they also pin the cubic
  coefficient a = -0.75.

Fixtures live in tests/golden/ (written by extract_from_pages.py).
"""

import numpy as np
import pytest

from conftest import load_golden

AFFINE = load_golden("affine_grid_examples.json")
SAMPLE = load_golden("grid_sample_examples.json")
RESIZE = load_golden("resize_examples.json")

# Printed values carry about 8 significant digits.
PRINT_TOL = 2e-6


@pytest.mark.parametrize("ex", AFFINE, ids=[e["name"] for e in AFFINE])
def test_affine_grid_examples(oracle_mod, ex):
    theta = np.array(ex["theta"], np.float32).reshape(ex["theta_shape"])
    grid = oracle_mod.affine_grid(theta, ex["size"], ex["align_corners"])
    ref = np.array(ex["grid"]).reshape(ex["grid_shape"])
    assert grid.shape == ref.shape
    err = np.abs(grid.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= PRINT_TOL, ex["citation"]


@pytest.mark.parametrize("ex", SAMPLE, ids=[e["name"] for e in SAMPLE])
def test_grid_sample_examples(oracle_mod, ex):
    X = np.array(ex["X"], np.float32).reshape(ex["X_shape"])
    G = np.array(ex["grid"], np.float32).reshape(ex["grid_shape"])
    # Attributes the example does not print take the page's defaults
    # (mode linear, padding zeros) and align_corners 0.
    mode = ex["mode"] or "linear"
    pad = ex["padding_mode"] or "zeros"
    ac = ex["align_corners"] or 0
    Y = oracle_mod.grid_sample(X, G, mode, pad, ac)
    ref = np.array(ex["Y"]).reshape(ex["Y_shape"])
    assert Y.shape == ref.shape
    if mode == "nearest":
        assert np.array_equal(Y.astype(np.float32), ref.astype(np.float32)), ex["citation"]
    else:
        err = np.abs(Y - ref) / np.maximum(1.0, np.abs(ref))
        assert err.max() <= PRINT_TOL, ex["citation"]


def test_examples_cover_every_mode_and_padding():
    modes = {(e["mode"] or "linear") for e in SAMPLE}
    pads = {(e["padding_mode"] or "zeros") for e in SAMPLE}
    assert modes == {"linear", "nearest", "cubic"}
    assert pads == {"zeros", "border", "reflection"}
    assert {e["X_shape"].__len__() for e in SAMPLE} == {4, 5}


def resize_positions(ctm, n_in, n_out, scale):
    """Resize page, coordinate_transformation_mode: output index -> input pixel.

    With a `scales` input the resized length is n_in * scale (unfloored); with
    `sizes` it is n_out.  That reading reproduces every example used here.
    """
    x = np.arange(n_out, dtype=np.float64)
    length_resized = n_in * scale
    if ctm == "half_pixel":
        return (x + 0.5) / scale - 0.5
    if ctm == "asymmetric":
        return x / scale
    if ctm == "align_corners":
        if length_resized <= 1:
            return np.zeros_like(x)
        return x * (n_in - 1) / (length_resized - 1)
    raise ValueError(ctm)


def sampling_compatible(ex):
    """Resize examples that are also border-padded GridSample calls: linear or
    cubic with the GridSample cubic coefficient, no exclude_outside, every
    axis given, and a coordinate mode that is an affine map of the index."""
    return (ex["mode"] in ("linear", "cubic") and ex["cubic_coeff_a"] in (None, -0.75)
            and not ex["exclude_outside"] and ex["axes"] is None
            and (ex["coordinate_transformation_mode"] or "half_pixel")
            in ("half_pixel", "asymmetric", "align_corners"))


RESIZE_SAMPLING = [e for e in RESIZE if sampling_compatible(e)]


def resize_as_sampling_grid(ex):
    data = np.array(ex["data"], np.float32).reshape(ex["data_shape"])
    H, W = data.shape[2:]
    if ex["scales"]:
        sh, sw = ex["scales"][2:]
        Ho, Wo = int(np.floor(H * sh)), int(np.floor(W * sw))
    else:
        Ho, Wo = ex["sizes"][2:]
        sh, sw = Ho / H, Wo / W
    ctm = ex["coordinate_transformation_mode"] or "half_pixel"
    py = resize_positions(ctm, H, Ho, sh)
    px = resize_positions(ctm, W, Wo, sw)
    # pixel position p of an n-pixel axis <-> normalised location (2p+1)/n - 1
    # under align_corners=0 (the pixel-edge convention of the GridSample page)
    G = np.zeros((1, Ho, Wo, 2), np.float32)
    G[0, :, :, 0] = ((2 * px + 1) / W - 1)[None, :]
    G[0, :, :, 1] = ((2 * py + 1) / H - 1)[:, None]
    return data, G


@pytest.mark.parametrize("ex", RESIZE_SAMPLING, ids=[e["name"] for e in RESIZE_SAMPLING])
def test_resize_examples_as_border_sampling(oracle_mod, ex):
    data, G = resize_as_sampling_grid(ex)
    Y = oracle_mod.grid_sample(data, G, ex["mode"], "border", 0)
    ref = np.array(ex["expected"]).reshape(Y.shape)
    err = np.abs(Y - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= PRINT_TOL, ex["citation"]


@pytest.mark.parametrize("ex", [e for e in RESIZE_SAMPLING if e["mode"] == "cubic"],
                         ids=[e["name"] for e in RESIZE_SAMPLING if e["mode"] == "cubic"])
def test_resize_cubic_examples_reject_other_paddings(oracle_mod, ex):
    """The same values are NOT reproduced by zero padding of the taps, so the
    examples really fix the per-tap border rule (reflection coincides with
    border on some of them, hence only zeros is required to differ)."""
    data, G = resize_as_sampling_grid(ex)
    Y = oracle_mod.grid_sample(data, G, "cubic", "zeros", 0)
    ref = np.array(ex["expected"]).reshape(Y.shape)
    assert np.abs(Y - ref).max() > 0.1
