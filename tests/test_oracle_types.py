"""The oracle on the element types the GridSample page allows beyond fp32.

* double X and double grid (the grid's coordinate steps then run in float64):
  the printed GridSample examples still hold to their printed precision;
* fp16 grid: widened exactly to fp32, so it equals the fp32 oracle on the
  same values;
* integer X (GridSample page, Outputs: interpolation in floating point, the
  result converted to the integer type): hand-worked values of the cast -- truncation
  toward zero, saturation at the type's range -- including a cubic overshoot
  worked out from Keys' weights by hand, and nearest copying integers exactly.
"""

import numpy as np
import pytest

from conftest import load_golden

SAMPLE = load_golden("grid_sample_examples.json")
PRINT_TOL = 2e-6


@pytest.mark.parametrize("ex", SAMPLE, ids=[e["name"] for e in SAMPLE])
def test_page_examples_in_double(oracle_mod, ex):
    X = np.array(ex["X"], np.float64).reshape(ex["X_shape"])
    G = np.array(ex["grid"], np.float64).reshape(ex["grid_shape"])
    Y = oracle_mod.grid_sample(X, G, ex["mode"] or "linear", ex["padding_mode"] or "zeros",
                               ex["align_corners"] or 0)
    ref = np.array(ex["Y"]).reshape(ex["Y_shape"])
    assert (np.abs(Y - ref) / np.maximum(1, np.abs(ref))).max() <= PRINT_TOL


def test_half_grid_is_widened_to_fp32(oracle_mod):
    rng = np.random.default_rng(3)
    X = rng.uniform(-1, 1, (2, 3, 6, 7)).astype(np.float32)
    G16 = rng.uniform(-1.2, 1.2, (2, 4, 5, 2)).astype(np.float16)
    for mode in ("nearest", "linear", "cubic"):
        a = oracle_mod.grid_sample(X, G16, mode, "reflection", 0)
        b = oracle_mod.grid_sample(X, G16.astype(np.float32), mode, "reflection", 0)
        assert np.array_equal(a, b)


def test_integer_cast_truncates_and_saturates(oracle_mod):
    to_int = oracle_mod.to_integer
    assert to_int(np.array([127.5, -127.5, 0.999, -0.999]), np.int16).tolist() == [127, -127, 0, 0]
    assert to_int(np.array([300.0, -300.0]), np.int8).tolist() == [127, -128]
    assert to_int(np.array([-5.0, 256.0, 255.9]), np.uint8).tolist() == [0, 255, 255]
    assert to_int(np.array([np.nan]), np.int32).tolist() == [0]


def test_uint8_midpoint(oracle_mod):
    # two pixels 0 and 255, align_corners=1, location 0 -> pixel coordinate
    # 0.5: 127.5 before the cast, 127 after it
    X = np.array([[[[0, 255]]]], np.uint8)
    G = np.array([[[[0.0, 0.0]]]], np.float32)
    Y = oracle_mod.grid_sample(X, G, "linear", "border", 1)
    assert Y[0, 0, 0, 0] == 127.5
    assert oracle_mod.to_integer(Y, np.uint8)[0, 0, 0, 0] == 127


def test_int8_cubic_overshoot_saturates(oracle_mod):
    # row -128 -128 127 127 127, align_corners=1, x = 0.125 -> p = 2.25:
    # taps 1..4 with Keys (a = -0.75) weights at t = 0.25:
    #   k(1.25) = -0.10546875, k(0.25) = 0.87890625,
    #   k(0.75) = 0.26171875,  k(1.75) = -0.03515625
    # value = 128 * 0.10546875 + 127 * (0.87890625 + 0.26171875 - 0.03515625)
    #       = 13.5 + 140.39453125 = 153.89453125 -> 127 after the cast
    X = np.array([-128, -128, 127, 127, 127], np.int8).reshape(1, 1, 1, 5)
    G = np.array([0.125, 0.0], np.float32).reshape(1, 1, 1, 2)
    Y = oracle_mod.grid_sample(X, G, "cubic", "border", 1)
    assert Y[0, 0, 0, 0] == 153.89453125
    assert oracle_mod.to_integer(Y, np.int8)[0, 0, 0, 0] == 127


def test_nearest_copies_large_integers(oracle_mod):
    # int32 values far beyond fp32's 24-bit mantissa survive exactly (float64
    # intermediates hold every int32)
    X = np.array([2**31 - 1, -2**31, 123456789], np.int32).reshape(1, 1, 1, 3)
    G = np.array([[-1.0, 0.0], [0.0, 0.0], [1.0, 0.0]], np.float32).reshape(1, 1, 3, 2)
    Y = oracle_mod.grid_sample(X, G, "nearest", "zeros", 1)
    assert oracle_mod.to_integer(Y, np.int32).reshape(-1).tolist() == [2**31 - 1, -2**31,
                                                                      123456789]


AFFINE = load_golden("affine_grid_examples.json")


@pytest.mark.parametrize("ex", AFFINE, ids=[e["name"] for e in AFFINE])
def test_affine_grid_examples_in_double(oracle_mod, ex):
    theta = np.array(ex["theta"], np.float64).reshape(ex["theta_shape"])
    g = oracle_mod.affine_grid(theta, ex["size"], ex["align_corners"])
    assert g.dtype == np.float64
    ref = np.array(ex["grid"]).reshape(ex["grid_shape"])
    assert (np.abs(g - ref) / np.maximum(1, np.abs(ref))).max() <= PRINT_TOL


@pytest.mark.parametrize("ac", [0, 1])
def test_affine_grid_double_is_a_linear_map_of_linspace(oracle_mod, ac):
    """Closed form in float64: positions are numpy.linspace over [-1, 1]
    (corner centres, ac=1) or its pixel centres (ac=0), mapped by theta."""
    rng = np.random.default_rng(9)
    theta = rng.normal(0, 1, (2, 3, 4))
    D, H, W = 3, 4, 5
    g = oracle_mod.affine_grid(theta, (2, 1, D, H, W), ac)

    def pos(m):
        if ac:
            return np.linspace(-1, 1, m) if m > 1 else np.zeros(1)
        return (2 * np.arange(m) + 1) / m - 1

    z, y, x = np.meshgrid(pos(D), pos(H), pos(W), indexing="ij")
    hom = np.stack([x, y, z, np.ones_like(x)], -1)
    ref = np.einsum("dhwj,nkj->ndhwk", hom, theta)
    assert np.abs(g - ref).max() <= 1e-14
