"""Resize on the GPU (gs_resize through the C ABI) against the CPU oracle.

Every printed Resize example, then seeded random inputs over every mode x
coordinate_transformation_mode x element type, with nearest_mode,
exclude_outside and cubic_coeff_a varied, at sizes that span several tiles
with ragged last tiles and plane counts that leave a remainder after the
plane groups: up- and downsampling, mixed scales, extents from sizes, 1-D,
2-D and 3-D resizes, leading axes folded into planes, the identity, strong
downsampling (the direct-gather path) and a non-default stream.
Tolerances: nearest bit-exact; fp32 linear 1e-5 * max|X|, cubic 1e-4 * max|X|;
fp16 / bf16 2e-2 relative and within one output ulp of the rounded oracle.
"""

import itertools

import numpy as np
import pytest

import oracle
from conftest import load_golden
from parity import check, from_gpu, note, torch_mod, x_to_gpu
from test_oracle_resize import example_output

pytestmark = pytest.mark.gpu

RESIZE = load_golden("resize_examples.json")
CTMS = ["half_pixel", "pytorch_half_pixel", "align_corners", "asymmetric"]
NEAREST = ["round_prefer_floor", "round_prefer_ceil", "floor", "ceil"]
KINDS = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()   # raises if the HIP library is not built
    return gsa


@pytest.mark.parametrize("ex", RESIZE, ids=[e["name"] for e in RESIZE])
def test_resize_page_examples(gsa, ex):
    note(ex["name"])
    X = np.array(ex["data"], np.float32).reshape(ex["data_shape"])
    Xg, _ = x_to_gpu(X, "f32")
    Y = from_gpu(gsa.resize(Xg, ex["scales"], ex["sizes"], ex["axes"], ex["mode"],
                            ex["coordinate_transformation_mode"] or "half_pixel",
                            ex["nearest_mode"] or "round_prefer_floor",
                            ex["cubic_coeff_a"] if ex["cubic_coeff_a"] is not None else -0.75,
                            ex["exclude_outside"],
                            ex["keep_aspect_ratio_policy"] or "stretch"))
    shape, ref = example_output(oracle, ex)
    check(Y, ref, ex["mode"], "f32", float(np.abs(X).max()), ex["name"])
    printed = np.array(ex["expected"]).reshape(ex["expected_shape"])
    got = Y[:, :, :printed.shape[2], :]  # one listing prints 7 of its 8 rows
    assert (np.abs(got - printed) / np.maximum(1, np.abs(printed))).max() <= 2e-6


def run_case(gsa, X, y_shape, scales, mode, ctm, nm="round_prefer_floor", a=-0.75, ex=0,
             kind="f32", stream=None):
    what = "%s %s->%s scales=%s %s %s a=%g ex=%d %s" % (mode, X.shape, tuple(y_shape), scales,
                                                         ctm, nm, a, ex, kind)
    note(what)
    Xg, Xw = x_to_gpu(X, kind)
    Y = from_gpu(gsa.resize_to(Xg, y_shape, scales, mode, ctm, nm, a, ex, stream=stream))
    ref = oracle.resize(Xw, y_shape, scales, mode, ctm, nm, a, ex)
    check(Y, ref, mode, kind, float(np.abs(Xw).max()), what)


# (input spatial, output spatial, scales or None) over (N, C) = (2, 3)
PATTERNS_2D = [
    ((37, 53), (74, 106), (2.0, 2.0)),
    ((37, 53), (18, 26), (0.5, 0.5)),
    ((37, 53), (50, 38), (1.37, 0.73)),
    ((37, 53), (41, 29), None),
    ((16, 64), (40, 160), (2.5, 2.5)),     # 16-byte rows (vector staging)
]


def scales4(sc):
    return None if sc is None else [1.0, 1.0, float(np.float32(sc[0])), float(np.float32(sc[1]))]


@pytest.mark.parametrize("kind,pat,ctm,nm", list(itertools.product(
    KINDS, range(len(PATTERNS_2D)), CTMS, NEAREST)))
def test_nearest_2d(gsa, kind, pat, ctm, nm):
    (h, w), (ho, wo), sc = PATTERNS_2D[pat]
    X = np.random.default_rng(100 + pat).uniform(-1, 1, (2, 3, h, w)).astype(np.float32)
    run_case(gsa, X, (2, 3, ho, wo), scales4(sc), "nearest", ctm, nm, kind=kind)


@pytest.mark.parametrize("kind,pat,ctm,mode,ex", list(itertools.product(
    KINDS, range(len(PATTERNS_2D)), CTMS, ["linear", "cubic"], [0, 1])))
def test_linear_cubic_2d(gsa, kind, pat, ctm, mode, ex):
    (h, w), (ho, wo), sc = PATTERNS_2D[pat]
    X = np.random.default_rng(200 + pat).uniform(-1, 1, (2, 3, h, w)).astype(np.float32)
    run_case(gsa, X, (2, 3, ho, wo), scales4(sc), mode, ctm, ex=ex, kind=kind)


@pytest.mark.parametrize("a", [-0.5, -0.6, -1.0])
def test_cubic_coefficients(gsa, a):
    X = np.random.default_rng(7).normal(0, 1, (1, 4, 29, 31)).astype(np.float32)
    for ex in (0, 1):
        run_case(gsa, X, (1, 4, 58, 40), [1, 1, 2.0, float(np.float32(1.3))], "cubic",
                 "half_pixel", a=a, ex=ex)


@pytest.mark.parametrize("mode,ctm", list(itertools.product(["nearest", "linear", "cubic"], CTMS)))
def test_many_tiles_and_planes(gsa, mode, ctm):
    X = np.random.default_rng(8).uniform(-1, 1, (3, 5, 150, 190)).astype(np.float32)
    run_case(gsa, X, (3, 5, 301, 233), None, mode, ctm)


@pytest.mark.parametrize("mode,kind", list(itertools.product(["nearest", "linear", "cubic"], KINDS)))
def test_one_axis(gsa, mode, kind):
    rng = np.random.default_rng(9)
    X = rng.uniform(-1, 1, (4, 7, 300)).astype(np.float32)
    run_case(gsa, X, (4, 7, 777), None, mode, "half_pixel", kind=kind)
    run_case(gsa, X, (4, 7, 113), [1.0, 1.0, float(np.float32(0.38))], mode, "align_corners",
             kind=kind)
    v = rng.uniform(-1, 1, (1000,)).astype(np.float32)
    run_case(gsa, v, (2500,), None, mode, "asymmetric", kind=kind)


@pytest.mark.parametrize("mode,ctm,kind", list(itertools.product(
    ["nearest", "linear", "cubic"], CTMS, KINDS)))
def test_three_axes(gsa, mode, ctm, kind):
    X = np.random.default_rng(10).uniform(-1, 1, (2, 3, 9, 10, 11)).astype(np.float32)
    run_case(gsa, X, (2, 3, 17, 20, 5), None, mode, ctm, kind=kind)
    run_case(gsa, X, (2, 3, 4, 23, 16), [1, 1, 0.5, 2.3, float(np.float32(1.5))], mode, ctm,
             kind=kind)


@pytest.mark.parametrize("mode", ["nearest", "linear", "cubic"])
def test_leading_axes_are_planes(gsa, mode):
    X = np.random.default_rng(11).uniform(-1, 1, (2, 3, 4, 10, 12)).astype(np.float32)
    run_case(gsa, X, (2, 3, 4, 20, 6), None, mode, "half_pixel")
    run_case(gsa, X, (2, 3, 4, 10, 25), None, mode, "align_corners")


@pytest.mark.parametrize("mode", ["nearest", "linear", "cubic"])
def test_identity(gsa, mode):
    X = np.random.default_rng(12).uniform(-1, 1, (2, 3, 33, 47)).astype(np.float32)
    Xg, _ = x_to_gpu(X, "f32")
    for sc in (None, [1.0, 1.0, 1.0, 1.0]):
        note("identity %s %s" % (mode, sc))
        Y = from_gpu(gsa.resize_to(Xg, X.shape, sc, mode, "half_pixel"))
        assert np.array_equal(Y, X.astype(np.float64))


@pytest.mark.parametrize("mode,kind", list(itertools.product(["nearest", "linear", "cubic"], KINDS)))
def test_strong_downsampling_direct_path(gsa, mode, kind):
    # a 64 x 16 output tile reads 512 x 128 input elements: beyond the LDS
    # budget, so the kernel gathers straight from the input
    X = np.random.default_rng(13).uniform(-1, 1, (1, 2, 512, 512)).astype(np.float32)
    run_case(gsa, X, (1, 2, 64, 64), [1, 1, 0.125, 0.125], mode, "half_pixel", kind=kind)
    run_case(gsa, X, (1, 2, 37, 300), None, mode, "asymmetric", kind=kind)


def test_empty_output(gsa):
    torch = torch_mod()
    X = torch.zeros((2, 3, 4, 5), device="cuda")
    Y = gsa.resize_to(X, (2, 3, 0, 10), None, "linear")
    assert tuple(Y.shape) == (2, 3, 0, 10)


def test_rejects_resized_leading_axis(gsa):
    torch = torch_mod()
    X = torch.zeros((2, 3, 4, 5, 6), device="cuda")
    with pytest.raises(gsa.GSError):
        gsa.resize_to(X, (4, 3, 4, 5, 6), None, "linear")


def test_non_default_stream(gsa):
    torch = torch_mod()
    X = np.random.default_rng(14).uniform(-1, 1, (2, 4, 40, 50)).astype(np.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run_case(gsa, X, (2, 4, 70, 90), None, "linear", "half_pixel", stream=s)
    torch.cuda.synchronize()
