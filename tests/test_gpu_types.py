"""GridSample of any rank and element type on the GPU (gs_grid_sample and the
2D/3D entries routed to the any-rank kernel) against the oracle.

The any-rank kernel computes the coordinate steps in the grid's precision and
the weighted sum in double in the order of the definition -- the oracle's
order -- so its outputs are compared BIT FOR BIT with the oracle's value after
the same final conversion: fp32 / fp16 / bf16 / double outputs rounded to
nearest (double -> fp32 -> half for the half types), integer outputs cast by
truncation toward zero with saturation (GridSample page, Outputs).

Cases: ranks 1, 4, 5 and 6 with every mode x padding x align_corners; double
X with double and fp32 grids in 1-D, 2D and 3D; fp16 and bf16 grids (widened
exactly to fp32); every integer type with values spanning its range;
non-finite locations; sizes that span several 256-location tiles with a
ragged tail and channel counts that leave a remainder after the channel
groups; launches large enough that blocks take whole channel loops in
batches, against one-channel launches and the oracle.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from parity import note, torch_mod

pytestmark = pytest.mark.gpu

MODES = ["nearest", "linear", "cubic"]
PADS = ["zeros", "border", "reflection"]


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def tgpu(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


FLOAT_KINDS = ("f32", "f16", "bf16", "f64")


def expected(ref: np.ndarray, kind: str) -> np.ndarray:
    """The oracle's float64 value after the output conversion of `kind`: a
    float64 array for the float kinds, the integer array for integer kinds."""
    if kind == "f64":
        return ref
    if kind == "f32":
        return ref.astype(np.float32).astype(np.float64)
    if kind == "f16":
        return ref.astype(np.float32).astype(np.float16).astype(np.float64)
    if kind == "bf16":
        bits = W.to_half_bits(ref.astype(np.float32), "bf16")
        return W.half_bits_to_f32(bits, "bf16").astype(np.float64)
    return oracle.to_integer(ref, np.dtype(kind))


def gpu_values(Y, kind):
    torch = torch_mod()
    torch.cuda.synchronize()
    if kind in FLOAT_KINDS:
        return Y.double().cpu().numpy()
    signed = {"uint16": torch.int16, "uint32": torch.int32, "uint64": torch.int64}
    if kind in signed:  # read the bits through the signed type of the same width
        return Y.view(signed[kind]).cpu().numpy().view(np.dtype(kind))
    return Y.cpu().numpy()


def run(gsa, X, G, mode, pad, ac, kind, grid_kind="f32", what=""):
    """X: numpy array of the element type (fp32 values for the half kinds,
    rounded here); G: fp32 or float64 numpy grid (rounded here for half
    grids)."""
    torch = torch_mod()
    note("%s %s %s/%s ac=%d X=%s grid=%s" % (what, kind, mode, pad, ac, X.shape, grid_kind))
    if kind in ("f16", "bf16"):
        bits = W.to_half_bits(X, kind)
        Xd = tgpu(bits.view(np.int16), torch.float16 if kind == "f16" else torch.bfloat16)
        Xo = W.half_bits_to_f32(bits, kind)
    elif kind in ("uint16", "uint32", "uint64"):
        tdt = getattr(torch, kind, None)
        if tdt is None:
            pytest.skip("torch has no %s" % kind)
        signed = {"uint16": np.int16, "uint32": np.int32, "uint64": np.int64}[kind]
        Xd = tgpu(X.view(signed), tdt)
        Xo = X
    else:
        Xd = tgpu(X)
        Xo = X
    if grid_kind in ("f16", "bf16"):
        gbits = W.to_half_bits(G, grid_kind)
        Gd = tgpu(gbits.view(np.int16), torch.float16 if grid_kind == "f16" else torch.bfloat16)
        Go = W.half_bits_to_f32(gbits, grid_kind)
    else:
        Gd = tgpu(G)
        Go = G
    Y = gsa.grid_sample(Xd, Gd, mode, pad, ac)
    got = gpu_values(Y, kind)
    ref = expected(oracle.grid_sample(Xo, Go, mode, pad, ac), kind)
    if kind in FLOAT_KINDS:
        bad = ~((got == ref) | (np.isnan(got) & np.isnan(ref)))
    else:
        bad = got != ref
    assert not bad.any(), "%s: %d of %d outputs differ, first at %s: %r vs %r" % (
        what, bad.sum(), bad.size, np.argwhere(bad)[0], got[bad][0], ref[bad][0])


def shapes(rank, seed):
    rng = np.random.default_rng(seed)
    if rank == 1:
        return (2, 5, 37), (2, 300, 1)
    if rank == 4:
        return (2, 3, 5, 6, 4, 7), (2, 3, 4, 5, 6, 4)
    if rank == 5:
        return (1, 2, 4, 3, 5, 3, 4), (1, 3, 2, 4, 3, 5, 5)
    return (1, 2, 3, 2, 3, 2, 3, 4), (1, 2, 3, 2, 3, 4, 5, 6)


@pytest.mark.parametrize("rank,mode,pad,ac", list(itertools.product(
    [1, 4, 5, 6], MODES, PADS, [0, 1])))
def test_any_rank_fp32(gsa, rank, mode, pad, ac):
    # cubic at ranks 5 and 6 sums 1,024 and 4,096 taps per output; its
    # per-axis tap tables sit in the lane's stack frame (indices bounded by
    # the tap digit, 0..3)
    xs, gsh = shapes(rank, rank)
    rng = np.random.default_rng(10 * rank + ac)
    X = rng.uniform(-1, 1, xs).astype(np.float32)
    G = rng.uniform(-1.3, 1.3, gsh).astype(np.float32)
    run(gsa, X, G, mode, pad, ac, "f32", what="rank %d" % rank)


@pytest.mark.parametrize("rank,mode,pad,ac", list(itertools.product(
    [1, 2, 3], MODES, PADS, [0, 1])))
def test_double_x_and_grid(gsa, rank, mode, pad, ac):
    rng = np.random.default_rng(40 + rank)
    xs = {1: (2, 5, 37), 2: (2, 5, 23, 29), 3: (2, 3, 7, 8, 9)}[rank]
    gsh = {1: (2, 300, 1), 2: (2, 17, 19, 2), 3: (2, 5, 6, 9, 3)}[rank]
    X = rng.normal(0, 1, xs)
    G = rng.uniform(-1.3, 1.3, gsh)
    run(gsa, X, G, mode, pad, ac, "f64", "f64", what="double")
    run(gsa, X, G.astype(np.float32), mode, pad, ac, "f64", "f32", what="double X, fp32 grid")
    run(gsa, X.astype(np.float32), G, mode, pad, ac, "f32", "f64", what="fp32 X, double grid")


@pytest.mark.parametrize("gk,mode,pad", list(itertools.product(["f16", "bf16"], MODES, PADS)))
def test_half_grids(gsa, gk, mode, pad):
    rng = np.random.default_rng(50)
    X = rng.uniform(-1, 1, (2, 5, 23, 29)).astype(np.float32)
    G = rng.uniform(-1.2, 1.2, (2, 17, 19, 2)).astype(np.float32)
    for ac in (0, 1):
        run(gsa, X, G, mode, pad, ac, "f32", gk, what="half grid")
        run(gsa, X, G, mode, pad, ac, "bf16", gk, what="half grid, bf16 X")


INT_KINDS = ["int8", "uint8", "int16", "uint16", "int32", "uint32", "int64", "uint64"]


@pytest.mark.parametrize("kind,mode,pad", list(itertools.product(INT_KINDS, MODES, PADS)))
def test_integer_types(gsa, kind, mode, pad):
    rng = np.random.default_rng(60)
    info = np.iinfo(kind)
    lo, hi = max(info.min, -2**40), min(info.max, 2**40)
    X = rng.integers(lo, hi, (2, 5, 23, 29), dtype=np.int64, endpoint=True).astype(kind)
    # a few plateaus at the extremes so cubic overshoot saturates
    X[:, :, 3:6, 3:9] = info.max
    X[:, :, 10:13, 4:8] = info.min
    G = rng.uniform(-1.2, 1.2, (2, 17, 19, 2)).astype(np.float32)
    for ac in (0, 1):
        run(gsa, X, G, mode, pad, ac, kind, what="integer")


def test_uint8_images_3d(gsa):
    rng = np.random.default_rng(61)
    X = rng.integers(0, 256, (2, 3, 9, 10, 11), dtype=np.uint8)
    G = rng.uniform(-1.1, 1.1, (2, 6, 7, 8, 3)).astype(np.float32)
    for mode, pad in itertools.product(MODES, PADS):
        run(gsa, X, G, mode, pad, 0, "uint8", what="uint8 3D")


def test_non_finite_locations(gsa):
    rng = np.random.default_rng(62)
    X = rng.uniform(-1, 1, (1, 3, 40)).astype(np.float32)
    G = rng.uniform(-1, 1, (1, 260, 1)).astype(np.float32)
    G[0, ::7, 0] = np.nan
    G[0, 1::11, 0] = np.inf
    G[0, 2::13, 0] = -np.inf
    G[0, 3::17, 0] = 3e38
    for mode, pad in itertools.product(MODES, PADS):
        run(gsa, X, G, mode, pad, 0, "f32", what="non-finite 1-D")
    Xi = rng.integers(-100, 100, (1, 3, 40)).astype(np.int16)
    run(gsa, Xi, G, "linear", "zeros", 1, "int16", what="non-finite int16")




@pytest.mark.parametrize("kind,rank,ac", list(itertools.product(["f64", "f16", "bf16"], [2, 3],
                                                                [0, 1])))
def test_affine_grid_types(gsa, kind, rank, ac):
    """AffineGrid with a double theta matches the float64 oracle bit for bit;
    with fp16 / bf16 theta, the fp32 oracle on the widened theta rounded once
    to the half type."""
    torch = torch_mod()
    note("affine_grid %s rank %d ac=%d" % (kind, rank, ac))
    rng = np.random.default_rng(70 + rank)
    theta = rng.normal(0, 1, (3, rank, rank + 1))
    size = (3, 2) + ((37, 45) if rank == 2 else (9, 10, 11))
    if kind == "f64":
        g = gsa.affine_grid(tgpu(theta), size, ac)
        got = g.cpu().numpy()
        ref = oracle.affine_grid(theta, size, ac)
        assert got.dtype == np.float64 and np.array_equal(got, ref)
        return
    bits = W.to_half_bits(theta.astype(np.float32), kind)
    tdt = torch.float16 if kind == "f16" else torch.bfloat16
    g = gsa.affine_grid(tgpu(bits.view(np.int16), tdt), size, ac)
    assert g.dtype == tdt
    got = g.view(torch.int16).cpu().numpy().view(np.uint16)
    ref32 = oracle.affine_grid(W.half_bits_to_f32(bits, kind), size, ac)
    assert np.array_equal(got, W.to_half_bits(ref32, kind))


# Enough locations that a launch reaches its block target with one channel
# group (each block takes every channel of its image), and channel counts
# that leave a remainder after the kernel's channel batches (8 / taps
# channels per batch; 2 for 8 taps).
BATCH_CASES = [
    # rank, mode, kind, X shape, grid shape
    (1, "linear", "f32", (1, 7, 5000), (1, 600000, 1)),
    (1, "nearest", "uint8", (1, 11, 5000), (1, 600000, 1)),
    (1, "cubic", "f32", (1, 5, 5000), (1, 600000, 1)),
    (2, "linear", "uint8", (1, 5, 64, 64), (1, 800, 800, 2)),
    (2, "linear", "f64", (1, 3, 64, 64), (1, 800, 800, 2)),
    (3, "linear", "f64", (1, 3, 16, 16, 16), (1, 86, 86, 86, 3)),
    (3, "linear", "uint8", (1, 5, 16, 16, 16), (1, 86, 86, 86, 3)),
]


@pytest.mark.parametrize("ci", range(len(BATCH_CASES)))
def test_channel_batches(gsa, ci):
    """The any-rank kernel with whole channel loops per block: bit-identical
    to one-channel launches (one channel per block, no batch) everywhere, and
    to the oracle on the first locations."""
    torch = torch_mod()
    rank, mode, kind, xs, gsh = BATCH_CASES[ci]
    rng = np.random.default_rng(70 + ci)
    note("channel batches rank %d %s %s X=%s grid=%s" % (rank, mode, kind, xs, gsh))
    if kind == "uint8":
        X = rng.integers(0, 256, xs, dtype=np.uint8)
    elif kind == "f64":
        X = rng.normal(0, 1, xs)
    else:
        X = rng.uniform(-1, 1, xs).astype(np.float32)
    G = rng.uniform(-1.1, 1.1, gsh).astype(np.float32)
    Xd, Gd = tgpu(X), tgpu(G)
    Y = gsa.grid_sample(Xd, Gd, mode, "zeros", 0)
    for c in range(xs[1]):
        Yc = gsa.grid_sample(Xd[:, c:c + 1].contiguous(), Gd, mode, "zeros", 0)
        assert torch.equal(Y[:, c:c + 1], Yc), "channel %d differs from its own launch" % c
    # the oracle on the first 2,000 locations (a grid of one row of them)
    flat = G.reshape(1, -1, rank)[:, :2000]
    sub = flat.reshape((1, 2000) + (1,) * (rank - 1) + (rank,))
    got = gpu_values(Y, kind).reshape(1, xs[1], -1)[:, :, :2000]
    ref = expected(oracle.grid_sample(X, sub, mode, "zeros", 0), kind).reshape(1, xs[1], -1)
    assert np.array_equal(got, ref), "%d of %d outputs differ from the oracle" % (
        (got != ref).sum(), got.size)
