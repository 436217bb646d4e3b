"""GPU path (through the C ABI) against the CPU oracle, element by element.

Sizes span several 256-location tiles with a ragged last tile, and channel
counts that leave a remainder after the kernels' channel groups.  Every
mode x padding x align_corners x element type runs in 2D and 3D; the fused
theta -> sample path must equal the unfused pair bit for bit.
"""

import itertools

import numpy as np
import pytest

import oracle
from conftest import load_golden
from parity import check, from_gpu, note, to_gpu_f32, torch_mod, x_to_gpu

pytestmark = pytest.mark.gpu

MODES = ["nearest", "linear", "cubic"]
PADS = ["zeros", "border", "reflection"]
KINDS = ["f32", "f16", "bf16"]


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()   # raises if the HIP library is not built
    return gsa


# ------------------------------------------------------------ page examples

AFFINE = load_golden("affine_grid_examples.json")
SAMPLE = load_golden("grid_sample_examples.json")


@pytest.mark.parametrize("ex", AFFINE, ids=[e["name"] for e in AFFINE])
def test_affine_grid_page_examples(gsa, ex):
    note(ex["name"])
    theta = np.array(ex["theta"], np.float32).reshape(ex["theta_shape"])
    g = gsa.affine_grid(to_gpu_f32(theta), ex["size"], ex["align_corners"])
    got = from_gpu(g)
    ref = oracle.affine_grid(theta, ex["size"], ex["align_corners"])
    assert np.array_equal(got, ref.astype(np.float64))
    printed = np.array(ex["grid"]).reshape(ex["grid_shape"])
    assert (np.abs(got - printed) / np.maximum(1, np.abs(printed))).max() <= 2e-6


@pytest.mark.parametrize("ex", SAMPLE, ids=[e["name"] for e in SAMPLE])
def test_grid_sample_page_examples(gsa, ex):
    note(ex["name"])
    X = np.array(ex["X"], np.float32).reshape(ex["X_shape"])
    G = np.array(ex["grid"], np.float32).reshape(ex["grid_shape"])
    mode, pad, ac = ex["mode"] or "linear", ex["padding_mode"] or "zeros", ex["align_corners"] or 0
    Y = from_gpu(gsa.grid_sample(to_gpu_f32(X), to_gpu_f32(G), mode, pad, ac))
    check(Y, oracle.grid_sample(X, G, mode, pad, ac), mode, "f32", np.abs(X).max(), ex["name"])
    printed = np.array(ex["Y"]).reshape(ex["Y_shape"])
    assert (np.abs(Y - printed) / np.maximum(1, np.abs(printed))).max() <= 2e-6


# -------------------------------------------------------------- AffineGrid

@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("size", [(3, 1, 37, 41), (2, 4, 1, 300), (1, 1, 129, 1), (2, 1, 5, 7, 9),
                                  (1, 1, 1, 1, 700), (2, 1, 17, 1, 19)])
def test_affine_grid_bit_exact(gsa, ac, size):
    note("affine_grid %s ac=%d" % (size, ac))
    r = len(size) - 2
    rng = np.random.default_rng(sum(size) + ac)
    theta = rng.normal(size=(size[0], r, r + 1)).astype(np.float32)
    got = from_gpu(gsa.affine_grid(to_gpu_f32(theta), size, ac))
    assert np.array_equal(got, oracle.affine_grid(theta, size, ac).astype(np.float64))


# ------------------------------------------------------------- GridSample

def random_case(rank, seed, lo=-1.3, hi=1.3):
    rng = np.random.default_rng(seed)
    if rank == 2:
        X = rng.uniform(-1, 1, (2, 11, 13, 17)).astype(np.float32)
        G = rng.uniform(lo, hi, (2, 19, 23, 2)).astype(np.float32)      # 437 locations
    else:
        X = rng.uniform(-1, 1, (2, 5, 6, 7, 9)).astype(np.float32)
        G = rng.uniform(lo, hi, (2, 5, 6, 11, 3)).astype(np.float32)    # 330 locations
    return X, G


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rank", [2, 3])
def test_grid_sample_matches_oracle(gsa, rank, mode, pad, ac, kind):
    note("grid_sample %dD %s/%s ac=%d %s" % (rank, mode, pad, ac, kind))
    X, G = random_case(rank, 1000 * rank + 17 * ac + 3 * MODES.index(mode) + PADS.index(pad))
    Xd, Xin = x_to_gpu(X, kind)
    Y = from_gpu(gsa.grid_sample(Xd, to_gpu_f32(G), mode, pad, ac))
    check(Y, oracle.grid_sample(Xin, G, mode, pad, ac), mode, kind, np.abs(Xin).max(),
          "%dD %s/%s/%d/%s" % (rank, mode, pad, ac, kind))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rank", [2, 3])
def test_grid_sample_direct_gather_path(gsa, rank, mode, pad, ac, kind):
    """Random locations over an image larger than any LDS staging box: every
    block takes the direct-gather loop."""
    note("direct path %dD %s/%s ac=%d %s" % (rank, mode, pad, ac, kind))
    rng = np.random.default_rng(3000 + 1000 * rank + 17 * ac + 3 * MODES.index(mode) + PADS.index(pad))
    if rank == 2:
        X = rng.uniform(-1, 1, (2, 11, 70, 90)).astype(np.float32)
        G = rng.uniform(-1.3, 1.3, (2, 19, 23, 2)).astype(np.float32)
    else:
        X = rng.uniform(-1, 1, (2, 5, 20, 24, 28)).astype(np.float32)
        G = rng.uniform(-1.3, 1.3, (2, 5, 6, 11, 3)).astype(np.float32)
    Xd, Xin = x_to_gpu(X, kind)
    Y = from_gpu(gsa.grid_sample(Xd, to_gpu_f32(G), mode, pad, ac))
    check(Y, oracle.grid_sample(Xin, G, mode, pad, ac), mode, kind, np.abs(Xin).max(),
          "direct %dD %s/%s/%d/%s" % (rank, mode, pad, ac, kind))


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
def test_direct_gather_channel_batches(gsa, mode, kind):
    """Random locations over a plane too large to stage (the direct-gather
    loop).  Cubic has 4,096 tiles here, so each block takes all 5 channels:
    two 2-channel batches and a remainder; nearest and linear split the
    channels over groups of 2.  Every mode equals one-channel launches bit
    for bit, and the oracle at 4,096 sampled outputs."""
    torch = torch_mod()
    note("direct-gather channel batches %s %s" % (mode, kind))
    rng = np.random.default_rng(77 + MODES.index(mode))
    X = rng.uniform(-1, 1, (1, 5, 200, 200)).astype(np.float32)
    G = rng.uniform(-1.2, 1.2, (1, 1024, 1024, 2)).astype(np.float32)
    Xd, Xin = x_to_gpu(X, kind)
    Gd = to_gpu_f32(G)
    Y = gsa.grid_sample(Xd, Gd, mode, "reflection", 1)
    for c in range(5):
        Yc = gsa.grid_sample(Xd[:, c:c + 1].contiguous(), Gd, mode, "reflection", 1)
        assert torch.equal(Y[:, c:c + 1], Yc), "channel %d differs from its own launch" % c
    flat = np.random.default_rng(78).integers(0, Y.numel(), 4096)
    ref = oracle.grid_sample_points(Xin, G, flat, mode, "reflection", 1)
    got = from_gpu(Y).reshape(-1)[flat]
    check(got, ref, mode, kind, np.abs(Xin).max(), "direct batches %s %s" % (mode, kind))


@pytest.mark.parametrize("mode,pad", list(itertools.product(MODES, PADS)))
def test_grid_sample_many_tiles(gsa, mode, pad):
    """Several tiles per image, ragged tail, channel count with a remainder."""
    note("many tiles %s/%s" % (mode, pad))
    rng = np.random.default_rng(5)
    X = rng.normal(size=(3, 19, 40, 53)).astype(np.float32)
    G = rng.uniform(-1.15, 1.15, (3, 67, 71, 2)).astype(np.float32)
    for ac in (0, 1):
        Y = from_gpu(gsa.grid_sample(to_gpu_f32(X), to_gpu_f32(G), mode, pad, ac))
        check(Y, oracle.grid_sample(X, G, mode, pad, ac), mode, "f32", np.abs(X).max(),
              "many tiles %s/%s/%d" % (mode, pad, ac))


# ------------------------------------------------------------------ fused

@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rank", [2, 3])
def test_fused_equals_unfused_and_oracle(gsa, rank, mode, pad, kind):
    note("fused %dD %s/%s %s" % (rank, mode, pad, kind))
    rng = np.random.default_rng(77 + rank)
    if rank == 2:
        X = rng.uniform(-1, 1, (3, 9, 21, 18)).astype(np.float32)
        out = (29, 31)
    else:
        X = rng.uniform(-1, 1, (2, 4, 7, 8, 9)).astype(np.float32)
        out = (6, 9, 10)
    n, c = X.shape[:2]
    theta = (np.concatenate([np.eye(rank), np.zeros((rank, 1))], 1)[None]
             + 0.3 * rng.normal(size=(n, rank, rank + 1))).astype(np.float32)
    Xd, Xin = x_to_gpu(X, kind)
    td = to_gpu_f32(theta)
    for ac in (0, 1):
        fused = gsa.affine_grid_sample_fused(td, Xd, out, mode, pad, ac)
        grid = gsa.affine_grid(td, (n, c) + out, ac)
        unfused = gsa.grid_sample(Xd, grid, mode, pad, ac)
        F, U = from_gpu(fused), from_gpu(unfused)
        assert np.array_equal(F, U), "fused differs from unfused"
        G = oracle.affine_grid(theta, (n, c) + out, ac)
        check(F, oracle.grid_sample(Xin, G, mode, pad, ac), mode, kind, np.abs(Xin).max(),
              "fused %dD %s/%s/%d" % (rank, mode, pad, ac))


def rotation3(rng, angle):
    """A rotation by `angle` about a random axis (Rodrigues)."""
    a = rng.normal(size=3)
    a /= np.linalg.norm(a)
    K = np.array([[0, -a[2], a[1]], [a[2], 0, -a[0]], [-a[1], a[0], 0]])
    return np.eye(3) + np.sin(angle) * K + (1 - np.cos(angle)) * K @ K


def theta3_family(rng, n):
    """3D affine matrices of every kind: near identity, large rotations with
    translation, zoom in and out (out: more input rows than a tile's staging
    plan holds, so those tiles gather directly), shear, a degenerate map
    (every output at one point), non-finite and huge entries."""
    out = []
    for b in range(n):
        kind = b % 9
        M = np.eye(3)
        t = rng.normal(0, 0.2, 3)
        if kind == 0:
            M = M + rng.normal(0, 0.1, (3, 3))
        elif kind == 1:
            M = rotation3(rng, rng.uniform(0.5, 1.2))
        elif kind == 2:
            M = 0.3 * rotation3(rng, 0.3)
        elif kind == 3:
            M = 3.0 * rotation3(rng, 0.4)
        elif kind == 4:
            M = M + np.triu(rng.normal(0, 0.8, (3, 3)), 1)
        elif kind == 5:
            M = np.zeros((3, 3))
        th = np.concatenate([M, t[:, None]], 1)
        if kind == 6:
            th[1, 2] = np.nan
        elif kind == 7:
            th[0, 0] = 1e30
        elif kind == 8:
            th = th + rng.normal(0, 0.5, th.shape)
        out.append(th)
    return np.stack(out).astype(np.float32)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("pad", ["zeros", "border"])
@pytest.mark.parametrize("mode", ["linear", "nearest"])
def test_fused_3d_equals_unfused_over_theta_kinds(gsa, mode, pad, ac, kind):
    """The 3D fused sampler equals AffineGrid + GridSample bit for bit over
    several tiles with ragged edges, extents of 1 and 2, and theta of every
    kind (staged and directly gathered tiles), and matches the oracle."""
    rng = np.random.default_rng(310 + 2 * ac + (pad == "border"))
    for xs, out in [((9, 3, 19, 21, 23), (17, 13, 70)), ((9, 2, 1, 5, 2), (1, 3, 40)),
                    ((9, 2, 2, 1, 37), (5, 2, 33))]:
        note("fused 3D theta kinds %s/%s ac=%d %s X=%s out=%s" % (mode, pad, ac, kind, xs, out))
        X = rng.uniform(-1, 1, xs).astype(np.float32)
        n, c = xs[:2]
        theta = theta3_family(rng, n)
        Xd, Xin = x_to_gpu(X, kind)
        td = to_gpu_f32(theta)
        fused = gsa.affine_grid_sample_fused(td, Xd, out, mode, pad, ac)
        grid = gsa.affine_grid(td, (n, c) + out, ac)
        unfused = gsa.grid_sample(Xd, grid, mode, pad, ac)
        F, U = from_gpu(fused), from_gpu(unfused)
        bad = ~((F == U) | (np.isnan(F) & np.isnan(U)))
        assert not bad.any(), "fused differs from unfused at %s" % (np.argwhere(bad)[0],)
        G = oracle.affine_grid(theta, (n, c) + out, ac)
        ok = np.isfinite(theta).all(axis=(1, 2)) & (np.abs(theta).max(axis=(1, 2)) < 1e6)
        check(F[ok], oracle.grid_sample(Xin[ok], G[ok], mode, pad, ac), mode, kind,
              np.abs(Xin).max(), "fused 3D theta kinds %s/%s/%d" % (mode, pad, ac))


# ------------------------------------------------------------- edge cases

@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("pad", PADS)
def test_non_finite_and_huge_locations(gsa, mode, pad):
    note("non-finite %s/%s" % (mode, pad))
    rng = np.random.default_rng(9)
    X = rng.uniform(-1, 1, (1, 3, 5, 6)).astype(np.float32)
    bad = np.array([np.nan, np.inf, -np.inf, 3e38, -3e38, 1e9, -1e9, 16777217.0, -16777219.0,
                    1e-40, -0.0], np.float32)
    G = np.zeros((1, 2, bad.size, 2), np.float32)
    G[0, 0, :, 0] = bad
    G[0, 0, :, 1] = 0.1
    G[0, 1, :, 0] = 0.2
    G[0, 1, :, 1] = bad
    for ac in (0, 1):
        Y = from_gpu(gsa.grid_sample(to_gpu_f32(X), to_gpu_f32(G), mode, pad, ac))
        ref = oracle.grid_sample(X, G, mode, pad, ac)
        assert np.all(np.isfinite(Y))
        check(Y, ref, mode, "f32", np.abs(X).max(), "non-finite %s/%s/%d" % (mode, pad, ac))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("pad", PADS)
@pytest.mark.parametrize("in_sp", [(1, 1), (1, 7), (6, 1), (2, 2)])
def test_tiny_and_unit_extents(gsa, mode, pad, in_sp):
    note("tiny %s %s/%s" % (in_sp, mode, pad))
    rng = np.random.default_rng(10)
    X = rng.uniform(-1, 1, (2, 3) + in_sp).astype(np.float32)
    G = rng.uniform(-2.5, 2.5, (2, 3, 5, 2)).astype(np.float32)
    for ac in (0, 1):
        Y = from_gpu(gsa.grid_sample(to_gpu_f32(X), to_gpu_f32(G), mode, pad, ac))
        check(Y, oracle.grid_sample(X, G, mode, pad, ac), mode, "f32", np.abs(X).max(),
              "tiny %s %s/%s/%d" % (in_sp, mode, pad, ac))


def test_unit_output_extents_and_single_channel(gsa):
    note("unit output extents")
    rng = np.random.default_rng(11)
    for x_shape, g_shape in [((1, 1, 9, 9), (1, 1, 1, 2)), ((4, 1, 9, 9), (4, 300, 1, 2)),
                             ((1, 67, 5, 5), (1, 1, 513, 2)), ((2, 2, 3, 4, 5), (2, 1, 1, 1, 3))]:
        X = rng.uniform(-1, 1, x_shape).astype(np.float32)
        G = rng.uniform(-1.2, 1.2, g_shape).astype(np.float32)
        for mode in MODES:
            Y = from_gpu(gsa.grid_sample(to_gpu_f32(X), to_gpu_f32(G), mode, "zeros", 0))
            check(Y, oracle.grid_sample(X, G, mode, "zeros", 0), mode, "f32", np.abs(X).max(),
                  "unit %s %s" % (x_shape, mode))


def test_empty_tensors_launch_nothing(gsa):
    note("empty tensors")
    torch = torch_mod()
    X = torch.zeros(0, 3, 4, 4, device="cuda")
    G = torch.zeros(0, 5, 5, 2, device="cuda")
    assert gsa.grid_sample(X, G).shape == (0, 3, 5, 5)
    X = torch.zeros(2, 0, 4, 4, device="cuda")
    G = torch.zeros(2, 5, 5, 2, device="cuda")
    assert gsa.grid_sample(X, G).shape == (2, 0, 5, 5)
    theta = torch.zeros(0, 2, 3, device="cuda")
    assert gsa.affine_grid(theta, (0, 1, 4, 4)).shape == (0, 4, 4, 2)
    # output left untouched when there is nothing to do
    out = torch.full((2, 3, 0, 5), 7.0, device="cuda")
    gsa.grid_sample(torch.zeros(2, 3, 4, 4, device="cuda"), torch.zeros(2, 0, 5, 2, device="cuda"),
                    out=out)


def test_errors_raise_through_binding(gsa):
    note("binding errors")
    torch = torch_mod()
    X = torch.zeros(2, 3, 4, 4, device="cuda")
    with pytest.raises(gsa.GSError):
        gsa.grid_sample(X, torch.zeros(3, 5, 5, 2, device="cuda"))      # batch mismatch
    with pytest.raises(gsa.GSError):
        gsa.grid_sample(X, torch.zeros(2, 5, 5, 2, device="cuda", dtype=torch.int32))  # integer grid
    with pytest.raises(gsa.GSError):
        gsa.grid_sample(X, torch.zeros(2, 5, 5, 2, device="cuda"), align_corners=3)
    with pytest.raises(gsa.GSError):
        gsa.grid_sample(torch.zeros(2, 3, 4, 0, device="cuda"), torch.zeros(2, 5, 5, 2, device="cuda"))


def test_non_default_stream(gsa):
    note("non-default stream")
    torch = torch_mod()
    X, G = random_case(2, 4242)
    Xd, Gd = to_gpu_f32(X), to_gpu_f32(G)
    ref = gsa.grid_sample(Xd, Gd, "cubic", "reflection", 1)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = gsa.grid_sample(Xd, Gd, "cubic", "reflection", 1)
    s.synchronize()
    assert torch.equal(out, ref)
