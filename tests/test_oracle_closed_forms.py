"""Oracle against closed forms and invariants of the grid generator and sampler.

AffineGrid page, Summary: the grid is theta applied to evenly spaced positions
over [-1, 1]; with align_corners=1 the ends are the corner-pixel centres (so the
first and last positions are exactly -1 and 1), with align_corners=0 they are
the outer pixel edges (so positions are pixel centres).

GridSample page, Summary and Attributes: identity transforms reproduce the
input; weights of every mode sum to one; zeros padding reads 0 outside the
image; border repeats the edge; reflection mirrors at the borders and repeats.
"""

import numpy as np
import pytest

MODES = ["nearest", "linear", "cubic"]


def evenly_spaced(m, ac):
    """numpy.linspace positions: ends at -1/1 (ac=1) or half a pixel inside."""
    if ac:
        return np.linspace(-1.0, 1.0, m) if m > 1 else np.zeros(1)
    return np.linspace(-1.0 + 1.0 / m, 1.0 - 1.0 / m, m)


# ---------------------------------------------------------------- AffineGrid

@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("spatial", [(5, 7), (1, 6), (6, 1), (3, 4, 5), (1, 1, 2)])
def test_affine_grid_is_linear_map_of_linspace(oracle_mod, ac, spatial):
    r = len(spatial)
    rng = np.random.default_rng(7 + ac + 10 * r)
    theta = rng.normal(size=(3, r, r + 1)).astype(np.float32)
    grid = oracle_mod.affine_grid(theta, (3, 2) + spatial, ac).astype(np.float64)
    # base position vector, innermost axis first
    axes = [evenly_spaced(m, ac) for m in spatial]
    mesh = np.meshgrid(*axes, indexing="ij")
    base = np.stack(mesh[::-1], axis=-1)                    # (*spatial, r)
    expect = np.einsum("...j,nkj->n...k", base, theta[:, :, :r].astype(np.float64))
    expect += theta[:, :, r].astype(np.float64).reshape((3,) + (1,) * r + (r,))
    scale = np.abs(theta).sum(axis=2).max()
    np.testing.assert_allclose(grid, expect, rtol=0, atol=4e-7 * max(1.0, scale))


@pytest.mark.parametrize("ac", [0, 1])
def test_affine_grid_identity_and_translation(oracle_mod, ac):
    for spatial in [(4, 6), (2, 3, 5)]:
        r = len(spatial)
        theta = np.zeros((2, r, r + 1), np.float32)
        theta[:, :, :r] = np.eye(r)
        theta[1, :, r] = np.arange(1, r + 1) * 0.25             # exact translation
        grid = oracle_mod.affine_grid(theta, (2, 1) + spatial, ac)
        axes = [evenly_spaced(m, ac) for m in spatial]
        base = np.stack(np.meshgrid(*axes, indexing="ij")[::-1], axis=-1)
        ulp = np.spacing(np.float32(2.0))
        np.testing.assert_allclose(grid[0], base, rtol=0, atol=ulp)
        np.testing.assert_allclose(grid[1], base + theta[1, :, r], rtol=0, atol=2 * ulp)
        if ac:
            # the ends of every axis are exactly -1 and 1
            for k in range(r):
                comp = grid[0][..., k]
                assert comp.min() == -1.0 and comp.max() == 1.0


# ---------------------------------------------------------------- GridSample

def identity_grid(oracle_mod, n, spatial, ac):
    r = len(spatial)
    theta = np.zeros((n, r, r + 1), np.float32)
    theta[:, :, :r] = np.eye(r)
    return oracle_mod.affine_grid(theta, (n, 1) + spatial, ac)


@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("spatial", [(16, 16), (64, 128), (256, 256), (9, 17, 33)])
def test_identity_nearest_reproduces_input_exactly(oracle_mod, ac, spatial):
    rng = np.random.default_rng(1)
    X = rng.uniform(-1, 1, (1, 2) + spatial).astype(np.float32)
    G = identity_grid(oracle_mod, 1, spatial, ac)
    for pad in ["zeros", "border", "reflection"]:
        Y = oracle_mod.grid_sample(X, G, "nearest", pad, ac)
        assert np.array_equal(Y, X.astype(np.float64))


@pytest.mark.parametrize("mode", ["linear", "cubic"])
@pytest.mark.parametrize("spatial", [(16, 16), (64, 128), (256, 256), (9, 17, 33)])
def test_identity_linear_cubic(oracle_mod, mode, spatial):
    if mode == "cubic" and len(spatial) == 3:
        spatial = (5, 9, 17)
    rng = np.random.default_rng(2)
    X = rng.uniform(-1, 1, (1, 2) + spatial).astype(np.float32)
    for ac in (0, 1):
        G = identity_grid(oracle_mod, 1, spatial, ac)
        Y = oracle_mod.grid_sample(X, G, mode, "zeros", ac)
        pow2 = all(m & (m - 1) == 0 for m in spatial)
        if ac == 0 and pow2:
            # for power-of-two extents the pixel centres (2i+1)/n - 1 are exact
            # in fp32 and map back onto integer coordinates exactly
            assert np.array_equal(Y, X.astype(np.float64))
        else:
            # fp32 rounding of the identity grid moves p by up to ~4e-6 px per
            # axis at n = 256; neighbouring pixels differ by up to 2 max|X|
            tol = len(spatial) * 1e-5 * np.abs(X).max()
            assert np.abs(Y - X).max() <= tol


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("rank", [2, 3])
def test_constant_input(oracle_mod, mode, ac, rank):
    rng = np.random.default_rng(3)
    spatial = (16,) * rank
    c = np.float32(0.6180339)
    X = np.full((2, 3) + spatial, c, np.float32)
    out = (4,) * rank
    # border and reflection: every tap reads c and the weights sum to one
    G = rng.uniform(-3, 3, (2,) + out + (rank,)).astype(np.float32)
    for pad in ["border", "reflection"]:
        Y = oracle_mod.grid_sample(X, G, mode, pad, ac)
        np.testing.assert_allclose(Y, float(c), rtol=1e-12, atol=0)
    # zeros: well inside -> c; far outside on any axis -> 0
    inside = rng.uniform(-0.5, 0.5, (2,) + out + (rank,)).astype(np.float32)
    np.testing.assert_allclose(oracle_mod.grid_sample(X, inside, mode, "zeros", ac), float(c),
                               rtol=1e-12, atol=0)
    outside = inside.copy()
    axis = rng.integers(0, rank, size=(2,) + out)
    sign = rng.choice([-1.0, 1.0], size=(2,) + out)
    far = rng.uniform(2.5, 40.0, size=(2,) + out)
    np.put_along_axis(outside, axis[..., None], (sign * far)[..., None].astype(np.float32), axis=-1)
    assert np.all(oracle_mod.grid_sample(X, outside, mode, "zeros", ac) == 0.0)


@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("rank", [2, 3])
def test_linear_reproduces_affine_ramps(oracle_mod, ac, rank):
    rng = np.random.default_rng(4 + rank)
    spatial = (7, 11) if rank == 2 else (5, 6, 7)
    coef = rng.normal(size=rank)
    offset = 0.3
    idx = np.meshgrid(*[np.arange(m) for m in spatial], indexing="ij")
    X = (offset + sum(coef[a] * idx[a] for a in range(rank))).astype(np.float32)
    X = np.ascontiguousarray(np.broadcast_to(X, (1, 2) + spatial))
    # locations whose pixel coordinates stay inside [0, n-1] on every axis
    lo = [-1.0 if ac else -1.0 + 1.0 / spatial[rank - 1 - k] for k in range(rank)]
    G = np.stack([rng.uniform(lo[k], -lo[k], (1, 6, 5) if rank == 2 else (1, 3, 4, 5))
                  for k in range(rank)], axis=-1).astype(np.float32)
    Y = oracle_mod.grid_sample(X, G, "linear", "zeros", ac)
    expect = np.full(G.shape[:-1], offset)
    for a in range(rank):
        g = G[..., rank - 1 - a].astype(np.float64)
        n = spatial[a]
        p = (g + 1) / 2 * (n - 1) if ac else ((g + 1) * n - 1) / 2
        expect = expect + coef[a] * p
    for ch in range(2):
        np.testing.assert_allclose(Y[:, ch], expect, rtol=0, atol=1e-5 * np.abs(X).max())


@pytest.mark.parametrize("mode", ["nearest", "linear"])
@pytest.mark.parametrize("rank", [2, 3])
def test_border_equals_sampling_clamped_location(oracle_mod, mode, rank):
    rng = np.random.default_rng(5)
    spatial = (6, 9) if rank == 2 else (4, 5, 6)
    X = rng.uniform(-1, 1, (2, 2) + spatial).astype(np.float32)
    G = rng.uniform(-4, 4, (2, 5, 7, rank) if rank == 2 else (2, 3, 4, 5, rank)).astype(np.float32)
    # with align_corners=1, g = +-1 are exactly the edge pixel centres
    Yb = oracle_mod.grid_sample(X, G, mode, "border", 1)
    Yz = oracle_mod.grid_sample(X, np.clip(G, -1, 1), mode, "zeros", 1)
    assert np.array_equal(Yb, Yz)


@pytest.mark.parametrize("mode", ["linear", "cubic"])
@pytest.mark.parametrize("ac", [0, 1])
def test_reflection_symmetry_and_period(oracle_mod, mode, ac):
    rng = np.random.default_rng(6 + ac)
    X = rng.uniform(-1, 1, (1, 2, 6, 9)).astype(np.float32)
    # multiples of 1/1024 keep -2-g, 2-g and g+4 exact in fp32
    G = (rng.integers(-3 * 1024, 3 * 1024, (1, 8, 8, 2)) / 1024.0).astype(np.float32)
    Y = oracle_mod.grid_sample(X, G, mode, "reflection", ac)
    tol = 1e-5 * np.abs(X).max() * (4 if mode == "cubic" else 1)
    for mapped in (-2.0 - G, 2.0 - G, G + 4.0, G - 4.0):
        Ym = oracle_mod.grid_sample(X, mapped.astype(np.float32), mode, "reflection", ac)
        np.testing.assert_allclose(Ym, Y, rtol=0, atol=tol)


def test_reflection_worked_text_case(oracle_mod):
    """GridSample page, padding_mode: with borders at -1 and 1 (align_corners=1
    on a 3-pixel axis gives pixel coordinates -1..1 after a shift of one), the
    location -3.5 folds to 1.5 and then to 0.5."""
    X = np.array([[[[0.0, 10.0, 20.0]]]], np.float32)   # pixels 0,1,2 <-> -1,0,1
    # pixel coordinate -3.5 - (-1) = -2.5  <->  g = -2.5 (n - 1 = 2 => p = g + 1)
    G = np.array([[[[-3.5, 0.0]]]], np.float32)
    Y = oracle_mod.grid_sample(X, G, "linear", "reflection", 1)
    # 0.5 in the shifted frame is pixel coordinate 1.5 -> halfway 10 and 20
    assert Y[0, 0, 0, 0] == pytest.approx(15.0, abs=1e-6)


@pytest.mark.parametrize("mode", MODES)
def test_channels_and_batch_are_independent(oracle_mod, mode):
    rng = np.random.default_rng(8)
    X = rng.uniform(-1, 1, (3, 4, 7, 8)).astype(np.float32)
    G = rng.uniform(-1.3, 1.3, (3, 5, 6, 2)).astype(np.float32)
    Y = oracle_mod.grid_sample(X, G, mode, "zeros", 0)
    pc = rng.permutation(4)
    pn = rng.permutation(3)
    assert np.array_equal(oracle_mod.grid_sample(X[:, pc], G, mode, "zeros", 0), Y[:, pc])
    assert np.array_equal(oracle_mod.grid_sample(X[pn], G[pn], mode, "zeros", 0), Y[pn])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("pad", ["zeros", "border", "reflection"])
def test_non_finite_and_huge_locations_are_safe(oracle_mod, mode, pad):
    rng = np.random.default_rng(9)
    X = rng.uniform(-1, 1, (1, 2, 5, 6)).astype(np.float32)
    bad = np.array([np.nan, np.inf, -np.inf, 3e38, -3e38, 1e9, -1e9, 16777217.0],
                   np.float32)
    G = np.zeros((1, 1, bad.size, 2), np.float32)
    G[0, 0, :, 0] = bad
    G[0, 0, :, 1] = 0.1
    Y = oracle_mod.grid_sample(X, G, mode, pad, 0)
    assert np.all(np.isfinite(Y))
    # non-finite locations read 0 (a memory-safety reading; the pages are silent)
    assert np.all(Y[0, :, 0, :3] == 0.0)
    if pad == "zeros":
        assert np.all(Y == 0.0)
    else:
        assert np.all(np.abs(Y) <= np.abs(X).max() * 1.6)
