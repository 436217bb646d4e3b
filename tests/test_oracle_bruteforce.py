"""Oracle against a dense-lattice brute force on tiny inputs.

The brute force writes every mode as one kernel k applied to the distance
from the sampling position p to *every* lattice point j of a padded copy of X:

    Y(p) = sum_j  prod_d k(p_d - j_d) * Xpad[j]

so it has no floor, no tap window and no per-tap bookkeeping.  The padded copy
comes from numpy.pad: 'constant' (zeros), 'edge' (border), and for reflection
'reflect' (mirror about the edge pixel centre, the align_corners=1 bounds) or
'symmetric' (mirror about the outer pixel edge, the align_corners=0 bounds).

Kernels: nearest = indicator of the closest lattice point, ties to the even
index; linear = the tent max(0, 1-|s|); cubic = Keys' cubic convolution kernel
with a = -0.75 (its values are fixed independently by the bicubic examples of
the GridSample page and the Resize cubic examples).

Sampling positions p are computed in fp32 from the normalised location, as
the un-normalisation fixed by the printed examples; this keeps nearest
comparisons exact.  Every mode x padding x align_corners combination runs in
1-D to 4-D, with fp32 and float64 grids, on extents 1..5 including extent-1
axes.
"""

import itertools

import numpy as np
import pytest

A = -0.75


def keys(s):
    x = np.abs(s)
    near = (A + 2) * x**3 - (A + 3) * x**2 + 1
    far = A * x**3 - 5 * A * x**2 + 8 * A * x - 4 * A
    return np.where(x <= 1, near, np.where(x < 2, far, 0.0))


def tent(s):
    return np.maximum(0.0, 1.0 - np.abs(s))


def nearest_kernel(s, j):
    """1 where j is the lattice point nearest to p = s + j (ties -> even j)."""
    a = np.abs(s)
    return np.where(a < 0.5, 1.0, np.where((a == 0.5) & (j % 2 == 0), 1.0, 0.0))


def pixel_position(g, n, ac, double=False):
    """Un-normalisation in the grid's precision (fp32, or float64 for a
    double grid)."""
    f = np.float64 if double else np.float32
    g = f(g)
    one = f(1)
    if ac:
        return ((g + one) / f(2)) * f(n - 1)
    return ((g + one) * f(n) - one) / f(2)


def pad_mode(padding, ac):
    if padding == "zeros":
        return "constant"
    if padding == "border":
        return "edge"
    return "reflect" if ac else "symmetric"


def brute_force(X, grid, mode, padding, ac):
    N, C = X.shape[:2]
    in_sp = X.shape[2:]
    double = grid.dtype == np.float64
    r = len(in_sp)
    out_sp = grid.shape[1:-1]
    # lattice large enough to hold every tap of every location in the tests
    L = 4 * max(in_sp) + 8
    Y = np.zeros((N, C) + tuple(out_sp))
    for n in range(N):
        Xp = np.pad(X[n].astype(np.float64), [(0, 0)] + [(L, L)] * r, mode=pad_mode(padding, ac))
        for o in itertools.product(*[range(m) for m in out_sp]):
            g = grid[(n,) + o]
            weights = []
            for a in range(r):
                # component k of the location vector addresses axis r-1-k
                p = float(pixel_position(g[r - 1 - a], in_sp[a], ac, double))
                j = np.arange(-L, in_sp[a] + L)
                s = p - j
                if mode == "nearest":
                    w = nearest_kernel(s, j)
                elif mode == "linear":
                    w = tent(s)
                else:
                    w = keys(s)
                weights.append(w)
            # outer product of the per-axis weights over the padded lattice
            W = weights[0]
            for w in weights[1:]:
                W = np.multiply.outer(W, w)
            Y[(n, slice(None)) + o] = np.tensordot(Xp, W, axes=r)
    return Y


COMBOS = list(itertools.product(["nearest", "linear", "cubic"], ["zeros", "border", "reflection"], [0, 1]))


@pytest.mark.parametrize("mode,padding,ac", COMBOS)
@pytest.mark.parametrize("rank", [1, 2, 3, 4])
@pytest.mark.parametrize("precision", ["f32", "f64"])
def test_oracle_matches_dense_lattice(oracle_mod, mode, padding, ac, rank, precision):
    """Every rank the page defines in general (1-D, 2-D, 3-D, 4-D here), with
    fp32 grids and X, and with float64 grids and X (coordinates in float64)."""
    rng = np.random.default_rng(100 + 7 * rank + 31 * ac)
    dt = np.float32 if precision == "f32" else np.float64
    for trial in range(4 if rank < 4 else 2):
        hi = 6 if rank < 4 else 4
        in_sp = tuple(int(v) for v in rng.integers(1, hi, size=rank))
        if trial == 0:
            in_sp = (1,) * rank                       # all extents 1
        out_sp = tuple(int(v) for v in rng.integers(1, 4 if rank < 4 else 3, size=rank))
        X = rng.uniform(-1, 1, size=(2, 2) + in_sp).astype(dt)
        G = rng.uniform(-1.7, 1.7, size=(2,) + out_sp + (rank,)).astype(dt)
        Y = oracle_mod.grid_sample(X, G, mode, padding, ac)
        B = brute_force(X, G, mode, padding, ac)
        if mode == "nearest":
            assert np.array_equal(Y, B), (in_sp, out_sp)
        else:
            np.testing.assert_allclose(Y, B, rtol=0, atol=1e-12, err_msg=str((in_sp, out_sp)))


def test_brute_force_nearest_tie_goes_to_even():
    # location exactly halfway between pixels 0 and 1 of a 2-wide row:
    # the GridSample page rounds it to the even index 0.
    X = np.array([[[[10.0, 20.0]]]], np.float32)
    G = np.array([[[[0.0, 0.0]]]], np.float32)     # p = 0.5 with align_corners=0
    assert brute_force(X, G, "nearest", "zeros", 0)[0, 0, 0, 0] == 10.0
