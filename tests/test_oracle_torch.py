"""Oracle cross-checked against the torch CPU functions the pages name under
"See also" (torch.nn.functional.affine_grid and grid_sample).

This is a black-box comparison on random inputs, not a pin of the values: the
comparator builds its grid with a different fp32 operation order, so nearest
is compared exactly only away from rounding ties, and linear / cubic within a
small tolerance.  It covers the combinations no printed example reaches
(cubic with border and reflection, nearest with border and reflection).
torch has no 3D cubic; those combinations are covered by the brute force.
"""

import itertools

import numpy as np
import pytest

torch = pytest.importorskip("torch")
F = torch.nn.functional

COMBOS_2D = list(itertools.product(["nearest", "linear", "cubic"],
                                   ["zeros", "border", "reflection"], [0, 1]))
COMBOS_3D = list(itertools.product(["nearest", "linear"], ["zeros", "border", "reflection"], [0, 1]))

TORCH_MODE = {"nearest": "nearest", "linear": "bilinear", "cubic": "bicubic"}


def torch_sample(X, G, mode, pad, ac):
    return F.grid_sample(torch.from_numpy(X).double(), torch.from_numpy(G).double(),
                         mode=TORCH_MODE[mode], padding_mode=pad,
                         align_corners=bool(ac)).numpy()


def tie_distance(G, in_sp, ac):
    """Distance of each location's pixel coordinate to the nearest .5 tie."""
    r = len(in_sp)
    d = np.full(G.shape[:-1], np.inf)
    for a in range(r):
        g = G[..., r - 1 - a].astype(np.float64)
        n = in_sp[a]
        p = (g + 1) / 2 * (n - 1) if ac else ((g + 1) * n - 1) / 2
        d = np.minimum(d, np.abs(np.abs(p - np.floor(p)) - 0.5))
        # reflection folds the location; folded ties sit at the same distance
    return d


@pytest.mark.parametrize("mode,pad,ac", COMBOS_2D + [("3d-" + m, p, a) for m, p, a in COMBOS_3D])
def test_oracle_agrees_with_torch_cpu(oracle_mod, mode, pad, ac):
    rank = 3 if mode.startswith("3d-") else 2
    mode = mode.replace("3d-", "")
    rng = np.random.default_rng(11 + 3 * ac)
    in_sp = (7, 9) if rank == 2 else (4, 5, 6)
    out = (6, 8) if rank == 2 else (3, 4, 5)
    X = rng.uniform(-1, 1, (2, 3) + in_sp).astype(np.float32)
    G = rng.uniform(-1.6, 1.6, (2,) + out + (rank,)).astype(np.float32)
    Y = oracle_mod.grid_sample(X, G, mode, pad, ac)
    T = torch_sample(X, G, mode, pad, ac)
    if mode == "nearest":
        safe = tie_distance(G, in_sp, ac) > 1e-4
        safe = np.broadcast_to(safe[:, None], Y.shape)
        assert safe.mean() > 0.9
        assert np.array_equal(Y[safe], T[safe])
    else:
        assert np.abs(Y - T).max() <= 1e-5 * np.abs(X).max()


@pytest.mark.parametrize("ac", [0, 1])
@pytest.mark.parametrize("size", [(3, 2, 5, 6), (2, 3, 4, 5, 6), (2, 1, 1, 7)])
def test_affine_grid_agrees_with_torch_cpu(oracle_mod, ac, size):
    r = len(size) - 2
    rng = np.random.default_rng(12 + ac)
    theta = rng.normal(size=(size[0], r, r + 1)).astype(np.float32)
    grid = oracle_mod.affine_grid(theta, size, ac)
    ref = F.affine_grid(torch.from_numpy(theta).double(), list(size), align_corners=bool(ac)).numpy()
    scale = np.abs(theta).sum(axis=2).max()
    assert np.abs(grid - ref).max() <= 4e-7 * max(1.0, scale)
