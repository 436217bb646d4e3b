"""The 2-D gather path (gs_grid_sample_2d_ws) against the oracle and against
the plain sampler.

* Random-flow grids (locations i.i.d. over [-1.2, 1.2]): the device probe
  must choose the gather path (its 64 verdict words, the workspace's first
  256 bytes, sum to 32 or more), and the result must equal gs_grid_sample_2d
  bit for bit -- the same taps, weights and fp32 sums in the same order -- and
  the oracle within the tolerances of tests/parity.py.  Every mode, padding,
  align_corners and element type; 64-byte channel slices (one, four, many)
  and 32-byte ones (three, one), fewer (image, slice) planes than XCDs and
  more; output rows that end in a ragged 64- or 128-location segment;
  non-finite locations.
* Near-identity affine grids: the probe keeps the staged sampler (verdicts
  sum below 32), and the result equals gs_grid_sample_2d bit for bit.  So do
  random flows over images small enough for a tile's LDS slot, grids with a
  few scattered tiles (the sampler gathers those from X), and grids mostly
  scattered with some smooth tiles (the gather kernel writes every output).
* The workspace's contents before the call do not matter, and the call
  replays correctly from a captured graph.
* Without a workspace, or one too small, the call is gs_grid_sample_2d.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, from_gpu, note, torch_mod, x_to_gpu

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


def verdict_sum(ws):
    """Probes (of 64) that found their tile scattered: the workspace's first
    256 bytes hold their verdict words."""
    return int(ws[:256].cpu().numpy().view(np.int32)[:64].sum())


def run_case(gsa, X32, G, kind, mode, pad, ac, expect_gather, what):
    torch = torch_mod()
    note("gather %s %s %s %s ac=%d X=%s G=%s" % (what, kind, mode, pad, ac, X32.shape, G.shape))
    Xd, Xo = x_to_gpu(X32, kind)
    Gd = torch.from_numpy(np.ascontiguousarray(G, np.float32)).cuda()
    need = gsa.grid_sample_2d_workspace_size(tuple(X32.shape), tuple(G.shape), gsa.dtype_code(Xd))
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Yw = gsa.grid_sample(Xd, Gd, mode, pad, ac, workspace=ws)
    Yp = gsa.grid_sample(Xd, Gd, mode, pad, ac)
    torch.cuda.synchronize()
    vs = verdict_sum(ws)
    assert (vs >= 32) == expect_gather, "verdicts %d" % vs
    a = Yw.view(torch.int16 if kind != "f32" else torch.int32).cpu().numpy()
    b = Yp.view(torch.int16 if kind != "f32" else torch.int32).cpu().numpy()
    ref = oracle.grid_sample(Xo, G, mode, pad, ac)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        i = tuple(bad[0])
        raise AssertionError("%s: %d elements differ from the plain sampler, first %s: %r vs %r, "
                             "oracle %r, location %r" % (what, len(bad), i, float(Yw[i]),
                                                         float(Yp[i]), ref[i], G[i[0], i[2], i[3]]))
    check(from_gpu(Yw), ref, mode, kind, float(np.abs(Xo).max()), what)


def random_grid(rng, n, ho, wo):
    return rng.uniform(-1.2, 1.2, (n, ho, wo, 2)).astype(np.float32)


# Input planes of more than 256 rows: the box of a tile's scattered
# locations spans more rows than the sampler stages (256), so the probes find
# every tile scattered, however few locations it holds.
CASES = [
    # n, c (f32), c (half), h, w, ho, wo
    (2, 16, 32, 320, 104, 9, 140),   # one 64-byte slice, three row segments, the last ragged
    (1, 24, 48, 330, 110, 17, 64),   # three 32-byte slices, one ragged row segment
    (3, 64, 128, 321, 101, 5, 13),   # 12 planes of 64-byte slices (XCD order), narrow rows
    (2, 8, 16, 337, 99, 4, 300),     # one 32-byte slice, three row segments
    (1, 128, 256, 326, 104, 1, 50),  # 8 slices, one row: one block per XCD (one counter)
    (1, 128, 256, 326, 104, 2, 50),  # 8 slices, two rows: two counters per XCD
]


@pytest.mark.parametrize("kind,ci,mode,pad,ac", list(itertools.product(
    ["f32", "f16", "bf16"], range(len(CASES)), MODES, PADS, [0, 1])))
def test_random_flow_takes_the_gather_path(gsa, kind, ci, mode, pad, ac):
    n, c32, c16, h, w, ho, wo = CASES[ci]
    c = c32 if kind == "f32" else c16
    rng = np.random.default_rng(1000 + ci)
    X = rng.uniform(-1, 1, (n, c, h, w)).astype(np.float32)
    G = random_grid(rng, n, ho, wo)
    run_case(gsa, X, G, kind, mode, pad, ac, True, "case %d" % ci)


@pytest.mark.parametrize("mode", MODES)
def test_non_finite_locations(gsa, mode):
    rng = np.random.default_rng(7)
    X = rng.uniform(-1, 1, (1, 8, 320, 100)).astype(np.float32)
    G = random_grid(rng, 1, 6, 20)
    G[0, 0, :4, 0] = np.nan
    G[0, 1, 2:5, 1] = np.inf
    G[0, 2, 7, :] = -np.inf
    run_case(gsa, X, G, "f32", mode, "reflection", 1, True, "non-finite")


def test_many_slices(gsa):
    """Few output rows, 32 channel slices walked in XCD order."""
    rng = np.random.default_rng(8)
    X = rng.uniform(-1, 1, (1, 256, 320, 91)).astype(np.float32)
    G = random_grid(rng, 1, 2, 40)
    run_case(gsa, X, G, "f32", "cubic", "border", 0, True, "many slices")


@pytest.mark.parametrize("mode", MODES)
def test_affine_grid_keeps_the_staged_sampler(gsa, mode):
    rng = np.random.default_rng(9)
    X = rng.uniform(-1, 1, (2, 16, 40, 48)).astype(np.float32)
    theta = np.tile(np.array([[0.9, 0.05, 0.02], [-0.04, 1.1, -0.03]], np.float32), (2, 1, 1))
    G = oracle.affine_grid(theta, (2, 16, 36, 44), 0).astype(np.float32)
    run_case(gsa, X, G, "f32", mode, "zeros", 0, False, "affine")


def test_small_image_keeps_the_staged_sampler(gsa):
    """A whole 23 x 37 plane fits a tile's LDS slot: scattered locations are
    still staged."""
    rng = np.random.default_rng(12)
    X = rng.uniform(-1, 1, (2, 16, 23, 37)).astype(np.float32)
    G = random_grid(rng, 2, 9, 70)
    run_case(gsa, X, G, "f32", "linear", "border", 1, False, "small image")


def centre_grid(n, ho, wo, zoom=1.0):
    """Pixel-centre locations (align_corners = 0) scaled by `zoom`: a grid
    every tile of which the sampler stages."""
    xs = ((2.0 * np.arange(wo) + 1.0) / wo - 1.0) * zoom
    ys = ((2.0 * np.arange(ho) + 1.0) / ho - 1.0) * zoom
    g = np.empty((n, ho, wo, 2), np.float32)
    g[..., 0] = xs[None, None, :]
    g[..., 1] = ys[None, :, None]
    return g


@pytest.mark.parametrize("kind,mode", list(itertools.product(["f32", "bf16"], MODES)))
def test_few_scattered_tiles_gather_from_x(gsa, kind, mode):
    """Random locations in the first 16 output rows of one image, a smooth
    grid elsewhere: two of the 64 probes find their tile scattered, so the
    sampler runs and gathers those tiles' taps from X; the result equals the
    plain sampler bit for bit."""
    rng = np.random.default_rng(21)
    X = rng.uniform(-1, 1, (2, 16, 320, 100)).astype(np.float32)
    G = centre_grid(2, 256, 64, 0.9)
    G[0, :16] = random_grid(rng, 1, 16, 64)[0]
    run_case(gsa, X, G, kind, mode, "border", 0, False, "few scattered")


@pytest.mark.parametrize("mode", MODES)
def test_mostly_scattered_with_staged_tiles_takes_the_gather_path(gsa, mode):
    """Random locations over the first 192 of 256 output rows of every image
    and a smooth grid below: the gather path writes every output, the
    staged tiles' included, with the same bits."""
    rng = np.random.default_rng(22)
    X = rng.uniform(-1, 1, (2, 16, 320, 100)).astype(np.float32)
    G = centre_grid(2, 256, 64, 0.9)
    G[:, :192] = random_grid(rng, 2, 192, 64)
    run_case(gsa, X, G, "f32", mode, "zeros", 1, True, "mostly scattered")


def test_workspace_contents_do_not_matter(gsa):
    """The call reads nothing a previous call, or garbage, left in the
    workspace: a smooth grid after a random one, and a random one after a
    smooth one, on the same workspace filled with 0xff first."""
    torch = torch_mod()
    rng = np.random.default_rng(23)
    X = torch.from_numpy(rng.uniform(-1, 1, (2, 16, 320, 100)).astype(np.float32)).cuda()
    Gs = torch.from_numpy(centre_grid(2, 256, 64, 0.9)).cuda()
    Gr = torch.from_numpy(random_grid(rng, 2, 256, 64)).cuda()
    need = gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(Gs.shape), 0)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for G, gather in ((Gs, False), (Gr, True), (Gs, False), (Gr, True)):
        note("workspace reuse, gather %s" % gather)
        Yw = gsa.grid_sample(X, G, "linear", "zeros", 0, workspace=ws)
        Yp = gsa.grid_sample(X, G, "linear", "zeros", 0)
        torch.cuda.synchronize()
        assert (verdict_sum(ws) >= 32) == gather
        assert torch.equal(Yw, Yp)


@pytest.mark.parametrize("kind", ["smooth", "random"])
def test_captured_graph_replays(gsa, kind):
    """The call captured in a graph and replayed, X changed in between:
    every replay equals the eager plain sampler on that X (the probe
    rewrites its verdicts and resets the gather kernel's counters each
    time; no memset node is recorded)."""
    torch = torch_mod()
    rng = np.random.default_rng(24)
    X = torch.from_numpy(rng.uniform(-1, 1, (2, 16, 320, 100)).astype(np.float32)).cuda()
    G = torch.from_numpy(centre_grid(2, 256, 64, 0.9) if kind == "smooth"
                         else random_grid(rng, 2, 256, 64)).cuda()
    need = gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(G.shape), 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Y = torch.empty((2, 16, 256, 64), device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gsa.grid_sample(X, G, "linear", "zeros", 0, out=Y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gsa.grid_sample(X, G, "linear", "zeros", 0, out=Y, workspace=ws)
    for rep in range(4):
        note("graph replay %d (%s grid)" % (rep, kind))
        X.copy_(torch.from_numpy(rng.uniform(-1, 1, tuple(X.shape)).astype(np.float32)).cuda())
        graph.replay()
        Yp = gsa.grid_sample(X, G, "linear", "zeros", 0)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yp), "replay %d differs from the eager result" % rep
        assert (verdict_sum(ws) >= 32) == (kind == "random")


def test_without_workspace_is_the_plain_sampler(gsa):
    torch = torch_mod()
    rng = np.random.default_rng(10)
    X = torch.from_numpy(rng.uniform(-1, 1, (1, 16, 100, 100)).astype(np.float32)).cuda()
    G = torch.from_numpy(random_grid(rng, 1, 8, 8)).cuda()
    a = gsa.grid_sample(X, G, "cubic", "zeros", 0, workspace=torch.empty(0, dtype=torch.uint8,
                                                                          device="cuda"))
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    b = gsa.grid_sample(X, G, "cubic", "zeros", 0, workspace=small)
    c = gsa.grid_sample(X, G, "cubic", "zeros", 0)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(b, c)
    assert int(small.sum()) == 0            # too small: untouched


def test_full_size_random_flow_all_elements(gsa):
    """The flow2d_bicubic workload at its full size through the gather path:
    the verdicts, bit-equality with the plain sampler, and every output
    against the oracle (its OpenMP build), image by image."""
    torch = torch_mod()
    wl = W.WORKLOADS["flow2d_bicubic"]
    inp = W.make_inputs(wl)
    note("gather full-size flow2d_bicubic")
    X = torch.from_numpy(inp["X"]).cuda()
    G = torch.from_numpy(inp["grid"]).cuda()
    need = gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(G.shape), gsa.dtype_code(X))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Yw = gsa.grid_sample(X, G, wl.mode, wl.padding, wl.align_corners, workspace=ws)
    Yp = gsa.grid_sample(X, G, wl.mode, wl.padding, wl.align_corners)
    torch.cuda.synchronize()
    assert verdict_sum(ws) >= 32
    assert torch.equal(Yw, Yp)
    del ws, Yp, X, G
    got = from_gpu(Yw)
    del Yw
    par = oracle.parallel()
    xmax = float(np.abs(inp["X"]).max())
    for b in range(got.shape[0]):
        ref = oracle.grid_sample(inp["X"][b:b + 1], inp["grid"][b:b + 1], wl.mode, wl.padding,
                                 wl.align_corners, lib=par)
        check(got[b:b + 1], ref, wl.mode, "f32", xmax, "gather full-size image %d" % b)
