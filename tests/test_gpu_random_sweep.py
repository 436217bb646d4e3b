"""Seeded random sweep of the sampler against the oracle.

Each case draws its own shapes and attributes from its seed: spatial rank,
mode, padding, align_corners, element type, batch, a channel count that
leaves a remainder after the kernels' channel groups, input and output
extents that do not divide the tiles (extents of 1 included), and one of
four grid kinds:

* i.i.d. locations over [-1.3, 1.3] (the direct-gather path);
* an affine map with a random zoom, rotation and shift (the LDS-staged path,
  with tiles partly or wholly outside the image);
* a smooth flow with a random amplitude, locally folding;
* a mixture: a smooth grid with a random share of its locations replaced by
  i.i.d. ones (staged and direct tiles in one launch).

2-D cases also run through the workspace entry (the gather path when the
probe finds the grid scattered) in a third of the cases, and the affine kind
also through the fused entry (bit-identical to the unfused pair).  The
tolerances are those of the other parity tests (tests/parity.py).

Further sweeps: Resize, the any-rank kernel, DeformConv and the gather path
(through the helpers of their own test files), and one graph holding every
entry point, replayed with new inputs.
"""

import numpy as np
import pytest

import oracle
from parity import check, from_gpu, note, to_gpu_f32, torch_mod, x_to_gpu

pytestmark = pytest.mark.gpu

MODES = ["nearest", "linear", "cubic"]
PADS = ["zeros", "border", "reflection"]
KINDS = ["f32", "f16", "bf16"]
GRIDS = ["iid", "affine", "flow", "mixed"]
N_CASES = 384


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def draw_case(seed):
    rng = np.random.default_rng(90000 + seed)
    rank = 3 if rng.random() < 0.3 else 2
    mode = MODES[rng.integers(3)]
    pad = PADS[rng.integers(3)]
    ac = int(rng.integers(2))
    kind = KINDS[rng.integers(3)]
    grid_kind = GRIDS[rng.integers(4)]
    n = int(rng.integers(1, 4))
    c = int(rng.choice([1, 3, 5, 8, 13, 24, 37, 64, 70]))
    if rank == 2:
        in_sp = tuple(int(rng.choice([1, 2, 7, 16, 33, 48, 65])) for _ in range(2))
        out_sp = tuple(int(rng.choice([1, 3, 17, 32, 40, 64, 129])) for _ in range(2))
    else:
        in_sp = tuple(int(rng.choice([1, 2, 5, 9, 16])) for _ in range(3))
        out_sp = tuple(int(rng.choice([1, 3, 4, 7, 12])) for _ in range(3))
    # keep the oracle's work small
    while n * c * int(np.prod(out_sp)) > 600_000:
        c = max(1, c // 2)
    return dict(rng=rng, rank=rank, mode=mode, pad=pad, ac=ac, kind=kind, grid_kind=grid_kind,
                n=n, c=c, in_sp=in_sp, out_sp=out_sp)


def base_grid(out_sp):
    """Pixel-centre positions over [-1, 1], innermost axis first in the last dim."""
    axes = [-1.0 + (2.0 * np.arange(m) + 1.0) / m for m in out_sp]
    mesh = np.meshgrid(*axes, indexing="ij")
    return np.stack(mesh[::-1], axis=-1)


def make_theta(rng, n, r):
    theta = np.zeros((n, r, r + 1))
    for b in range(n):
        zoom = np.exp(rng.uniform(-0.7, 0.7))
        q, _ = np.linalg.qr(rng.normal(size=(r, r)))
        angle_mix = rng.uniform(0, 0.6)
        m = (1 - angle_mix) * np.eye(r) + angle_mix * q
        theta[b, :, :r] = zoom * m
        theta[b, :, r] = rng.uniform(-0.4, 0.4, r)
    return theta.astype(np.float32)


def make_grid(case):
    rng, n, r, out_sp = case["rng"], case["n"], case["rank"], case["out_sp"]
    shape = (n,) + out_sp + (r,)
    kind = case["grid_kind"]
    if kind == "iid":
        return rng.uniform(-1.3, 1.3, shape).astype(np.float32), None
    if kind == "affine":
        theta = make_theta(rng, n, r)
        return oracle.affine_grid(theta, (n, 1) + out_sp, case["ac"]).astype(np.float32), theta
    g = np.broadcast_to(base_grid(out_sp), shape).astype(np.float64).copy()
    amp = rng.uniform(0.02, 0.25)
    for b in range(n):
        for k in range(r):
            u = rng.uniform(-2, 2, r)
            phase = rng.uniform(0, 2 * np.pi)
            arg = sum(u[a] * g[b, ..., a] for a in range(r))
            g[b, ..., k] += amp * np.sin(2 * np.pi * arg + phase)
    if kind == "mixed":
        share = rng.uniform(0.05, 0.9)
        hit = rng.random(g.shape[:-1]) < share
        g[hit] = rng.uniform(-1.3, 1.3, (int(hit.sum()), r))
    return g.astype(np.float32), None


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case_matches_oracle(gsa, seed):
    case = draw_case(seed)
    rng, r = case["rng"], case["rank"]
    mode, pad, ac, kind = case["mode"], case["pad"], case["ac"], case["kind"]
    X = rng.uniform(-1, 1, (case["n"], case["c"]) + case["in_sp"]).astype(np.float32)
    G, theta = make_grid(case)
    use_ws = r == 2 and rng.random() < 1 / 3
    what = "seed %d: %dD %s/%s ac=%d %s grid=%s X=%s out=%s ws=%s" % (
        seed, r, mode, pad, ac, kind, case["grid_kind"], X.shape, case["out_sp"], use_ws)
    note(what)
    Xd, Xin = x_to_gpu(X, kind)
    ref = oracle.grid_sample(Xin, G, mode, pad, ac)
    Gd = to_gpu_f32(G)
    Y = from_gpu(gsa.grid_sample(Xd, Gd, mode, pad, ac, workspace="auto" if use_ws else None))
    check(Y, ref, mode, kind, np.abs(Xin).max(), what)
    if theta is not None:
        td = to_gpu_f32(theta)
        F = from_gpu(gsa.affine_grid_sample_fused(td, Xd, case["out_sp"], mode, pad, ac))
        U = from_gpu(gsa.grid_sample(Xd, gsa.affine_grid(td, X.shape[:2] + case["out_sp"], ac),
                                     mode, pad, ac))
        assert np.array_equal(F, U), what + ": fused differs from unfused"
        check(F, ref, mode, kind, np.abs(Xin).max(), what + " (fused)")


# ------------------------------------------------------------------ Resize

CTMS = ["half_pixel", "pytorch_half_pixel", "align_corners", "asymmetric"]
NEAREST = ["round_prefer_floor", "round_prefer_ceil", "floor", "ceil"]


@pytest.mark.parametrize("seed", range(128))
def test_random_resize_matches_oracle(gsa, seed):
    """Random Resize: 1 to 3 resized trailing axes, scales from 0.3 to 3.1
    (the output extent floor(n * scale)) or free output extents, every mode,
    coordinate transformation, nearest rounding, cubic coefficient and
    exclude_outside, and element type."""
    from test_gpu_resize import run_case

    rng = np.random.default_rng(91000 + seed)
    r = int(rng.choice([1, 2, 2, 3]))
    lead = tuple(int(v) for v in rng.integers(1, 4, 2))
    in_sp = tuple(int(rng.integers(1, 40 if r < 3 else 12)) for _ in range(r))
    mode = MODES[rng.integers(3)]
    kind = KINDS[rng.integers(3)]
    ctm = CTMS[rng.integers(4)]
    nm = NEAREST[rng.integers(4)]
    a = float(rng.choice([-0.5, -0.75]))
    ex = int(rng.integers(2))
    if rng.random() < 0.6:
        sc = [float(np.float32(rng.uniform(0.3, 3.1))) for _ in range(r)]
        out_sp = tuple(max(1, int(np.floor(n * s))) for n, s in zip(in_sp, sc))
        scales = [1.0] * len(lead) + sc
    else:
        out_sp = tuple(int(rng.integers(1, 60 if r < 3 else 14)) for _ in range(r))
        scales = None
    X = rng.uniform(-1, 1, lead + in_sp).astype(np.float32)
    run_case(gsa, X, lead + out_sp, scales, mode, ctm, nm, a, ex, kind=kind)


# ---------------------------------------------------- any rank, any type

TYPE_KINDS = ["f64", "f32", "f16", "int8", "uint8", "int16", "int32"]
GRID_KINDS = ["f32", "f64", "f16", "bf16"]


@pytest.mark.parametrize("seed", range(128))
def test_random_any_rank_type_matches_oracle(gsa, seed):
    """Random GridSample through the any-rank kernel: ranks 1 to 4, float and
    integer element types, fp32 / double / half grids; compared bit for bit
    after the output conversion (as the other any-rank tests)."""
    from test_gpu_types import run

    rng = np.random.default_rng(92000 + seed)
    r = int(rng.choice([1, 2, 3, 4]))
    mode = MODES[rng.integers(3)] if r < 4 else MODES[rng.integers(2)]
    pad = PADS[rng.integers(3)]
    ac = int(rng.integers(2))
    kind = TYPE_KINDS[rng.integers(len(TYPE_KINDS))]
    grid_kind = GRID_KINDS[rng.integers(len(GRID_KINDS))]
    if r in (2, 3) and kind in ("f32", "f16") and grid_kind == "f32":
        grid_kind = "f64"  # those go to the tuned kernels; keep this sweep on the any-rank one
    lim = {1: 300, 2: 24, 3: 9, 4: 5}[r]
    n, c = int(rng.integers(1, 3)), int(rng.integers(1, 6))
    in_sp = tuple(int(rng.integers(1, lim)) for _ in range(r))
    out_sp = tuple(int(rng.integers(1, lim)) for _ in range(r))
    if kind in ("f64", "f32", "f16"):
        X = rng.uniform(-2, 2, (n, c) + in_sp)
        X = X.astype(np.float64 if kind == "f64" else np.float32)
    else:
        info = np.iinfo(np.dtype(kind))
        X = rng.integers(max(info.min, -(1 << 20)), min(info.max, 1 << 20), (n, c) + in_sp,
                         endpoint=True).astype(np.dtype(kind))
    G = rng.uniform(-1.3, 1.3, (n,) + out_sp + (r,))
    G = G if grid_kind == "f64" else G.astype(np.float32)
    run(gsa, X, G, mode, pad, ac, kind, grid_kind, what="sweep seed %d rank %d" % (seed, r))


# -------------------------------------------------------------- DeformConv

@pytest.mark.parametrize("seed", range(96))
def test_random_deform_conv_matches_oracle(gsa, seed):
    """Random 2-D DeformConv: channel counts that do and do not fill the
    channels-last chunks, groups and offset groups, strides, pads,
    dilations, kernel sizes up to 5, optional mask and bias, with and without
    a workspace, fp32 / fp16 / bf16 (the derived tolerance of the DeformConv
    tests)."""
    from test_gpu_deform import case, run

    rng = np.random.default_rng(93000 + seed)
    grp = int(rng.choice([1, 1, 2, 4]))
    cg = int(rng.choice([1, 3, 8, 16, 24, 40]))
    c = grp * cg
    og = int(rng.choice([d for d in range(1, c + 1) if c % d == 0][:4]))
    oc = grp * int(rng.choice([1, 5, 32, 70, 150]))
    kh, kw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    st = [int(v) for v in rng.integers(1, 3, 2)]
    dl = [int(v) for v in rng.integers(1, 3, 2)]
    pd = [int(v) for v in rng.integers(0, 3, 4)]
    n = int(rng.integers(1, 3))
    h = int(rng.integers(dl[0] * (kh - 1) + 1, 24))
    w = int(rng.integers(dl[1] * (kw - 1) + 1, 24))
    kind = KINDS[rng.integers(3)]
    with_mask, with_bias = bool(rng.integers(2)), bool(rng.integers(2))
    X, Wt, off, B, M = case(94000 + seed, n, c, h, w, oc, kh, kw, st, pd, dl, grp, og,
                            with_mask, with_bias)
    run(gsa, X, Wt, off, B, M, kind, st, pd, dl, grp, og,
        what="sweep seed %d" % seed, no_workspace=bool(rng.integers(2)))


# ------------------------------------------------------------- gather path

@pytest.mark.parametrize("seed", range(64))
def test_random_gather_path_matches_oracle(gsa, seed):
    """Random scattered grids over planes taller than the sampler stages (the
    probe chooses the gather path): channel counts that fill 32- or 64-byte
    slices, one to three images, output rows that leave ragged row segments;
    the gather path equals the plain sampler bit for bit and the oracle
    within tolerance."""
    from test_gpu_gather import run_case as run_gather_case

    rng = np.random.default_rng(95000 + seed)
    kind = KINDS[rng.integers(3)]
    per_slice = 8 if kind == "f32" else 16          # channels in 32 bytes
    c = per_slice * int(rng.choice([1, 2, 3, 4, 6, 8]))
    n = int(rng.integers(1, 4))
    h, w = int(rng.integers(300, 340)), int(rng.integers(60, 130))
    ho, wo = int(rng.integers(1, 24)), int(rng.integers(1, 300))
    mode, pad, ac = MODES[rng.integers(3)], PADS[rng.integers(3)], int(rng.integers(2))
    X = rng.uniform(-1, 1, (n, c, h, w)).astype(np.float32)
    G = rng.uniform(-1.2, 1.2, (n, ho, wo, 2)).astype(np.float32)
    run_gather_case(gsa, X, G, kind, mode, pad, ac, True, "sweep seed %d" % seed)


# ------------------------------------------------------------ graph capture

def test_entry_points_captured_in_a_graph(gsa):
    """AffineGrid, the sampler (unfused and fused), Resize and DeformConv with
    a workspace captured in one graph and replayed four times, inputs changed
    in between with eager work and synchronisations between the replays:
    every replay equals the eager calls on the same inputs bit for bit (the
    library records no memset)."""
    torch = torch_mod()
    rng = np.random.default_rng(96000)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    X = dev(rng.uniform(-1, 1, (2, 16, 40, 44)))
    theta = dev(np.eye(2, 3)[None] + 0.1 * rng.normal(size=(2, 2, 3)))
    Xr = dev(rng.uniform(-1, 1, (2, 3, 30, 34)))
    Xd = dev(rng.uniform(-1, 1, (1, 16, 12, 13)))
    Wd = dev(rng.uniform(-1, 1, (24, 16, 3, 3)))
    Od = dev(rng.uniform(-2, 2, (1, 18, 12, 13)))
    Md = dev(rng.uniform(0, 1, (1, 9, 12, 13)))
    Bd = dev(rng.uniform(-1, 1, 24))
    grid = torch.empty((2, 36, 40, 2), device="cuda")
    Y1 = torch.empty((2, 16, 36, 40), device="cuda")
    Y2 = torch.empty_like(Y1)
    Y3 = torch.empty((2, 3, 61, 50), device="cuda")
    Y4 = torch.empty((1, 24, 12, 13), device="cuda")
    ws = torch.empty(gsa.deform_conv_workspace_size((1, 16, 12, 13), (24, 16, 3, 3), 0, None,
                                                   [1, 1, 1, 1], None, 1, 1),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0

    def calls():
        gsa.affine_grid(theta, (2, 16, 36, 40), 0, out=grid)
        gsa.grid_sample(X, grid, "linear", "border", 0, out=Y1)
        gsa.affine_grid_sample_fused(theta, X, (36, 40), "cubic", "reflection", 0, out=Y2)
        gsa.resize_to(Xr, (2, 3, 61, 50), None, "cubic", "half_pixel", out=Y3)
        gsa.deform_conv(Xd, Wd, Od, Bd, Md, pads=[1, 1, 1, 1], out=Y4, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    outs = (Y1, Y2, Y3, Y4)
    for rep in range(4):
        note("multi-entry graph replay %d" % rep)
        for t in (X, theta, Xr, Xd, Od):
            t.copy_(dev(rng.uniform(-1, 1, tuple(t.shape)) * (0.1 if t is theta else 1.0)
                        + (np.eye(2, 3)[None] if t is theta else 0.0)))
        graph.replay()
        got = [y.clone() for y in outs]
        torch.cuda.synchronize()
        calls()   # eager, same inputs
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, outs)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager call" % (rep, k)


# ---------------------------------------------------------- extreme shapes

EXTREME = [
    # N, C, input spatial, output spatial
    (300, 3, (5, 5), (4, 6)),            # many images of one small tile each
    (1, 3000, (3, 4), (2, 3)),           # thousands of channels, tiny planes
    (2, 5, (1, 1000), (1, 999)),         # one-row images
    (2, 5, (1000, 1), (999, 1)),         # one-column images
    (1, 2, (700, 3), (2, 900)),          # tall input, wide output
    (1, 1, (1, 1), (50, 70)),            # one-pixel input
    (1, 2, (1, 1, 300), (1, 1, 299)),    # 3-D line
    (1, 3, (40, 1, 2), (3, 50, 2)),      # 3-D with unit axes
    (64, 1, (2, 2, 2), (3, 3, 3)),       # 3-D, many tiny volumes
]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("ci", range(len(EXTREME)))
def test_extreme_shapes(gsa, ci, mode, kind):
    n, c, in_sp, out_sp = EXTREME[ci]
    rng = np.random.default_rng(97000 + ci)
    r = len(in_sp)
    pad, ac = PADS[ci % 3], ci % 2
    X = rng.uniform(-1, 1, (n, c) + in_sp).astype(np.float32)
    G = rng.uniform(-1.2, 1.2, (n,) + out_sp + (r,)).astype(np.float32)
    what = "extreme %d: X=%s out=%s %s/%s ac=%d %s" % (ci, X.shape, out_sp, mode, pad, ac, kind)
    note(what)
    Xd, Xin = x_to_gpu(X, kind)
    Y = from_gpu(gsa.grid_sample(Xd, to_gpu_f32(G), mode, pad, ac))
    check(Y, oracle.grid_sample(Xin, G, mode, pad, ac), mode, kind, np.abs(Xin).max(), what)
