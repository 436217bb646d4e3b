"""Pointers aligned only to their element size.

A caller of the C ABI may pass any pointer into a buffer, and torch views with
a storage offset do the same.  The library checks each pointer before it takes
a 16-byte (or 8-byte) access path and otherwise takes the element-wise one.
Every case runs an entry point twice on the same values: once with each
tensor at the start of its own allocation (aligned to at least 256 bytes),
once with each tensor, inputs and output alike, one element past an aligned
base.  The outputs must agree bit for bit: both access paths load and store
the same elements, and the arithmetic of an output does not depend on which
one ran.  The aligned outputs of the sampler and Resize cases are also held to
the oracle (tolerances of the other parity tests); DeformConv's aligned
outputs are covered by its own parity tests.  A workspace that is not
256-byte aligned is not used: the call runs the path that needs none, with
the same outputs as a call without a workspace.
"""

import numpy as np
import pytest

import oracle
from parity import check, note, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def shifted_empty(shape, dtype):
    """An uninitialised tensor whose data starts one element past a 16-byte
    aligned base."""
    torch = torch_mod()
    n = int(np.prod(shape)) if len(shape) else 1
    buf = torch.empty(n + 1, dtype=dtype, device="cuda")
    v = buf[1:].view(tuple(shape))
    assert buf.data_ptr() % 16 == 0 and v.data_ptr() % 16 != 0
    return v


def shifted(t):
    """A copy of device tensor t one element past a 16-byte aligned base."""
    v = shifted_empty(tuple(t.shape), t.dtype)
    v.copy_(t)
    return v


def same_bits(a, b, what):
    torch = torch_mod()
    assert a.dtype == b.dtype and a.shape == b.shape, what
    if a.dtype.is_floating_point:
        ia = a.contiguous().view(torch.uint8)
        ib = b.contiguous().view(torch.uint8)
    else:
        ia, ib = a, b
    assert torch.equal(ia, ib), "%s: outputs differ between aligned and shifted pointers" % what


def gpu(a, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(dtype) if dtype is not None else t


def affine_theta(rng, n, r):
    eye = np.concatenate([np.eye(r), np.zeros((r, 1))], 1)[None].repeat(n, 0)
    return (eye + 0.1 * rng.normal(size=eye.shape)).astype(np.float32)


KINDS = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def host_values(Xd):
    return Xd.float().cpu().numpy()


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["linear", "nearest", "cubic"])
@pytest.mark.parametrize("grid_kind", ["affine", "iid"])
def test_sampler_2d(gsa, kind, mode, grid_kind):
    torch = torch_mod()
    what = "2-D sampler %s %s grid=%s" % (kind, mode, grid_kind)
    note(what)
    rng = np.random.default_rng(7100)
    X = gpu(rng.uniform(-1, 1, (2, 6, 40, 64)).astype(np.float32), getattr(torch, KINDS[kind]))
    if grid_kind == "affine":
        G = oracle.affine_grid(affine_theta(rng, 2, 2), (2, 6, 24, 32), 0).astype(np.float32)
    else:
        G = rng.uniform(-1.1, 1.1, (2, 24, 32, 2)).astype(np.float32)
    Gd = gpu(G)
    Ya = gsa.grid_sample(X, Gd, mode, "zeros", 0)
    Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
    gsa.grid_sample(shifted(X), shifted(Gd), mode, "zeros", 0, out=Ys)
    torch.cuda.synchronize()
    same_bits(Ya, Ys, what)
    Xh = host_values(X)
    ref = oracle.grid_sample(Xh, G, mode, "zeros", 0)
    check(Ya.double().cpu().numpy(), ref, mode, kind, float(np.abs(Xh).max()), what)


@pytest.mark.parametrize("mode", ["linear", "nearest"])
def test_sampler_3d_and_fused(gsa, mode):
    torch = torch_mod()
    rng = np.random.default_rng(7200)
    for r, xs, out in [(2, (2, 5, 40, 64), (24, 32)), (3, (1, 3, 8, 16, 16), (4, 8, 16))]:
        what = "%d-D sampler and fused %s" % (r, mode)
        note(what)
        X = gpu(rng.uniform(-1, 1, xs).astype(np.float32))
        theta = affine_theta(rng, xs[0], r)
        th = gpu(theta)
        Fa = gsa.affine_grid_sample_fused(th, X, out, mode, "border", 0)
        Fs = shifted_empty(tuple(Fa.shape), Fa.dtype)
        gsa.affine_grid_sample_fused(shifted(th), shifted(X), out, mode, "border", 0, out=Fs)
        Ga = gsa.affine_grid(th, xs[:2] + out, 0)
        Gs = shifted_empty(tuple(Ga.shape), Ga.dtype)
        gsa.affine_grid(shifted(th), xs[:2] + out, 0, out=Gs)
        Ya = gsa.grid_sample(X, Ga, mode, "border", 0)
        Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
        gsa.grid_sample(shifted(X), Gs, mode, "border", 0, out=Ys)
        torch.cuda.synchronize()
        same_bits(Fa, Fs, what + " (fused)")
        same_bits(Ga, Gs, what + " (AffineGrid)")
        same_bits(Ya, Ys, what + " (unfused)")
        G = oracle.affine_grid(theta, xs[:2] + out, 0)
        Xh = X.cpu().numpy()
        ref = oracle.grid_sample(Xh, G, mode, "border", 0)
        check(Fa.double().cpu().numpy(), ref, mode, "f32", float(np.abs(Xh).max()), what)


@pytest.mark.parametrize("kind", ["f64", "int8"])
def test_any_rank_kernel(gsa, kind):
    """Rank 1 with double or int8 data (element loads of 8 and 1 bytes)."""
    torch = torch_mod()
    what = "any-rank kernel %s" % kind
    note(what)
    rng = np.random.default_rng(7300)
    if kind == "f64":
        Xn = rng.uniform(-2, 2, (2, 3, 50))
    else:
        Xn = rng.integers(-128, 128, (2, 3, 50)).astype(np.int8)
    G = rng.uniform(-1.2, 1.2, (2, 40, 1))
    X, Gd = gpu(Xn), gpu(G)
    Ya = gsa.grid_sample(X, Gd, "linear", "reflection", 1)
    Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
    gsa.grid_sample(shifted(X), shifted(Gd), "linear", "reflection", 1, out=Ys)
    torch.cuda.synchronize()
    same_bits(Ya, Ys, what)
    ref = oracle.grid_sample(Xn.astype(np.float64), G, "linear", "reflection", 1)
    if kind == "int8":
        ref = oracle.to_integer(ref, np.dtype(np.int8))
    assert np.array_equal(Ya.cpu().numpy(), ref), what


def test_gather_path_and_unaligned_workspace(gsa):
    """The gather path (a workspace, a scattered grid over tall planes) with a
    shifted X; a shifted workspace runs the plain sampler instead."""
    from test_gpu_gather import verdict_sum

    torch = torch_mod()
    what = "gather path"
    note(what)
    rng = np.random.default_rng(7400)
    X = gpu(rng.uniform(-1, 1, (1, 16, 300, 64)).astype(np.float32))
    G = gpu(rng.uniform(-1.2, 1.2, (1, 8, 64, 2)).astype(np.float32))
    need = gsa.grid_sample_2d_workspace_size(tuple(X.shape), tuple(G.shape), 0)
    assert need > 0
    plain = gsa.grid_sample(X, G, "linear", "zeros", 0)
    Ya = gsa.grid_sample(X, G, "linear", "zeros", 0, workspace="auto")
    Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    gsa.grid_sample(shifted(X), shifted(G), "linear", "zeros", 0, out=Ys, workspace=ws)
    wbuf = torch.empty(need + 1, dtype=torch.uint8, device="cuda")
    Yw = gsa.grid_sample(X, G, "linear", "zeros", 0, workspace=wbuf[1:])
    torch.cuda.synchronize()
    assert verdict_sum(ws) >= 32, "the probe did not choose the gather path"
    same_bits(Ya, Ys, what)
    same_bits(plain, Ya, what + " against the plain sampler")
    same_bits(plain, Yw, what + " with a shifted workspace")


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("mode", ["nearest", "linear", "cubic"])
def test_resize(gsa, kind, mode):
    torch = torch_mod()
    rng = np.random.default_rng(7500)
    for xs, ys, scales in [((2, 3, 20, 32), (2, 3, 40, 64), [1.0, 1.0, 2.0, 2.0]),
                           ((1, 2, 6, 8, 16), (1, 2, 12, 16, 32), [1.0, 1.0, 2.0, 2.0, 2.0])]:
        what = "Resize %s %s %s -> %s" % (kind, mode, xs, ys)
        note(what)
        X = gpu(rng.uniform(-1, 1, xs).astype(np.float32), getattr(torch, KINDS[kind]))
        Ya = gsa.resize_to(X, ys, scales, mode, "half_pixel")
        Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
        gsa.resize_to(shifted(X), ys, scales, mode, "half_pixel", out=Ys)
        torch.cuda.synchronize()
        same_bits(Ya, Ys, what)
        Xh = host_values(X)
        ref = oracle.resize(Xh, ys, scales, mode, "half_pixel")
        check(Ya.double().cpu().numpy(), ref, mode, kind, float(np.abs(Xh).max()), what)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_deform_conv(gsa, kind):
    """Both DeformConv kernels (with a workspace: channels-last copy and
    packed W; without: planes) and the allocation-free entry point, with X,
    W, offset, mask, B and Y shifted; a shifted workspace runs the kernel
    that needs none."""
    torch = torch_mod()
    rng = np.random.default_rng(7600)
    dt = torch.float32 if kind == "f32" else torch.bfloat16
    n, c, h, w, oc, k = 2, 16, 12, 12, 32, 3
    X = gpu(rng.uniform(-1, 1, (n, c, h, w)).astype(np.float32), dt)
    Wt = gpu(rng.uniform(-0.2, 0.2, (oc, c, k, k)).astype(np.float32), dt)
    off = gpu(rng.normal(0, 1, (n, 2 * k * k, h, w)).astype(np.float32), dt)
    M = gpu(rng.uniform(0, 1, (n, k * k, h, w)).astype(np.float32), dt)
    B = gpu(rng.uniform(-0.1, 0.1, (oc,)).astype(np.float32), dt)
    kw = dict(strides=[1, 1], pads=[1, 1, 1, 1], dilations=[1, 1])
    shifted_in = [shifted(t) for t in (X, Wt, off, B, M)]
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    for name, ws in [("workspace", None), ("no workspace", empty)]:
        what = "DeformConv %s %s" % (kind, name)
        note(what)
        Ya = gsa.deform_conv(X, Wt, off, B, M, workspace=ws, **kw)
        Ys = shifted_empty(tuple(Ya.shape), Ya.dtype)
        gsa.deform_conv(*shifted_in, workspace=ws, out=Ys, **kw)
        torch.cuda.synchronize()
        same_bits(Ya, Ys, what)
        if name == "no workspace":
            direct = Ya
        else:
            cl = Ya
    what = "DeformConv %s shifted workspace" % kind
    note(what)
    need = gsa.deform_conv_workspace_size(tuple(X.shape), tuple(Wt.shape), gsa.dtype_code(X), **kw)
    assert need > 0
    wbuf = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    Yw = gsa.deform_conv(X, Wt, off, B, M, workspace=wbuf[1:need + 1], **kw)
    what_na = "DeformConv %s allocation-free" % kind
    note(what_na)
    Na = gsa.deform_conv_noalloc(X, Wt, off, B, M, **kw)
    Ns = shifted_empty(tuple(Na.shape), Na.dtype)
    gsa.deform_conv_noalloc(*shifted_in, out=Ns, **kw)
    torch.cuda.synchronize()
    same_bits(direct, Yw, what)
    same_bits(cl, Na, what_na + " against the workspace call")
    same_bits(Na, Ns, what_na)
