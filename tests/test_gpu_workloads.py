"""The synthetic workloads (five sampler, five Resize, three of other ranks
and element types, a DeformConv layer) on the GPU against the oracle.

* reduced shapes (same distributions, several tiles, ragged tails): every
  output element is compared;
* full shapes, in exactly the launches the benchmark times: every output
  element of the sampler, Resize and other-type workloads is compared, image
  by image (or plane by plane), against the OpenMP build of the oracle (the
  same sources as the serial oracle, bit-identical values); the DeformConv
  layer compares 32,768 random outputs plus the first and last outputs of
  every image, computed one by one.
"""

import numpy as np
import pytest

import oracle
import workloads as W
from parity import check, from_gpu, note, to_gpu_f32, torch_mod, x_to_gpu
from test_gpu_deform import deform_rel_tol

pytestmark = pytest.mark.gpu

REDUCED = {
    "stn2d_tiny": ((2, 3, 16, 16), (5, 6)),
    "stn2d_batch": ((3, 10, 37, 45), (39, 41)),
    "flow2d_bicubic": ((2, 9, 40, 44), (35, 37)),
    "vol3d": ((2, 5, 13, 14, 15), (11, 12, 13)),
    "flow2d_half": ((2, 12, 40, 48), (33, 35)),
}


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def mode_list(w):
    return [(w.mode, w.padding)] + list(w.extra_modes)


def run_gpu(gsa, w, inp, kind, mode, pad, ac, fused):
    """The same calls the benchmark makes: theta -> grid -> sample, or fused."""
    Xd, Xin = x_to_gpu(inp["X"], kind)
    n, c = inp["x_shape"][:2]
    if inp["theta"] is not None:
        td = to_gpu_f32(inp["theta"])
        if fused:
            Y = gsa.affine_grid_sample_fused(td, Xd, inp["out_spatial"], mode, pad, ac)
        else:
            grid = gsa.affine_grid(td, (n, c) + tuple(inp["out_spatial"]), ac)
            Y = gsa.grid_sample(Xd, grid, mode, pad, ac)
    else:
        Y = gsa.grid_sample(Xd, to_gpu_f32(inp["grid"]), mode, pad, ac)
    return Y, Xin


def oracle_grid(inp, ac):
    if inp["theta"] is not None:
        n, c = inp["x_shape"][:2]
        return oracle.affine_grid(inp["theta"], (n, c) + tuple(inp["out_spatial"]), ac)
    return inp["grid"]


def cases(reduced: bool):
    out = []
    for name, w in W.WORKLOADS.items():
        for kind in w.dtypes:
            for mode, pad in mode_list(w):
                acs = (0, 1) if name == "stn2d_tiny" else (w.align_corners,)
                for ac in acs:
                    fused_opts = (False, True) if w.grid_kind.startswith("affine") else (False,)
                    for fused in fused_opts:
                        out.append(pytest.param(name, kind, mode, pad, ac, fused,
                                                id="%s-%s-%s-%s-ac%d%s" % (
                                                    name, kind, mode, pad, ac,
                                                    "-fused" if fused else "")))
    return out


@pytest.mark.parametrize("name,kind,mode,pad,ac,fused", cases(True))
def test_workload_reduced_all_elements(gsa, name, kind, mode, pad, ac, fused):
    w = W.WORKLOADS[name]
    x_shape, out_sp = REDUCED[name]
    note("reduced %s %s %s/%s ac=%d fused=%s x=%s out=%s" % (name, kind, mode, pad, ac, fused,
                                                             x_shape, out_sp))
    inp = W.make_inputs(w, x_shape, out_sp)
    Y, Xin = run_gpu(gsa, w, inp, kind, mode, pad, ac, fused)
    ref = oracle.grid_sample(Xin, oracle_grid(inp, ac), mode, pad, ac)
    check(from_gpu(Y), ref, mode, kind, np.abs(Xin).max(), name)


def sample_indices(n, c, count, k, seed):
    rng = np.random.default_rng(seed)
    total = n * c * count
    idx = [rng.integers(0, total, size=k)]
    for b in range(n):
        for ch in (0, c - 1):
            base = (b * c + ch) * count
            idx.append(base + np.arange(min(count, 64)))
            idx.append(base + count - 1 - np.arange(min(count, 64)))
    return np.unique(np.concatenate(idx))


@pytest.mark.parametrize("name,kind,mode,pad,ac,fused",
                         [p for p in cases(False) if "tiny" not in p.id])
def test_workload_full_size_all_elements(gsa, name, kind, mode, pad, ac, fused):
    w = W.WORKLOADS[name]
    note("full %s %s %s/%s ac=%d fused=%s x=%s" % (name, kind, mode, pad, ac, fused, w.x_shape))
    inp = W.make_inputs(w)
    Y, Xin = run_gpu(gsa, w, inp, kind, mode, pad, ac, fused)
    got = from_gpu(Y)
    del Y
    par = oracle.parallel()
    n, c = w.x_shape[:2]
    if inp["theta"] is not None:
        G = oracle.affine_grid(inp["theta"], (n, c) + tuple(inp["out_spatial"]), ac, lib=par)
    else:
        G = inp["grid"]
    xmax = np.abs(Xin).max()
    for b in range(n):
        ref = oracle.grid_sample(Xin[b:b + 1], G[b:b + 1], mode, pad, ac, lib=par)
        check(got[b:b + 1], ref, mode, kind, xmax, "full %s image %d" % (name, b))


# ------------------------------------------------------------------ Resize

RESIZE_REDUCED = {
    "resize2d_up2_linear": (3, 5, 37, 45),
    "resize2d_up2_nearest": (3, 5, 37, 45),
    "resize2d_up2_cubic": (3, 5, 37, 45),
    "resize2d_down2_linear": (3, 5, 74, 90),
    "resize3d_up2_linear": (2, 3, 9, 10, 11),
}


def resize_gpu(gsa, w, X):
    """The call the benchmark makes (scales on the trailing axes)."""
    rank = X.ndim
    axes = list(range(rank - len(w.scales), rank))
    return gsa.resize(x_to_gpu(X, "f32")[0], scales=list(w.scales), axes=axes, mode=w.mode,
                      coordinate_transformation_mode=w.coordinate_transformation_mode)


@pytest.mark.parametrize("name", list(W.RESIZE_WORKLOADS))
def test_resize_workload_reduced_all_elements(gsa, name):
    w = W.RESIZE_WORKLOADS[name]
    X = W.make_resize_input(w, RESIZE_REDUCED[name])
    note("reduced %s x=%s" % (name, X.shape))
    Y = resize_gpu(gsa, w, X)
    ref = oracle.resize(X, tuple(Y.shape), w.full_scales(), w.mode,
                        w.coordinate_transformation_mode)
    check(from_gpu(Y), ref, w.mode, "f32", np.abs(X).max(), name)


@pytest.mark.parametrize("name", list(W.RESIZE_WORKLOADS))
def test_resize_workload_full_size_all_elements(gsa, name):
    w = W.RESIZE_WORKLOADS[name]
    note("full %s x=%s" % (name, w.x_shape))
    X = W.make_resize_input(w)
    Y = resize_gpu(gsa, w, X)
    got = from_gpu(Y)
    del Y
    par = oracle.parallel()
    shape = got.shape
    xmax = np.abs(X).max()
    # the leading axis keeps its extent (scale 1): compare one slice at a time
    for b in range(shape[0]):
        ref = oracle.resize(X[b:b + 1], (1,) + shape[1:], w.full_scales(), w.mode,
                            w.coordinate_transformation_mode, lib=par)
        check(got[b:b + 1], ref, w.mode, "f32", xmax, "full %s slice %d" % (name, b))


# ----------------------------------------------- other ranks and element types

TYPE_REDUCED = {
    "stn2d_u8": ((3, 3, 45, 53), (41, 47)),
    "signal1d_f32": ((3, 5, 300), (257,)),
    "vol3d_f64": ((2, 3, 9, 10, 11), (7, 8, 9)),
}


def type_expected(ref, x):
    """The oracle's float64 value after the output conversion of X's type
    (the any-rank kernel matches it bit for bit)."""
    if x.dtype == np.uint8:
        return oracle.to_integer(ref, np.uint8)
    if x.dtype == np.float32:
        return ref.astype(np.float32)
    return ref


def type_gpu(gsa, w, inp):
    torch = torch_mod()
    n, c = inp["x_shape"][:2]
    X = torch.from_numpy(inp["X"]).cuda()
    if inp["theta"] is not None:
        grid = gsa.affine_grid(torch.from_numpy(inp["theta"]).cuda(),
                               (n, c) + tuple(inp["out_spatial"]), w.align_corners)
        g_ref = oracle.affine_grid(inp["theta"], (n, c) + tuple(inp["out_spatial"]),
                                   w.align_corners)
    else:
        grid = torch.from_numpy(inp["grid"]).cuda()
        g_ref = inp["grid"]
    return gsa.grid_sample(X, grid, w.mode, w.padding, w.align_corners), g_ref


@pytest.mark.parametrize("name", list(W.TYPE_WORKLOADS))
def test_type_workload_reduced_all_elements(gsa, name):
    w = W.TYPE_WORKLOADS[name]
    x_shape, out_sp = TYPE_REDUCED[name]
    note("reduced %s x=%s out=%s" % (name, x_shape, out_sp))
    inp = W.make_type_inputs(w, x_shape, out_sp)
    Y, g_ref = type_gpu(gsa, w, inp)
    torch_mod().cuda.synchronize()
    got = Y.cpu().numpy()
    ref = type_expected(oracle.grid_sample(inp["X"], g_ref, w.mode, w.padding, w.align_corners),
                        inp["X"])
    assert np.array_equal(got, ref), name


@pytest.mark.parametrize("name", list(W.TYPE_WORKLOADS))
def test_type_workload_full_size_all_elements(gsa, name):
    w = W.TYPE_WORKLOADS[name]
    note("full %s x=%s" % (name, w.x_shape))
    inp = W.make_type_inputs(w)
    Y, g_ref = type_gpu(gsa, w, inp)
    torch_mod().cuda.synchronize()
    got = Y.cpu().numpy()
    del Y
    par = oracle.parallel()
    X = inp["X"]
    for b in range(X.shape[0]):
        ref = type_expected(oracle.grid_sample(X[b:b + 1], g_ref[b:b + 1], w.mode, w.padding,
                                               w.align_corners, lib=par), X)
        assert np.array_equal(got[b:b + 1], ref), "%s image %d" % (name, b)


# ------------------------------------------------------------------ DeformConv

def deform_dev(inp, kind):
    torch = torch_mod()
    out, exact = {}, {}
    for k, a in inp.items():
        if kind == "f32":
            out[k], exact[k] = torch.from_numpy(a).cuda(), a
        else:
            bits = W.to_half_bits(a, kind)
            out[k] = torch.from_numpy(bits.view(np.int16)).cuda().view(
                torch.float16 if kind == "f16" else torch.bfloat16)
            exact[k] = W.half_bits_to_f32(bits, kind)
    return out, exact


def deform_check(got, ref, S, kind, K, what):
    rel = deform_rel_tol(kind, K)
    ulp = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[kind]
    tol = rel * S + ulp * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    assert (err <= tol).all(), "%s: max err/tol %.3g" % (what, (err / tol).max())


@pytest.mark.parametrize("name,kind", [(n, k) for n, w in W.DEFORM_WORKLOADS.items()
                                       for k in w.dtypes])
def test_deform_workload_reduced_all_elements(gsa, name, kind):
    w = W.DEFORM_WORKLOADS[name]
    xs = (2, 24, 19, 21)
    ws = (40, 24) + tuple(w.w_shape[2:])
    note("reduced %s %s x=%s w=%s" % (name, kind, xs, ws))
    d, e = deform_dev(W.make_deform_inputs(w, xs, ws), kind)
    Y = gsa.deform_conv(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=list(w.pads),
                        group=w.group, offset_group=w.offset_group)
    got = Y.double().cpu().numpy()
    args = dict(pads=list(w.pads), group=w.group, offset_group=w.offset_group)
    ref = oracle.deform_conv(e["X"], e["W"], e["offset"], e["B"], e["mask"], **args)
    S = oracle.deform_conv(np.abs(e["X"]), np.abs(e["W"]), e["offset"], None, np.abs(e["mask"]),
                           **args) + np.abs(e["B"]).reshape(1, -1, 1, 1)
    deform_check(got, ref, S, kind, int(np.prod(ws[1:])), name)


@pytest.mark.parametrize("name,kind", [(n, k) for n, w in W.DEFORM_WORKLOADS.items()
                                       for k in w.dtypes])
def test_deform_workload_full_size_sampled(gsa, name, kind):
    w = W.DEFORM_WORKLOADS[name]
    note("full %s %s x=%s" % (name, kind, w.x_shape))
    d, e = deform_dev(W.make_deform_inputs(w), kind)
    Y = gsa.deform_conv(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=list(w.pads),
                        group=w.group, offset_group=w.offset_group)
    n, oc, oh, ow = w.out_shape()
    idx = sample_indices(n, oc, oh * ow, 32768, w.seed)
    torch = torch_mod()
    got = Y.reshape(-1)[torch.from_numpy(idx).cuda()].double().cpu().numpy()
    del Y
    args = dict(pads=list(w.pads), group=w.group, offset_group=w.offset_group, flat_index=idx,
                lib=oracle.parallel())
    ref = oracle.deform_conv(e["X"], e["W"], e["offset"], e["B"], e["mask"], **args)
    S = oracle.deform_conv(np.abs(e["X"]), np.abs(e["W"]), e["offset"], None, np.abs(e["mask"]),
                           **args) + np.abs(e["B"])[(idx // (oh * ow)) % oc]
    deform_check(got, ref, S, kind, int(np.prod(w.w_shape[1:])), "full " + name)
