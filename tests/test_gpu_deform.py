"""DeformConv on the GPU (gs_deform_conv through the C ABI) against the oracle.

* The four printed examples (2-D fp32: the matrix-core kernel).
* 2-D fp32 / fp16 / bf16 (matrix cores) over output-channel counts that take
  one or two 128- / 256-row tiles with a ragged last one, output planes that
  end in a ragged 64-position tile, K not a multiple of 32, strides, pads,
  dilations, conv groups, offset groups spanning one or two groups per conv
  group, kernels whose sampling table fits LDS and ones that sample on the
  fly (7x7), with and without mask and bias.  Tolerance per output, from the
  sum of the absolute values of its terms S (the oracle on |X|, |W|, |mask|,
  plus |B|): fp32 2e-5 * S; fp16 and bf16 (u + (K + 8) * 2^-24) * S, where
  u = 2^-11 (fp16) or 2^-8 (bf16) bounds the one rounding of each sampled
  value to the data type before its product (exact in fp32), K products per
  output are accumulated in fp32 (at most K roundings of 2^-24 relative to
  S), and 8 more cover the fp32 interpolation and mask products; plus one
  unit in the last place of the output type.  Below the smallest normal
  value (2^-14 for fp16, 2^-126 for bf16) the types have a fixed spacing
  (2^-24, 2^-133), so a relative bound does not hold there: each sampled
  value's rounding adds up to half that spacing times |W| of its product,
  and the output's rounding one spacing.
* 2-D cases whose conv and offset groups hold multiples of 8 channels run on
  the channels-last copy of X by default: channel counts that fill whole
  chunks and ones padded up to the next chunk, offset groups that change
  within a kernel position's chunks, kernels too large for the sampling
  table, and (fp16 / bf16 with more than 128 output channels per group) the
  8-wave blocks with 64-channel chunks; the same cases with an empty
  workspace take the gather kernel instead.
* double data and 1-D / 3-D data (the direct kernel, summing in double in the
  oracle's order): bit for bit after the output conversion.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from conftest import load_golden
from parity import note, torch_mod

pytestmark = pytest.mark.gpu

DEFORM = load_golden("deform_conv_examples.json")


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def to_dev(a, kind):
    """Device tensor of kind from fp32 / float64 values, and the exact values
    the oracle sees."""
    torch = torch_mod()
    if a is None:
        return None, None
    if kind == "f64":
        return torch.from_numpy(np.ascontiguousarray(a, np.float64)).cuda(), np.asarray(a, np.float64)
    a32 = np.ascontiguousarray(a, np.float32)
    if kind == "f32":
        return torch.from_numpy(a32).cuda(), a32
    bits = W.to_half_bits(a32, kind)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(
        torch.float16 if kind == "f16" else torch.bfloat16)
    return t, W.half_bits_to_f32(bits, kind)


def rounded(ref, kind):
    if kind == "f64":
        return ref
    if kind == "f32":
        return ref.astype(np.float32).astype(np.float64)
    if kind == "f16":
        return ref.astype(np.float32).astype(np.float16).astype(np.float64)
    return W.half_bits_to_f32(W.to_half_bits(ref.astype(np.float32), "bf16"), "bf16").astype(np.float64)


def deform_rel_tol(kind, K):
    """Bound on |gpu - oracle| / S for K products per output (see above)."""
    if kind == "f32":
        return 2e-5
    u = 2.0 ** -11 if kind == "f16" else 2.0 ** -8
    return u + (K + 8) * 2.0 ** -24


def run(gsa, X, Wt, off, B, mask, kind, st=None, pd=None, dl=None, grp=1, og=1, exact=False,
        what="", no_workspace=False):
    torch = torch_mod()
    note("deform %s %s X=%s W=%s st=%s pd=%s dl=%s group=%d og=%d mask=%s bias=%s ws=%s" % (
        what, kind, X.shape, Wt.shape, st, pd, dl, grp, og, mask is not None, B is not None,
        not no_workspace))
    (Xd, Xo), (Wd, Wo), (Od, Oo), (Bd, Bo), (Md, Mo) = (to_dev(a, kind) for a in (X, Wt, off, B, mask))
    ws = torch.empty(0, dtype=torch.uint8, device="cuda") if no_workspace else None
    Y = gsa.deform_conv(Xd, Wd, Od, Bd, Md, st, pd, dl, grp, og, workspace=ws)
    torch.cuda.synchronize()
    got = Y.double().cpu().numpy()
    ref = oracle.deform_conv(Xo, Wo, Oo, Bo, Mo, st, pd, dl, grp, og)
    if exact:
        bad = got != rounded(ref, kind)
        assert not bad.any(), "%s: %d of %d differ" % (what, bad.sum(), bad.size)
        return
    S = oracle.deform_conv(np.abs(Xo), np.abs(Wo), Oo, None,
                           None if Mo is None else np.abs(Mo), st, pd, dl, grp, og)
    if Bo is not None:
        S = S + np.abs(Bo).reshape((1, -1) + (1,) * (S.ndim - 2))
    K = int(np.prod(Wt.shape[1:]))  # products summed per output
    rel = deform_rel_tol(kind, K)
    ulp = {"f32": 0.0, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[kind]
    # fixed spacing below the smallest normal value: half of it per sampled
    # value (times |W| of its product), one for the output
    sub = {"f32": 0.0, "f16": 2.0 ** -24, "bf16": 2.0 ** -133}[kind]
    wsum = np.abs(np.asarray(Wo, np.float64)).reshape(Wo.shape[0], -1).sum(1)
    wsum = wsum.reshape((1, -1) + (1,) * (ref.ndim - 2))
    tol = rel * S + ulp * np.abs(ref) + sub * (0.5 * wsum + 1.0) + 1e-30
    err = np.abs(got - ref)
    assert (err <= tol).all(), "%s: max err/tol %.3g at %s" % (
        what, (err / tol).max(), np.unravel_index((err / tol).argmax(), err.shape))


def arr(ex, key):
    t = ex[key]
    return None if t is None else np.array(t["values"], np.float32).reshape(t["shape"])


@pytest.mark.parametrize("ex", DEFORM, ids=[e["name"] for e in DEFORM])
def test_page_examples(gsa, ex):
    run(gsa, arr(ex, "X"), arr(ex, "W"), arr(ex, "offset"), arr(ex, "B"), arr(ex, "mask"), "f32",
        pd=ex["pads"], og=ex["offset_group"] or 1, what=ex["name"])
    torch = torch_mod()
    Xd, Wd, Od = (torch.from_numpy(arr(ex, k)).cuda() for k in ("X", "W", "offset"))
    Bd = None if ex["B"] is None else torch.from_numpy(arr(ex, "B")).cuda()
    Md = None if ex["mask"] is None else torch.from_numpy(arr(ex, "mask")).cuda()
    Y = gsa.deform_conv(Xd, Wd, Od, Bd, Md, pads=ex["pads"], offset_group=ex["offset_group"] or 1)
    printed = arr(ex, "Y")
    assert np.abs(Y.cpu().numpy() - printed).max() <= 2e-6 * max(1.0, np.abs(printed).max())


def case(seed, n, c, h, w, oc, kh, kw, st, pd, dl, grp, og, with_mask, with_bias, off_scale=2.0):
    rng = np.random.default_rng(seed)
    X = rng.uniform(-1, 1, (n, c, h, w)).astype(np.float32)
    Wt = rng.uniform(-1, 1, (oc, c // grp, kh, kw)).astype(np.float32)
    oh = (h + pd[0] + pd[2] - (dl[0] * (kh - 1) + 1)) // st[0] + 1
    ow = (w + pd[1] + pd[3] - (dl[1] * (kw - 1) + 1)) // st[1] + 1
    off = rng.uniform(-off_scale, off_scale, (n, og * kh * kw * 2, oh, ow)).astype(np.float32)
    mask = rng.uniform(0, 1, (n, og * kh * kw, oh, ow)).astype(np.float32) if with_mask else None
    B = rng.uniform(-1, 1, oc).astype(np.float32) if with_bias else None
    return X, Wt, off, B, mask


CASES_2D = [
    # n, c, h, w, oc, kh, kw, strides, pads, dilations, group, offset_group
    (2, 8, 12, 13, 6, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1, 1),
    (1, 16, 20, 21, 160, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1, 2),       # 256-row tile
    (1, 12, 15, 17, 300, 3, 3, (2, 1), (1, 0, 2, 1), (1, 2), 1, 1),       # 2 tiles, ragged
    (2, 6, 11, 9, 4, 3, 2, (1, 2), (0, 1, 1, 0), (2, 1), 2, 3),           # groups, og span 2
    (1, 5, 16, 16, 7, 7, 7, (1, 1), (3, 3, 3, 3), (1, 1), 1, 1),          # 49 taps: no table
    (1, 3, 33, 35, 129, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 1, 3),        # 1x1, og = C
]


@pytest.mark.parametrize("kind,ci,mask,bias", list(itertools.product(
    ["f32", "f16", "bf16"], range(len(CASES_2D)), [False, True], [False, True])))
def test_2d_matrix_cores(gsa, kind, ci, mask, bias):
    n, c, h, w, oc, kh, kw, st, pd, dl, grp, og = CASES_2D[ci]
    X, Wt, off, B, M = case(100 + ci, n, c, h, w, oc, kh, kw, st, pd, dl, grp, og, mask, bias)
    run(gsa, X, Wt, off, B, M, kind, list(st), list(pd), list(dl), grp, og, what="2-D case %d" % ci)


@pytest.mark.parametrize("ci,mask", list(itertools.product(range(len(CASES_2D)), [False, True])))
def test_2d_double_exact(gsa, ci, mask):
    n, c, h, w, oc, kh, kw, st, pd, dl, grp, og = CASES_2D[ci]
    X, Wt, off, B, M = case(200 + ci, n, c, h, w, oc, kh, kw, st, pd, dl, grp, og, mask, True)
    f = lambda a: None if a is None else a.astype(np.float64)
    run(gsa, f(X), f(Wt), f(off) + 1e-9, f(B), f(M), "f64", list(st), list(pd), list(dl), grp, og,
        exact=True, what="2-D double %d" % ci)


@pytest.mark.parametrize("kind,rank", list(itertools.product(["f32", "f16", "bf16", "f64"], [1, 3])))
def test_1d_3d_direct_exact(gsa, kind, rank):
    rng = np.random.default_rng(300 + rank)
    if rank == 1:
        xs, ws, st, pd, dl = (2, 6, 40), (6, 3, 4), [2], [1, 2], [2]
    else:
        xs, ws, st, pd, dl = (1, 4, 6, 7, 8), (4, 2, 2, 3, 2), [1, 2, 1], [1, 0, 1, 0, 1, 1], [1, 1, 2]
    grp, og = 2, 2
    outs = oracle.deform_conv_output_shape(xs[2:], ws[2:], st, pd, dl)
    K = int(np.prod(ws[2:]))
    X = rng.uniform(-1, 1, xs)
    Wt = rng.uniform(-1, 1, ws)
    off = rng.uniform(-2, 2, (xs[0], og * K * rank) + outs)
    M = rng.uniform(0, 1, (xs[0], og * K) + outs)
    B = rng.uniform(-1, 1, ws[0])
    if kind != "f64":
        X, Wt, off, M, B = (a.astype(np.float32) for a in (X, Wt, off, M, B))
    run(gsa, X, Wt, off, B, M, kind, st, pd, dl, grp, og, exact=True, what="%d-D direct" % rank)


CASES_CL = [
    # n, c, h, w, oc, kh, kw, strides, pads, dilations, group, offset_group
    (2, 64, 9, 70, 33, 3, 3, (1, 1), (0, 1, 0, 1), (1, 1), 1, 1),          # 2 chunks/tap, ragged tile
    (1, 40, 14, 15, 70, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1, 5),         # Cg padded, og varies
    (2, 32, 10, 11, 300, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 2, 2),        # groups, 256-row tiles
    (1, 16, 18, 19, 24, 7, 7, (1, 1), (3, 3, 3, 3), (1, 1), 1, 1),         # 49 taps: no table
    (1, 24, 8, 9, 9, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 3, 3),            # 8 of 32 channels used
    (1, 48, 12, 13, 130, 3, 2, (1, 2), (2, 0, 1, 1), (2, 1), 2, 6),        # og span 3 per group
    (2, 32, 10, 10, 40, 2, 2, (1, 1), (1, 0, 0, 1), (1, 1), 1, 2),         # og changes inside a chunk
    (1, 32, 14, 15, 144, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 1, 1),        # wide: 8 waves, no table
    (1, 96, 9, 11, 200, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1, 3),         # wide, og changes in a chunk
    (1, 32, 8, 9, 160, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), 1, 1),          # wide, a single chunk
]


@pytest.mark.parametrize("kind,ci,ws", list(itertools.product(
    ["f32", "f16", "bf16"], range(len(CASES_CL)), [True, False])))
def test_2d_channels_last(gsa, kind, ci, ws):
    n, c, h, w, oc, kh, kw, st, pd, dl, grp, og = CASES_CL[ci]
    assert gsa.deform_conv_workspace_size(
        (n, c, h, w), (oc, c // grp, kh, kw), {"f32": 0, "f16": 1, "bf16": 2}[kind], list(st),
        list(pd), list(dl), grp, og) > 0
    X, Wt, off, B, M = case(400 + ci, n, c, h, w, oc, kh, kw, st, pd, dl, grp, og, True, True)
    run(gsa, X, Wt, off, B, M, kind, list(st), list(pd), list(dl), grp, og,
        what="2-D channels-last case %d" % ci, no_workspace=not ws)


def test_channels_last_non_finite_x(gsa):
    """An infinite X value outside every sample's support leaves the outputs
    finite (corners outside the image, or of zero weight from outside, read
    no X); one inside the support of a sample makes it non-finite as in the
    oracle."""
    torch = torch_mod()
    n, c, h, w, oc = 1, 8, 6, 7, 4
    X = np.zeros((n, c, h, w), np.float32)
    X[0, 3, 5, 6] = np.inf
    Wt = np.ones((oc, c, 1, 1), np.float32)
    off = np.zeros((n, 2, h, w), np.float32)
    off[0, :, 0, 0] = 100.0                 # far outside: reads nothing
    off[0, 0, 2, 2] = 0.5                   # between rows 2 and 3: finite
    Y = gsa.deform_conv(torch.from_numpy(X).cuda(), torch.from_numpy(Wt).cuda(),
                        torch.from_numpy(off).cuda())
    got = Y.cpu().numpy()
    ref = oracle.deform_conv(X, Wt, off)
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
