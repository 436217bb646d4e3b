"""DeformConv oracle pinned to what the DeformConv page and mathematics fix.

* DeformConv page, Examples: the four printed outputs (padding, no padding,
  mask and bias, two offset groups).  One listing prints its offset tensor
  with channels 3 and 4 elided; the fixture stores them as zeros, a reading
  the printed output is consistent with.
* Closed forms: with zero offsets and no mask DeformConv is a convolution --
  torch CPU conv1d / conv2d / conv3d with strides, pads, dilations and
  groups (the convolution meaning of the attributes the page does not list);
  integer offsets shift the input (zero-filled); a constant mask scales the
  result without the bias; offset groups split the input channels into
  contiguous blocks, each with its own offsets and mask (sums of smaller
  deformable convolutions).
* Brute force: the linear interpolation written as a tent kernel applied to
  the distance to every input element (no floor, no corner bookkeeping).
* Planted mistakes in a copy of deform_conv.c, each rejected.
"""

import itertools
import os

import numpy as np
import pytest

from conftest import ROOT, load_golden

DEFORM = load_golden("deform_conv_examples.json")
PRINT_TOL = 2e-6
SRC = os.path.join(ROOT, "oracle", "deform_conv.c")


def arr(ex, key):
    t = ex[key]
    return None if t is None else np.array(t["values"], np.float32).reshape(t["shape"])


def check_example(om, ex, lib=None):
    Y = om.deform_conv(arr(ex, "X"), arr(ex, "W"), arr(ex, "offset"), arr(ex, "B"),
                       arr(ex, "mask"), pads=ex["pads"], offset_group=ex["offset_group"] or 1,
                       lib=lib)
    ref = arr(ex, "Y").astype(np.float64)
    if Y.shape != ref.shape:
        return "%s: shape %s vs %s" % (ex["name"], Y.shape, ref.shape)
    err = (np.abs(Y - ref) / np.maximum(1, np.abs(ref))).max()
    return None if err <= PRINT_TOL else "%s: error %.3g" % (ex["name"], err)


@pytest.mark.parametrize("ex", DEFORM, ids=[e["name"] for e in DEFORM])
def test_page_examples(oracle_mod, ex):
    assert check_example(oracle_mod, ex) is None, ex["citation"]


def test_elided_channels_are_recorded():
    ex = DEFORM[0]
    assert ex["offset"]["elided_channels"] == [3, 4]


def conv_ok(om, lib=None):
    """Zero offsets, no mask: torch conv with the same attributes."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(5)
    cases = [
        (2, (4, 9, 11), (6, 2, 3, 2), (2, 1), (1, 0, 2, 1), (1, 2), 2),
        (1, (3, 7, 8), (3, 3, 3, 3), (1, 1), (1, 1, 1, 1), (1, 1), 1),
        (1, (4, 13), (2, 4, 3), (3,), (2, 1), (2,), 1),
        (1, (2, 5, 6, 7), (2, 1, 2, 3, 2), (1, 2, 1), (0, 1, 1, 1, 0, 0), (1, 1, 2), 2),
    ]
    for n, xs, ws, st, pd, dl, grp in cases:
        r = len(xs) - 1
        X = rng.uniform(-1, 1, (n,) + xs).astype(np.float32)
        W = rng.uniform(-1, 1, ws).astype(np.float32)
        B = rng.uniform(-1, 1, ws[0]).astype(np.float32)
        K = int(np.prod(ws[2:]))
        outs = om.deform_conv_output_shape(xs[1:], ws[2:], st, pd, dl)
        off = np.zeros((n, K * r) + outs, np.float32)
        Y = om.deform_conv(X, W, off, B, None, st, pd, dl, grp, 1, lib=lib)
        Xt = torch.from_numpy(X).double()
        # torch pads symmetrically: pad explicitly (begin, end per axis)
        pad_list = []
        for a in reversed(range(r)):
            pad_list += [pd[a], pd[r + a]]
        Xp = F.pad(Xt, pad_list)
        conv = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}[r]
        ref = conv(Xp, torch.from_numpy(W).double(), torch.from_numpy(B).double(), stride=st,
                   dilation=dl, groups=grp).numpy()
        if ref.shape != Y.shape or np.abs(Y - ref).max() > 1e-12:
            return "conv %s" % (xs,)
    return None


def test_zero_offsets_are_a_convolution(oracle_mod):
    assert conv_ok(oracle_mod) is None


def shift_ok(om, lib=None):
    """Integer offsets (dy, dx) on every tap: the convolution of X shifted
    (no padding, so every regular position lies on the shifted image)."""
    rng = np.random.default_rng(6)
    X = rng.uniform(-1, 1, (1, 2, 7, 9)).astype(np.float32)
    W = rng.uniform(-1, 1, (3, 2, 3, 3)).astype(np.float32)
    for dy, dx in ((1, 0), (0, -2), (2, 3), (-1, -1)):
        off = np.zeros((1, 18, 5, 7), np.float32)
        off[:, 0::2] = dy
        off[:, 1::2] = dx
        Y = om.deform_conv(X, W, off, None, None, lib=lib)
        Xs = np.zeros_like(X)
        src = X[:, :, max(dy, 0):7 + min(dy, 0), max(dx, 0):9 + min(dx, 0)]
        Xs[:, :, max(-dy, 0):max(-dy, 0) + src.shape[2], max(-dx, 0):max(-dx, 0) + src.shape[3]] = src
        ref = om.deform_conv(Xs, W, np.zeros_like(off), None, None, lib=lib)
        if np.abs(Y - ref).max() > 1e-12:
            return "shift %d %d" % (dy, dx)
    return None


def test_integer_offsets_shift_the_input(oracle_mod):
    assert shift_ok(oracle_mod) is None


def mask_ok(om, lib=None):
    rng = np.random.default_rng(7)
    X = rng.uniform(-1, 1, (2, 4, 6, 7)).astype(np.float32)
    W = rng.uniform(-1, 1, (4, 2, 2, 3)).astype(np.float32)
    B = rng.uniform(-1, 1, 4).astype(np.float32)
    off = rng.uniform(-2, 2, (2, 2 * 6 * 2, 5, 5)).astype(np.float32)
    base = om.deform_conv(X, W, off, B, None, None, None, None, 2, 2, lib=lib)
    m = np.full((2, 2 * 6, 5, 5), 0.375, np.float32)
    Y = om.deform_conv(X, W, off, B, m, None, None, None, 2, 2, lib=lib)
    Bc = B.astype(np.float64)[None, :, None, None]
    if np.abs((Y - Bc) - 0.375 * (base - Bc)).max() > 1e-12:
        return "mask scaling"
    return None


def test_constant_mask_scales(oracle_mod):
    assert mask_ok(oracle_mod) is None


def groups_ok(om, lib=None):
    """offset_group = C: each input channel with its own offsets and mask is
    a single-channel deformable convolution; the output is their sum."""
    rng = np.random.default_rng(8)
    C = 3
    X = rng.uniform(-1, 1, (1, C, 6, 7)).astype(np.float32)
    W = rng.uniform(-1, 1, (2, C, 2, 2)).astype(np.float32)
    off = rng.uniform(-1.5, 1.5, (1, C * 4 * 2, 5, 6)).astype(np.float32)
    mask = rng.uniform(0, 1, (1, C * 4, 5, 6)).astype(np.float32)
    Y = om.deform_conv(X, W, off, None, mask, None, None, None, 1, C, lib=lib)
    ref = 0
    for c in range(C):
        ref = ref + om.deform_conv(X[:, c:c + 1], W[:, c:c + 1], off[:, c * 8:(c + 1) * 8], None,
                                   mask[:, c * 4:(c + 1) * 4], lib=lib)
    if np.abs(Y - ref).max() > 1e-12:
        return "offset groups"
    # offset_group 2 over 4 channels: contiguous channel blocks {0,1}, {2,3}
    X = rng.uniform(-1, 1, (1, 4, 6, 7)).astype(np.float32)
    W = rng.uniform(-1, 1, (2, 4, 2, 2)).astype(np.float32)
    off = rng.uniform(-1.5, 1.5, (1, 2 * 4 * 2, 5, 6)).astype(np.float32)
    mask = rng.uniform(0, 1, (1, 2 * 4, 5, 6)).astype(np.float32)
    Y = om.deform_conv(X, W, off, None, mask, None, None, None, 1, 2, lib=lib)
    ref = sum(om.deform_conv(X[:, 2 * g:2 * g + 2], W[:, 2 * g:2 * g + 2], off[:, g * 8:(g + 1) * 8],
                             None, mask[:, g * 4:(g + 1) * 4], lib=lib) for g in range(2))
    if np.abs(Y - ref).max() > 1e-12:
        return "offset groups of two channels"
    return None


def test_offset_groups_split_channels(oracle_mod):
    assert groups_ok(oracle_mod) is None


def brute_force(X, W, off, mask, st, pd, dl):
    """2-D, group 1, offset_group 1, fp32 locations: tent kernel over every
    input element."""
    N, C, H, Wd = X.shape
    OC, _, KH, KW = W.shape
    OH, OW = off.shape[2:]
    Y = np.zeros((N, OC, OH, OW))
    hs, ws = np.arange(H), np.arange(Wd)
    for n, oh, ow in itertools.product(range(N), range(OH), range(OW)):
        for i, j in itertools.product(range(KH), range(KW)):
            k = i * KW + j
            py = np.float32(oh * st[0] - pd[0] + i * dl[0]) + np.float32(off[n, 2 * k, oh, ow])
            px = np.float32(ow * st[1] - pd[1] + j * dl[1]) + np.float32(off[n, 2 * k + 1, oh, ow])
            wy = np.maximum(0, 1 - np.abs(float(py) - hs))
            wx = np.maximum(0, 1 - np.abs(float(px) - ws))
            samp = np.einsum("nchw,h,w->nc", X[n:n + 1].astype(np.float64), wy, wx)[0]
            m = 1.0 if mask is None else float(mask[n, k, oh, ow])
            Y[n, :, oh, ow] += (W[:, :, i, j].astype(np.float64) * (m * samp)[None, :]).sum(1)
    return Y


def brute_ok(om, lib=None):
    rng = np.random.default_rng(9)
    for st, pd, dl in (((1, 1), (1, 0, 1, 2), (1, 1)), ((2, 1), (0, 1, 0, 1), (1, 2))):
        X = rng.uniform(-1, 1, (1, 2, 5, 6)).astype(np.float32)
        W = rng.uniform(-1, 1, (2, 2, 2, 3)).astype(np.float32)
        outs = om.deform_conv_output_shape((5, 6), (2, 3), st, pd, dl)
        off = rng.uniform(-3, 3, (1, 12) + outs).astype(np.float32)
        mask = rng.uniform(0, 1, (1, 6) + outs).astype(np.float32)
        Y = om.deform_conv(X, W, off, None, mask, st, pd, dl, lib=lib)
        if np.abs(Y - brute_force(X, W, off, mask, st, pd, dl)).max() > 1e-12:
            return "brute force %s" % (st,)
    return None


def test_brute_force(oracle_mod):
    assert brute_ok(oracle_mod) is None


def test_double_locations(oracle_mod):
    """float64 data takes its locations in float64: an offset that fp32 would
    round moves the sample accordingly."""
    X = np.array([0.0, 1.0, 0.0, 0.0], np.float64).reshape(1, 1, 1, 4)
    W = np.ones((1, 1, 1, 1))
    off = np.zeros((1, 2, 1, 4))
    off[0, 1, 0, 0] = 1e-9             # x offset of output 0: lost in fp32 (0 + 1e-9)
    Y = oracle_mod.deform_conv(X, W, off)
    assert Y[0, 0, 0, 0] == 1e-9
    Yf = oracle_mod.deform_conv(X.astype(np.float32), W.astype(np.float32),
                                off.astype(np.float32))
    assert Yf[0, 0, 0, 0] == np.float64(np.float32(1e-9)) * 1.0


def battery(om, lib):
    for ex in DEFORM:
        msg = check_example(om, ex, lib)
        if msg:
            return msg
    for check in (conv_ok, shift_ok, mask_ok, groups_ok, brute_ok):
        msg = check(om, lib)
        if msg:
            return msg
    return None


MUTANTS = [
    ("offset components swapped", "P->offset[((n * P->og + g) * K * r + k * r + a)",
     "P->offset[((n * P->og + g) * K * r + k * r + (r - 1 - a))"),
    ("regular position without the pad",
     "oi[a] * P->strides[a] - P->pads[a] + ki[a] * P->dilations[a]",
     "oi[a] * P->strides[a] + ki[a] * P->dilations[a]"),
    ("dilation ignored", "oi[a] * P->strides[a] - P->pads[a] + ki[a] * P->dilations[a]",
     "oi[a] * P->strides[a] - P->pads[a] + ki[a]"),
    ("linear weights swapped", "w *= bit ? frac[a] : 1.0 - frac[a];",
     "w *= bit ? 1.0 - frac[a] : frac[a];"),
    ("zero extension replaced by a clamp", "valid = valid && i >= 0 && i < in_sp[a];",
     "i = i < 0 ? 0 : (i >= in_sp[a] ? in_sp[a] - 1 : i);"),
    ("mask channel of the wrong group", "v *= P->mask[((n * P->og + g) * K + k) * out_count + o];",
     "v *= P->mask[((n * P->og + 0) * K + k) * out_count + o];"),
    ("offset group by modulo", "const int64_t g = c / P->Cog;", "const int64_t g = c % P->og;"),
    ("weights of the wrong kernel position", "acc += P->Wt[(oc * P->Cg + cl) * K + k] * v;",
     "acc += P->Wt[(oc * P->Cg + cl) * K + (K - 1 - k)] * v;"),
    ("bias dropped", "acc += P->B[oc];", "acc += 0.0 * P->B[oc];"),
]


def test_unmodified_oracle_passes_battery(oracle_mod):
    assert battery(oracle_mod, None) is None


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle_mod, tmp_path, desc, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + desc
    mutant = tmp_path / "deform_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = oracle_mod.build(deform_src=str(mutant), out=str(tmp_path / "libmutant.so"))
    lib = oracle_mod.load_library(so)
    assert battery(oracle_mod, lib) is not None, "no pin rejects the mutant: " + desc
