"""The C-ABI library loads, exports what include/gsample.h declares, and
rejects bad arguments before any launch (no GPU is touched by these tests:
every call here fails validation or has nothing to do)."""

import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "gsample.h")


@pytest.fixture(scope="module")
def gs():
    from spatial_transformer_grid_amd import _binding

    if not os.path.exists(_binding.LIB_PATH):
        from spatial_transformer_grid_amd import build

        build.build()
    return _binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(gs_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "gs_abi_version", "gs_status_string", "gs_affine_grid", "gs_grid_sample_2d",
        "gs_grid_sample_3d", "gs_affine_grid_sample_fused", "gs_resize", "gs_resize_output_shape",
        "gs_grid_sample", "gs_deform_conv", "gs_deform_conv_workspace_size",
        "gs_grid_sample_2d_ws", "gs_grid_sample_2d_workspace_size", "gs_deform_conv_noalloc"])


def test_library_exports_every_declared_symbol(gs):
    handle = gs.lib()
    for name in declared_functions():
        assert hasattr(handle, name), name
    assert set(declared_functions()) == set(gs.SIGNATURES)


def test_abi_version_and_status_strings(gs):
    lib = gs.lib()
    assert lib.gs_abi_version() == 2
    for code in range(8):
        s = lib.gs_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.gs_status_string(99).decode() == "unknown status"


def test_library_shares_torchs_hip_runtime_whatever_the_import_order(gs):
    """Loading the library before torch is imported still leaves one HIP
    runtime in the process (a fresh interpreter, so the order is the one
    under test); with two, every launch on a torch stream fails."""
    import subprocess
    import sys

    code = ("import sys\n"
            "import spatial_transformer_grid_amd as g\n"
            "assert 'torch' not in sys.modules\n"
            "g.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({m.split()[-1] for m in maps if 'libamdhip64' in m.split()[-1]}))\n")
    env = dict(os.environ, PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def sample2d(gs, **kw):
    a = dict(X=FAKE, x_dtype=gs.GS_F32, x_shape=[2, 3, 4, 5], grid=FAKE, grid_dtype=gs.GS_F32,
             grid_shape=[2, 6, 7, 2], mode=0, padding=0, ac=0, Y=FAKE)
    a.update(kw)
    return gs.lib().gs_grid_sample_2d(a["X"], a["x_dtype"], gs.int64_array(a["x_shape"]), a["grid"],
                                      a["grid_dtype"], gs.int64_array(a["grid_shape"]), a["mode"],
                                      a["padding"], a["ac"], a["Y"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x_dtype=12), 3),
    (dict(x_dtype=-1), 3),
    (dict(grid_dtype=4), 3),
    (dict(grid_dtype=5), 3),
    (dict(mode=3), 4),
    (dict(mode=-1), 4),
    (dict(padding=3), 4),
    (dict(ac=2), 4),
    (dict(grid_shape=[3, 6, 7, 2]), 2),          # batch mismatch
    (dict(grid_shape=[2, 6, 7, 3]), 2),          # last grid dim must be 2
    (dict(x_shape=[2, -3, 4, 5]), 2),
    (dict(grid_shape=[2, 6, -7, 2]), 2),
    (dict(x_shape=[2, 3, 0, 5]), 2),             # empty image, non-empty output
    (dict(X=None), 1),
    (dict(Y=None), 1),
    (dict(grid=None), 1),
    (dict(x_shape=[2, 3, 1 << 15, 1 << 14]), 6),  # input plane above 2^28: GS_ERR_TOO_LARGE
    (dict(grid_shape=[2, 1 << 15, 1 << 14, 2]), 6),
])
def test_grid_sample_2d_rejects(gs, kw, status):
    assert sample2d(gs, **kw) == status


@pytest.mark.parametrize("kw", [
    dict(x_shape=[0, 3, 4, 5], grid_shape=[0, 6, 7, 2]),
    dict(x_shape=[2, 0, 4, 5]),
    dict(grid_shape=[2, 0, 7, 2]),
    dict(grid_shape=[2, 6, 0, 2], X=None, Y=None, grid=None),
])
def test_empty_work_returns_ok_without_launch(gs, kw):
    assert sample2d(gs, **kw) == 0


def test_grid_sample_3d_shape_rules(gs):
    lib = gs.lib()
    f = lambda xs, gsh, **k: lib.gs_grid_sample_3d(
        FAKE, 0, gs.int64_array(xs), FAKE, 0, gs.int64_array(gsh), k.get("mode", 0), 0, 0, FAKE, None)
    assert f([1, 2, 3, 4, 5], [1, 2, 3, 4, 2]) == 2
    assert f([1, 2, 3, 4, 5], [2, 2, 3, 4, 3]) == 2
    assert f([1, 2, 3, 4, 5], [1, 2, 3, 4, 3], mode=5) == 4
    assert f([1, 2, 3, 4, 5], [1, 0, 3, 4, 3]) == 0


def test_affine_grid_rejects(gs):
    lib = gs.lib()
    f = lambda size, n=None, dt=0, ac=0, theta=FAKE, grid=FAKE: lib.gs_affine_grid(
        theta, dt, gs.int64_array(size), len(size) if n is None else n, ac, grid, None)
    assert f([2, 3, 4, 5], n=3) == 2
    assert f([2, 3, 4, 5], dt=4) == 3          # integer theta
    assert f([2, 3, 4, 5], dt=12) == 3
    assert f([2, 3, 4, 5], ac=-1) == 4
    assert f([2, 3, -4, 5]) == 2
    assert f([2, 3, 4, 5], theta=None) == 1
    assert f([2, 3, 4, 5], grid=None) == 1
    assert f([0, 3, 4, 5], theta=None, grid=None) == 0
    assert f([2, 3, 1 << 16, 1 << 16]) == gs.GS_ERR_TOO_LARGE
    assert lib.gs_affine_grid(FAKE, 0, None, 4, 0, FAKE, None) == 1


def test_fused_rejects(gs):
    lib = gs.lib()

    def f(xs, out, rank=None, theta=FAKE, dt=0, xdt=0, mode=0):
        return lib.gs_affine_grid_sample_fused(theta, dt, FAKE, xdt, gs.int64_array(xs),
                                               len(xs) if rank is None else rank,
                                               gs.int64_array(out), mode, 0, 0, FAKE, None)

    assert f([1, 2, 3, 4], [5, 6], rank=3) == 2
    assert f([1, 2, 3, 4], [5, 6], dt=2) == 3
    assert f([1, 2, 3, 4], [5, 6], xdt=9) == 3
    assert f([1, 2, 3, 4], [5, 6], mode=9) == 4
    assert f([1, 2, 3, 4], [5, 6], theta=None) == 1
    assert f([1, 2, 3, 4], [0, 6], theta=None) == 0
    assert f([1, 2, 3, 4], [5, -6]) == 2


def test_binding_refuses_host_tensors(gs):
    torch = pytest.importorskip("torch")
    from spatial_transformer_grid_amd import grid_sample

    with pytest.raises(ValueError):
        grid_sample(torch.zeros(1, 1, 2, 2), torch.zeros(1, 2, 2, 2))


def resize_call(gs, x_shape, y_shape, scales=None, X=FAKE, Y=FAKE, dt=0, mode=0, ct=0, nm=0,
                a=-0.75, ex=0, rank=None):
    lib = gs.lib()
    sc = (ctypes.c_float * len(scales))(*scales) if scales is not None else None
    return lib.gs_resize(X, dt, gs.int64_array(x_shape), len(x_shape) if rank is None else rank,
                         gs.int64_array(y_shape), sc, mode, ct, nm, a, ex, Y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), 3),
    (dict(mode=3), 4),
    (dict(ct=4), 4),
    (dict(ct=-1), 4),
    (dict(nm=4), 4),
    (dict(ex=2), 4),
    (dict(a=float("nan")), 4),
    (dict(scales=[1.0, 1.0, 0.0, 2.0]), 4),
    (dict(scales=[1.0, 1.0, float("inf"), 2.0]), 4),
    (dict(rank=0), 2),
    (dict(rank=9), 2),
    (dict(X=None), 1),
    (dict(Y=None), 1),
])
def test_resize_rejects(gs, kw, status):
    assert resize_call(gs, [2, 3, 4, 5], [2, 3, 8, 10], **kw) == status


def test_resize_shape_rules(gs):
    # only the last three axes may change
    assert resize_call(gs, [2, 3, 4, 5, 6], [4, 3, 4, 5, 6]) == 2
    assert resize_call(gs, [2, 3, 4, 5, 6], [2, 3, 4, 5, 6], scales=[1.5, 1, 1, 1, 1]) == 2
    assert resize_call(gs, [2, 3, -4, 5], [2, 3, 8, 10]) == 2
    assert resize_call(gs, [2, 3, 0, 5], [2, 3, 8, 10]) == 2        # empty input, output not
    assert resize_call(gs, [2, 3, 4, 5], [2, 3, 0, 10], X=None, Y=None) == 0
    assert resize_call(gs, [0, 3, 4, 5], [0, 3, 8, 10], X=None, Y=None) == 0
    assert resize_call(gs, [1, 1, 1 << 15, 1 << 14], [1, 1, 2, 2]) == gs.GS_ERR_TOO_LARGE


def test_resize_output_shape_matches_oracle(gs, oracle_mod):
    """The library's host shape rule (Summary, keep_aspect_ratio_policy)
    agrees with the oracle's on the page examples and on random cases."""
    from conftest import load_golden
    from spatial_transformer_grid_amd import resize_output_shape

    cases = []
    for ex in load_golden("resize_examples.json"):
        cases.append((ex["data_shape"], ex["scales"], ex["sizes"], ex["axes"],
                      ex["keep_aspect_ratio_policy"] or "stretch"))
    rng = np.random.default_rng(5)
    for _ in range(200):
        rank = int(rng.integers(1, 6))
        shape = [int(v) for v in rng.integers(1, 40, rank)]
        count = int(rng.integers(1, rank + 1))
        axes = [int(a) for a in rng.permutation(rank)[:count]]
        axes = [a - rank if rng.random() < 0.3 else a for a in axes]
        if rng.random() < 0.5:
            scales = [float(np.float32(v)) for v in rng.uniform(0.05, 4.0, count)]
            cases.append((shape, scales, None, axes, "stretch"))
        else:
            sizes = [int(v) for v in rng.integers(0, 60, count)]
            pol = ["stretch", "not_larger", "not_smaller"][int(rng.integers(0, 3))]
            cases.append((shape, None, sizes, axes, pol))
    for shape, sc, sz, axes, pol in cases:
        ref = oracle_mod.resize_output_shape(shape, scales=sc, sizes=sz, axes=axes,
                                             keep_aspect_ratio_policy=pol)
        got = resize_output_shape(shape, sc, sz, axes, pol)
        assert got == ref, (shape, sc, sz, axes, pol)


def test_resize_output_shape_rejects(gs):
    lib = gs.lib()
    f = lambda xs, axes, sc=None, sz=None, pol=0, n=None: lib.gs_resize_output_shape(
        gs.int64_array(xs), len(xs), gs.int64_array(axes) if axes is not None else None,
        len(axes) if n is None and axes is not None else (n if n is not None else len(xs)),
        (ctypes.c_float * 4)(*sc) if sc is not None else None,
        gs.int64_array(sz) if sz is not None else None, pol, (ctypes.c_int64 * 8)())
    assert f([2, 3], [0, 0], sc=[1, 1]) == 2          # repeated axis
    assert f([2, 3], [0, 2], sc=[1, 1]) == 2          # axis out of range
    assert f([2, 3], [0, 1], sc=[1, 1], sz=[1, 1]) == 4
    assert f([2, 3], [0, 1]) == 1
    assert f([2, 3], [0, 1], sc=[1, -1]) == 4
    assert f([2, 3], [0, 1], sz=[1, -1]) == 2
    assert f([2, 3], [0, 1], sz=[1, 1], pol=3) == 4
    assert f([2, 3], None, sc=[1, 1], n=1) == 2       # no axes: one value per axis


def test_grid_sample_any_rank_rejects(gs):
    lib = gs.lib()

    def f(xs, gsh, rank=None, xdt=0, gdt=0, X=FAKE, Y=FAKE, grid=FAKE):
        return lib.gs_grid_sample(X, xdt, gs.int64_array(xs), len(xs) if rank is None else rank,
                                  grid, gdt, gs.int64_array(gsh), 0, 0, 0, Y, None)

    assert f([1, 2, 3], [1, 4, 1], rank=2) == 2              # x_rank below 3
    assert f([1] * 9, [1] * 8 + [7], rank=9) == 2             # more than 6 spatial axes
    assert f([1, 2, 3], [1, 4, 2]) == 2                       # last grid dim must be r
    assert f([1, 2, 3], [2, 4, 1]) == 2                       # batch mismatch
    assert f([1, 2, 3], [1, 4, 1], xdt=13) == 3
    assert f([1, 2, 3], [1, 4, 1], gdt=4) == 3                # integer grids are not allowed
    assert f([1, 2, 3], [1, 4, 1], grid=None) == 1
    assert f([1, 2, 3], [1, 0, 1], X=None, Y=None, grid=None) == 0
    assert f([1, 2, 1 << 28], [1, 4, 1], xdt=3) == gs.GS_ERR_TOO_LARGE  # 2^28 doubles: above 2^30 bytes


def test_binding_dtype_codes(gs):
    torch = pytest.importorskip("torch")
    assert gs.dtype_code(torch.zeros(1, dtype=torch.uint8)) == gs.GS_U8
    assert gs.dtype_code(torch.zeros(1, dtype=torch.float64)) == gs.GS_F64
    assert gs.dtype_code(torch.zeros(1, dtype=torch.int64)) == gs.GS_I64
    with pytest.raises(TypeError):
        gs.dtype_code(torch.zeros(1, dtype=torch.bool))


def test_deform_conv_rejects(gs):
    lib = gs.lib()

    def f(xs, ws, dt=0, X=FAKE, W=FAKE, off=FAKE, Y=FAKE, st=None, pd=None, dl=None, grp=1,
          og=1, rank=None):
        a = lambda v: gs.int64_array(v) if v is not None else None
        return lib.gs_deform_conv(X, dt, gs.int64_array(xs), len(xs) if rank is None else rank, W,
                                  gs.int64_array(ws), off, None, None, a(st), a(pd), a(dl), grp,
                                  og, Y, None, 0, None)

    assert f([1, 4, 8, 8], [6, 4, 3, 3], dt=5) == 3              # integer data
    assert f([1, 4, 8, 8], [6, 4, 3, 3], rank=6) == 2
    assert f([1, 4, 8, 8], [6, 3, 3, 3]) == 2                     # W's C/group
    assert f([1, 4, 8, 8], [5, 2, 3, 3], grp=2) == 2              # oC % group
    assert f([1, 4, 8, 8], [6, 4, 3, 3], og=3) == 2               # C % offset_group
    assert f([1, 4, 8, 8], [6, 4, 3, 3], grp=0) == 4
    assert f([1, 4, 8, 8], [6, 4, 3, 3], st=[0, 1]) == 4
    assert f([1, 4, 8, 8], [6, 4, 3, 3], pd=[0, -1, 0, 0]) == 4
    assert f([1, 4, 2, 8], [6, 4, 3, 3]) == 2                     # padded input too small
    assert f([1, 4, 8, 8], [6, 4, 3, 3], X=None) == 1
    assert f([1, 4, 8, 8], [6, 4, 3, 3], off=None) == 1
    assert f([0, 4, 8, 8], [6, 4, 3, 3], X=None, W=None, off=None, Y=None) == 0
    assert f([1, 4, 1 << 24, 2], [6, 4, 3, 1]) == gs.GS_ERR_TOO_LARGE
    assert lib.gs_deform_conv(FAKE, 0, gs.int64_array([1, 4, 8, 8]), 4, FAKE,
                              gs.int64_array([6, 4, 3, 3]), FAKE, None, None, None, None, None, 1,
                              1, FAKE, None, -1, None) == 4         # negative workspace size


def test_deform_conv_workspace_size(gs):
    """Channels-last copies of X and of W (kernel-position major, channels
    rounded up to 32), each rounded up to 256 bytes; none when the conv or
    offset groups are not multiples of 8 channels, for double or for 1-D and
    3-D data."""
    ws = gs.deform_conv_workspace_size
    up = lambda b: (b + 255) // 256 * 256
    # 2 x 64 x 10 x 12 bf16, W 48 x 64 x 3 x 3: X 2*64*120*2 bytes, W with
    # its 48 output channels padded to 64
    assert ws([2, 64, 10, 12], [48, 64, 3, 3], gs.GS_BF16, pads=[1, 1, 1, 1]) == \
        up(2 * 64 * 120 * 2) + up(64 * 9 * 64 * 2)
    # fp32, 40 channels per group, 2 groups of 8 output channels: each group's
    # rows padded to 32, its channels to 64
    assert ws([1, 80, 7, 7], [16, 40, 3, 3], gs.GS_F32, group=2, offset_group=2) == \
        up(80 * 49 * 4) + up(2 * 32 * 9 * 64 * 4)
    assert ws([1, 12, 7, 7], [16, 12, 3, 3], gs.GS_F32) == 0                    # 12 channels
    assert ws([1, 16, 7, 7], [16, 16, 3, 3], gs.GS_F32, offset_group=4) == 0    # 4 per offset group
    assert ws([1, 16, 7, 7], [16, 16, 3, 3], gs.GS_F64) == 0
    assert ws([1, 16, 7], [16, 16, 3], gs.GS_F32) == 0
    assert ws([1, 16, 7, 7, 7], [16, 16, 3, 3, 3], gs.GS_F32) == 0
    with pytest.raises(gs.GSError):
        ws([1, 16, 2, 7], [16, 16, 3, 3], gs.GS_F32)                          # input too small


def test_grid_sample_2d_workspace_size(gs):
    """An 8,448-byte header (probe verdicts, tile counters) plus X in
    channels-last slices; none when the channels do not fill 32-byte slices,
    for types the gather path does not take, or when an image or its output
    planes exceed 2^31 bytes."""
    ws = gs.grid_sample_2d_workspace_size
    assert ws((16, 128, 256, 256), (16, 256, 256, 2), gs.GS_F32) == 8448 + 16 * 128 * 256 * 256 * 4
    assert ws((2, 16, 5, 7), (2, 3, 4, 2), gs.GS_BF16) == 8448 + 2 * 16 * 35 * 2
    assert ws((2, 8, 5, 7), (2, 3, 4, 2), gs.GS_F32) == 8448 + 2 * 8 * 35 * 4
    assert ws((2, 24, 5, 7), (2, 3, 4, 2), gs.GS_F32) == 8448 + 2 * 24 * 35 * 4  # 32-byte slices
    assert ws((2, 12, 5, 7), (2, 3, 4, 2), gs.GS_F32) == 0     # 48-byte pixel runs
    assert ws((2, 8, 5, 7), (2, 3, 4, 2), gs.GS_F16) == 0      # 16-byte pixel runs
    assert ws((2, 8, 5, 7), (2, 3, 4, 2), gs.GS_F64) == 0
    assert ws((1, 64, 8192, 8192), (1, 4, 4, 2), gs.GS_F32) == 0  # 16 GiB image
    # tall, narrow outputs over many slices (each image's Y just below
    # 2^31 bytes): 8 images x 128 slices x (2^18 - 1) rows is more tiles than
    # the gather kernel hands out (2^27), so only the plain sampler runs (no
    # workspace); 4 images fit
    tall = (1 << 18) - 1
    assert ws((8, 4096, 4, 4), (8, tall, 1, 2), gs.GS_F16) == 0
    assert ws((4, 4096, 4, 4), (4, tall, 1, 2), gs.GS_F16) == 8448 + 4 * 4096 * 16 * 2
    with pytest.raises(gs.GSError):
        ws((2, 8, 5, 7), (3, 3, 4, 2), gs.GS_F32)              # batch mismatch


def test_deform_conv_noalloc_rejects_beyond_its_array(gs):
    """A layer whose channels-last scratch exceeds the library's 64 MiB
    array is rejected before anything is enqueued (host-side check)."""
    f = gs.lib().gs_deform_conv_noalloc
    a = gs.int64_array
    st = f(FAKE, gs.GS_F32, a([8, 512, 64, 64]), 4, FAKE, a([16, 512, 3, 3]), FAKE, None, None,
           None, None, None, 1, 1, FAKE, None)
    assert st == gs.GS_ERR_TOO_LARGE
    st = f(FAKE, 99, a([8, 512, 64, 64]), 4, FAKE, a([16, 512, 3, 3]), FAKE, None, None, None,
           None, None, 1, 1, FAKE, None)
    assert st == gs.GS_ERR_DTYPE
