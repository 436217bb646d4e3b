"""Inputs of more than 2^31 elements on the GPU.

X holds (N, C, spatial) with N * C * spatial beyond 2^31 (fp16 / int8, about
2.3 GB to 4.6 GB), generated on the device from a seeded generator; the
outputs are small.  Planes past the 2^31-element mark are addressed through
64-bit image and channel offsets, and each plane through its own 32-bit
buffer range.  Sampled (image, channel) planes of the output are compared
with the oracle run on those planes alone (the oracle samples each plane
independently, so a plane and its grid give the same values as the whole
tensor).  Tolerances are those of the other parity tests.
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


def device_x(shape, dtype, seed):
    """X of `shape` on the device, values uniform in [-1, 1) (floats) or over
    the type's range (int8), from a seeded generator on the device."""
    torch = torch_mod()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    if dtype == torch.int8:
        return torch.randint(-128, 128, shape, generator=gen, dtype=torch.int8, device="cuda")
    x = torch.empty(shape, dtype=dtype, device="cuda")
    x.uniform_(-1.0, 1.0, generator=gen)
    return x


def planes_to_check(n, c):
    """(image, channel) pairs: both ends of each image's channel range and
    the ones around the 2^31-element boundary of the whole tensor."""
    pairs = {(0, 0), (0, c - 1), (n - 1, 0), (n - 1, c - 1), (n - 1, c // 2)}
    return sorted(pairs)


def host_plane(X, b, ch):
    torch = torch_mod()
    p = X[b:b + 1, ch:ch + 1]
    return p.float().cpu().numpy() if X.dtype != torch.int8 else p.cpu().numpy()


@pytest.mark.parametrize("mode", ["nearest", "linear", "cubic"])
def test_sampler_2d_beyond_2_31_elements(gsa, mode):
    torch = torch_mod()
    n, c, h, w = 2, 1100, 1024, 1024          # 2.31e9 elements, fp16
    assert n * c * h * w > 2 ** 31
    note("large 2-D sampler %s X=(%d,%d,%d,%d) fp16" % (mode, n, c, h, w))
    X = device_x((n, c, h, w), torch.float16, 11)
    rng = np.random.default_rng(12)
    G = rng.uniform(-1.1, 1.1, (n, 16, 16, 2)).astype(np.float32)
    Y = gsa.grid_sample(X, torch.from_numpy(G).cuda(), mode, "border", 0)
    torch.cuda.synchronize()
    for b, ch in planes_to_check(n, c):
        xp = host_plane(X, b, ch)
        ref = oracle.grid_sample(xp, G[b:b + 1], mode, "border", 0)
        got = Y[b:b + 1, ch:ch + 1].double().cpu().numpy()
        check(got, ref, mode, "f16", float(np.abs(xp).max()), "plane (%d, %d)" % (b, ch))
    del X, Y
    torch.cuda.empty_cache()


def test_fused_and_3d_beyond_2_31_elements(gsa):
    torch = torch_mod()
    n, c, d, h, w = 2, 1100, 16, 256, 256     # 2.31e9 elements, fp16
    note("large 3-D fused sampler X=(%d,%d,%d,%d,%d) fp16" % (n, c, d, h, w))
    X = device_x((n, c, d, h, w), torch.float16, 13)
    theta = np.concatenate([np.eye(3), np.zeros((3, 1))], 1)[None].repeat(n, 0)
    theta = (theta + 0.05 * np.random.default_rng(14).normal(size=theta.shape)).astype(np.float32)
    out = (4, 8, 8)
    Y = gsa.affine_grid_sample_fused(torch.from_numpy(theta).cuda(), X, out, "linear", "zeros", 0)
    torch.cuda.synchronize()
    G = oracle.affine_grid(theta, (n, 1) + out, 0)
    for b, ch in planes_to_check(n, c):
        xp = host_plane(X, b, ch)
        ref = oracle.grid_sample(xp, G[b:b + 1], "linear", "zeros", 0)
        got = Y[b:b + 1, ch:ch + 1].double().cpu().numpy()
        check(got, ref, "linear", "f16", float(np.abs(xp).max()), "plane (%d, %d)" % (b, ch))
    del X, Y
    torch.cuda.empty_cache()


def test_resize_beyond_2_31_elements(gsa):
    torch = torch_mod()
    n, c, h, w = 2, 1100, 1024, 1024
    note("large Resize X=(%d,%d,%d,%d) fp16" % (n, c, h, w))
    X = device_x((n, c, h, w), torch.float16, 15)
    Y = gsa.resize_to(X, (n, c, 16, 12), None, "linear", "half_pixel")
    torch.cuda.synchronize()
    for b, ch in planes_to_check(n, c):
        xp = host_plane(X, b, ch)
        ref = oracle.resize(xp, (1, 1, 16, 12), None, "linear", "half_pixel")
        got = Y[b:b + 1, ch:ch + 1].double().cpu().numpy()
        check(got, ref, "linear", "f16", float(np.abs(xp).max()), "plane (%d, %d)" % (b, ch))
    del X, Y
    torch.cuda.empty_cache()


def test_any_rank_int8_beyond_2_31_elements(gsa):
    """int8 X through the any-rank kernel (bit for bit after the integer
    cast, as the other any-rank tests)."""
    torch = torch_mod()
    n, c, h, w = 2, 1100, 1024, 1024
    note("large any-rank int8 X=(%d,%d,%d,%d)" % (n, c, h, w))
    X = device_x((n, c, h, w), torch.int8, 16)
    rng = np.random.default_rng(17)
    G = rng.uniform(-1.1, 1.1, (n, 8, 8, 2)).astype(np.float32)
    Y = gsa.grid_sample(X, torch.from_numpy(G).cuda(), "linear", "reflection", 1)
    torch.cuda.synchronize()
    for b, ch in planes_to_check(n, c):
        xp = host_plane(X, b, ch)
        ref = oracle.to_integer(oracle.grid_sample(xp, G[b:b + 1], "linear", "reflection", 1),
                                np.dtype(np.int8))
        got = Y[b:b + 1, ch:ch + 1].cpu().numpy()
        assert np.array_equal(got, ref), "plane (%d, %d)" % (b, ch)
    del X, Y
    torch.cuda.empty_cache()
