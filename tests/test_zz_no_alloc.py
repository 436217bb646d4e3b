"""gs_deform_conv_noalloc (the library's own scratch array, no allocation)
against gs_deform_conv with a caller-owned workspace, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (and another
element type), each compared bit for bit with gs_deform_conv given a
workspace: both run the same kernels on the same data.  A shape that needs no
scratch (double data, the direct kernel) runs too, and one that needs more
than the array holds is rejected before anything is enqueued.
"""

import numpy as np
import pytest

import workloads as W
from parity import note, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import spatial_transformer_grid_amd as gsa

    gsa.lib()
    return gsa


def layer(dw, x_shape, w_shape, tdt):
    torch = torch_mod()
    inp = W.make_deform_inputs(dw, x_shape, w_shape)
    return {k: torch.from_numpy(v).cuda().to(tdt) for k, v in inp.items()}


def both(gsa, d, pads):
    torch = torch_mod()
    ws_bytes = gsa.deform_conv_workspace_size(tuple(d["X"].shape), tuple(d["W"].shape),
                                              gsa.dtype_code(d["X"]), None, pads)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    ref = gsa.deform_conv(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=pads,
                          workspace=ws)
    got = gsa.deform_conv_noalloc(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=pads)
    torch.cuda.synchronize()
    return got, ref, ws_bytes


def test_two_calls_match_the_workspace_entry_point(gsa):
    torch = torch_mod()
    dw = W.DEFORM_WORKLOADS["dcn2d_resnet"]
    pads = list(dw.pads)
    cases = [
        ("dcn2d_resnet bf16, full size", dw.x_shape, dw.w_shape, torch.bfloat16),
        ("smaller fp32 layer", (2, 48, 21, 19), (40, 48, 3, 3), torch.float32),
    ]
    for what, xs, wsh, tdt in cases:
        note("noalloc %s X=%s W=%s" % (what, xs, wsh))
        d = layer(dw, xs, wsh, tdt)
        got, ref, need = both(gsa, d, pads)
        assert 0 < need <= 64 << 20, need
        assert torch.equal(got, ref), what


def test_shape_without_scratch_runs_as_the_plain_call(gsa):
    torch = torch_mod()
    rng = np.random.default_rng(9)
    note("noalloc double data (direct kernel)")
    X = torch.from_numpy(rng.uniform(-1, 1, (1, 4, 9, 8))).cuda()
    Wt = torch.from_numpy(rng.uniform(-1, 1, (3, 4, 3, 3))).cuda()
    off = torch.from_numpy(rng.normal(0, 1, (1, 18, 7, 6))).cuda()
    got = gsa.deform_conv_noalloc(X, Wt, off)
    ref = gsa.deform_conv(X, Wt, off)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_beyond_the_array_is_rejected(gsa):
    torch = torch_mod()
    # X alone is 8 * 512 * 64 * 64 * 4 bytes = 64 MiB: with packed W it needs more
    X = torch.zeros((8, 512, 64, 64), device="cuda")
    Wt = torch.zeros((16, 512, 3, 3), device="cuda")
    off = torch.zeros((8, 18, 62, 62), device="cuda")
    Y = torch.full((8, 16, 62, 62), 7.0, device="cuda")
    with pytest.raises(gsa.GSError) as e:
        gsa.deform_conv_noalloc(X, Wt, off, out=Y)
    assert e.value.status == 6  # GS_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())  # nothing written


def test_captured_in_a_graph(gsa):
    """The callers this entry point is for include code under graph capture:
    after one eager call (which looks the array's address up), the call is
    captured in a graph and replayed three times with new inputs, each replay
    equal bit for bit to gs_deform_conv with a workspace on the same inputs."""
    torch = torch_mod()
    dw = W.DEFORM_WORKLOADS["dcn2d_resnet"]
    pads = list(dw.pads)
    d = layer(dw, (2, 32, 20, 18), (48, 32, 3, 3), torch.bfloat16)
    Y = torch.empty((2, 48, 20, 18), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gsa.deform_conv_noalloc(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=pads, out=Y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gsa.deform_conv_noalloc(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=pads, out=Y)
    rng = np.random.default_rng(31)
    for rep in range(3):
        note("noalloc graph replay %d" % rep)
        for k in ("X", "offset", "mask"):
            d[k].copy_(torch.from_numpy(rng.uniform(-1, 1, tuple(d[k].shape)).astype(np.float32)))
        graph.replay()
        got = Y.clone()
        torch.cuda.synchronize()
        ref = gsa.deform_conv(d["X"], d["W"], d["offset"], d["B"], d["mask"], pads=pads)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "replay %d" % rep
