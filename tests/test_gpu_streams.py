"""Calls in flight on several streams at once.

The library keeps no state between calls, and the entry points with a
workspace keep theirs in the caller's buffer, so calls enqueued on different
streams and running at the same time must give exactly the results of the
same calls run one after another.  Each round enqueues, on four streams and
without synchronising between launches, the 2-D sampler (staged path), the
gather path with its own workspace, the fused 3-D sampler, a 2-D Resize and
DeformConv with its own workspace, each on its own inputs; the outputs are
compared bit for bit with the sequential results on the default stream.
"""

import numpy as np
import pytest

import oracle
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


def make_jobs(gsa, seed):
    """(name, callable(out) that enqueues the call on the current stream,
    output shape and dtype) for one set of seeded inputs."""
    torch = torch_mod()
    rng = np.random.default_rng(seed)
    cuda = lambda a, dt=None: (torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
                               if dt is not None else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    jobs = []
    # staged 2-D sampler over an affine grid
    th = np.concatenate([np.eye(2), np.zeros((2, 1))], 1)[None].repeat(4, 0)
    th = (th + 0.1 * rng.normal(size=th.shape)).astype(np.float32)
    X1 = cuda(rng.uniform(-1, 1, (4, 16, 96, 96)).astype(np.float32))
    G1 = cuda(oracle.affine_grid(th, (4, 16, 80, 80), 0))
    jobs.append(("sampler", lambda out: gsa.grid_sample(X1, G1, "linear", "zeros", 0, out=out),
                 (4, 16, 80, 80), torch.float32))
    # gather path with a workspace of its own
    X2 = cuda(rng.uniform(-1, 1, (2, 32, 300, 64)).astype(np.float32), torch.bfloat16)
    G2 = cuda(rng.uniform(-1.2, 1.2, (2, 16, 64, 2)).astype(np.float32))
    ws2 = torch.empty(gsa.grid_sample_2d_workspace_size(tuple(X2.shape), tuple(G2.shape),
                                                        gsa.dtype_code(X2)),
                      dtype=torch.uint8, device="cuda")
    jobs.append(("gather", lambda out: gsa.grid_sample(X2, G2, "cubic", "reflection", 1, out=out,
                                                       workspace=ws2),
                 (2, 32, 16, 64), torch.bfloat16))
    # fused 3-D sampler
    t3 = np.concatenate([np.eye(3), np.zeros((3, 1))], 1)[None].repeat(2, 0)
    t3 = (t3 + 0.1 * rng.normal(size=t3.shape)).astype(np.float32)
    T3 = cuda(t3)
    X3 = cuda(rng.uniform(-1, 1, (2, 8, 16, 32, 32)).astype(np.float32))
    jobs.append(("fused 3-D", lambda out: gsa.affine_grid_sample_fused(T3, X3, (16, 32, 32), "linear",
                                                                        "border", 0, out=out),
                 (2, 8, 16, 32, 32), torch.float32))
    # 2-D Resize
    X4 = cuda(rng.uniform(-1, 1, (3, 8, 64, 48)).astype(np.float32), torch.float16)
    jobs.append(("resize", lambda out: gsa.resize_to(X4, (3, 8, 128, 96), [1.0, 1.0, 2.0, 2.0],
                                                     "cubic", "half_pixel", out=out),
                 (3, 8, 128, 96), torch.float16))
    # DeformConv with a workspace of its own
    X5 = cuda(rng.uniform(-1, 1, (2, 32, 16, 16)).astype(np.float32), torch.bfloat16)
    W5 = cuda(rng.uniform(-0.1, 0.1, (64, 32, 3, 3)).astype(np.float32), torch.bfloat16)
    O5 = cuda(rng.normal(0, 1, (2, 18, 16, 16)).astype(np.float32), torch.bfloat16)
    M5 = cuda(rng.uniform(0, 1, (2, 9, 16, 16)).astype(np.float32), torch.bfloat16)
    kw = dict(strides=[1, 1], pads=[1, 1, 1, 1], dilations=[1, 1])
    ws5 = torch.empty(gsa.deform_conv_workspace_size(tuple(X5.shape), tuple(W5.shape),
                                                     gsa.dtype_code(X5), **kw),
                      dtype=torch.uint8, device="cuda")
    jobs.append(("deform", lambda out: gsa.deform_conv(X5, W5, O5, None, M5, out=out, workspace=ws5,
                                                       **kw),
                 (2, 64, 16, 16), torch.bfloat16))
    return jobs


def bits(t):
    torch = torch_mod()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_calls_on_four_streams_match_sequential_calls(gsa):
    torch = torch_mod()
    sets = [make_jobs(gsa, 8800 + i) for i in range(4)]
    # sequential reference on the default stream
    ref = []
    for jobs in sets:
        outs = []
        for name, fn, shape, dt in jobs:
            y = torch.empty(shape, dtype=dt, device="cuda")
            fn(y)
            outs.append(y)
        ref.append(outs)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for rnd in range(3):
        note("streams round %d" % rnd)
        got = [[torch.full(shape, float("nan"), dtype=dt, device="cuda") for _, _, shape, dt in jobs]
               for jobs in sets]
        torch.cuda.synchronize()
        # interleave the launches over the streams: job j of set i on stream (i + rnd) % 4
        for j in range(len(sets[0])):
            for i, jobs in enumerate(sets):
                with torch.cuda.stream(streams[(i + rnd) % 4]):
                    jobs[j][1](got[i][j])
        torch.cuda.synchronize()
        for i, jobs in enumerate(sets):
            for j, (name, _, _, _) in enumerate(jobs):
                assert torch.equal(bits(got[i][j]), bits(ref[i][j])), (
                    "round %d, input set %d, %s: differs from the sequential call" % (rnd, i, name))


def test_calls_from_four_host_threads_match_sequential_calls(gsa):
    """The same jobs from four host threads at once, each thread on its own
    stream and with its own inputs and workspaces (ctypes releases the
    interpreter lock during the calls, so the library's entry points run
    concurrently), ten rounds per thread."""
    import threading

    torch = torch_mod()
    sets = [make_jobs(gsa, 8900 + i) for i in range(4)]
    ref = []
    for jobs in sets:
        outs = []
        for name, fn, shape, dt in jobs:
            y = torch.empty(shape, dtype=dt, device="cuda")
            fn(y)
            outs.append(y)
        ref.append(outs)
    torch.cuda.synchronize()
    note("host threads")
    errors = []

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            jobs = sets[i]
            outs = [torch.empty(shape, dtype=dt, device="cuda") for _, _, shape, dt in jobs]
            for rnd in range(10):
                with torch.cuda.stream(stream):
                    for j, (_, fn, _, _) in enumerate(jobs):
                        outs[j].fill_(float("nan"))
                        fn(outs[j])
                stream.synchronize()
                for j, (name, _, _, _) in enumerate(jobs):
                    if not torch.equal(bits(outs[j]), bits(ref[i][j])):
                        errors.append("thread %d round %d %s differs" % (i, rnd, name))
        except Exception as e:  # reported by the main thread
            errors.append("thread %d: %r" % (i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors[:5]
