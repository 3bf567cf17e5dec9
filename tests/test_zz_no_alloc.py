"""The no-allocation synchronisation (ddp_sync_allreduce_avg_noalloc), called
through the C ABI, against ddp_sync_allreduce_avg on the same inputs, bit for
bit: two calls in a row, the second on a smaller plan (the static buffer
keeps the first call's larger tables); random plans with empty and short
buckets over N = 2..64 and every dtype pair; and a HIP graph that captured
the call, replayed with new gradient values written in between."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, random_inputs, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _noalloc(ddp, plan, flats, out, order, stream=None):
    """ddp_sync_allreduce_avg_noalloc straight through ctypes."""
    ptrs = (ctypes.c_void_p * len(flats))(*[ctypes.c_void_p(t.data_ptr()) for t in flats])
    st = ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)
    code = 1 if out.dtype.itemsize == 2 else 0
    rc = ddp.lib.ddp_sync_allreduce_avg_noalloc(plan.handle, ptrs, len(flats),
                                                {"seq": 0, "ring": 1}[order], code,
                                                ctypes.c_void_p(out.data_ptr()), st)
    assert rc == 0, ddp.status_string(rc)


def _bits(torch, t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _workload(torch, ddp, name):
    wl = W.workload(name)
    plan = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    flats = []
    for r in range(wl.n_ranks):
        t = torch.empty(plan.total, dtype=tdt, device="cuda:0")
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    return plan, flats


def test_two_calls_second_smaller(env):
    """many-small (761 buckets: three batches of bases, 732 K tiles), then
    ResNet-50 (5 buckets, 100 K tiles) in the same buffer."""
    torch, ddp = env
    for name in ("many_small", "resnet50"):
        plan, flats = _workload(torch, ddp, name)
        got = torch.full((plan.total,), float("nan"), device="cuda:0")
        want = torch.full((plan.total,), float("nan"), device="cuda:0")
        print(f"{name}: no-allocation sync, ring", flush=True)
        _noalloc(ddp, plan, flats, got, "ring")
        ddp.sync_allreduce_avg(plan, flats, want, "ring")
        torch.cuda.synchronize()
        assert torch.equal(_bits(torch, got), _bits(torch, want)), name
        del flats, got, want
        torch.cuda.empty_cache()


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")],
                         ids=lambda p: f"{p[0]}-{p[1]}")
@pytest.mark.parametrize("N", [2, 3, 5, 8, 13, 17, 64])
def test_random_plans(env, pair, N):
    """Plans with empty parameters, buckets shorter than a tile and tiles that
    meet three or more ring chunks; also against the oracle.  Each case runs
    after the previous one left larger or smaller tables in the buffer."""
    torch, ddp = env
    in_dt, out_dt = pair
    rng = np.random.default_rng(1000 + N)
    eb = 4 if in_dt == "f32" else 2
    for case in range(3):
        sizes = [int(x) for x in rng.choice([0, 1, 3, 17, 255, 600, 5000, 40000, 100000],
                                            size=int(rng.integers(5, 40)))]
        if sum(sizes) == 0:
            sizes[0] = 1
        cap = int(rng.choice([64, 4096, 1 << 16, 1 << 20]))
        plan = ddp.plan_buckets(sizes, cap, in_dt)
        op = oracle.plan_cap(sizes, cap, eb)
        xs = random_inputs(rng, N, plan.total, in_dt)
        flats = [to_dev(x, torch) for x in xs]
        tout = torch.float32 if out_dt == "f32" else torch.bfloat16
        got = torch.full((plan.total,), float("nan"), dtype=tout, device="cuda:0")
        want = torch.full((plan.total,), float("nan"), dtype=tout, device="cuda:0")
        for order in ("ring", "seq"):
            _noalloc(ddp, plan, flats, got, order)
            ddp.sync_allreduce_avg(plan, flats, want, order)
            torch.cuda.synchronize()
            assert torch.equal(_bits(torch, got), _bits(torch, want)), (N, pair, case, order)
            assert_bits_equal(to_host(got, torch), oracle.sync_avg(op, xs, order, in_dt, out_dt),
                              f"N={N} {pair} case {case} {order}")


def test_graph_replays(env):
    """The call captured into a HIP graph (the caller that cannot allocate),
    replayed three times with new gradients written eagerly in between; every
    replay equals the eager ddp_sync_allreduce_avg of the same values."""
    torch, ddp = env
    sizes = [70000, 3, 0, 123457, 4096, 999]
    plan = ddp.plan_buckets(sizes, 1 << 18, "f32")
    N = 6
    flats = [torch.empty(plan.total, device="cuda:0") for _ in range(N)]
    out = torch.empty(plan.total, device="cuda:0")
    want = torch.empty(plan.total, device="cuda:0")
    side = torch.cuda.Stream()
    for r, f in enumerate(flats):
        W.device_normal_(f, r, 5, 1e-3)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _noalloc(ddp, plan, flats, out, "ring", stream=side)
    for rep in range(3):
        for r, f in enumerate(flats):
            W.device_normal_(f, 100 * rep + r, 5, 1e-3)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ddp.sync_allreduce_avg(plan, flats, want, "ring")
        torch.cuda.synchronize()
        assert torch.equal(_bits(torch, out), _bits(torch, want)), rep
    del graph
