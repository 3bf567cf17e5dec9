"""Capture and overlap ("(24) NCCL通信与分布式数据并行", sections 十 and 十一).

* A whole step -- flatten every rank, one-launch synchronisation, unflatten --
  captured into a HIP graph (through torch's graph API; the library launches
  on the capturing stream and allocates nothing once the plan is prepared and
  the bindings exist).  The graph is replayed several times with new
  gradient values written eagerly between replays, and every replay is
  compared bit for bit with the same step run eagerly, and with the oracle.
* The two-bucket schedule: the DEEP_COMM bucket averaged on an update stream
  while a compute kernel runs on the compute stream, then FIRST_COMM; the
  result equals the serial synchronisation bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def test_captured_step_replays_match_eager_and_oracle(env):
    torch, ddp = env
    sizes = [p.numel for p in W.many_small(n=3000)]
    N, cap = 4, 1 << 20
    lp = ddp.plan_buckets(sizes, cap, "f32")
    op = oracle.plan_cap(sizes, cap, 4)
    lp.prepare(N)   # every table the captured RING syncs read, uploaded before capture
    dev = "cuda:0"
    grads = [[torch.empty(n, dtype=torch.float32, device=dev) for n in sizes] for _ in range(N)]
    flats = [torch.empty(lp.total, dtype=torch.float32, device=dev) for _ in range(N)]
    out = torch.empty(lp.total, dtype=torch.float32, device=dev)
    res = [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]
    binds = [ddp.bind_params(lp, grads[r]) for r in range(N)]
    rbind = ddp.bind_params(lp, res)

    def step():
        for r in range(N):
            ddp.flatten(lp, binds[r], flats[r])
        ddp.sync_allreduce_avg(lp, flats, out, "ring")
        ddp.unflatten(lp, rbind, out)

    def fill(seed):
        rng = np.random.default_rng(seed)
        host = []
        for r in range(N):
            hr = []
            for g, n in zip(grads[r], sizes):
                h = (rng.standard_normal(n) * 1e-3).astype(np.float32)
                g.copy_(to_dev(h, torch))
                hr.append(h)
            host.append(hr)
        return host

    fill(0)
    step()                       # warm up on the side of the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for rep in range(4):
        host = fill(100 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replay = [to_host(t, torch) for t in res]
        step()                   # the same step, eagerly
        torch.cuda.synchronize()
        eager = [to_host(t, torch) for t in res]
        want = oracle.unflatten(op, oracle.sync_avg(op, [oracle.flatten(op, h) for h in host], "ring"))
        for p in range(0, len(sizes), 7):
            assert_bits_equal(replay[p], eager[p], f"replay {rep} param {p}")
            assert_bits_equal(replay[p], want[p], f"replay {rep} param {p} vs oracle")


def test_two_bucket_overlap_matches_serial(env):
    torch, ddp = env
    wl = W.workload("resnet50")
    lp = ddp.plan_two_bucket(wl.numel, wl.regions, "f32")
    op = oracle.plan_two_bucket(wl.numel, wl.regions)
    assert lp.n_buckets == 2
    dev = "cuda:0"
    flats = []
    for r in range(wl.n_ranks):
        t = torch.empty(lp.total, dtype=torch.float32, device=dev)
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    serial = torch.empty(lp.total, dtype=torch.float32, device=dev)
    overlapped = torch.full((lp.total,), float("nan"), dtype=torch.float32, device=dev)
    ddp.sync_allreduce_avg(lp, flats, serial, "ring")
    torch.cuda.synchronize()
    a = torch.randn(2048, 2048, device=dev, dtype=torch.bfloat16)
    b = torch.randn(2048, 2048, device=dev, dtype=torch.bfloat16)
    comp, upd = torch.cuda.Stream(), torch.cuda.Stream()
    (deep_len, deep_base, _, _), (first_len, first_base, _, _) = lp.bucket(0), lp.bucket(1)
    comp.wait_stream(torch.cuda.current_stream())
    upd.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(comp):
        for _ in range(4):
            c = torch.mm(a, b)          # stands in for the first layer's backward
    with torch.cuda.stream(upd):
        ddp.bucket_allreduce_avg([f[deep_base:deep_base + deep_len] for f in flats],
                                 overlapped[deep_base:deep_base + deep_len], "ring")
    upd.wait_stream(comp)
    with torch.cuda.stream(upd):
        ddp.bucket_allreduce_avg([f[first_base:first_base + first_len] for f in flats],
                                 overlapped[first_base:first_base + first_len], "ring")
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    assert_bits_equal(to_host(overlapped, torch), to_host(serial, torch), "overlapped")
    host = [to_host(f, torch) for f in flats]
    assert_bits_equal(to_host(serial, torch), oracle.sync_avg(op, host, "ring"), "two-bucket oracle")
