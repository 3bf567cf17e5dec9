"""The mean all-reduce at its two small call sites, against the oracle, bit
for bit:

* the BN running statistics of "(24) NCCL通信与分布式数据并行" section 十二:
  every BN layer's running mean and running variance of ResNet-50, stored
  back to back as one contiguous range (2 x 26,560 f32 values per rank),
  averaged over 8 virtual ranks -- on its own buffers and as a range inside
  a larger per-rank model-state buffer at an unaligned offset;
* the validation record of section 十三: 3 scalars per rank (loss, top-1,
  top-5 accumulated), averaged over 8 virtual ranks;

each through the per-bucket call, a prepared one-bucket sync (make_sync) and
a captured HIP graph replayed with new values written in between.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

N = 8


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _bn_channels():
    wl = W.workload("resnet50")
    return sum(p.numel for p in wl.params if p.region == W.REGION_BN_WEIGHT)


def _stats(rng, channels):
    """Per-rank running mean (any sign) then running variance (positive)."""
    mean = rng.standard_normal(channels) * 0.3
    var = np.abs(rng.standard_normal(channels)) + 0.5
    return np.concatenate([mean, var]).astype(np.float32)


def _record(rng):
    """Per-rank loss, top-1 and top-5 accuracies of one validation pass."""
    return np.array([rng.uniform(1.0, 3.0), rng.uniform(0.5, 0.8), rng.uniform(0.8, 0.95)],
                    np.float32)


def test_bn_channel_count():
    assert _bn_channels() == 26560


@pytest.mark.parametrize("site", ["bn_running_stats", "metric_record"])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_small_mean_all_reduce(env, site, order):
    torch, ddp = env
    rng = np.random.default_rng(23 if site == "metric_record" else 29)
    make = (lambda: _record(rng)) if site == "metric_record" else \
        (lambda: _stats(rng, _bn_channels()))
    xs = [make() for _ in range(N)]
    L = xs[0].size
    want = oracle.bucket_avg(xs, order)
    ins = [to_dev(x, torch) for x in xs]
    out = torch.full((L,), float("nan"), device="cuda:0")
    ddp.bucket_allreduce_avg(ins, out, order)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out, torch), want, f"{site} {order} per-bucket call")

    plan = ddp.plan_buckets([L], 1 << 40, "f32")
    out.fill_(float("nan"))
    sync = ddp.make_sync(plan, ins, out, order)
    sync()
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out, torch), want, f"{site} {order} prepared")

    # captured once, replayed with new values each time
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gsync = ddp.make_sync(plan, ins, out, order, stream=side)
    gsync()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gsync()
    for rep in range(3):
        xs = [make() for _ in range(N)]
        for t, x in zip(ins, xs):
            t.copy_(to_dev(x, torch))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(to_host(out, torch), oracle.bucket_avg(xs, order),
                          f"{site} {order} graph replay {rep}")
    del graph


@pytest.mark.parametrize("order", ["seq", "ring"])
def test_bn_stats_inside_model_state(env, order):
    """The statistics as a range of a larger per-rank state buffer (weights
    first, then the running statistics, at an element offset that is not a
    multiple of 4), averaged in place into rank 0's buffer."""
    torch, ddp = env
    rng = np.random.default_rng(31)
    C = _bn_channels()
    off = 1_000_003
    states = []
    xs = []
    for _ in range(N):
        s = rng.standard_normal(off + 2 * C + 7).astype(np.float32)
        xs.append(_stats(rng, C))
        s[off:off + 2 * C] = xs[-1]
        states.append(to_dev(s, torch))
    before = [to_host(s, torch) for s in states]
    ddp.bucket_allreduce_avg([s[off:off + 2 * C] for s in states], states[0][off:off + 2 * C],
                             order)
    torch.cuda.synchronize()
    got = to_host(states[0], torch)
    assert_bits_equal(got[off:off + 2 * C], oracle.bucket_avg(xs, order), f"in place {order}")
    # nothing outside the range moved, on any rank
    assert np.array_equal(got[:off].view(np.uint32), before[0][:off].view(np.uint32))
    assert np.array_equal(got[off + 2 * C:].view(np.uint32),
                          before[0][off + 2 * C:].view(np.uint32))
    for r in range(1, N):
        assert np.array_equal(to_host(states[r], torch).view(np.uint32),
                              before[r].view(np.uint32))
