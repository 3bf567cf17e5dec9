"""GPU parity of ddp_accumulate (local accumulation of no_sync micro-steps,
"DDP" (sgdbs.github.io, AI_Infra/1.DataParallel) section 5.2) and of the whole
no_sync scenario: M micro-steps accumulated per virtual rank, then one
synchronisation, bit for bit against the oracle."""
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


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n_bufs", [1, 2, 5, 8, 64])
def test_accumulate_parity(env, dt, n_bufs):
    torch, ddp = env
    rng = np.random.default_rng(n_bufs + len(dt))
    for L in (1, 3, 7, 256, 511, 4099, 100_003):
        d = random_inputs(rng, n_bufs, L, dt)
        s = random_inputs(rng, n_bufs, L, dt)
        dd = [to_dev(x, torch) for x in d]
        sd = [to_dev(x, torch) for x in s]
        ddp.accumulate(dd, sd)
        torch.cuda.synchronize()
        for k in range(n_bufs):
            want = d[k].copy()
            oracle.accumulate(want, s[k], dt)
            assert_bits_equal(to_host(dd[k], torch), want, f"{dt} n={n_bufs} L={L} k={k}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_accumulate_misaligned_and_self(env, dt):
    torch, ddp = env
    rng = np.random.default_rng(9)
    L = 10_001
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    d, s = random_inputs(rng, 3, L, dt), random_inputs(rng, 3, L, dt)
    dd, sd = [], []
    for k in range(3):
        bd = torch.empty(L + 4, dtype=tdt, device="cuda:0")
        bs = torch.empty(L + 4, dtype=tdt, device="cuda:0")
        bd[1:1 + L].copy_(to_dev(d[k], torch))
        bs[3:3 + L].copy_(to_dev(s[k], torch))
        dd.append(bd[1:1 + L])
        sd.append(bs[3:3 + L])
    ddp.accumulate(dd, sd)
    torch.cuda.synchronize()
    for k in range(3):
        want = d[k].copy()
        oracle.accumulate(want, s[k], dt)
        assert_bits_equal(to_host(dd[k], torch), want, "misaligned")
    # a destination that is its own source doubles
    x = to_dev(d[0], torch)
    ddp.accumulate([x], [x])
    torch.cuda.synchronize()
    want = d[0].copy()
    oracle.accumulate(want, d[0].copy(), dt)
    assert_bits_equal(to_host(x, torch), want, "self")


def test_accumulate_rejects_overlap(env):
    torch, ddp = env
    a = torch.zeros(1000, device="cuda:0")
    with pytest.raises(ddp.DDPError) as ei:
        ddp.accumulate([a[:500]], [a[100:600]])
    assert ei.value.status == 4


@pytest.mark.parametrize("name,order", [("resnet50", "ring"), ("resnet50", "seq"),
                                        ("many_small", "ring")])
def test_no_sync_micro_steps_then_one_sync(env, name, order):
    torch, ddp = env
    wl = W.workload(name)
    lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
    op = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
    M, N, P = 3, wl.n_ranks, op.total
    micro = []
    for m in range(M):
        step = []
        for r in range(N):
            t = torch.empty(P, dtype=torch.float32, device="cuda:0")
            W.device_normal_(t, r, wl.stream + 100 * (m + 1), wl.sigma)
            step.append(t)
        micro.append(step)
    local = [t.clone() for t in micro[0]]
    for m in range(1, M):
        ddp.accumulate(local, micro[m])
    out = torch.empty(P, dtype=torch.float32, device="cuda:0")
    ddp.sync_allreduce_avg(lp, local, out, order)
    torch.cuda.synchronize()
    host = [[to_host(t, torch) for t in step] for step in micro]
    want = oracle.no_sync_then_sync(op, host, order)
    assert_bits_equal(to_host(out, torch), want, f"{name} {order} no_sync")
    del micro, local, out
    torch.cuda.empty_cache()
