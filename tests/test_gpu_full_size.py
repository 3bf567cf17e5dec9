"""Every output element of the multi-GB workloads compared with the oracle,
bit for bit, by streaming the device buffers to the host piece by piece
(tests/gpu_stream.py) and folding each piece with the oracle's piece form
on host threads.

* the one-launch synchronisation (ddp_sync_allreduce_avg): GPT-1.3B with
  the 146-bucket cap plan and with the two-bucket DEEP_COMM / FIRST_COMM
  split (N = 8, ring), Llama-7B (N = 8, bf16, sequential and ring);
* the one-kernel synchronisation over per-parameter tensors
  (ddp_param_sync_run): GPT-1.3B (ring) and Llama-7B (bf16, both orders);
* the average folded into two momentum-SGD steps: flat (ddp_sync_sgd_update,
  Llama-7B, both orders) and per parameter (ddp_param_sgd_run, Llama-7B,
  ring), parameters and momentum of every element.

Gradients come from torch's seeded device generator (workloads
.device_normal_); the oracle reads the same device values back.
"""
import time

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_stream import StreamedCheck
from gpu_util import assert_bits_equal, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _tdt(torch, dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


def _plans(ddp, wl):
    if wl.two_bucket:
        return (ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype),
                oracle.plan_two_bucket(wl.numel, wl.regions))
    return (ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype),
            oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes))


def _same(got, want, what):
    view = np.uint16 if got.dtype == np.uint16 else np.uint32
    if not np.array_equal(got.view(view), want.view(view)):
        assert_bits_equal(got, want, what)


def _avg_check(N, orders, in_dt, out_dt, what):
    """meta = (bucket length, position of the run's first element in it);
    hosts: x0..x{N-1} the ranks' inputs, one output per order."""
    def check(meta, off, hosts):
        L, lo = meta
        xs = [hosts[f"x{r}"] for r in range(N)]
        for o in orders:
            want = oracle.bucket_range_avg(xs, L, lo + off, o, in_dt, out_dt)
            _same(hosts[o], want, f"{what} {o}: bucket of {L} at {lo + off}")
    return check


def _report(what, n, t0):
    print(f"{what}: {n} elements compared in {time.perf_counter() - t0:.1f} s", flush=True)


def _flats(torch, wl, total):
    flats = []
    for r in range(wl.n_ranks):
        t = torch.empty(total, dtype=_tdt(torch, wl.dtype), device="cuda:0")
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    return flats


@pytest.mark.parametrize("name,orders", [("gpt1p3b", ("ring",)),
                                         ("gpt1p3b_two_bucket", ("ring",)),
                                         ("llama7b", ("seq", "ring"))])
def test_sync_every_element(env, name, orders):
    torch, ddp = env
    wl = W.workload(name)
    lp, op = _plans(ddp, wl)
    assert lp.buckets() == op.buckets
    flats = _flats(torch, wl, lp.total)
    outs = {o: torch.full((lp.total,), float("nan"), dtype=_tdt(torch, wl.out_dtype),
                          device="cuda:0") for o in orders}
    print(f"{name}: sync {orders}", flush=True)
    for o in orders:
        ddp.sync_allreduce_avg(lp, flats, outs[o], o)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    check = _avg_check(wl.n_ranks, orders, wl.dtype, wl.out_dtype, name)
    with StreamedCheck(torch, check) as sc:
        for L, base in zip(op.bucket_len, op.bucket_base):
            views = {f"x{r}": f[base:base + L] for r, f in enumerate(flats)}
            views.update({o: outs[o][base:base + L] for o in orders})
            sc.add((L, 0), views)
        n = sc.finish()
    _report(name, n, t0)
    assert n == lp.total
    del flats, outs
    torch.cuda.empty_cache()


def _param_stores(torch, wl, P):
    """Each rank's gradients as per-parameter tensors cut from one store in
    registration order (views, as autograd leaves separate tensors)."""
    reg_off = np.cumsum([0] + wl.numel[:-1]).astype(np.int64)
    stores = []
    for r in range(wl.n_ranks):
        t = torch.empty(P, dtype=_tdt(torch, wl.dtype), device="cuda:0")
        W.device_normal_(t, r, wl.stream, wl.sigma)
        stores.append(t)
    views = lambda t: [t[o:o + n] for o, n in zip(reg_off, wl.numel)]   # noqa: E731
    return stores, views


def _param_runs(op):
    """(parameter, bucket length, offset in bucket) of every parameter."""
    lens = op.bucket_len
    return [(p, lens[b], off) for p, (b, off) in enumerate(op.param_location())]


@pytest.mark.parametrize("name,orders", [("gpt1p3b", ("ring",)), ("llama7b", ("seq", "ring"))])
def test_param_sync_every_element(env, name, orders):
    torch, ddp = env
    wl = W.workload(name)
    lp, op = _plans(ddp, wl)
    stores, views = _param_stores(torch, wl, lp.total)
    grads = [views(t) for t in stores]
    binds = [ddp.bind_params(lp, g) for g in grads]
    outs = {}
    print(f"{name}: per-parameter sync {orders}", flush=True)
    for o in orders:
        store = torch.full((lp.total,), float("nan"), dtype=_tdt(torch, wl.out_dtype),
                           device="cuda:0")
        outs[o] = views(store)
        ps = ddp.param_sync(lp, binds, ddp.bind_params(lp, outs[o]), o)
        ps()
        torch.cuda.synchronize()
        del ps
    t0 = time.perf_counter()
    check = _avg_check(wl.n_ranks, orders, wl.dtype, wl.out_dtype, f"{name} per-parameter")
    with StreamedCheck(torch, check) as sc:
        for p, L, off in _param_runs(op):
            if wl.numel[p] == 0:
                continue
            v = {f"x{r}": grads[r][p] for r in range(wl.n_ranks)}
            v.update({o: outs[o][p] for o in orders})
            sc.add((L, off), v)
        n = sc.finish()
    _report(f"{name} per-parameter", n, t0)
    assert n == lp.total
    del stores, grads, outs, binds
    torch.cuda.empty_cache()


def _sgd_check(N, order, lr, mu, steps, what):
    """hosts: x0..x{N-1}, p0 (parameters before), p and m (after `steps`
    steps); the oracle averages the piece, then applies its SGD step."""
    def check(meta, off, hosts):
        L, lo = meta
        avg = oracle.bucket_range_avg([hosts[f"x{r}"] for r in range(N)], L, lo + off, order,
                                      "bf16", "bf16")
        wp = hosts["p0"].copy()
        wm = np.zeros_like(wp)
        for _ in range(steps):
            oracle.sgd_step(wp, avg, lr, "bf16", wm, mu)
        _same(hosts["p"], wp, f"{what} params: bucket of {L} at {lo + off}")
        _same(hosts["m"], wm, f"{what} momentum: bucket of {L} at {lo + off}")
    return check


def test_fused_sgd_every_element_llama(env):
    """ddp_sync_sgd_update at the Llama-7B size: bf16 gradients of 8 ranks,
    27 GB each of f32 parameters and momentum, two momentum steps per order."""
    torch, ddp = env
    wl = W.workload("llama7b")
    lp, op = _plans(ddp, wl)
    P = lp.total
    flats = _flats(torch, wl, P)
    p0 = torch.empty(P, dtype=torch.float32, device="cuda:0")
    W.device_normal_(p0, 99, 7, 1.0)
    params = torch.empty_like(p0)
    mbuf = torch.empty_like(p0)
    for order in ("seq", "ring"):
        print(f"llama7b fused SGD {order}", flush=True)
        params.copy_(p0)
        mbuf.zero_()
        for _ in range(2):
            ddp.sync_sgd_update(lp, flats, params, 0.1, order, momentum_buf=mbuf, momentum=0.9)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with StreamedCheck(torch, _sgd_check(wl.n_ranks, order, 0.1, 0.9, 2,
                                             f"llama7b fused {order}")) as sc:
            for L, base in zip(op.bucket_len, op.bucket_base):
                v = {f"x{r}": f[base:base + L] for r, f in enumerate(flats)}
                v.update(p0=p0[base:base + L], p=params[base:base + L], m=mbuf[base:base + L])
                sc.add((L, 0), v)
            n = sc.finish()
        _report(f"llama7b fused SGD {order}", n, t0)
        assert n == P
    del flats, p0, params, mbuf
    torch.cuda.empty_cache()


def test_param_sgd_every_element_llama(env):
    """ddp_param_sgd_run at the Llama-7B size: per-parameter bf16 gradients
    of 8 ranks, per-parameter f32 parameters and momentum, two momentum
    steps in ring order."""
    torch, ddp = env
    wl = W.workload("llama7b")
    lp, op = _plans(ddp, wl)
    P = lp.total
    stores, views = _param_stores(torch, wl, P)
    grads = [views(t) for t in stores]
    p0 = torch.empty(P, dtype=torch.float32, device="cuda:0")
    W.device_normal_(p0, 99, 7, 1.0)
    pstore = p0.clone()
    mstore = torch.zeros_like(p0)
    step = ddp.param_sgd(lp, [ddp.bind_params(lp, g) for g in grads],
                         ddp.bind_params(lp, views(pstore)), ddp.bind_params(lp, views(mstore)),
                         None, "ring")
    print("llama7b per-parameter fused SGD ring", flush=True)
    for _ in range(2):
        step(0.1, 0.9)
    torch.cuda.synchronize()
    del step
    t0 = time.perf_counter()
    p0s, ps, ms = views(p0), views(pstore), views(mstore)
    with StreamedCheck(torch, _sgd_check(wl.n_ranks, "ring", 0.1, 0.9, 2,
                                         "llama7b per-parameter fused ring")) as sc:
        for p, L, off in _param_runs(op):
            if wl.numel[p] == 0:
                continue
            v = {f"x{r}": grads[r][p] for r in range(wl.n_ranks)}
            v.update(p0=p0s[p], p=ps[p], m=ms[p])
            sc.add((L, off), v)
        n = sc.finish()
    _report("llama7b per-parameter fused SGD ring", n, t0)
    assert n == P
    del stores, grads, p0, pstore, mstore
    torch.cuda.empty_cache()
