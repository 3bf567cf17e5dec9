"""Seeded random plans against the oracle, bit for bit: cap-mode plans with
tiny caps (hundreds of buckets) and zero-size parameters (empty buckets),
two-bucket plans with random region tags, N = 1..10, every dtype pair, both
orders -- through the one-launch sync, the per-bucket calls, the fused SGD
step and flatten/unflatten.  Also two different plans synchronising
concurrently on two streams."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, random_inputs, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")]


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _random_case(rng):
    n = int(rng.integers(1, 120))
    numel = [int(v) for v in rng.integers(0, 3000, n)]
    for _ in range(int(rng.integers(0, 4))):
        numel[int(rng.integers(0, n))] = 0
    in_dt, out_dt = PAIRS[int(rng.integers(0, 3))]
    N = int(rng.integers(1, 11))
    if N == 1:
        out_dt = in_dt
    eb = 4 if in_dt == "f32" else 2
    if rng.random() < 0.25:
        regions = [int(v) for v in rng.integers(0, 6, n)]
        return numel, ("two", regions), in_dt, out_dt, N, eb
    cap = int(rng.choice([1, 8, 64, 1000, 4096, 40000, int(rng.integers(1, 30000))]))
    return numel, ("cap", cap), in_dt, out_dt, N, eb


@pytest.mark.parametrize("seed", range(12))
def test_random_plans(env, seed):
    torch, ddp = env
    rng = np.random.default_rng(1234 + seed)
    for case in range(8):
        numel, mode, in_dt, out_dt, N, eb = _random_case(rng)
        if mode[0] == "cap":
            lp = ddp.plan_buckets(numel, mode[1], in_dt)
            op = oracle.plan_cap(numel, mode[1], eb)
        else:
            lp = ddp.plan_two_bucket(numel, mode[1], in_dt)
            op = oracle.plan_two_bucket(numel, mode[1])
        assert lp.buckets() == op.buckets
        P = op.total
        tag = f"seed={seed} case={case} N={N} {in_dt}->{out_dt} {mode[0]} P={P} B={op.n_buckets}"
        print(tag, flush=True)
        xs = random_inputs(rng, N, P, in_dt)
        ts = [to_dev(x, torch) for x in xs]
        odt = torch.float32 if out_dt == "f32" else torch.bfloat16
        out = torch.empty(P, dtype=odt, device="cuda:0")
        for order in ("seq", "ring"):
            want = oracle.sync_avg(op, xs, order, in_dt, out_dt)
            ddp.sync_allreduce_avg(lp, ts, out, order)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(out, torch), want, "sync " + tag)
            per = torch.empty_like(out)
            for b in range(lp.n_buckets):
                ln, base, _, _ = lp.bucket(b)
                ddp.bucket_allreduce_avg([t[base:base + ln] for t in ts], per[base:base + ln], order,
                                         length=ln)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(per, torch), want, "per-bucket " + tag)
        if P and case % 2 == 0:
            p0 = rng.standard_normal(P).astype(np.float32)
            params = to_dev(p0, torch)
            ddp.sync_sgd_update(lp, ts, params, 0.02, "ring", out_dtype=out_dt)
            torch.cuda.synchronize()
            wp = p0.copy()
            oracle.sync_sgd(op, xs, "ring", wp, 0.02, in_dt, out_dt)
            assert_bits_equal(to_host(params, torch), wp, "sgd " + tag)
        if P and case % 3 == 0:
            tdt = torch.float32 if in_dt == "f32" else torch.bfloat16
            grads_h = [random_inputs(rng, 1, n, in_dt)[0] for n in numel]
            grads = [to_dev(g, torch) if g.size else torch.empty(0, dtype=tdt, device="cuda:0")
                     for g in grads_h]
            bd = ddp.bind_params(lp, grads)
            flat = torch.empty(P, dtype=tdt, device="cuda:0")
            ddp.flatten(lp, bd, flat)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(flat, torch), oracle.flatten(op, grads_h), "flatten " + tag)


def test_two_plans_on_two_streams(env):
    torch, ddp = env
    rng = np.random.default_rng(77)
    cases = []
    for k in range(2):
        numel = [int(v) for v in rng.integers(1000, 200000, 40)]
        lp = ddp.plan_buckets(numel, 1 << 20)
        op = oracle.plan_cap(numel, 1 << 20, 4)
        xs = random_inputs(rng, 4 + 3 * k, op.total, "f32")
        ts = [to_dev(x, torch) for x in xs]
        out = torch.empty(op.total, dtype=torch.float32, device="cuda:0")
        cases.append((lp, op, xs, ts, out, torch.cuda.Stream()))
    torch.cuda.synchronize()
    for _ in range(3):
        for lp, op, xs, ts, out, s in cases:
            with torch.cuda.stream(s):
                ddp.sync_allreduce_avg(lp, ts, out, "ring")
    torch.cuda.synchronize()
    for lp, op, xs, ts, out, s in cases:
        assert_bits_equal(to_host(out, torch), oracle.sync_avg(op, xs, "ring"), "two streams")


@pytest.mark.parametrize("seed", range(4))
def test_random_plans_many_ranks(env, seed):
    """N = 9..64 (the looped kernel): tiny caps, so chunks are shorter than a
    tile and most tiles meet two or more ring segments."""
    torch, ddp = env
    rng = np.random.default_rng(9000 + seed)
    for case in range(4):
        n = int(rng.integers(1, 60))
        numel = [int(v) for v in rng.integers(0, 4000, n)]
        N = int(rng.choice([9, 11, 12, 16, 23, 33, 64]))
        in_dt, out_dt = PAIRS[int(rng.integers(0, 3))]
        eb = 4 if in_dt == "f32" else 2
        cap = int(rng.choice([64, 1000, 4096, 20000]))
        lp = ddp.plan_buckets(numel, cap, in_dt)
        op = oracle.plan_cap(numel, cap, eb)
        P = op.total
        tag = f"seed={seed} case={case} N={N} {in_dt}->{out_dt} cap={cap} P={P} B={op.n_buckets}"
        print(tag, flush=True)
        xs = random_inputs(rng, N, P, in_dt)
        ts = [to_dev(x, torch) for x in xs]
        odt = torch.float32 if out_dt == "f32" else torch.bfloat16
        out = torch.empty(P, dtype=odt, device="cuda:0")
        for order in ("seq", "ring"):
            ddp.sync_allreduce_avg(lp, ts, out, order)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(out, torch), oracle.sync_avg(op, xs, order, in_dt, out_dt),
                              "sync " + tag)
