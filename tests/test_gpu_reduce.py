"""GPU parity of ddp_bucket_allreduce_avg against the CPU oracle, bit for bit.

Covers every rank count with an unrolled kernel (2..8), the looped kernel
(9, 16, 64), N = 1, lengths that are empty, shorter than one vector, one tile
and a ragged tail, several tiles and a ragged tail; all three dtype pairs;
both summation orders; IEEE special values; misaligned buffers (per-element
kernel); in-place output; guard bands around the output.
"""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import assert_bits_equal, random_inputs, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")]
ORDERS = ["seq", "ring"]
# lengths: empty, shorter than one 16-byte vector, ragged tails, one and many
# tiles (a tile is 256 f32 or 512 bf16 elements)
LENGTHS = [0, 1, 3, 5, 63, 2048, 2049, 4103, 3 * 4096 + 5, 100_003]
RANKS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 64]


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _run(env, xs, order, in_dt, out_dt, out=None, rank_tensors=None, length=None):
    torch, ddp = env
    ts = rank_tensors if rank_tensors is not None else [to_dev(x, torch) for x in xs]
    L = xs[0].size if length is None else length
    if out is None:
        out = torch.empty(L, dtype=torch.float32 if out_dt == "f32" else torch.bfloat16,
                          device="cuda:0")
    ddp.bucket_allreduce_avg(ts, out, order, length=L)
    torch.cuda.synchronize()
    return to_host(out, torch), out


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
@pytest.mark.parametrize("N", RANKS)
def test_bucket_parity(env, N, pair):
    in_dt, out_dt = pair
    torch, ddp = env
    rng = np.random.default_rng(1000 * N + len(in_dt) + 7 * len(out_dt))
    for L in LENGTHS:
        xs = random_inputs(rng, N, L, in_dt)
        for order in ORDERS:
            if N == 1 and in_dt != out_dt:
                with pytest.raises(ddp.DDPError) as ei:
                    _run(env, xs, order, in_dt, out_dt)
                assert ei.value.status == 2
                continue
            got, _ = _run(env, xs, order, in_dt, out_dt)
            want = oracle.bucket_avg(xs, order, in_dt, out_dt)
            assert_bits_equal(got, want, f"N={N} L={L} {order} {in_dt}->{out_dt}")


def _specials_f32(rng, N, L):
    xs = random_inputs(rng, N, L, "f32", 1.0)
    spec = np.array([0.0, -0.0, 1.4e-45, -1.4e-45, 1.1754942e-38, 5.9e-39, 3.4028235e38,
                     -3.4028235e38, np.inf, -np.inf, np.nan, 1e-30, 65504.0], dtype=np.float32)
    for r in range(N):
        idx = rng.integers(0, L, L // 3)
        xs[r][idx] = spec[rng.integers(0, spec.size, idx.size)]
    # a block of elements that are -0 on every rank
    for r in range(N):
        xs[r][100:140] = -0.0
        xs[r][200:240] = 1.4e-45          # smallest subnormal everywhere
    return xs


@pytest.mark.parametrize("N", [2, 3, 4, 8, 11])
@pytest.mark.parametrize("order", ORDERS)
def test_special_values(env, N, order):
    rng = np.random.default_rng(N)
    L = 4096 * 2 + 13
    xs = _specials_f32(rng, N, L)
    for out_dt in ("f32", "bf16"):
        got, _ = _run(env, xs, order, "f32", out_dt)
        want = oracle.bucket_avg(xs, order, "f32", out_dt)
        assert_bits_equal(got, want, f"specials N={N} {order} ->{out_dt}")
    got, _ = _run(env, xs, order, "f32", "f32")
    zero_bits = got[100:140].view(np.uint32)
    assert (zero_bits == (0x80000000 if order == "ring" else 0)).all()
    # subnormals are kept, not flushed: N * 2^-149 / N rounds back to 2^-149
    assert (got[200:240].view(np.uint32) == 1).all()


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
@pytest.mark.parametrize("order", ORDERS)
def test_ranks_at_different_offsets(env, pair, order):
    torch, ddp = env
    in_dt, out_dt = pair
    rng = np.random.default_rng(5)
    N, L = 5, 9001
    xs = random_inputs(rng, N, L, in_dt)
    tdt = torch.float32 if in_dt == "f32" else torch.bfloat16
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    ts = []
    for r, x in enumerate(xs):
        big = torch.empty(L + 8, dtype=tdt, device="cuda:0")
        off = 1 + (r % 3)                              # never 16-byte aligned
        big[off:off + L].copy_(to_dev(x, torch))
        ts.append(big[off:off + L])
    obig = torch.empty(L + 8, dtype=odt, device="cuda:0")
    out = obig[3:3 + L]
    got, _ = _run(env, xs, order, in_dt, out_dt, out=out, rank_tensors=ts)
    assert_bits_equal(got, oracle.bucket_avg(xs, order, in_dt, out_dt), "misaligned")


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
@pytest.mark.parametrize("order", ORDERS)
def test_shared_misalignment_peels_the_head(env, pair, order):
    """Every rank buffer and the output start the same number of elements past
    a 16-byte boundary (a bucket at an unpadded offset of equally aligned
    flat buffers): the head goes element-wise, the rest to the vector
    kernel, and ring chunks stay those of the whole bucket."""
    torch, ddp = env
    in_dt, out_dt = pair
    rng = np.random.default_rng(6)
    vec = 4 if in_dt == "f32" else 8
    tdt = torch.float32 if in_dt == "f32" else torch.bfloat16
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    for N in (2, 3, 8, 12):
        for off in range(1, vec):
            for L in (1, vec - off, vec, 257, 4099, 70001):
                xs = random_inputs(rng, N, L, in_dt)
                ts = []
                for x in xs:
                    big = torch.empty(L + 16, dtype=tdt, device="cuda:0")
                    big[off:off + L].copy_(to_dev(x, torch))
                    ts.append(big[off:off + L])
                obig = torch.empty(L + 16, dtype=odt, device="cuda:0")
                tag = f"N={N} off={off} L={L}"
                got, _ = _run(env, xs, order, in_dt, out_dt, out=obig[off:off + L], rank_tensors=ts)
                want = oracle.bucket_avg(xs, order, in_dt, out_dt)
                assert_bits_equal(got, want, tag)
                if in_dt == out_dt:   # in place into rank 0's buffer
                    ddp.bucket_allreduce_avg(ts, ts[0], order)
                    torch.cuda.synchronize()
                    assert_bits_equal(to_host(ts[0], torch), want, "in place " + tag)
            # the same offset from a 16-byte boundary, different ones from a 128-byte one
            L = 30011
            xs = random_inputs(rng, N, L, in_dt)
            ts = []
            for r, x in enumerate(xs):
                o = (r * vec) % 64 + 1
                big = torch.empty(L + 80, dtype=tdt, device="cuda:0")
                big[o:o + L].copy_(to_dev(x, torch))
                ts.append(big[o:o + L])
            obig = torch.empty(L + 16, dtype=odt, device="cuda:0")
            got, _ = _run(env, xs, order, in_dt, out_dt, out=obig[1:1 + L], rank_tensors=ts)
            assert_bits_equal(got, oracle.bucket_avg(xs, order, in_dt, out_dt), f"N={N} mixed")


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("k", [0, 3])
def test_in_place_output(env, order, k):
    torch, ddp = env
    rng = np.random.default_rng(11 + k)
    N, L = 4, 3 * 4096 + 17
    xs = random_inputs(rng, N, L, "f32")
    ts = [to_dev(x, torch) for x in xs]
    got, _ = _run(env, xs, order, "f32", "f32", out=ts[k], rank_tensors=ts)
    assert_bits_equal(got, oracle.bucket_avg(xs, order), "in place")


@pytest.mark.parametrize("pad", [0, 1, 4])
def test_guard_bands_around_output_untouched(env, pad):
    torch, ddp = env
    rng = np.random.default_rng(pad)
    N, L = 8, 4096 * 3 + 3
    xs = random_inputs(rng, N, L, "f32")
    big = torch.full((L + 64,), -7.25, dtype=torch.float32, device="cuda:0")
    out = big[pad:pad + L]
    for order in ORDERS:
        got, _ = _run(env, xs, order, "f32", "f32", out=out)
        assert_bits_equal(got, oracle.bucket_avg(xs, order), "guarded")
        h = to_host(big, torch)
        assert (h[:pad] == -7.25).all() and (h[pad + L:] == -7.25).all()


def test_partial_overlap_is_rejected_and_nothing_written(env):
    torch, ddp = env
    N, L = 2, 1024
    a = torch.zeros(2 * L, dtype=torch.float32, device="cuda:0")
    b = torch.ones(L, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ddp.DDPError) as ei:
        ddp.bucket_allreduce_avg([a[:L], b], a[4:4 + L], "seq")
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert float(a.abs().sum()) == 0.0


def test_same_result_on_repeat_and_on_a_side_stream(env):
    torch, ddp = env
    rng = np.random.default_rng(3)
    xs = random_inputs(rng, 8, 50_001, "f32")
    first, _ = _run(env, xs, "ring", "f32", "f32")
    s = torch.cuda.Stream()
    ts = [to_dev(x, torch) for x in xs]
    out = torch.empty(50_001, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ddp.bucket_allreduce_avg(ts, out, "ring")
    s.synchronize()
    assert_bits_equal(to_host(out, torch), first, "side stream")


def test_one_plan_ring_tables_per_rank_count(env):
    """The RING table of a plan is per rank count: one plan synchronised with
    N = 2, 3, 5, 8, 12, then 3 and 8 again, matches the oracle every time."""
    torch, ddp = env
    rng = np.random.default_rng(31)
    numel = [int(v) for v in rng.integers(1, 40000, 60)]
    for dt, eb in (("f32", 4), ("bf16", 2)):
        lp = ddp.plan_buckets(numel, 96 << 10, dt)
        op = oracle.plan_cap(numel, 96 << 10, eb)
        xs = random_inputs(rng, 12, op.total, dt)
        ts = [to_dev(x, torch) for x in xs]
        out = torch.empty(op.total, dtype=ts[0].dtype, device="cuda:0")
        for n in (2, 3, 5, 8, 12, 3, 8):
            print(f"{dt} N={n}", flush=True)
            lp.prepare(n)
            ddp.sync_allreduce_avg(lp, ts[:n], out, "ring")
            torch.cuda.synchronize()
            assert_bits_equal(to_host(out, torch), oracle.sync_avg(op, xs[:n], "ring", dt, dt),
                              f"{dt} N={n}")


def test_occupancy_policy_changes_no_bit(env):
    """Both occupancy policies give the same bits (reduce in both orders, the
    fused SGD step, flatten)."""
    torch, ddp = env
    rng = np.random.default_rng(5)
    numel = [int(v) for v in rng.integers(1, 50000, 80)]
    lp = ddp.plan_buckets(numel, 200 << 10)
    op = oracle.plan_cap(numel, 200 << 10, 4)
    xs = random_inputs(rng, 6, op.total, "f32")
    ts = [to_dev(x, torch) for x in xs]
    p0 = rng.standard_normal(op.total).astype(np.float32)
    grads = [to_dev(g, torch) for g in random_inputs(rng, 1, op.total, "f32")[0:1]]
    views = list(torch.split(grads[0], numel))
    got = {}
    try:
        for policy in ("shared", "tuned"):
            ddp.set_occupancy(policy)
            for order in ("seq", "ring"):
                out = torch.empty(op.total, dtype=torch.float32, device="cuda:0")
                ddp.sync_allreduce_avg(lp, ts, out, order)
                got[(policy, order)] = to_host(out, torch)
            params, mom = to_dev(p0, torch), torch.zeros(op.total, device="cuda:0")
            ddp.sync_sgd_update(lp, ts, params, 0.05, "ring", momentum_buf=mom, momentum=0.9)
            got[(policy, "sgd")] = to_host(params, torch)
            flat = torch.empty(op.total, dtype=torch.float32, device="cuda:0")
            ddp.flatten(lp, ddp.bind_params(lp, views), flat)
            got[(policy, "flatten")] = to_host(flat, torch)
    finally:
        ddp.set_occupancy("tuned")
    for what in ("seq", "ring", "sgd", "flatten"):
        assert_bits_equal(got[("shared", what)], got[("tuned", what)], what)
    assert_bits_equal(got[("tuned", "ring")], oracle.sync_avg(op, xs, "ring"), "ring vs oracle")


def test_prepared_sync_matches_direct_call(env):
    torch, ddp = env
    import workloads as W
    wl = W.workload("tiny")
    lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes)
    xs = [W.host_rank_flat(wl, r) for r in range(wl.n_ranks)]
    ts = [to_dev(x, torch) for x in xs]
    a = torch.empty(lp.total, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for order in ORDERS:
        call = ddp.make_sync(lp, ts, a, order)
        call()
        call()
        ddp.sync_allreduce_avg(lp, ts, b, order)
        torch.cuda.synchronize()
        assert_bits_equal(to_host(a, torch), to_host(b, torch), f"prepared {order}")


def test_concurrent_first_use_of_ring_tables(env):
    """Four host threads synchronise one fresh plan at the same time, each with
    its own rank count and stream, so the per-rank-count RING tables are built
    concurrently (under the plan's lock); every result matches the oracle."""
    import threading
    torch, ddp = env
    rng = np.random.default_rng(44)
    numel = [int(v) for v in rng.integers(1, 30000, 70)]
    lp = ddp.plan_buckets(numel, 120 << 10)
    op = oracle.plan_cap(numel, 120 << 10, 4)
    xs = random_inputs(rng, 8, op.total, "f32")
    ts = [to_dev(x, torch) for x in xs]
    counts = (3, 5, 7, 8)
    outs = {n: torch.empty(op.total, dtype=torch.float32, device="cuda:0") for n in counts}
    streams = {n: torch.cuda.Stream() for n in counts}
    torch.cuda.synchronize()
    start, errors = threading.Barrier(len(counts)), []

    def run(n):
        try:
            start.wait()
            for _ in range(3):
                ddp.sync_allreduce_avg(lp, ts[:n], outs[n], "ring", stream=streams[n])
            streams[n].synchronize()
        except Exception as e:   # reported below, in the main thread
            errors.append((n, e))

    threads = [threading.Thread(target=run, args=(n,)) for n in counts]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for n in counts:
        assert_bits_equal(to_host(outs[n], torch), oracle.sync_avg(op, xs[:n], "ring"), f"N={n}")


def test_object_policies_and_bucket_calls_change_no_bit(env):
    """A plan's own occupancy policy (shared, tuned, default) gives the bits of
    the oracle and leaves the process-wide policy alone; the plan's buckets
    averaged one call each (ddp_sync_allreduce_avg_bucket, last layers
    first) give the one-launch bits; a per-parameter sync with its own
    policy gives the same bits as with the default."""
    torch, ddp = env
    rng = np.random.default_rng(55)
    numel = [int(v) for v in rng.integers(1, 40000, 60)]
    lp = ddp.plan_buckets(numel, 150 << 10)
    op = oracle.plan_cap(numel, 150 << 10, 4)
    xs = random_inputs(rng, 5, op.total, "f32")
    ts = [to_dev(x, torch) for x in xs]
    want = {o: oracle.sync_avg(op, xs, o) for o in ("seq", "ring")}
    for policy in ("shared", "tuned", "default"):
        lp.set_occupancy(policy)
        for order in ("seq", "ring"):
            out = torch.full((op.total,), float("nan"), device="cuda:0")
            ddp.sync_allreduce_avg(lp, ts, out, order)
            per = torch.full((op.total,), float("nan"), device="cuda:0")
            for b in range(lp.n_buckets):
                ddp.sync_allreduce_avg_bucket(lp, b, ts, per, order)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(out, torch), want[order], f"{policy} {order}")
            assert_bits_equal(to_host(per, torch), want[order], f"{policy} {order} per bucket")
        assert ddp.get_occupancy() == "tuned"
    # per-parameter sync: its own policy against the default
    grads = [list(torch.split(t, numel)) for t in ts]
    binds = [ddp.bind_params(lp, g) for g in grads]
    outs = {}
    for policy in ("default", "shared"):
        res = [torch.empty(n, device="cuda:0") for n in numel]
        ps = ddp.param_sync(lp, binds, ddp.bind_params(lp, res), "ring")
        ps.set_occupancy(policy)
        assert ps.get_occupancy() == policy
        ps()
        torch.cuda.synchronize()
        outs[policy] = np.concatenate([to_host(r, torch) for r in res])
    assert_bits_equal(outs["shared"], outs["default"], "per-parameter sync policies")
    assert ddp.get_occupancy() == "tuned"


@pytest.mark.parametrize("N,pair", [pytest.param(N, pair, id=f"{N}-{pair[0]}-{pair[1]}")
                                    for N in (1, 2, 3, 8, 13, 24)
                                    for pair in (("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"))
                                    if N > 1 or pair[0] == pair[1]])   # one rank keeps its dtype
def test_bucket_calls_every_dtype_pair(env, pair, N):
    """ddp_sync_allreduce_avg_bucket over every bucket of random plans (empty
    parameters, buckets shorter than a tile, buckets at unaligned offsets),
    every dtype pair, N from 1 to 24, both orders: the oracle's bits, and an
    output outside the bucket left untouched."""
    torch, ddp = env
    in_dt, out_dt = pair
    rng = np.random.default_rng(600 + N)
    eb = 4 if in_dt == "f32" else 2
    sizes = [int(x) for x in rng.choice([0, 1, 3, 17, 255, 600, 5000, 40000], size=30)]
    sizes[0] = max(sizes[0], 1)
    cap = 8192
    lp = ddp.plan_buckets(sizes, cap, in_dt)
    op = oracle.plan_cap(sizes, cap, eb)
    xs = random_inputs(rng, N, op.total, in_dt)
    ts = [to_dev(x, torch) for x in xs]
    tout = torch.float32 if out_dt == "f32" else torch.bfloat16
    for order in ("seq", "ring"):
        want = oracle.sync_avg(op, xs, order, in_dt, out_dt)
        out = torch.full((op.total,), float("nan"), dtype=tout, device="cuda:0")
        for b in range(lp.n_buckets):
            ddp.sync_allreduce_avg_bucket(lp, b, ts, out, order)
        torch.cuda.synchronize()
        assert_bits_equal(to_host(out, torch), want, f"N={N} {pair} {order}")
        # one bucket alone writes only its own range
        b = lp.n_buckets // 2
        ln, base, _, _ = lp.bucket(b)
        one = torch.full((op.total,), float("nan"), dtype=tout, device="cuda:0")
        ddp.sync_allreduce_avg_bucket(lp, b, ts, one, order)
        torch.cuda.synchronize()
        got = to_host(one, torch)
        assert_bits_equal(got[base:base + ln], want[base:base + ln], f"bucket {b}")
        rest = np.concatenate([got[:base], got[base + ln:]])
        nan = ((rest & 0x7F80) == 0x7F80) & ((rest & 0x7F) != 0) if rest.dtype == np.uint16 \
            else np.isnan(rest)
        assert nan.all(), "a bucket call wrote outside its bucket"
