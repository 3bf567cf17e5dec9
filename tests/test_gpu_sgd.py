"""GPU parity of ddp_sync_sgd_update (average folded into one SGD step)
against the oracle's synchronisation followed by its SGD step, bit for bit:
parameters, momentum buffer and the stored average, for every rank count
1..9, 13, 16, 40 and 64 (N > 8: the looped kernel), all dtype pairs, both orders, with and without
momentum and average output, buffers off 16-byte boundaries (all at one offset,
or each at its own), in-place average output,
the ResNet-50 and many-small workloads at full size, and Llama-7B (bf16
gradients, 27 GB of f32 parameters) on sampled positions."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, random_inputs, sample_positions, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _case(env, sizes, N, in_dt, out_dt, order, mom, write_avg, seed, misalign=False,
          in_place=False, xs=None, cap=1 << 16):
    torch, ddp = env
    rng = np.random.default_rng(seed)
    eb = 4 if in_dt == "f32" else 2
    lp = ddp.plan_buckets(sizes, cap, in_dt)
    op = oracle.plan_cap(sizes, cap, eb)
    P = op.total
    xs = xs if xs is not None else random_inputs(rng, N, P, in_dt)
    p0 = rng.standard_normal(P).astype(np.float32)
    m0 = (rng.standard_normal(P) * 1e-3).astype(np.float32)
    lr, mu = 0.05, 0.9
    tdt = torch.float32 if in_dt == "f32" else torch.bfloat16
    odt = torch.float32 if out_dt == "f32" else torch.bfloat16
    # element offsets of (rank r's buffer - r % 3, params, momentum, average)
    offs = misalign if isinstance(misalign, tuple) else (1, 1, 1, 1) if misalign else (0, 0, 0, 0)
    ranks = []
    for r, x in enumerate(xs):
        off = offs[0] + (r % 3 if isinstance(misalign, tuple) else 0)
        big = torch.empty(P + 8, dtype=tdt, device="cuda:0")
        big[off:off + P].copy_(to_dev(x, torch))
        ranks.append(big[off:off + P])
    pb = torch.empty(P + 8, dtype=torch.float32, device="cuda:0")
    params = pb[offs[1]:offs[1] + P]
    params.copy_(to_dev(p0, torch))
    mb = torch.empty(P + 8, dtype=torch.float32, device="cuda:0")
    mbuf = mb[offs[2]:offs[2] + P] if mom else None
    if mom:
        mbuf.copy_(to_dev(m0, torch))
    gout = None
    if in_place:
        gout = ranks[N - 1]
    elif write_avg:
        gb = torch.empty(P + 8, dtype=odt, device="cuda:0")
        gout = gb[offs[3]:offs[3] + P]
    ddp.sync_sgd_update(lp, ranks, params, lr, order, grad_out=gout, momentum_buf=mbuf,
                        momentum=mu, out_dtype=out_dt)
    torch.cuda.synchronize()
    wp = p0.copy()
    wm = m0.copy() if mom else None
    wavg = oracle.sync_sgd(op, xs, order, wp, lr, in_dt, out_dt, wm, mu)
    tag = f"N={N} {in_dt}->{out_dt} {order} mom={mom} avg={write_avg} mis={misalign} inpl={in_place}"
    assert_bits_equal(to_host(params, torch), wp, "params " + tag)
    if mom:
        assert_bits_equal(to_host(mbuf, torch), wm, "momentum " + tag)
    if gout is not None:
        assert_bits_equal(to_host(gout, torch), wavg, "average " + tag)


SIZES = [1000, 3, 77, 5000, 1, 2049, 300, 12345]


# N = 1 has no dtype change (DDP_ERR_UNSUPPORTED), so f32->bf16 starts at N = 2
CASES = [(N, pair) for N in list(range(1, 10)) + [13, 16, 40, 64]
         for pair in (("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"))
         if not (N == 1 and pair[0] != pair[1])]


@pytest.mark.parametrize("N,pair", CASES, ids=lambda c: str(c))
def test_fused_sgd_parity(env, N, pair):
    in_dt, out_dt = pair
    for order in ("seq", "ring"):
        for mom in (False, True):
            for write_avg in (False, True):
                _case(env, SIZES, N, in_dt, out_dt, order, mom, write_avg, seed=N * 10 + mom)


@pytest.mark.parametrize("order", ["seq", "ring"])
def test_fused_sgd_misaligned_and_in_place(env, order):
    _case(env, SIZES, 4, "f32", "f32", order, True, True, seed=1, misalign=True)
    _case(env, SIZES, 8, "bf16", "bf16", order, True, True, seed=2, misalign=True)
    _case(env, SIZES, 4, "f32", "f32", order, True, False, seed=3, in_place=True)


@pytest.mark.parametrize("total", [1, 3, 7, 8, 9, 255, 257, 511, 512, 513, 777])
def test_fused_sgd_short_totals(env, total):
    """Totals shorter than a vector, a tile (256 f32 / 512 bf16 elements) and
    a little past one: the lanes past the end, the split bf16 layout's second
    group and the per-element paths, in both orders, N = 3, 8 and 12."""
    sizes = [total] if total < 9 else [total // 3, total - total // 3]
    for k, (N, in_dt, out_dt) in enumerate([(3, "bf16", "bf16"), (8, "bf16", "bf16"),
                                            (12, "bf16", "bf16"), (8, "f32", "f32"),
                                            (8, "f32", "bf16")]):
        for order in ("seq", "ring"):
            _case(env, sizes, N, in_dt, out_dt, order, True, True, seed=total * 7 + k, cap=64)


MIXED = [(0, 1, 2, 3), (1, 3, 0, 1), (2, 0, 3, 0), (3, 2, 1, 2)]


@pytest.mark.parametrize("order", ["seq", "ring"])
@pytest.mark.parametrize("offs", MIXED, ids=lambda o: "off" + "".join(map(str, o)))
def test_fused_sgd_mixed_alignment(env, order, offs):
    """Every buffer at its own element offset from a 16-byte boundary (rank
    buffers among themselves too): the vector kernels read and write at
    element alignment, through the unrolled (N <= 8) and looped kernels."""
    for k, (N, in_dt, out_dt) in enumerate([(4, "f32", "f32"), (8, "bf16", "bf16"),
                                            (5, "f32", "bf16"), (12, "f32", "f32"),
                                            (12, "bf16", "bf16")]):
        for mom in (False, True):
            _case(env, SIZES, N, in_dt, out_dt, order, mom, True, seed=40 + k, misalign=offs)


@pytest.mark.parametrize("name", ["resnet50", "many_small"])
def test_fused_sgd_workload_full(env, name):
    torch, ddp = env
    wl = W.workload(name)
    lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
    op = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
    P = op.total
    flats = []
    for r in range(wl.n_ranks):
        t = torch.empty(P, dtype=torch.float32, device="cuda:0")
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    host = [to_host(t, torch) for t in flats]
    params = torch.empty(P, dtype=torch.float32, device="cuda:0")
    W.device_normal_(params, 99, 7, 1.0)
    mbuf = torch.zeros(P, dtype=torch.float32, device="cuda:0")
    p0 = to_host(params, torch)
    for order in wl.orders:
        wp, wm = p0.copy(), np.zeros(P, np.float32)
        params.copy_(to_dev(p0, torch))
        mbuf.zero_()
        for step in range(2):
            ddp.sync_sgd_update(lp, flats, params, 0.1, order, momentum_buf=mbuf, momentum=0.9)
            oracle.sync_sgd(op, host, order, wp, 0.1, momentum_buf=wm, momentum=0.9)
        torch.cuda.synchronize()
        assert_bits_equal(to_host(params, torch), wp, f"{name} {order} params")
        assert_bits_equal(to_host(mbuf, torch), wm, f"{name} {order} momentum")
    del flats, params, mbuf
    torch.cuda.empty_cache()


def test_fused_sgd_rejects_overlaps(env):
    torch, ddp = env
    lp = ddp.plan_buckets([100, 28], 1 << 20)
    a = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    b = torch.zeros(128, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ddp.DDPError) as ei:
        ddp.sync_sgd_update(lp, [a[:128], b], a[64:192], 0.1)
    assert ei.value.status == 4
    m = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ddp.DDPError) as ei:
        ddp.sync_sgd_update(lp, [a[:128], b], m[:128], 0.1, momentum_buf=m[64:192])
    assert ei.value.status == 4


def test_fused_sgd_llama_sampled(env):
    """The fused step at the Llama-7B size: bf16 gradients of 8 ranks, f32
    parameters and momentum (27 GB each), two momentum steps in both orders,
    checked on positions covering every bucket and ring-chunk edge plus
    random ones."""
    torch, ddp = env
    wl = W.workload("llama7b")
    lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, "bf16")
    op = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, 2)
    P = op.total
    flats = []
    for r in range(wl.n_ranks):
        t = torch.empty(P, dtype=torch.bfloat16, device="cuda:0")
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    params = torch.empty(P, dtype=torch.float32, device="cuda:0")
    mbuf = torch.empty(P, dtype=torch.float32, device="cuda:0")
    rng = np.random.default_rng(71)
    pos = sample_positions(op.bucket_base, op.bucket_len, wl.n_ranks, P, rng)
    idx = torch.from_numpy(pos).to("cuda:0")
    vals = np.stack([to_host(f.index_select(0, idx), torch) for f in flats], axis=1)
    base = np.array(op.bucket_base, dtype=np.int64)
    lens = np.array(op.bucket_len, dtype=np.int64)
    b_of = np.searchsorted(base, pos, side="right") - 1
    for order in ("seq", "ring"):
        print(f"llama7b fused SGD {order}", flush=True)
        W.device_normal_(params, 99, 7, 1.0)
        mbuf.zero_()
        wp = to_host(params.index_select(0, idx), torch).copy()
        wm = np.zeros(pos.size, np.float32)
        avg = oracle.sampled_avg(vals, pos - base[b_of], lens[b_of], order, "bf16", "bf16")
        for _ in range(2):
            ddp.sync_sgd_update(lp, flats, params, 0.1, order, momentum_buf=mbuf, momentum=0.9)
            oracle.sgd_step(wp, avg, 0.1, "bf16", wm, 0.9)
        torch.cuda.synchronize()
        assert_bits_equal(to_host(params.index_select(0, idx), torch), wp, f"llama7b {order} params")
        assert_bits_equal(to_host(mbuf.index_select(0, idx), torch), wm, f"llama7b {order} momentum")
    del flats, params, mbuf, idx
    torch.cuda.empty_cache()
