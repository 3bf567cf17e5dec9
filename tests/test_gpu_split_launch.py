"""Grids too large for one dispatch.

A dispatch counts its grid in 32-bit work-items, so the library gives one
launch at most 2^30 work-items and runs a larger grid as consecutive
launches on the same stream, each told the grid-wide index of its first
block (the environment variable DDP_MAX_LAUNCH_ITEMS lowers the limit).
These tests check that the split changes no bit:

* the launch count: kernel nodes of captured graphs, for the one-launch
  synchronisation, an unaligned single bucket (head block in the last
  launch), ranks at mixed offsets, the fused SGD step (buffers on and off
  16-byte boundaries), accumulate and flatten, each replay equal to the
  eager call;
* the parity suites (flat and per-parameter) once more in a child process whose limit is 4096
  work-items (64 reduce blocks, 8 copy units per launch), so that every
  small case spans many launches and is compared with the oracle there;
* at the real limit: N = 2 f32 ranks of 4.3 G elements (past element 2^32,
  where the one-launch sync, the head-peeled and mixed-offset buckets, the
  fused step with buffers on and off 16-byte boundaries and accumulate
  split), checked on sampled positions around every launch edge, bucket edge
  and ring-chunk edge against the oracle.
"""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, sample_positions, to_host, torch_cuda

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = "DDP_MAX_LAUNCH_ITEMS"
CHILD_LIMIT = 4096


def launch_items():
    """The library's launch limit for this process (same rule as the library:
    at most 2^30, at least 4096, a multiple of 4096)."""
    v = 1 << 30
    s = os.environ.get(ENV)
    if s:
        try:
            x = int(s)
        except ValueError:
            x = 0
        if 0 < x < v:
            v = max(x, 4096)
    return v // 4096 * 4096


def launches(blocks, threads):
    per = launch_items() // threads
    return -(-blocks // per)


def copy_units_per_launch(esize):
    """Copy units one flatten/unflatten launch takes (same rule as the
    library): the work-item limit's worth of 256-thread blocks, one per 8 KiB
    of a 4096-element unit, rounded down to whole rounds of 8 runs of up to
    64 consecutive units."""
    cap = launch_items() // (256 * (4096 * esize // 8192))
    run = min(64, cap // 8)
    return cap // (8 * run) * (8 * run)


@pytest.fixture(scope="module")
def env():
    torch = torch_cuda()
    import gradient_allreduce_averaging_amd as ddp
    return torch, ddp


def _kernel_nodes(torch, fn):
    """Captures fn() into a graph; returns (kernel node count, graph)."""
    hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has already loaded
    fn()                                    # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    raw = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(raw, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(raw, nodes, ctypes.byref(n)) == 0
    kernels = 0
    for k in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[k]), ctypes.byref(t)) == 0
        kernels += t.value == 0          # hipGraphNodeTypeKernel
    g.instantiate()
    return kernels, g


def _replay_equals_eager(torch, g, fn, outs, what, reset=None):
    """Replays g and runs fn() eagerly from the same state; the outputs agree."""
    def start():
        if reset:
            reset()
        else:
            for o in outs:
                o.fill_(float("nan"))
    start()
    g.replay()
    torch.cuda.synchronize()
    got = [to_host(o, torch).copy() for o in outs]
    start()
    fn()
    torch.cuda.synchronize()
    for a, o in zip(got, outs):
        assert_bits_equal(a, to_host(o, torch), what)


def test_launch_count_follows_the_item_limit(env):
    torch, ddp = env
    dev = "cuda:0"
    sizes = [p.numel for p in W.many_small(n=400)]
    N = 4
    lp = ddp.plan_buckets(sizes, 1 << 20, "f32")
    lp.prepare(N)
    P = lp.total
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    flats = [torch.empty(P + 64, device=dev).normal_(0, 1e-3, generator=gen) for _ in range(N)]
    out = torch.empty(P + 64, device=dev)
    print(f"launch limit {launch_items()} work-items, P={P}", flush=True)

    def sync():
        ddp.sync_allreduce_avg(lp, [f[:P] for f in flats], out[:P], "ring")
    k, g = _kernel_nodes(torch, sync)
    assert k == launches(-(-P // 256), 64), ("sync", k)
    _replay_equals_eager(torch, g, sync, [out], "sync replay")

    # a bucket 12 bytes past a 128-byte boundary: 29 head elements, head block last
    L = P - 3

    def head():
        ddp.bucket_allreduce_avg([f[3:] for f in flats], out[3:], "ring", length=L)
    k, g = _kernel_nodes(torch, head)
    assert k == launches(-(-(L - 29) // 256) + 1, 64), ("head", k)
    _replay_equals_eager(torch, g, head, [out], "head replay")

    # ranks at different offsets from a 16-byte boundary: the vector kernel on
    # the output's alignment (here 0 head elements), loads at element alignment
    def mixed():
        ddp.bucket_allreduce_avg([f[r:] for r, f in enumerate(flats)], out, "ring", length=L)
    k, g = _kernel_nodes(torch, mixed)
    assert k == launches(-(-L // 256), 64), ("mixed offsets", k)
    _replay_equals_eager(torch, g, mixed, [out], "mixed-offset replay")

    params = torch.empty(P, device=dev).normal_(0, 1, generator=gen)
    mom = torch.zeros(P, device=dev)
    p0 = params.clone()

    def sgd_reset():
        params.copy_(p0)
        mom.zero_()
        torch.cuda.synchronize()

    def sgd():
        ddp.sync_sgd_update(lp, [f[:P] for f in flats], params, 0.1, "ring", momentum_buf=mom,
                            momentum=0.9)
    k, g = _kernel_nodes(torch, sgd)
    assert k == launches(-(-P // 256), 64), ("sgd", k)
    _replay_equals_eager(torch, g, sgd, [params, mom], "fused SGD replay", sgd_reset)

    # rank buffers off a 16-byte boundary: still the vector kernel
    def sgd_mixed():
        ddp.sync_sgd_update(lp, [f[1:P + 1] for f in flats], params, 0.1, "ring",
                            momentum_buf=mom, momentum=0.9)
    k, g = _kernel_nodes(torch, sgd_mixed)
    assert k == launches(-(-P // 256), 64), ("sgd, ranks off 16 B", k)
    _replay_equals_eager(torch, g, sgd_mixed, [params, mom], "SGD replay, ranks off 16 B", sgd_reset)

    # parameters and momentum off a 16-byte boundary (1 and 3 elements): the
    # same vector grid, stores at element alignment
    pbig = torch.empty(P + 4, device=dev)
    p_off = pbig[1:P + 1]
    mbig = torch.zeros(P + 4, device=dev)
    m_off = mbig[3:P + 3]

    def p_reset():
        p_off.copy_(p0)
        m_off.zero_()
        torch.cuda.synchronize()

    def sgd_off():
        ddp.sync_sgd_update(lp, [f[:P] for f in flats], p_off, 0.1, "ring", momentum_buf=m_off,
                            momentum=0.9)
    k, g = _kernel_nodes(torch, sgd_off)
    assert k == launches(-(-P // 256), 64), ("sgd, parameters off 16 B", k)
    _replay_equals_eager(torch, g, sgd_off, [p_off, m_off], "SGD replay, parameters off 16 B", p_reset)

    acc_dst = [torch.empty(P, device=dev) for _ in range(2)]

    def acc_reset():
        for d, f in zip(acc_dst, flats):
            d.copy_(f[:P])
        torch.cuda.synchronize()

    def acc():
        ddp.accumulate(acc_dst, [f[:P] for f in flats[2:]])
    k, g = _kernel_nodes(torch, acc)
    assert k == launches(-(-P // 256), 64), ("accumulate", k)
    _replay_equals_eager(torch, g, acc, acc_dst, "accumulate replay", acc_reset)

    grads = [torch.empty(n, device=dev).normal_(0, 1, generator=gen) for n in sizes]
    bind = ddp.bind_params(lp, grads)

    def flat():
        ddp.flatten(lp, bind, out[:P])
    k, g = _kernel_nodes(torch, flat)
    units = sum(-(-n // 4096) for n in sizes)
    # plus the edge pass when a parameter starts or the plan ends off a
    # 16-byte boundary of the flat buffer
    starts, pos = [], 0
    for n in reversed(sizes):      # the cap plan's flat order
        if n:
            starts.append(pos)
        pos += n
    base = out.data_ptr()
    edge = any((base + 4 * f) % 16 for f in starts + [pos])
    # the edge work rides as extra blocks at the end of the last copy launch
    # when they fit under the work-item limit, else it is a launch of its own
    per = copy_units_per_launch(4)
    run = min(64, launch_items() // 512 // 8)
    n_last = units - (-(-units // per) - 1) * per
    # whole rounds of 8 runs, then the rest shared out in 8 runs of ceil(rest / 8)
    whole, rest = divmod(n_last, 8 * run)
    bulk_last = (whole * run + -(-rest // 8)) * 8 * 2          # 2 blocks per f32 unit
    eblocks = -(-8 * (len(starts) + 1) // 256)
    alone = edge and (bulk_last + eblocks) * 256 > launch_items()
    assert k == -(-units // per) + alone, ("flatten", k, edge, alone)
    _replay_equals_eager(torch, g, flat, [out], "flatten replay")
    del flats, out, params, mom, acc_dst, grads
    torch.cuda.empty_cache()


@pytest.mark.skipif(os.environ.get(ENV) is not None, reason="already in the child process")
def test_parity_suites_with_split_launches(env):
    torch, _ = env
    torch.cuda.empty_cache()
    suites = ["tests/test_gpu_reduce.py", "tests/test_gpu_sgd.py", "tests/test_gpu_accumulate.py",
              "tests/test_gpu_flatten.py", "tests/test_gpu_fuzz.py",
              "tests/test_gpu_graph_overlap.py", "tests/test_gpu_param_sync.py",
              "tests/test_gpu_split_launch.py"]
    cmd = [sys.executable, "-u", "-m", "pytest", "-x", "-q", "-m", "gpu", "-p", "no:cacheprovider",
           "-k", "not llama and not real_limit and not gpt", *suites]
    child_env = dict(os.environ, **{ENV: str(CHILD_LIMIT)})
    print("child:", " ".join(cmd[3:]), f"with {ENV}={CHILD_LIMIT}", flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=child_env, capture_output=True, text=True, timeout=420)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-2000:]).strip()
    print(tail.splitlines()[-1] if tail else "", flush=True)
    assert r.returncode == 0, tail
    assert " passed" in r.stdout


def _sampled(torch, flats, pos):
    idx = torch.from_numpy(pos).to(flats[0].device)
    return np.stack([to_host(f.index_select(0, idx), torch) for f in flats], axis=1), idx


def _near(points, lo, hi, width=70):
    return {p + d for p in points for d in range(-width, width + 1) if lo <= p + d < hi}


def test_real_limit_past_element_2_32(env):
    torch, ddp = env
    dev = "cuda:0"
    numel = [2_150_000_003, 2_150_000_000]        # reversed: buckets of 2.15 G each
    N = 2
    lp = ddp.plan_buckets(numel, 25 << 20, "f32")
    op = oracle.plan_cap(numel, 25 << 20, 4)
    assert lp.buckets() == op.buckets
    P = op.total
    assert -(-P // 256) > (1 << 30) // 64, "the one-launch sync must need two launches"
    print(f"real limit: N={N} P={P}", flush=True)
    flats = []
    for r in range(N):
        t = torch.empty(P, dtype=torch.float32, device=dev)
        W.device_normal_(t, 40 + r, 9, 1e-3)
        flats.append(t)
    out = torch.empty(P, dtype=torch.float32, device=dev)
    base = np.array(op.bucket_base, dtype=np.int64)
    lens = np.array(op.bucket_len, dtype=np.int64)
    rng = np.random.default_rng(2 ** 32)
    pos = set(sample_positions(op.bucket_base, op.bucket_len, N, P, rng, n_random=8000).tolist())
    pos |= _near([1 << 32, P - 1], 0, P)          # the sync's launch edge (tile 2^24), the end
    pos = np.array(sorted(pos), dtype=np.int64)
    vals, idx = _sampled(torch, flats, pos)
    b_of = np.searchsorted(base, pos, side="right") - 1

    print("real limit: one-launch sync, ring f32 and seq f32->bf16", flush=True)
    ddp.sync_allreduce_avg(lp, flats, out, "ring")
    torch.cuda.synchronize()
    avg_ring = oracle.sampled_avg(vals, pos - base[b_of], lens[b_of], "ring")
    assert_bits_equal(to_host(out.index_select(0, idx), torch), avg_ring, "sync ring")
    out16 = torch.empty(P, dtype=torch.bfloat16, device=dev)
    ddp.sync_allreduce_avg(lp, flats, out16, "seq")
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out16.index_select(0, idx), torch),
                      oracle.sampled_avg(vals, pos - base[b_of], lens[b_of], "seq", "f32", "bf16"),
                      "sync seq bf16")
    del out16

    print("real limit: one bucket 12 bytes past a 128-byte boundary", flush=True)
    L = P - 3
    h = 29
    jpos = set(int(p) - 3 for p in pos if p >= 3)
    jpos |= _near([h + (1 << 32), 0, L - 1], 0, L)
    C = -(-L // N)
    jpos |= _near([C * k for k in range(N + 1)], 0, L)
    jpos = np.array(sorted(jpos), dtype=np.int64)
    jvals, jidx = _sampled(torch, flats, jpos + 3)
    out.fill_(float("nan"))
    ddp.bucket_allreduce_avg([f[3:] for f in flats], out[3:], "ring", length=L)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out.index_select(0, jidx), torch),
                      oracle.sampled_avg(jvals, jpos, np.full(jpos.size, L), "ring"),
                      "head-peeled bucket")
    del jidx

    print("real limit: ranks at different offsets from a 16-byte boundary", flush=True)
    L2 = P - 2
    spos = set(int(x) for x in rng.integers(0, L2, 4000))
    spos |= _near([1 << 32, 0, L2 - 1, L2 // 2], 0, L2)
    spos = np.array(sorted(spos), dtype=np.int64)
    sv = np.stack([to_host(flats[r].index_select(0, torch.from_numpy(spos + 1 + r).to(dev)), torch)
                   for r in range(N)], axis=1)
    ddp.bucket_allreduce_avg([flats[0][1:], flats[1][2:]], out, "ring", length=L2)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(out.index_select(0, torch.from_numpy(spos).to(dev)), torch),
                      oracle.sampled_avg(sv, spos, np.full(spos.size, L2), "ring"),
                      "mixed offsets")
    del out
    torch.cuda.empty_cache()

    print("real limit: fused SGD step, parameters and momentum off a 16-byte boundary", flush=True)
    p3big = torch.empty(P + 4, dtype=torch.float32, device=dev)
    p3 = p3big[1:P + 1]                           # 4 bytes past a 16-byte boundary
    W.device_normal_(p3, 78, 3, 1.0)
    m3big = torch.zeros(P + 4, dtype=torch.float32, device=dev)
    m3 = m3big[3:P + 3]                           # 12 bytes past one
    wp3 = to_host(p3.index_select(0, idx), torch).copy()
    wm3 = np.zeros(pos.size, np.float32)
    ddp.sync_sgd_update(lp, flats, p3, 0.1, "ring", momentum_buf=m3, momentum=0.9)
    oracle.sgd_step(wp3, avg_ring, 0.1, "f32", wm3, 0.9)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(p3.index_select(0, idx), torch), wp3, "offset SGD params")
    assert_bits_equal(to_host(m3.index_select(0, idx), torch), wm3, "offset SGD momentum")
    del p3, p3big, m3, m3big
    torch.cuda.empty_cache()

    print("real limit: fused SGD step with momentum", flush=True)
    params = torch.empty(P, dtype=torch.float32, device=dev)
    W.device_normal_(params, 77, 3, 1.0)
    mom = torch.zeros(P, dtype=torch.float32, device=dev)
    wp = to_host(params.index_select(0, idx), torch).copy()
    wm = np.zeros(pos.size, np.float32)
    for _ in range(2):
        ddp.sync_sgd_update(lp, flats, params, 0.1, "ring", momentum_buf=mom, momentum=0.9)
        oracle.sgd_step(wp, avg_ring, 0.1, "f32", wm, 0.9)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(params.index_select(0, idx), torch), wp, "fused SGD params")
    assert_bits_equal(to_host(mom.index_select(0, idx), torch), wm, "fused SGD momentum")
    del params, mom

    print("real limit: accumulate", flush=True)
    ddp.accumulate([flats[0]], [flats[1]])
    torch.cuda.synchronize()
    want = vals[:, 0].copy()
    oracle.accumulate(want, vals[:, 1].copy())
    assert_bits_equal(to_host(flats[0].index_select(0, idx), torch), want, "accumulate")
    del flats, idx
    torch.cuda.empty_cache()
