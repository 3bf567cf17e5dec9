"""The C ABI on the host (no GPU): the library loads and exports every
symbol ``include/ddp.h`` declares, its planner matches the oracle's plan on
every workload and on random fuzz, and invalid arguments come back as status
codes before any GPU work is queued."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ddp = pytest.importorskip("gradient_allreduce_averaging_amd")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "ddp.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddp_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 15
    raw = ctypes.CDLL(ddp.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_abi_version_and_status_strings():
    assert ddp.abi_version() == 1
    for code in range(8):
        assert ddp.status_string(code)


def _lib_plan_buckets(plan):
    return plan.buckets()


@pytest.mark.parametrize("name", W.WORKLOADS)
def test_planner_matches_oracle_on_workloads(name):
    wl = W.workload(name)
    if wl.two_bucket:
        lp = ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype)
        op = oracle.plan_two_bucket(wl.numel, wl.regions)
    else:
        lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
        op = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
    assert lp.n_buckets == op.n_buckets
    assert lp.total == op.total
    assert _lib_plan_buckets(lp) == op.buckets
    for b in range(op.n_buckets):
        ln, base, _, _ = lp.bucket(b)
        assert (ln, base) == (op.bucket_len[b], op.bucket_base[b])
    loc = op.param_location()
    for p in range(0, len(wl.numel), max(1, len(wl.numel) // 500)):
        assert lp.param(p) == loc[p]


def test_resnet50_bucket_lengths():
    # the 25 MiB plan of the standard ResNet-50 shapes, fixed by the readings
    wl = W.workload("resnet50")
    lp = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, "f32")
    assert [lp.bucket(b)[0] for b in range(lp.n_buckets)] == \
        [6_515_688, 4_462_592, 6_300_160, 6_112_256, 2_166_336]


def test_planner_fuzz_matches_oracle():
    rng = np.random.default_rng(42)
    for trial in range(400):
        n = int(rng.integers(1, 80))
        numel = [int(v) for v in rng.integers(0, 3000, n)]
        if trial % 7 == 0:
            numel[int(rng.integers(0, n))] = 0
        dt = "f32" if trial % 2 else "bf16"
        eb = 4 if dt == "f32" else 2
        cap = int(rng.choice([1, 2, 3, 4, 100, 1000, 4096, 10 ** 5, int(rng.integers(1, 20000))]))
        lp = ddp.plan_buckets(numel, cap, dt)
        op = oracle.plan_cap(numel, cap, eb)
        assert lp.buckets() == op.buckets, (numel, cap, dt)
        regions = [int(v) for v in rng.integers(0, 6, n)]
        lp2 = ddp.plan_two_bucket(numel, regions, dt)
        op2 = oracle.plan_two_bucket(numel, regions)
        assert lp2.buckets() == op2.buckets


def test_plan_errors():
    L = ddp.lib
    h = ctypes.c_void_p()
    one = (ctypes.c_int64 * 1)(5)
    neg = (ctypes.c_int64 * 2)(5, -1)
    assert L.ddp_plan_buckets(one, 0, 100, 0, ctypes.byref(h)) == 1
    assert L.ddp_plan_buckets(one, 1, 0, 0, ctypes.byref(h)) == 1
    assert L.ddp_plan_buckets(one, 1, 100, 7, ctypes.byref(h)) == 1
    assert L.ddp_plan_buckets(neg, 2, 100, 0, ctypes.byref(h)) == 1
    assert L.ddp_plan_buckets(None, 1, 100, 0, ctypes.byref(h)) == 1
    assert L.ddp_plan_buckets(one, 1, 100, 0, None) == 1
    huge = (ctypes.c_int64 * 2)(2 ** 62, 2 ** 62)
    assert L.ddp_plan_buckets(huge, 2, 100, 0, ctypes.byref(h)) == 3
    reg = (ctypes.c_uint8 * 1)(9)
    assert L.ddp_plan_two_bucket(one, reg, 1, 0, ctypes.byref(h)) == 1
    assert L.ddp_plan_num_buckets(None) == -1
    assert L.ddp_plan_total(None) == -1
    p = ddp.plan_buckets([3, 4], 1 << 20)
    ln = ctypes.c_int64()
    assert L.ddp_plan_bucket(p.handle, 1, ctypes.byref(ln), None, None, None) == 1
    assert L.ddp_plan_bucket(p.handle, -1, ctypes.byref(ln), None, None, None) == 1
    assert L.ddp_plan_param(p.handle, 2, None, None) == 1
    assert L.ddp_plan_slot_param(p.handle, 0, None) == 1
    # rank counts outside 1..64 and a null plan are rejected before any HIP call
    assert L.ddp_plan_prepare_ranks(None, 2) == 1
    assert L.ddp_plan_prepare_ranks(p.handle, 0) == 1
    assert L.ddp_plan_prepare_ranks(p.handle, 65) == 1
    assert L.ddp_plan_prepare(None) == 1
    with pytest.raises(ddp.DDPError):
        ddp.plan_buckets([1, 2], 0)


def test_reduce_argument_errors_are_host_side():
    # fake device addresses: every case below must be rejected before any
    # HIP call is made (this host has no GPU)
    L = ddp.lib
    P = lambda *a: (ctypes.c_void_p * len(a))(*[ctypes.c_void_p(x) for x in a])   # noqa: E731
    out = ctypes.c_void_p(0x100000)
    two = P(0x200000, 0x300000)
    assert L.ddp_bucket_allreduce_avg(two, 0, 16, 0, 0, 0, out, None) == 1      # N < 1
    assert L.ddp_bucket_allreduce_avg(two, 65, 16, 0, 0, 0, out, None) == 2     # N > max
    assert L.ddp_bucket_allreduce_avg(two, 2, -1, 0, 0, 0, out, None) == 1      # len < 0
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 5, 0, 0, out, None) == 1      # order
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 0, 1, 0, out, None) == 2      # bf16 -> f32
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 0, 3, 0, out, None) == 1      # bad dtype
    assert L.ddp_bucket_allreduce_avg(None, 2, 16, 0, 0, 0, out, None) == 1
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 0, 0, 0, None, None) == 1
    assert L.ddp_bucket_allreduce_avg(P(0x200000, 0), 2, 16, 0, 0, 0, out, None) == 1
    assert L.ddp_bucket_allreduce_avg(P(0x200002, 0x300000), 2, 16, 0, 0, 0, out, None) == 1
    # N == 1 with a dtype change has no bitwise identity to return
    assert L.ddp_bucket_allreduce_avg(P(0x200000), 1, 16, 0, 0, 1, out, None) == 2
    # partial overlap of out and an input; exact aliasing is allowed
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 0, 0, 0, ctypes.c_void_p(0x200010), None) == 4
    assert L.ddp_bucket_allreduce_avg(two, 2, 16, 0, 0, 1, ctypes.c_void_p(0x200000), None) == 4
    # empty bucket: nothing to do, no GPU touched
    assert L.ddp_bucket_allreduce_avg(two, 2, 0, 1, 0, 0, out, None) == 0
    assert L.ddp_bucket_allreduce_avg(None, 2, 0, 1, 0, 0, None, None) == 0   # torch's empty tensors
    assert L.ddp_bucket_allreduce_avg(None, 0, 0, 1, 0, 0, None, None) == 1
    assert L.ddp_sync_allreduce_avg(None, two, 2, 0, 0, out, None) == 1
    p = ddp.plan_buckets([3, 4], 1 << 20)
    assert L.ddp_sync_allreduce_avg(p.handle, P(0x200000), 1, 0, 1, out, None) == 2
    assert L.ddp_sync_allreduce_avg(p.handle, two, 2, 0, 0, ctypes.c_void_p(0x200004), None) == 4
    pb = ddp.plan_buckets([3, 4], 1 << 20, "bf16")
    assert L.ddp_sync_allreduce_avg(pb.handle, two, 2, 0, 0, out, None) == 2   # bf16 -> f32


def test_noalloc_sync_argument_errors_are_host_side():
    """The no-allocation sync validates like ddp_sync_allreduce_avg, and a
    plan whose RING tables exceed its static buffer (DDP_NOALLOC_SCRATCH_BYTES
    = 64 MiB: about 16 M tiles) is refused before any GPU call."""
    L = ddp.lib
    P = lambda *a: (ctypes.c_void_p * len(a))(*[ctypes.c_void_p(x) for x in a])   # noqa: E731
    f = L.ddp_sync_allreduce_avg_noalloc
    two = P(0x200000, 0x300000)
    out = ctypes.c_void_p(0x400000)
    assert f(None, two, 2, 1, 0, out, None) == 1
    p = ddp.plan_buckets([3, 4], 1 << 20)
    assert f(p.handle, two, 0, 1, 0, out, None) == 1
    assert f(p.handle, two, 2, 2, 0, out, None) == 1                           # bad order
    assert f(p.handle, P(0x200000), 1, 1, 1, out, None) == 2
    assert f(p.handle, two, 2, 1, 0, ctypes.c_void_p(0x200004), None) == 4
    pb = ddp.plan_buckets([3, 4], 1 << 20, "bf16")
    assert f(pb.handle, two, 2, 1, 0, out, None) == 2                          # bf16 -> f32
    # 2^32 + 1 f32 elements: 16 M + 1 tiles of 256, more words than the buffer holds
    big = ddp.plan_buckets([1 << 31, (1 << 31) + 1], 1 << 40)
    far = P(0x100000000000, 0x200000000000)
    assert f(big.handle, far, 2, 1, 0, ctypes.c_void_p(0x300000000000), None) == 7
    assert ddp.status_string(7) != ddp.status_string(6)


def test_flatten_argument_errors():
    L = ddp.lib
    p = ddp.plan_buckets([3, 4], 1 << 20)
    assert L.ddp_flatten(None, None, -1, ctypes.c_void_p(0x1000), 0, None) == 1
    assert L.ddp_flatten(p.handle, None, -1, ctypes.c_void_p(0x1000), 0, None) == 1
    assert L.ddp_bind_params(p.handle, None, None, None) == 1


def test_fused_sgd_argument_errors_are_host_side():
    L = ddp.lib
    P = lambda *a: (ctypes.c_void_p * len(a))(*[ctypes.c_void_p(x) for x in a])   # noqa: E731
    p = ddp.plan_buckets([100, 28], 1 << 20)            # 128 f32 elements = 512 B
    two = P(0x200000, 0x300000)
    ok_param = ctypes.c_void_p(0x400000)
    f = L.ddp_sync_sgd_update
    assert f(None, two, 2, 0, 0, None, ok_param, None, 0.1, 0.0, None) == 1
    assert f(p.handle, two, 2, 0, 0, None, None, None, 0.1, 0.0, None) == 1          # no params
    assert f(p.handle, two, 2, 0, 0, None, ctypes.c_void_p(0x400002), None, 0.1, 0.0, None) == 1
    assert f(p.handle, two, 2, 0, 0, None, ctypes.c_void_p(0x200100), None, 0.1, 0.0, None) == 4
    assert f(p.handle, two, 2, 0, 0, None, ok_param, ctypes.c_void_p(0x400100), 0.1, 0.0, None) == 4
    assert f(p.handle, two, 2, 0, 0, ctypes.c_void_p(0x400080), ok_param, None, 0.1, 0.0, None) == 4
    assert f(p.handle, two, 2, 0, 0, None, ok_param, ctypes.c_void_p(0x300000), 0.1, 0.0, None) == 4
    assert f(p.handle, P(0x200000), 1, 0, 1, None, ok_param, None, 0.1, 0.0, None) == 2   # N=1 f32->bf16
    assert f(p.handle, two, 65, 0, 0, None, ok_param, None, 0.1, 0.0, None) == 2


def test_accumulate_argument_errors_are_host_side():
    L = ddp.lib
    P = lambda *a: (ctypes.c_void_p * len(a))(*[ctypes.c_void_p(x) for x in a])   # noqa: E731
    f = L.ddp_accumulate
    assert f(P(0x1000), P(0x2000), 0, 16, 0, None) == 1
    assert f(P(0x1000), P(0x2000), 1, -1, 0, None) == 1
    assert f(P(0x1000), P(0x2000), 1, 16, 7, None) == 1
    assert f(P(0x1000), P(0x2000), 65, 16, 0, None) == 2
    assert f(None, None, 1, 0, 0, None) == 0                       # empty: nothing to do
    assert f(P(0x1000), P(0x1010), 1, 16, 0, None) == 4           # partial overlap
    assert f(P(0x1000, 0x1020), P(0x8000, 0x9000), 2, 16, 0, None) == 4   # dst overlap
    assert f(P(0x1000, 0x2000), P(0x2000, 0x9000), 2, 16, 0, None) == 4   # dst[0] is src[1]
    assert f(P(0x1002), P(0x2000), 1, 16, 0, None) == 1           # f32 misaligned to 2 B


def test_param_sync_argument_errors_are_host_side():
    L = ddp.lib
    p = ddp.plan_buckets([100, 28], 1 << 20)
    pb = ddp.plan_buckets([100, 28], 1 << 20, "bf16")
    ranks = (ctypes.c_void_p * 2)(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000))
    outb = ctypes.c_void_p(0x3000)
    res = ctypes.c_void_p()
    f = L.ddp_param_sync_create
    assert f(None, ranks, 2, outb, 1, 0, ctypes.byref(res)) == 1
    assert f(p.handle, None, 2, outb, 1, 0, ctypes.byref(res)) == 1
    assert f(p.handle, ranks, 2, None, 1, 0, ctypes.byref(res)) == 1
    assert f(p.handle, ranks, 2, outb, 1, 0, None) == 1
    assert f(p.handle, ranks, 0, outb, 1, 0, ctypes.byref(res)) == 1
    assert f(p.handle, ranks, 2, outb, 7, 0, ctypes.byref(res)) == 1      # order
    assert f(p.handle, ranks, 2, outb, 1, 9, ctypes.byref(res)) == 1      # dtype
    assert f(p.handle, ranks, 65, outb, 1, 0, ctypes.byref(res)) == 2
    assert f(pb.handle, ranks, 2, outb, 1, 0, ctypes.byref(res)) == 2     # bf16 -> f32
    assert f(p.handle, ranks, 1, outb, 1, 1, ctypes.byref(res)) == 2      # one rank, f32 -> bf16
    assert not res.value
    assert L.ddp_param_sync_run(None, None) == 1
    assert L.ddp_param_sync_run_buckets(None, 0, 1, None) == 1
    assert L.ddp_param_sgd_run(None, 0.1, 0.0, None) == 1
    assert L.ddp_param_sgd_run_buckets(None, 0, 1, 0.1, 0.0, None) == 1
    assert L.ddp_param_sgd_create(p.handle, ranks, 2, None, None, None, 1, 0, ctypes.byref(res)) == 1
    L.ddp_param_sync_free(None)


def test_occupancy_policy_round_trip():
    L = ddp.lib
    assert ddp.get_occupancy() == "tuned"
    assert L.ddp_set_occupancy(2) == 1
    assert L.ddp_set_occupancy(-1) == 1
    ddp.set_occupancy("shared")
    assert ddp.get_occupancy() == "shared"
    ddp.set_occupancy("tuned")
    assert ddp.get_occupancy() == "tuned"
    with pytest.raises(ValueError):
        ddp.set_occupancy("fast")


def test_object_occupancy_policies_round_trip():
    """A plan carries its own policy; setting it leaves the process-wide one
    alone.  DEFAULT (2) is valid for objects, not process-wide."""
    L = ddp.lib
    p = ddp.plan_buckets([3, 4], 1 << 20)
    assert p.get_occupancy() == "default"
    for pol in ("shared", "tuned", "default"):
        p.set_occupancy(pol)
        assert p.get_occupancy() == pol
        assert ddp.get_occupancy() == "tuned"
    assert L.ddp_plan_set_occupancy(p.handle, 3) == 1
    assert L.ddp_plan_set_occupancy(None, 0) == 1
    assert L.ddp_plan_get_occupancy(None) == 2
    assert L.ddp_param_sync_set_occupancy(None, 0) == 1
    assert L.ddp_param_sync_get_occupancy(None) == 2
    with pytest.raises(KeyError):
        p.set_occupancy("fast")


def test_bucket_sync_argument_errors_are_host_side():
    L = ddp.lib
    P = lambda *a: (ctypes.c_void_p * len(a))(*[ctypes.c_void_p(x) for x in a])   # noqa: E731
    f = L.ddp_sync_allreduce_avg_bucket
    p = ddp.plan_buckets([3, 4, 5], 16)          # three buckets of one parameter each
    two = P(0x200000, 0x300000)
    out = ctypes.c_void_p(0x400000)
    assert p.n_buckets == 3
    assert f(None, 0, two, 2, 1, 0, out, None) == 1
    assert f(p.handle, -1, two, 2, 1, 0, out, None) == 1
    assert f(p.handle, 3, two, 2, 1, 0, out, None) == 1
    assert f(p.handle, 0, two, 2, 2, 0, out, None) == 1                  # bad order
    assert f(p.handle, 0, P(0x200000), 1, 1, 1, out, None) == 2          # N = 1, f32 -> bf16
    assert f(p.handle, 0, two, 2, 1, 0, ctypes.c_void_p(0x200004), None) == 4
