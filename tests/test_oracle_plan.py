"""P7: the oracle's bucket plans.

Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel) sections 3.2
and 4.2 (parameters reversed, packed into ~25 MB buckets, the last layer in
the first bucket, each bucket one contiguous flat tensor); [TR24] "(24)
NCCL通信与分布式数据并行" section 八 (two buckets: DEEP_COMM = the deep
convolution gradients, FIRST_COMM = BN, FC and first-conv gradients as one
contiguous region span).

Hand-worked cases pin the cap rule; invariants (partition, contiguity, cap
bound, greedy maximality, reverse order) are checked on every workload.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def test_hand_worked_cap_example():
    # numel [3, 5, 2, 7, 1], f32, cap 40 B = 10 elements.
    # reversed: p4(1) p3(7) p2(2) -> 10 elements, p1 would make 15 -> close;
    # then p1(5) p0(3).
    plan = oracle.plan_cap([3, 5, 2, 7, 1], 40, 4)
    assert plan.buckets == [[4, 3, 2], [1, 0]]
    assert plan.bucket_len == [10, 8]
    assert plan.bucket_base == [0, 10]
    assert plan.param_location() == [(1, 5), (1, 0), (0, 8), (0, 1), (0, 0)]


def test_hand_worked_oversize_parameter_gets_its_own_bucket():
    plan = oracle.plan_cap([100, 1, 1], 40, 4)
    assert plan.buckets == [[2, 1], [0]]
    plan = oracle.plan_cap([1, 100, 1], 40, 4)
    assert plan.buckets == [[2], [1], [0]]


def test_cap_counts_bytes_of_the_gradient_dtype():
    # a 20 B cap holds one 4-element f32 tensor (16 B) but two bf16 ones (16 B)
    assert oracle.plan_cap([4, 4, 4], 20, 4).buckets == [[2], [1], [0]]
    assert oracle.plan_cap([4, 4, 4], 20, 2).buckets == [[2, 1], [0]]
    assert oracle.plan_cap([4, 4, 4], 24, 2).buckets == [[2, 1, 0]]


def test_cap_below_every_parameter_gives_one_bucket_each_in_reverse():
    plan = oracle.plan_cap([5, 6, 7], 4, 4)
    assert plan.buckets == [[2], [1], [0]]


def test_exactly_full_bucket_does_not_close_early():
    assert oracle.plan_cap([5, 5, 5], 40, 4).buckets == [[2, 1], [0]]


def test_invalid_arguments_raise():
    with pytest.raises(ValueError):
        oracle.plan_cap([1, 2], 0, 4)
    with pytest.raises(ValueError):
        oracle.plan_cap([1, -2], 8, 4)
    with pytest.raises(ValueError):
        oracle.plan_two_bucket([1, 2], [0, 9])


def check_plan_invariants(plan, numel, cap_bytes=None, elem_bytes=None):
    n = len(numel)
    seen = [p for b in plan.buckets for p in b]
    assert sorted(seen) == list(range(n))                     # a partition
    loc = plan.param_location()
    base = plan.bucket_base
    spans = sorted((base[b] + off, base[b] + off + numel[p]) for p, (b, off) in enumerate(loc))
    pos = 0
    for lo, hi in spans:                                       # contiguous, no gaps/overlap
        assert lo == pos
        pos = hi
    assert pos == sum(numel) == sum(plan.bucket_len)
    if cap_bytes is not None:
        assert seen == list(range(n))[::-1]                    # reverse registration order
        assert plan.buckets[0][0] == n - 1                     # last layer in bucket 0
        for b, ps in enumerate(plan.buckets):
            nbytes = sum(numel[p] for p in ps) * elem_bytes
            assert nbytes <= cap_bytes or len(ps) == 1
            if b + 1 < len(plan.buckets):                      # greedy: the next one did not fit
                nxt = plan.buckets[b + 1][0]
                assert nbytes + numel[nxt] * elem_bytes > cap_bytes


@pytest.mark.parametrize("name", W.WORKLOADS)
def test_invariants_on_every_workload(name):
    wl = W.workload(name)
    if wl.two_bucket:
        plan = oracle.plan_two_bucket(wl.numel, wl.regions)
        check_plan_invariants(plan, wl.numel)
    else:
        plan = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
        check_plan_invariants(plan, wl.numel, wl.bucket_cap_bytes, wl.in_bytes)


def test_random_fuzz_invariants():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(1, 60))
        numel = [int(v) for v in rng.integers(0, 1000, n)]
        cap = int(rng.integers(1, 5000))
        eb = int(rng.choice([2, 4]))
        check_plan_invariants(oracle.plan_cap(numel, cap, eb), numel, cap, eb)


def test_two_bucket_resnet50_regions():
    wl = W.workload("resnet50")
    plan = oracle.plan_two_bucket(wl.numel, wl.regions)
    assert plan.n_buckets == 2
    deep, first = plan.buckets
    names = [p.name for p in wl.params]
    # DEEP_COMM: every conv except the stem, in registration order
    assert [names[p] for p in deep] == [p.name for p in wl.params
                                        if ".conv" in p.name or "downsample.0" in p.name]
    assert deep == sorted(deep)
    # FIRST_COMM: BN biases, BN weights, fc bias, fc weight, stem conv
    regs = [wl.regions[p] for p in first]
    assert regs == sorted(regs)
    assert names[first[-1]] == "conv1.weight"
    assert names[first[-2]] == "fc.weight" and names[first[-3]] == "fc.bias"
    check_plan_invariants(plan, wl.numel)


def test_two_bucket_gpt_split_sizes_follow_the_region_tags():
    wl = W.workload("gpt1p3b_two_bucket")
    plan = oracle.plan_two_bucket(wl.numel, wl.regions)
    deep = sum(p.numel for p in wl.params if p.region == W.REGION_DEEP)
    assert plan.bucket_len == [deep, wl.total - deep]
    assert plan.bucket_len == [1_208_401_920, 107_321_344]


def test_two_bucket_drops_an_empty_bucket():
    plan = oracle.plan_two_bucket([3, 4], [oracle.DEEP, oracle.DEEP])
    assert plan.buckets == [[0, 1]]


def test_flatten_unflatten_round_trip_bits():
    wl = W.workload("tiny")
    plan = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, 4)
    rng = np.random.default_rng(1)
    grads = [rng.standard_normal(n).astype(np.float32) for n in wl.numel]
    flat = oracle.flatten(plan, grads)
    # reversed order: the bias (registered last) comes first in the bucket
    assert np.array_equal(flat[:10], grads[1]) and np.array_equal(flat[10:], grads[0])
    back = oracle.unflatten(plan, flat)
    for a, b in zip(back, grads):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_hand_worked_flatten_across_buckets():
    """Sizes [3, 5, 2, 4], cap 24 bytes of f32 (6 elements): walking from the
    last parameter, p3 + p2 fill bucket 0 exactly, p1 would overflow it and
    opens bucket 1, p0 would overflow that and opens bucket 2.  Every element
    of the flat buffer is written out by hand (value 10*p + j)."""
    sizes = [3, 5, 2, 4]
    plan = oracle.plan_cap(sizes, 24, 4)
    assert plan.buckets == [[3, 2], [1], [0]]
    assert plan.bucket_base == [0, 6, 11]
    grads = [np.array([10 * p + j for j in range(n)], dtype=np.float32) for p, n in enumerate(sizes)]
    flat = oracle.flatten(plan, grads)
    assert flat.tolist() == [30, 31, 32, 33, 20, 21,
                             10, 11, 12, 13, 14,
                             0, 1, 2]
    back = oracle.unflatten(plan, np.arange(14, dtype=np.float32))
    assert [b.tolist() for b in back] == [[11, 12, 13], [6, 7, 8, 9, 10], [4, 5], [0, 1, 2, 3]]
