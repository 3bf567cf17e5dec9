"""Pins of the oracle's SGD step, the optimizer update the 1/N average is
folded into ("(24) NCCL通信与分布式数据并行", section 九, note on removing the
separate scale kernel; update rule theta <- theta - eta * g of "DDP"
(sgdbs.github.io, AI_Infra/1.DataParallel), section 5.3).

* exact rational results on dyadic inputs (plain and with momentum, two steps)
* the two-rounding error bound on random inputs
* lr = 0 leaves the parameters untouched
* bf16 gradients are widened exactly before the step
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

U = Fraction(1, 2 ** 24)


def _dyadic(rng, n, scale=256):
    return np.array([int(v) / scale for v in rng.integers(-200, 201, n)], dtype=np.float32)


def test_plain_step_exact_on_dyadic_inputs():
    rng = np.random.default_rng(0)
    p0 = _dyadic(rng, 500)
    g = _dyadic(rng, 500)
    for lr in (0.5, 0.125, 2.0 ** -10):
        p = p0.copy()
        oracle.sgd_step(p, g, lr)
        for a, b, c in zip(p, p0, g):
            assert Fraction(float(a)) == Fraction(float(b)) - Fraction(lr) * Fraction(float(c))


def test_momentum_two_steps_exact_on_dyadic_inputs():
    rng = np.random.default_rng(1)
    p = _dyadic(rng, 300)
    g1, g2 = _dyadic(rng, 300), _dyadic(rng, 300)
    m = np.zeros_like(p)
    lr, mu = 0.25, 0.5
    P0 = [Fraction(float(x)) for x in p]
    oracle.sgd_step(p, g1, lr, momentum_buf=m, momentum=mu)
    oracle.sgd_step(p, g2, lr, momentum_buf=m, momentum=mu)
    for i in range(300):
        v1 = Fraction(float(g1[i]))
        p1 = P0[i] - Fraction(lr) * v1
        v2 = Fraction(mu) * v1 + Fraction(float(g2[i]))
        p2 = p1 - Fraction(lr) * v2
        assert Fraction(float(m[i])) == v2
        assert Fraction(float(p[i])) == p2


def test_random_step_within_two_roundings():
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(2000).astype(np.float32)
    g = (rng.standard_normal(2000) * 1e-3).astype(np.float32)
    lr = 0.1
    p = p0.copy()
    oracle.sgd_step(p, g, lr)
    lrf = Fraction(float(np.float32(lr)))
    for a, b, c in zip(p, p0, g):
        s = lrf * Fraction(float(c))
        exact = Fraction(float(b)) - s
        bound = abs(s) * U + (abs(exact) + abs(s) * U) * U
        assert abs(Fraction(float(a)) - exact) <= bound


def test_zero_learning_rate_keeps_parameters():
    rng = np.random.default_rng(3)
    p0 = rng.standard_normal(1000).astype(np.float32)
    p = p0.copy()
    oracle.sgd_step(p, rng.standard_normal(1000).astype(np.float32), 0.0)
    assert np.array_equal(p.view(np.uint32), p0.view(np.uint32))


def test_bf16_gradient_is_widened_exactly():
    rng = np.random.default_rng(4)
    h = (rng.integers(0, 1 << 16, 700, dtype=np.uint32) & 0xBFFF).astype(np.uint16)
    wide = (h.astype(np.uint32) << np.uint32(16)).view(np.float32)
    p0 = rng.standard_normal(700).astype(np.float32)
    a, b = p0.copy(), p0.copy()
    oracle.sgd_step(a, h, 0.01, "bf16")
    oracle.sgd_step(b, wide, 0.01, "f32")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_sync_then_step_composes():
    wl = W.workload("tiny")
    plan = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, 4)
    xs = [W.host_rank_flat(wl, r) for r in range(wl.n_ranks)]
    p = np.random.default_rng(5).standard_normal(plan.total).astype(np.float32)
    q = p.copy()
    avg = oracle.sync_sgd(plan, xs, "ring", p, 0.05)
    oracle.sgd_step(q, oracle.sync_avg(plan, xs, "ring"), 0.05)
    assert np.array_equal(p, q) and np.array_equal(avg, oracle.sync_avg(plan, xs, "ring"))


def test_bad_arguments():
    with pytest.raises(ValueError):
        oracle.sgd_step(np.zeros(3, np.float32), np.zeros(4, np.float32), 0.1)
