"""Pins of the oracle's local accumulation (no_sync micro-steps of "DDP"
(sgdbs.github.io, AI_Infra/1.DataParallel), section 5.2): gradients add up
locally across micro-batches and are synchronised once, so the result is
the rank average of every micro-batch gradient.

* exact integer sums; the bf16 path is one f32 add and one rounding
* IEEE specials
* no_sync then one sync == (1/N) sum_r sum_m g[r][m] exactly on dyadic
  inputs (N a power of two), for both summation orders
"""
from fractions import Fraction

import numpy as np

import oracle


def test_f32_exact_integer_sums():
    rng = np.random.default_rng(0)
    a = rng.integers(-10 ** 6, 10 ** 6, 1000).astype(np.float32)
    b = rng.integers(-10 ** 6, 10 ** 6, 1000).astype(np.float32)
    d = a.copy()
    oracle.accumulate(d, b)
    assert np.array_equal(d, (a.astype(np.float64) + b).astype(np.float32))


def test_bf16_is_one_f32_add_then_rne():
    rng = np.random.default_rng(1)
    a = (rng.integers(0, 1 << 16, 3000, dtype=np.uint32) & 0xBFFF).astype(np.uint16)
    b = (rng.integers(0, 1 << 16, 3000, dtype=np.uint32) & 0xBFFF).astype(np.uint16)
    wa = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    wb = (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    d = a.copy()
    oracle.accumulate(d, b, "bf16")
    assert np.array_equal(d, oracle.rne_bf16((wa + wb).astype(np.float32)))


def test_specials():
    d = np.array([np.inf, np.inf, 1.4e-45, -0.0, np.nan], np.float32)
    oracle.accumulate(d, np.array([1.0, -np.inf, 1.4e-45, -0.0, 1.0], np.float32))
    assert d[0] == np.inf and np.isnan(d[1]) and d.view(np.uint32)[2] == 2
    assert np.signbit(d[3]) and np.isnan(d[4])


def test_no_sync_then_sync_is_the_average_of_every_micro_gradient():
    rng = np.random.default_rng(2)
    sizes = [37, 5, 120]
    plan = oracle.plan_cap(sizes, 200, 4)
    N, M = 4, 3
    micro = [[np.array([int(v) / 64 for v in rng.integers(-500, 500, sum(sizes))], np.float32)
              for _ in range(N)] for _ in range(M)]
    for order in ("seq", "ring"):
        got = oracle.no_sync_then_sync(plan, micro, order)
        for i in range(sum(sizes)):
            exact = sum(Fraction(float(micro[m][r][i])) for m in range(M) for r in range(N)) / N
            assert Fraction(float(got[i])) == exact
