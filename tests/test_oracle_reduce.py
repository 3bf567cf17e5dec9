"""Pins of the oracle's reduce + scale against what the pages and IEEE-754 fix.

Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel);
[TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn).

* P2  sum-then-divide pseudocode of [TR24] section 一: zero-initialised sum in
      rank order, then divide by N; exact on exact inputs.
* P3  the data-parallel identity of [DDP] section 一: the average of the
      per-rank gradients g_k = (N/B) sum_{i in S_k} grad l_i equals the
      full-batch gradient (1/B) sum_i grad l_i -- exactly on dyadic inputs
      with N a power of two, and within the recursive-summation error bound
      (Higham, Accuracy and Stability of Numerical Algorithms, 2nd ed., sec. 4.2)
      on random inputs, checked in exact rational arithmetic.
* P9  the 1/N scale equals a correctly rounded division for N = 1, 2, 4, 8
      ([DDP] section 4.2 divides, [TR24] section 九 multiplies by 1/N).
* P10 N = 1 is the identity, bit for bit ([TR24] section 九 returns early).
* P11 IEEE special values.
* bf16: widen exactly, FP32 fold, one round-to-nearest-even at the end.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

U = Fraction(1, 2 ** 24)        # unit roundoff of binary32


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


# ----------------------------------------------------------------- P2
@pytest.mark.parametrize("N", [2, 4, 8])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p2_sum_then_divide_exact_on_small_integers(N, order):
    rng = np.random.default_rng(N)
    xs = [rng.integers(-50, 50, 333).astype(np.float32) for _ in range(N)]
    got = oracle.bucket_avg(xs, order)
    for i in range(333):
        want = Fraction(sum(int(x[i]) for x in xs), N)
        assert Fraction(float(got[i])) == want


def test_p2_zero_initialised_sum_makes_negative_zero_positive():
    z = _f32([-0.0, -0.0, 1.0])
    seq = oracle.bucket_avg([z, z, z, z], "seq")
    ring = oracle.bucket_avg([z, z, z, z], "ring")
    # grad_sync = zeros_like(...) then += each rank: +0 + -0 = +0
    assert not np.signbit(seq[0]) and not np.signbit(seq[1])
    # the ring fold starts from a rank's own value: -0 + -0 = -0
    assert np.signbit(ring[0]) and np.signbit(ring[1])
    assert seq[2] == 1.0 and ring[2] == 1.0


# ----------------------------------------------------------------- P3
def _identity_case(N, B, L, seed):
    """Per-sample gradients d_i (dyadic), shards of B/N samples per rank."""
    rng = np.random.default_rng(seed)
    d = [[Fraction(int(v), 256) for v in rng.integers(-64, 65, L)] for _ in range(B)]
    m = B // N
    g = []
    for k in range(N):
        shard = range(k * m, (k + 1) * m)
        g.append([Fraction(N, B) * sum(d[i][j] for i in shard) for j in range(L)])
    full = [sum(d[i][j] for i in range(B)) / B for j in range(L)]
    return g, full


@pytest.mark.parametrize("N,B", [(2, 8), (4, 16), (8, 32), (8, 64)])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p3_rank_average_equals_full_batch_gradient_exactly(N, B, order):
    L = 37
    g, full = _identity_case(N, B, L, seed=N * 100 + B)
    xs = []
    for k in range(N):
        row = np.array([float(v) for v in g[k]], dtype=np.float32)
        assert all(Fraction(float(a)) == b for a, b in zip(row, g[k]))   # exact in f32
        xs.append(row)
    got = oracle.bucket_avg(xs, order)
    for j in range(L):
        assert Fraction(float(got[j])) == full[j]


def _error_bound(xs_col, N):
    # fold: N-1 rounded additions (the +0 start is exact); then fl(1/N) and
    # one rounded product:  |y - s/N| <= gamma_{N-1} sum|x| / N (1+u)^2
    #                                    + |s/N| ((1+u)^2 - 1)
    k = N - 1
    gamma = (k * U) / (1 - k * U)
    s = sum(Fraction(float(v)) for v in xs_col)
    sabs = sum(abs(Fraction(float(v))) for v in xs_col)
    return s / N, gamma * sabs / N * (1 + U) ** 2 + abs(s / N) * ((1 + U) ** 2 - 1)


@pytest.mark.parametrize("N", [2, 3, 5, 6, 7, 8, 16])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p3_random_inputs_within_summation_error_bound(N, order):
    rng = np.random.default_rng(17 * N)
    L = 200
    xs = [(rng.standard_normal(L) * 1e-3).astype(np.float32) for _ in range(N)]
    got = oracle.bucket_avg(xs, order)
    for j in range(L):
        exact, bound = _error_bound([x[j] for x in xs], N)
        assert abs(Fraction(float(got[j])) - exact) <= bound


def test_p3_bound_is_tight_enough_to_catch_a_dropped_term():
    # a plausible mistake (one rank left out of the sum) breaks the bound
    rng = np.random.default_rng(5)
    N, L = 4, 50
    xs = [(rng.standard_normal(L) * 1e-3).astype(np.float32) for _ in range(N)]
    wrong = ((xs[0] + xs[1] + xs[2]) * np.float32(0.25)).astype(np.float32)
    bad = 0
    for j in range(L):
        exact, bound = _error_bound([x[j] for x in xs], N)
        bad += abs(Fraction(float(wrong[j])) - exact) > bound
    assert bad > L // 2


# ----------------------------------------------------------------- P9
def _one_hot_rank(x0, N):
    return [np.asarray(x0, dtype=np.float32)] + [np.zeros(len(x0), np.float32)] * (N - 1)


_SCALE_VALUES = np.concatenate([
    np.random.default_rng(9).standard_normal(2000).astype(np.float32),
    np.array([1.0, 3.0, 7.0, 1e-38, 1.1754944e-38, 3e-45, 1.4e-45, 3.4028235e38,
              -2.5, 6.0e-39], dtype=np.float32)])


@pytest.mark.parametrize("N", [1, 2, 4, 8])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p9_power_of_two_scale_is_a_correctly_rounded_division(N, order):
    got = oracle.bucket_avg(_one_hot_rank(_SCALE_VALUES, N), order)
    want = (_SCALE_VALUES / np.float32(N)).astype(np.float32)
    assert np.array_equal(_bits(got), _bits(want))


@pytest.mark.parametrize("N", [3, 5, 6, 7])
def test_p9_other_n_within_two_units_of_roundoff(N):
    # the bits for these N are defined only by the multiply-by-fl(1/N) reading;
    # what the mathematics fixes is closeness to x/N
    x = _SCALE_VALUES[np.abs(_SCALE_VALUES) > 1e-30]
    got = oracle.bucket_avg(_one_hot_rank(x, N), "ring")
    for a, y in zip(x, got):
        exact = Fraction(float(a)) / N
        assert abs(Fraction(float(y)) - exact) <= abs(exact) * (2 * U + U * U)


# ----------------------------------------------------------------- P10
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p10_single_rank_is_bitwise_identity(order):
    pats = np.array([0x80000000, 0x00000000, 0x00000001, 0x7F800000, 0xFF800000,
                     0x7FC00001, 0xFFA00000, 0x3F800000, 0x807FFFFF], dtype=np.uint32)
    x = np.concatenate([pats, np.random.default_rng(2).integers(0, 2 ** 32, 1000,
                                                                 dtype=np.uint32)])
    got = oracle.bucket_avg([x.view(np.float32)], order)
    assert np.array_equal(got.view(np.uint32), x)


# ----------------------------------------------------------------- P11
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_p11_special_values(order):
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    a = _f32([inf, inf, nan, 1.0, 1.4e-45, 3.4028235e38, -inf])
    b = _f32([1.0, -inf, 2.0, nan, 1.4e-45, 3.4028235e38, -5.0])
    got = oracle.bucket_avg([a, b], order)
    assert got[0] == inf
    assert np.isnan(got[1])                     # inf + -inf
    assert np.isnan(got[2]) and np.isnan(got[3])
    assert _bits(got[4:5])[0] == 1              # 2 * 2^-149 * 0.5: subnormals kept
    assert got[5] == inf                        # the sum overflows before the scale
    assert got[6] == -inf


def test_p11_nan_in_one_rank_reaches_every_position_of_its_element_only():
    rng = np.random.default_rng(4)
    xs = [rng.standard_normal(64).astype(np.float32) for _ in range(8)]
    xs[5][17] = np.nan
    for order in ("seq", "ring"):
        got = oracle.bucket_avg(xs, order)
        assert np.isnan(got[17]) and np.isfinite(np.delete(got, 17)).all()


# ----------------------------------------------------------------- bf16
def _widen(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("N", [2, 3, 8])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_bf16_path_is_fp32_fold_of_widened_inputs_then_one_rounding(N, order):
    rng = np.random.default_rng(N)
    hs = [rng.integers(0, 2 ** 16, 999, dtype=np.uint16) for _ in range(N)]
    hs = [np.where((h & 0x7F80) == 0x7F80, h & 0x807F, h).astype(np.uint16) for h in hs]  # finite
    got = oracle.bucket_avg(hs, order, "bf16", "bf16")
    f32 = oracle.bucket_avg([_widen(h) for h in hs], order, "f32", "f32")
    assert np.array_equal(got, oracle.rne_bf16(f32))
    got_f32_in = oracle.bucket_avg([_widen(h) for h in hs], order, "f32", "bf16")
    assert np.array_equal(got_f32_in, got)


def test_bf16_exact_identity_on_dyadic_inputs():
    # bf16 holds 8 significant bits: small integers are exact, so is their mean
    rng = np.random.default_rng(8)
    N = 8
    ints = [rng.integers(-100, 100, 300) for _ in range(N)]
    hs = [(np.asarray(i, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16) for i in ints]
    for order in ("seq", "ring"):
        got = _widen(oracle.bucket_avg(hs, order, "bf16", "bf16"))
        for j in range(300):
            exact = Fraction(sum(int(i[j]) for i in ints), N)
            # exact mean rounded once to bf16 (8 significant bits), ties to even
            assert abs(Fraction(float(got[j])) - exact) <= abs(exact) * Fraction(1, 256)


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_sampled_elements_equal_the_whole_bucket_average(pair, order):
    """sampled_avg (single elements given by value, position and bucket
    length, as the full-size GPU tests sample them) equals the pinned
    bucket_avg at those positions, across buckets of several lengths."""
    in_dt, out_dt = pair
    rng = np.random.default_rng(7)
    for N in (1, 2, 3, 5, 8):
        if N == 1 and in_dt != out_dt:
            continue
        lens = [1, 7, 64, 1001]
        bufs = []
        for L in lens:
            x = [rng.standard_normal(L).astype(np.float32) for _ in range(N)]
            if in_dt == "bf16":
                x = [oracle.rne_bf16(v) for v in x]
            bufs.append(x)
        whole = [oracle.bucket_avg(x, order, in_dt, out_dt) for x in bufs]
        pick = [(b, int(i)) for b, L in enumerate(lens) for i in rng.integers(0, L, 5)]
        vals = np.stack([np.array([bufs[b][r][i] for r in range(N)]) for b, i in pick])
        got = oracle.sampled_avg(vals, np.array([i for _, i in pick]),
                                 np.array([lens[b] for b, _ in pick]), order, in_dt, out_dt)
        want = np.array([whole[b][i] for b, i in pick], dtype=got.dtype)
        assert np.array_equal(got.view(np.uint16 if out_dt == "bf16" else np.uint32),
                              want.view(np.uint16 if out_dt == "bf16" else np.uint32)), (N, order)


@pytest.mark.parametrize("pair", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")])
@pytest.mark.parametrize("order", ["seq", "ring"])
def test_bucket_pieces_equal_the_whole_bucket_average(pair, order):
    """bucket_range_avg (a bucket checked piece by piece, as the full-size
    GPU tests stream it) equals the pinned bucket_avg on every piece, for
    pieces that start and end inside ring chunks, on chunk edges, empty
    pieces and the whole bucket; the pieces of a cut concatenate to it."""
    in_dt, out_dt = pair
    view = np.uint16 if out_dt == "bf16" else np.uint32
    rng = np.random.default_rng(11)
    for N in (1, 2, 3, 5, 8, 9):
        if N == 1 and in_dt != out_dt:
            continue
        for L in (1, 7, 64, 1001):
            x = [rng.standard_normal(L).astype(np.float32) for _ in range(N)]
            if in_dt == "bf16":
                x = [oracle.rne_bf16(v) for v in x]
            whole = oracle.bucket_avg(x, order, in_dt, out_dt)
            cuts = sorted({0, L, *(int(c) for c in rng.integers(0, L + 1, 4)),
                           min(L, -(-L // N)), min(L, 2 * -(-L // N))})
            pieces = [oracle.bucket_range_avg([v[a:b] for v in x], L, a, order, in_dt, out_dt)
                      for a, b in zip(cuts[:-1], cuts[1:])]
            assert np.array_equal(np.concatenate(pieces).view(view), whole.view(view)), (N, L)
            for _ in range(6):
                a = int(rng.integers(0, L + 1))
                b = int(rng.integers(a, L + 1))
                got = oracle.bucket_range_avg([v[a:b] for v in x], L, a, order, in_dt, out_dt)
                assert np.array_equal(got.view(view), whole[a:b].view(view)), (N, L, a, b)


def test_bucket_piece_rejects_a_range_outside_the_bucket():
    x = [np.zeros(5, np.float32)] * 2
    for lo, L in ((-1, 10), (6, 10), (3, 7)):
        with pytest.raises(ValueError):
            oracle.bucket_range_avg(x, L, lo, "ring")
