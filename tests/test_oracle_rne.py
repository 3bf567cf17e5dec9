"""P8: the oracle's f32 -> bf16 rounding is round-to-nearest, ties to even.

Checked against (a) a second formulation that picks the nearer of the two
neighbouring bf16 values by exact distance (IEEE-754 2019, section 4.3.1:
ties go to the even significand; overflow beyond the largest finite value
goes to infinity as if the exponent were unbounded), and (b) torch's CPU
``to(torch.bfloat16)`` as a library routine.

Coverage: every one of the 65,536 upper halves combined with every low-half
class the rounding decision depends on (0, just above 0, just below the
midpoint, the midpoint, just above it, all ones), plus 2,000,000 random
patterns.
"""
import numpy as np
import pytest

import oracle

LOW_CLASSES = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                       dtype=np.uint32)


def _patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    structured = (hi[:, None] | LOW_CLASSES[None, :]).reshape(-1)
    rnd = np.random.default_rng(123).integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([structured, rnd])


def _nearest_even_reference(u):
    """Independent rounding by distance, for finite f32 patterns u."""
    y = u.view(np.float32).astype(np.float64)
    sign = u & np.uint32(0x80000000)
    mag = u & np.uint32(0x7FFFFFFF)
    lo_pat = mag >> np.uint32(16)                  # bf16 magnitude toward zero
    hi_pat = lo_pat + np.uint32(1)                 # next bf16 magnitude up
    lo_val = (lo_pat << np.uint32(16)).view(np.float32).astype(np.float64)
    hi_val = np.where(hi_pat == 0x7F80, 2.0 ** 128,   # unbounded-exponent successor
                      (hi_pat << np.uint32(16)).view(np.float32).astype(np.float64))
    a = np.abs(y)
    d_lo = a - lo_val                               # exact in binary64
    d_hi = hi_val - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo_pat & np.uint32(1)) == 1))
    mag_out = np.where(pick_hi, hi_pat, lo_pat)
    return ((sign >> np.uint32(16)) | mag_out).astype(np.uint16)


def test_p8_rne_matches_nearest_by_distance():
    u = _patterns()
    finite = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    uf = u[finite]
    got = oracle.rne_bf16(uf.view(np.float32))
    want = _nearest_even_reference(uf)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [hex(int(uf[i])) for i in bad[:5]]


def test_p8_infinities_and_nans():
    u = _patterns()
    special = u[(u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)]
    got = oracle.rne_bf16(special.view(np.float32))
    is_nan = (special & np.uint32(0x7FFFFF)) != 0
    # infinities map to bf16 infinities of the same sign
    assert np.array_equal(got[~is_nan], (special[~is_nan] >> np.uint32(16)).astype(np.uint16))
    # NaNs stay NaN (exponent all ones, nonzero significand), sign kept
    g = got[is_nan]
    assert ((g & 0x7F80) == 0x7F80).all() and ((g & 0x7F) != 0).all()
    assert np.array_equal(g >> 15, (special[is_nan] >> np.uint32(31)).astype(np.uint16))


def test_p8_agrees_with_torch_cpu_conversion():
    torch = pytest.importorskip("torch")
    u = _patterns()
    finite = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    x = u[finite].view(np.float32)
    t = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.rne_bf16(x), t)


def test_p8_a_truncating_rounding_would_fail():
    # the pin is sharp: truncation differs on the midpoint-plus class
    x = np.array([0x3F808001], dtype=np.uint32).view(np.float32)
    assert oracle.rne_bf16(x)[0] == 0x3F81
    assert (np.array([0x3F808001], dtype=np.uint32) >> 16)[0] == 0x3F80
