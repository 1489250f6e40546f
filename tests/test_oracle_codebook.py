"""Pins of the oracle's NF4 codebook and thresholds (CPU only).

The pages print no codebook table, so the pins are the properties they state:
16 levels from N(0,1) quantiles with equal probability mass per bin, dense
near zero, normalised to [-1, 1], exact zero ([QLoRA note] "2. NF4";
[Paper note] "关键设计 1"; [Digest] "数学公式与关键细节" item 1).  The quantile
function is checked against two routines that share nothing with the oracle's
(scipy's ``ndtri`` and a bisection over ``math.erfc``).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4


def phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def phi_inv_bisect(p):
    """Quantile by bisection on erfc-based Phi, run until the bracket stops shrinking."""
    lo, hi = -40.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            return mid
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid


def test_ends_and_exact_zero():
    q = nf4.codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert q[0] == np.float32(-1.0)
    assert q[15] == np.float32(1.0)
    assert q[7] == np.float32(0.0) and not np.signbit(q[7])
    assert np.all(np.diff(q) > 0), "levels must be strictly increasing"
    assert len(set(q.tolist())) == 16


def test_denser_near_zero():
    q = nf4.codebook().astype(np.float64)
    neg_gaps = np.diff(q[:8])[::-1]       # gaps moving away from zero on the negative side
    pos_gaps = np.diff(q[7:])             # gaps moving away from zero on the positive side
    assert np.all(np.diff(neg_gaps) > 0)
    assert np.all(np.diff(pos_gaps) > 0)


def test_equal_probability_mass_per_bin():
    # Undo the normalisation and check that consecutive levels on each half are
    # equally spaced in probability (equal-mass bins), using erfc-based Phi.
    q = nf4.codebook_levels_f64()
    z = nf4._phi_inv(nf4.DELTA)
    pos = [phi(v * z) for v in q[7:]]          # 0.5, ..., delta
    neg = [phi(-v * z) for v in q[:8][::-1]]   # 0.5, ..., delta
    for probs, n in ((pos, 8), (neg, 7)):
        steps = np.diff(probs)
        assert np.allclose(steps, (nf4.DELTA - 0.5) / n, rtol=0, atol=1e-12)


def test_outer_level_is_centre_of_top_bin():
    # 16 equal-mass bins over (0, 1): the top bin is [15/16, 1]; its centre is delta.
    assert nf4.DELTA == (15.0 / 16.0 + 1.0) / 2.0


@pytest.mark.parametrize("name", ["scipy_ndtri", "erfc_bisection"])
def test_independent_quantile_routines_agree(name):
    if name == "scipy_ndtri":
        from scipy.special import ndtri
        alt = lambda p: float(ndtri(p))  # noqa: E731
    else:
        alt = phi_inv_bisect
    assert np.array_equal(nf4.codebook(alt).view(np.uint32), nf4.codebook().view(np.uint32))


def test_threshold_definition():
    q = nf4.codebook()
    T = nf4.thresholds()
    t = nf4.threshold_midpoints()
    for j in range(15):
        exact = (Fraction(float(q[j])) + Fraction(float(q[j + 1]))) / 2
        assert Fraction(t[j]) == exact                     # the double midpoint is exact
        assert Fraction(float(T[j])) <= exact
        nxt = np.nextafter(T[j], np.float32(np.inf))
        assert Fraction(float(nxt)) > exact                 # largest float32 <= midpoint
        # for float32 x around the midpoint, x > T_j  <=>  x > t_j exactly
        x = T[j]
        for _ in range(3):
            x = np.nextafter(x, np.float32(-np.inf))
        for _ in range(7):
            assert (x > T[j]) == (Fraction(float(x)) > exact)
            x = np.nextafter(x, np.float32(np.inf))


def test_some_midpoints_are_ties():
    # Ties are reachable: several midpoints are exactly representable in float32.
    q = nf4.codebook()
    t = nf4.threshold_midpoints()
    representable = [j for j in range(15) if float(np.float32(t[j])) == t[j]]
    assert 7 in representable   # between q[7] = 0 and q[8]: half a float32 is a float32
    assert len(representable) >= 3
    assert q[7] == 0
