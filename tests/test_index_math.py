"""The sparse decode's ownership quotient, checked exactly on the host.

The fp8 sparse path finds the owner and local index of a global position g
as floor(g / n) = trunc(fma(g, 1/n, 2^-20)), with 1/n the correctly rounded
float64 reciprocal and one rounding for the fused multiply-add.  Claimed
exact for 0 <= g < 2^31 and 1 <= n <= 4096 (the bounds the entry points
enforce).  The fused operation is emulated here with exact rationals and a
single round-to-nearest to float64, over every n in range at the multiples of
n and their neighbours (where a truncation would first go wrong) up to
2^31 - 1, and at random positions.
"""

from fractions import Fraction

import numpy as np

EPS = Fraction(1, 1 << 20)


def fused_quotient(g, n):
    inv = 1.0 / float(n)                       # IEEE division: correctly rounded
    exact = Fraction(g) * Fraction(inv) + EPS  # fma: one rounding of the exact value
    return int(float(exact))                   # float(Fraction) rounds to nearest even; int truncates


def test_quotient_exact_at_every_boundary():
    top = (1 << 31) - 1
    bad = []
    for n in range(1, 4097):
        kmax = top // n
        for k in (1, 2, 3, kmax // 2, kmax - 1, kmax):
            for g in (k * n - 1, k * n, k * n + 1):
                if 0 <= g <= top and fused_quotient(g, n) != g // n:
                    bad.append((g, n))
        for g in (0, top, top - 1):
            if fused_quotient(g, n) != g // n:
                bad.append((g, n))
    assert not bad, bad[:10]


def test_quotient_exact_at_random_positions():
    rng = np.random.default_rng(7)
    ns = rng.integers(1, 4097, size=20000)
    gs = rng.integers(0, 1 << 31, size=20000)
    bad = [(int(g), int(n)) for g, n in zip(gs, ns) if fused_quotient(int(g), int(n)) != int(g) // int(n)]
    assert not bad, bad[:10]


def test_plain_truncation_would_fail():
    """Without the 2^-20 nudge, some multiples of n fall just below the next
    integer after rounding: the guard is needed."""
    fails = 0
    for n in range(1, 4097):
        for k in (1000, (1 << 31) // n - 1):
            g = k * n
            if int(g * (1.0 / n)) != k:
                fails += 1
    assert fails > 0
