"""The encoder's quotient without a divider, checked on the host.

The rANS coding step ("CacheGen实战" section 1, grouped entropy coding; the
12-bit static rANS reading) needs floor(x / f) for a state x < f * 2^20
(after renormalisation, so x < 2^32) and a frequency 1 <= f <= 4096. The
GPU encoder computes it as trunc(fl64(x) * RU(1/f)), where RU(1/f) is 1/f
rounded up to binary64 (1/f rounded to nearest, moved up one ulp when
f * RN(1/f) < 1). This test restates that construction in numpy and
compares it with exact integer division at the values where a quotient
could first go wrong -- x = k*f - 1 and x = k*f, one below and at each
multiple -- for every f, at the bottom, middle and top of the state range.
"""
from fractions import Fraction

import numpy as np


def ru_recip(f: int) -> np.float64:
    r = np.float64(1.0) / np.float64(f)
    if Fraction(float(r)) * f < 1:
        r = np.nextafter(r, np.float64(np.inf))
    assert Fraction(float(r)) * f >= 1
    assert Fraction(float(np.nextafter(r, np.float64(-np.inf)))) * f < 1
    return r


def test_reciprocals_round_up():
    for f in (1, 2, 3, 5, 7, 255, 1000, 4095, 4096):
        r = ru_recip(f)
        assert Fraction(float(r)) >= Fraction(1, f)


def multiples(f: int) -> np.ndarray:
    top = min(f << 20, 1 << 32) // f  # x < f * 2^20 and x < 2^32
    ks = np.unique(np.concatenate([
        np.arange(1, 66, dtype=np.int64),
        np.arange((1 << 16) // f, (1 << 16) // f + 66, dtype=np.int64),
        np.arange(max(1, top - 300), top + 1, dtype=np.int64),
        np.linspace(1, top, 200).astype(np.int64)]))
    x = np.concatenate([ks * f - 1, ks * f])
    x = x[(x >= 0) & (x < min(f << 20, 1 << 32))]
    return np.unique(x).astype(np.uint64)


def test_quotient_exact_at_boundaries_for_every_frequency():
    bad = []
    for f in range(1, 4097):
        r = ru_recip(f)
        x = multiples(f)
        got = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
        want = x // np.uint64(f)
        if not np.array_equal(got, want):
            i = int(np.argmax(got != want))
            bad.append((f, int(x[i]), int(got[i]), int(want[i])))
    assert not bad, bad[:5]


def test_quotient_exact_at_the_range_extremes():
    # the largest states each frequency allows, and the smallest states
    for f in (1, 2, 3, 4095, 4096, 2731, 3277):
        r = ru_recip(f)
        hi = min(f << 20, 1 << 32)
        x = np.arange(max(0, hi - 5000), hi, dtype=np.uint64)
        x = np.concatenate([x, np.arange(0, 5000, dtype=np.uint64),
                            np.arange(1 << 16, (1 << 16) + 5000, dtype=np.uint64)])
        got = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
        assert np.array_equal(got, x // np.uint64(f)), f


def test_rounded_to_nearest_reciprocal_would_fail():
    """The rounding up matters: with RN(1/f) some frequency's quotient is
    one short just at a multiple (so the test above can tell the two apart)."""
    short = 0
    for f in range(1, 4097):
        r = np.float64(1.0) / np.float64(f)
        x = multiples(f)
        got = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
        short += int(np.count_nonzero(got != x // np.uint64(f)))
    assert short > 0
