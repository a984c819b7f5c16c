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

The encoder's LDS table stores that reciprocal rounded up further to 36
significant bits, with 4096 - f in the 16 low mantissa bits; its symbol
entries are (16 f - 1) mod 2^16 | b << 16, which give the renormalisation
test on the state's high half and, by their order, the escape decision.
Both are checked here as well.
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


# The constants table the encoder keeps in LDS holds, per frequency, one
# binary64 word: RU(1/f) rounded up further to 36 significant bits, with
# 4096 - f in the 16 low mantissa bits that frees. The value read back is
# then slightly above RU(1/f); the quotient must still be exact.

def packed_recip(f: int) -> np.float64:
    u = int(np.array([ru_recip(f)], dtype=np.float64).view(np.uint64)[0])
    u = ((u + 0xFFFF) & ~0xFFFF) | (4096 - f)
    return np.array([u], dtype=np.uint64).view(np.float64)[0]


def test_packed_reciprocal_carries_4096_minus_f():
    for f in range(1, 4097):
        u = int(np.array([packed_recip(f)], dtype=np.float64).view(np.uint64)[0])
        assert u & 0xFFFF == 4096 - f
        # still at or above 1/f, and within 2^-35 relative of it
        r = Fraction(float(packed_recip(f)))
        assert r >= Fraction(1, f)
        assert (r * f - 1) < Fraction(1, 1 << 35)


def test_packed_quotient_exact_at_boundaries_for_every_frequency():
    bad = []
    for f in range(1, 4097):
        r = packed_recip(f)
        x = multiples(f)
        got = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
        if not np.array_equal(got, x // np.uint64(f)):
            bad.append(f)
    assert not bad, bad[:5]


def test_packed_quotient_exact_at_the_range_extremes():
    for f in (1, 2, 3, 4095, 4096, 2731, 3277, 4093):
        r = packed_recip(f)
        hi = min(f << 20, 1 << 32)
        x = np.concatenate([np.arange(max(0, hi - 20000), hi, dtype=np.uint64),
                            np.arange(1 << 16, (1 << 16) + 5000, dtype=np.uint64)])
        got = np.trunc(x.astype(np.float64) * r).astype(np.uint64)
        assert np.array_equal(got, x // np.uint64(f)), f


def test_renormalisation_test_on_the_high_half():
    """x >= f * 2^20 exactly when (x >> 16) > (16 f - 1) mod 2^16, for every
    f in 1..4096 and every high half of a 32-bit state (f = 4096: never)."""
    hi = np.arange(1 << 16, dtype=np.uint64)
    for f in range(1, 4097):
        lo16 = (16 * f - 1) & 0xFFFF
        # the smallest and largest x of each high half decide the same way
        for low in (0, 0xFFFF):
            x = (hi << np.uint64(16)) | np.uint64(low)
            assert np.array_equal(x >= np.uint64(f << 20), hi > np.uint64(lo16)), f


def test_escape_entry_is_above_every_coded_symbol():
    """The encoder tells an escaping lane by its symbol entry
    (16 f - 1) mod 2^16 | b << 16 being at or above the escape's (symbol
    255, last in cumulative order): every other coded symbol (f > 0) has a
    smaller start b, so a smaller entry. Tables from the oracle's
    normalisation, plain and robust, over random and degenerate counts."""
    from oracle import oracle as O
    rng = np.random.default_rng(5)
    cases = [np.zeros(256, dtype=np.uint64)]
    for k in range(300):
        c = np.zeros(256, dtype=np.uint64)
        width = int(rng.integers(1, 256))
        idx = rng.choice(256, size=width, replace=False)
        c[idx] = rng.integers(1, 10 ** int(rng.integers(1, 7)), size=width).astype(np.uint64)
        cases.append(c)
    checked = 0
    for c in cases:
        for robust in (False, True):
            f = O.normalize(c, robust=robust).astype(np.int64)
            b = np.concatenate([[0], np.cumsum(f)[:-1]])
            e = ((16 * f - 1) & 0xFFFF) | (b << 16)
            if f[255] == 0:
                assert not robust
                continue
            coded = (f > 0) & (np.arange(256) < 255)
            assert np.all(e[coded] < e[255])
            assert e[255] < 0xFFFFFFFF  # below the invalid marker
            checked += 1
    assert checked > 300
