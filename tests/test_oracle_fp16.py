"""Pins the oracle's own binary16 <-> binary32 conversion to numpy's."""
import numpy as np

from oracle import oracle as O


def test_half_to_float_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.half_to_float_array(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # signs of NaNs survive
    assert np.array_equal(np.signbit(got[nan]), np.signbit(ref[nan]))


def _check_f2h(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    got = O.float_to_half_array(f)
    ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, (f[~nan][bad[:5]], got[~nan][bad[:5]], ref[~nan][bad[:5]])


def test_float_to_half_strided_bit_patterns():
    # every 4099th bit pattern of binary32: all exponents, signs, NaN/Inf
    bits = np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32)
    _check_f2h(bits.view(np.float32))


def test_float_to_half_ties_and_neighbours():
    # midpoints between consecutive finite halves and their float neighbours:
    # the cases where round-half-even decides
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: the midpoint has <= 12 significant bits
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    for v in (mid, up, dn, -mid, -up, -dn, lo.astype(np.float32)):
        _check_f2h(v)
    _check_f2h(np.array([65504, 65519.99, 65520, 65536, 1e30, np.inf, -np.inf, 0.0, -0.0,
                         2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 * (1 - 2 ** -11)],
                        dtype=np.float32))
