"""Quantizer and reconstruction pins ("CacheGen实战" section 1: one step per
layer group; section 3.1: step presets)."""
import numpy as np
import pytest

from oracle import oracle as O

PRESETS = [0.3, 0.8, 1.2, 0.5, 1.0, 1.5, 0.8, 1.5, 2.0]


def h(v):
    return int(np.float16(v).view(np.uint16))


def test_closed_forms():
    # step 1 on integers is the identity
    for v in [0, 1, -1, 7, -300, 2048, -2048, 32767 // 2]:
        assert O.quantize(h(v), 1.0)[0] == int(np.float16(v))
    # exact ties round to even
    assert [O.quantize(h(v), 1.0)[0] for v in (0.5, 1.5, 2.5, -2.5, -0.5, 3.5)] == [0, 2, 2, -2, 0, 4]
    # a power-of-two step gives an exact quotient
    assert O.quantize(h(3.0), 0.5)[0] == 6
    assert O.quantize(h(0.75), 0.5)[0] == 2      # 1.5 -> 2
    assert O.quantize(h(1.25), 0.5)[0] == 2      # 2.5 -> 2
    # saturation and special values
    assert O.quantize(h(65504), 0.3) == (32767, 1, 0)
    assert O.quantize(h(-65504), 0.3) == (-32768, 1, 0)
    assert O.quantize(0x7C00, 1.0) == (32767, 1, 0)       # +inf
    assert O.quantize(0xFC00, 1.0) == (-32768, 1, 0)      # -inf
    assert O.quantize(0x7E00, 1.0) == (0, 0, 1)           # NaN
    assert O.quantize(0x8000, 1.0) == (0, 0, 0)           # -0
    # 32767.5 is a tie between 32767 and 32768: even is 32768 -> saturates
    assert O.quantize(h(65504), 65504 / 32767.5)[0] == 32767


@pytest.mark.parametrize("step", PRESETS + [0.37, 3.3e-3, 7.77, 1e-3])
def test_fp32_division_pinned_by_fp64(step):
    """fl32(x/s) equals fl32(fl64(x)/fl64(s)): double rounding through
    binary64 is innocuous for a binary32 quotient (53 >= 2*24+2), so numpy's
    float64 route is an independent pin of the oracle's binary32 divide."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = x.view(np.float16).astype(np.float64)
    s32 = np.float32(step)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (xf / np.float64(s32)).astype(np.float32)
        r = np.rint(v)
        ref = np.where(np.isnan(r), 0, np.clip(np.nan_to_num(r, posinf=1e9, neginf=-1e9), -32768, 32767))
    got = O.quantize_array(x, step)
    assert np.array_equal(got, ref.astype(np.int32))


@pytest.mark.parametrize("step", PRESETS + [0.37])
def test_dequant_matches_numpy(step):
    q = np.arange(-32768, 32768, dtype=np.int32)
    got = O.dequantize_array(q, step)
    with np.errstate(over="ignore"):
        ref = (q.astype(np.float32) * np.float32(step)).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("step", PRESETS)
def test_error_bound_all_halves(step):
    """|x_hat - x| <= step/2 + 1 fp16 ulp on every unsaturated finite input."""
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = x.view(np.float16).astype(np.float64)
    q = O.quantize_array(x, step)
    xh = O.dequantize_array(q, step).view(np.float16).astype(np.float64)
    fin = np.isfinite(xf) & (np.abs(xf / step) <= 32767.0)
    big = np.maximum(np.abs(xf), np.abs(xh))
    ulp = np.spacing(big.astype(np.float16)).astype(np.float64)
    with np.errstate(invalid="ignore"):
        err = np.abs(xh - xf)
    assert np.all(err[fin] <= np.float64(np.float32(step)) / 2 + ulp[fin] + 1e-12)


def test_dequant_rounds_twice():
    """fl32(1035 * 1.1f) is exactly 1138.5, a tie in binary16 that goes to the
    even 1138; a single rounding of the exact product (1138.50002...) would
    give 1139."""
    assert np.float32(1035) * np.float32(1.1) == np.float32(1138.5)
    assert O.dequantize(1035, 1.1) == int(np.float16(1138).view(np.uint16))
    assert O.dequantize(-1035, 1.1) == int(np.float16(-1138).view(np.uint16))


def test_integer_identity_step_one():
    x = np.arange(-2048, 2049).astype(np.float16).view(np.uint16)
    q = O.quantize_array(x, 1.0)
    assert np.array_equal(O.dequantize_array(q, 1.0), x)


def test_wrap16():
    assert O.wrap16(32767 + 1) == -32768
    assert O.wrap16(-32768 - 1) == 32767
    assert O.wrap16(32767 - (-32768)) == -1
    assert O.wrap16(-32768 - 32767) == 1
    assert O.wrap16(5) == 5
