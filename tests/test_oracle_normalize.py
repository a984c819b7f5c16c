"""12-bit table normalisation: closed forms and invariants."""
import numpy as np
import pytest

from oracle import oracle as O


def counts(d):
    c = np.zeros(256, dtype=np.uint64)
    for k, v in d.items():
        c[k] = v
    return c


def test_closed_forms():
    assert np.all(O.normalize(np.full(256, 7, dtype=np.uint64)) == 16)
    f = O.normalize(counts({127: 5}))
    assert f[127] == 4096 and f.sum() == 4096
    f = O.normalize(counts({126: 9, 128: 9}))
    assert f[126] == 2048 and f[128] == 2048
    f = O.normalize(counts({3: 1, 200: 10 ** 6}))
    assert f[3] == 1 and f[200] == 4095
    # no observations: all mass on the zero delta
    f = O.normalize(np.zeros(256, dtype=np.uint64))
    assert f[127] == 4096 and f.sum() == 4096
    # deficit goes to the most frequent symbol; ties -> lowest index
    f = O.normalize(counts({10: 3, 20: 3, 30: 3}))
    assert list(f[[10, 20, 30]]) == [1366, 1365, 1365]


def test_surplus_taken_from_largest():
    # 200 singletons each bumped to f=1 plus one dominant symbol
    c = np.zeros(256, dtype=np.uint64)
    c[:200] = 1
    c[250] = 10 ** 9
    f = O.normalize(c)
    assert f.sum() == 4096
    assert np.all(f[:200] == 1)
    assert f[250] == 4096 - 200


@pytest.mark.parametrize("seed", range(40))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    k = rng.integers(1, 257)
    c = np.zeros(256, dtype=np.uint64)
    idx = rng.choice(256, size=k, replace=False)
    kind = seed % 3
    if kind == 0:
        c[idx] = rng.integers(1, 1000, size=k)
    elif kind == 1:
        c[idx] = np.floor(np.exp(rng.uniform(0, 20, size=k))).astype(np.uint64) + 1
    else:  # Laplacian-like delta histogram around symbol 127
        d = np.rint(rng.laplace(0, rng.uniform(0.2, 30), size=100000)).astype(int)
        d = np.clip(d, -128, 128)
        sym = np.where(np.abs(d) <= 127, d + 127, 255)
        c = np.bincount(sym, minlength=256).astype(np.uint64)
    f = O.normalize(c)
    n = float(c.sum())
    assert int(f.sum()) == 4096
    assert np.array_equal(f > 0, c > 0)
    # every frequency is within one unit of its proportional share, except the
    # symbol that absorbed the rounding deficit or surplus
    share = c.astype(np.float64) * 4096 / n
    dev = f.astype(np.float64) - share
    off = np.nonzero((c > 0) & ((dev > 1.0 + 1e-9) | (dev <= -1.0)))[0]
    assert len(off) <= 1, off
