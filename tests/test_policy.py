"""Level policies (host only): the bandwidth thresholds of "CacheGen实战" 2.2
(comparison operators garbled on the page; reading: > 5 Gbit/s high, > 1 to 5
balanced, else fast), the recency schedule of dynamic bit allocation, and the
host-side record picking and segmenting of the policy driver."""
import math
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_compression_encode_amd", "libcg.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")


def test_select_level_thresholds():
    from kv_cache_compression_encode_amd import cg as C
    cases = [(20.0, 0), (5.0001, 0), (5.0, 1), (3.0, 1), (1.0001, 1), (1.0, 2), (0.1, 2), (0.0, 2),
             (-1.0, 2), (math.nan, 2), (math.inf, 0)]
    for bw, lvl in cases:
        assert C.cg_select_level(bw) == lvl, bw


def test_recency_levels():
    from kv_cache_compression_encode_amd import cg as C
    lv = C.cg_recency_levels(10, 2, 6)
    # distance from the newest chunk: 9 .. 0
    assert lv.tolist() == [2, 2, 2, 2, 1, 1, 1, 1, 0, 0]
    assert C.cg_recency_levels(3, 0, 0).tolist() == [2, 2, 2]
    assert C.cg_recency_levels(3, 5, 9).tolist() == [0, 0, 0]
    assert C.cg_recency_levels(1, 1, 1).tolist() == [0]
    for bad in ((0, 1, 2), (5, 3, 2), (5, -1, 2)):
        with pytest.raises(C.CgError):
            C.cg_recency_levels(*bad)


def test_pick_records_and_transfer_time():
    from kv_cache_compression_encode_amd import policy as P
    rng = np.random.default_rng(0)
    conts = []
    for k in range(3):
        sizes = rng.integers(1, 50, 4) * 256
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64)
        conts.append((rng.integers(0, 256, int(offs[-1]), dtype=np.uint8), offs))
    levels = np.array([2, 0, 1, 0], dtype=np.int32)
    recs, offs, tor = P.pick_records(conts, levels)
    assert tor.tolist() == levels.tolist()
    for c, k in enumerate(levels):
        d, o = conts[k]
        assert np.array_equal(recs[int(offs[c]):int(offs[c + 1])], d[int(o[c]):int(o[c + 1])])
    trace = [10.0, 1.0, 2.0, 8.0]
    want = sum(float(offs[c + 1] - offs[c]) * 8 / (trace[c] * 1e9) for c in range(4))
    assert P.transfer_seconds(offs, trace) == pytest.approx(want)


def test_levels_for_bandwidth_and_segments():
    from kv_cache_compression_encode_amd import policy as P, synth
    tr = synth.bandwidth_trace(64, seed=1)
    lv = P.levels_for_bandwidth(tr)
    assert set(lv.tolist()) == {0, 1, 2}  # the trace visits every band
    assert all(lv[i] == (0 if tr[i] > 5 else 1 if tr[i] > 1 else 2) for i in range(64))
    segs = P.recency_segments([2, 2, 1, 1, 1, 0])
    assert segs == [(0, 2, 2), (2, 5, 1), (5, 6, 0)]
