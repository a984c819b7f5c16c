"""Level-mix decode where the decoder puts several records in one workgroup
("CacheGen实战" 2.1: every chunk stored at three quality levels, 2.2: the
level picked per chunk; 2.3: parallel GPU decode). The shape is large enough
that the block planner gives two records per workgroup, and each block of
records is launched once per table set, decoding only its set's records:
the result must not depend on how the levels of neighbouring records mix or
on the order of the references. Byte-exact against the oracle's per-chunk
decode."""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SHAPES = [
    # L, H, D, T, CC (15 chunks), records per decode workgroup
    (16, 8, 128, 600, 40, 2),
    (16, 64, 64, 150, 10, 3),
]
LEVELS = [(3, [0] * 16, [0.5]), (4, [0] * 8 + [1] * 8, [0.8, 1.2])]


@pytest.fixture(scope="module", params=SHAPES, ids=["2-records", "3-records"])
def two_levels(request):
    U.need_gpu()
    torch = U.torch
    O = U.O
    L, H, D, T, CC, rpb = request.param
    print("shape", request.param, flush=True)
    levels = [U.C.Level(lid, lg, st) for lid, lg, st in LEVELS]
    assert U.C.cg_decode_plan(U.C.shape(L, H, D, T, CC), levels, -(-T // CC))[0] == rpb
    X = synth.random_kv(L, H, D, T, 81)
    shp = U.C.shape(L, H, D, T, CC)
    cd = U.codec.Codec(shp)
    x = U.to_dev(X)
    oshp = O.shape(L, H, D, T, CC)
    gl, tabs, outs, oracle = [], [], [], []
    for lid, lg, st in LEVELS:
        lv = U.C.Level(lid, lg, st)
        t = cd.build_tables(x, lv)
        out, offs = cd.encode(x, lv, t)
        assert cd.read_status() == 0
        gl.append(lv)
        tabs.append(t)
        outs.append((out, offs))
        blob, _ = O.build_tables(oshp, lid, lg, st, X)
        data, ooffs = O.encode_all(oshp, blob, X)
        assert np.array_equal(offs.cpu().numpy().astype(np.uint64), ooffs)
        oracle.append((blob, data, ooffs))
    torch.cuda.synchronize()
    return cd, gl, tabs, outs, oshp, oracle, (L, H, D, T, CC)


def expected(oshp, oracle, mix, dims):
    O = U.O
    L, H, D, T, CC = dims
    ref = np.zeros((L, 2, H, T, D), dtype=np.uint16)
    for c, m in enumerate(mix):
        blob, data, offs = oracle[int(m)]
        assert O.decode_chunk(oshp, blob, data[int(offs[c]):int(offs[c + 1])], ref) == O.OK
    return ref


@pytest.mark.parametrize("pattern", ["runs", "alternating", "random-reversed"])
def test_level_mix_in_shared_blocks(two_levels, pattern):
    cd, gl, tabs, outs, oshp, oracle, dims = two_levels
    T, CC = dims[3], dims[4]
    n = -(-T // CC)
    if pattern == "runs":
        mix = np.array([0] * 7 + [1] * 8)
    elif pattern == "alternating":
        mix = np.arange(n) % 2
    else:
        mix = np.random.default_rng(82).integers(0, 2, n)
    order = list(range(n))[::-1] if pattern == "random-reversed" else list(range(n))
    parts = [(outs[int(mix[c])][0], outs[int(mix[c])][1], [c], int(mix[c])) for c in order]
    refs, nr = cd.make_refs(parts)
    y = cd.decode(gl, tabs, refs, nr)
    assert cd.read_status() == 0
    assert np.array_equal(y.cpu().numpy().view(np.uint16), expected(oshp, oracle, mix, dims))


def test_table_index_out_of_range_with_levels(two_levels):
    cd, gl, tabs, outs, oshp, oracle, _ = two_levels
    out, offs = outs[0]
    parts = [(out, offs, [0, 1], 0), (out, offs, [2], 2), (out, offs, [3], 0)]  # table 2: only 2 passed
    refs, nr = cd.make_refs(parts)
    cd.decode(gl, tabs, refs, nr)
    assert cd.read_status() == U.C.CG_ERR_INVALID_ARG
