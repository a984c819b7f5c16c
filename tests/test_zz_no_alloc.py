"""cg_build_tables_noalloc (symbol counts in the library's static device
array) against cg_build_tables (counts in a caller workspace): two calls in a
row on one GPU, the second on a smaller tensor, give byte-identical tables
blobs (format and lookup sections) and counters; a shape whose counts exceed
the array is refused before any launch."""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth

from tests import gpu_util as U

pytestmark = pytest.mark.gpu
C, torch = U.C, U.torch


def both(L, H, D, T, Cc, lg, steps, X, flags=0):
    shp = C.shape(L, H, D, T, Cc)
    lv = C.Level(5, lg, steps)
    cd = U.codec.Codec(shp)
    x = U.to_dev(X)
    st_ws = torch.zeros(4, dtype=torch.int64, device="cuda")
    st_na = torch.zeros(4, dtype=torch.int64, device="cuda")
    want = cd.build_tables(x, lv, stats=st_ws, flags=flags)
    got = torch.full((cd.tables_bytes(lv),), 0xA5, dtype=torch.uint8, device="cuda")
    C.cg_build_tables_noalloc(shp, lv, x, got, flags, st_na)
    torch.cuda.synchronize()
    return U.u8(want), U.u8(got), st_ws.cpu().numpy(), st_na.cpu().numpy()


def test_noalloc_matches_workspace_build_twice_smaller_second():
    U.need_gpu()
    cfg = synth.CONFIGS["tiny"]
    lvd = cfg.levels[0]
    X1 = synth.generate(cfg)
    w, g, sw, sn = both(cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens,
                        list(lvd.layer_group), list(lvd.steps), X1)
    assert np.array_equal(w, g) and np.array_equal(sw, sn)
    # second call on the same GPU: fewer layers, heads and tokens, so the
    # array still holds the larger first call's counts past the new ones
    X2 = synth.random_kv(2, 1, 64, 300, 71, scale=20.0)
    w, g, sw, sn = both(2, 1, 64, 300, 100, [0, 1], [0.3, 1.2], X2)
    assert np.array_equal(w, g) and np.array_equal(sw, sn)
    assert int(sn[0]) == X2.size


def test_noalloc_robust_tables():
    U.need_gpu()
    X = synth.random_kv(3, 2, 64, 400, 72, scale=6.0)
    w, g, sw, sn = both(3, 2, 64, 400, 128, [0, 0, 1], [0.5, 1.5], X, flags=C.CG_TABLES_ROBUST)
    assert np.array_equal(w, g) and np.array_equal(sw, sn)


def test_noalloc_refuses_counts_larger_than_its_array():
    # 64 groups x 2 x 8 heads x 128 dims x 256 counts x 4 bytes = 64 MiB
    shp = C.shape(64, 8, 128, 1024, 256)
    lv = C.Level(1, list(range(64)), [0.5] * 64)
    assert C.cg_build_workspace_bytes(shp, 64) > C.CG_NOALLOC_SCRATCH_BYTES
    rc = C.lib().cg_build_tables_noalloc(C.ctypes.byref(shp), C.ctypes.byref(lv.c), 256, 256, 0, None, None,
                                         None)
    assert rc == C.CG_ERR_UNSUPPORTED
