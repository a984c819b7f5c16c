"""The decode dispatch plan (host logic, no GPU): records per workgroup as
cg_decode launches them, planned for 256 compute units (an MI355X)."""
import os

import pytest

from kv_cache_compression_encode_amd import synth

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "kv_cache_compression_encode_amd", "libcg.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")
CUS = 256


def plan(L, H, D, T, Cc, groups):
    from kv_cache_compression_encode_amd import cg as C
    lg = [min(l * groups // L, groups - 1) for l in range(L)]
    lv = C.Level(3, lg, [0.5 + 0.1 * g for g in range(groups)])
    return C.cg_decode_plan(C.shape(L, H, D, T, Cc), [lv], -(-T // Cc), CUS)


def test_few_workgroups_take_one_record_each():
    # 2 table sets x 4 records all run at once on the 256 compute units: the shortest
    # workgroup (one record, one chain per wavefront) gives the shortest run
    assert plan(16, 1, 64, 1024, 256, 1) == (1, 0, 1)
    from kv_cache_compression_encode_amd import cg as C
    cfg = synth.CONFIGS["tiny"]
    lv = cfg.levels[0]
    assert C.cg_decode_plan(C.shape(4, 2, 64, 1024, 256), [C.Level(lv.level_id, lv.layer_group, lv.steps)], 4,
                            CUS) == (1, 0, 1)


def test_many_sets_fill_workgroups_with_three_records():
    # 128 table sets of a 16-layer group: three records per workgroup
    # (48 groups = three chains on each of 16 wavefronts)
    assert plan(16, 64, 64, 35, 3, 1) == (3, 12, 1)
    assert plan(16, 64, 64, 26, 2, 1) == (3, 9, 1)
    assert plan(16, 32, 64, 181, 16, 1) == (3, 9, 1)


def test_34b_workload_plan():
    from kv_cache_compression_encode_amd import cg as C
    cfg = synth.CONFIGS["34b"]
    lv = cfg.levels[0]
    got = C.cg_decode_plan(C.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens),
                           [C.Level(lv.level_id, lv.layer_group, lv.steps)], cfg.n_chunks, CUS)
    # 15 of the 22 records in triples, the rest (with the 512-token last
    # chunk) in pairs
    assert got == (3, 15, 2)
    r1, split, r2 = got
    assert split % r1 == 0 and 1 <= r2 <= r1 <= 3


def test_more_layers_per_group_than_wavefronts_allow_fewer_records():
    # 33 layers in one group: three records would need 99 chains > 48
    r1, _, r2 = plan(33, 64, 64, 35, 3, 1)
    assert r1 == 1 and r2 == 1


def test_layer_group_wider_than_a_workgroup_round():
    # 64 layers in one group: one record per workgroup, decoded in two rounds
    # of up to 48 chains (16 wavefronts x 3)
    assert plan(64, 8, 128, 4096, 512, 1) == (1, 0, 1)
    r1, _, r2 = plan(100, 2, 64, 333, 33, 2)
    assert r1 == 1 and r2 == 1


def test_plan_follows_the_compute_unit_count():
    from kv_cache_compression_encode_amd import cg as C
    lv = C.Level(3, [0] * 16, [0.5])
    shp = C.shape(16, 64, 64, 35, 3)
    # few units: the largest blocks; as many units as workgroups of one
    # record: one record each
    assert C.cg_decode_plan(shp, [lv], 12, 8)[0] == 3
    assert C.cg_decode_plan(shp, [lv], 12, 4096) == (1, 0, 1)


def test_plan_argument_checks():
    from kv_cache_compression_encode_amd import cg as C
    lv = C.Level(1, [0] * 4, [0.5])
    with pytest.raises(RuntimeError):
        C.cg_decode_plan(C.shape(4, 2, 64, 1024, 256), [lv], 0)
    with pytest.raises(RuntimeError):
        C.cg_decode_plan(C.shape(4, 2, 65, 1024, 256), [lv], 4)
