"""GPU path (through the C ABI) against the oracle, element by element and
byte by byte: tables, chunk records, reconstructed fp16 values, counters."""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth

from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [
    # (name, L, H, D, T, C, layer_group, steps, seed)
    ("tiny-config", None, None, None, None, None, None, None, None),
    ("one-token", 1, 1, 64, 1, 1, [0], [0.5], 1),
    ("ragged-chunks", 3, 2, 128, 300, 64, [0, 1, 1], [0.37, 1.1], 2),
    ("chunk-7", 2, 1, 64, 37, 7, [0, 0], [1.0], 3),
    ("d192-single-chunk", 1, 3, 192, 100, 100, [0], [0.3], 4),
    ("many-layers", 17, 1, 64, 129, 128, [l // 6 for l in range(17)], [0.3, 0.8, 1.2], 5),
    # layer groups wider than one workgroup round (16 wavefronts x 3 chains):
    # 64 layers in one group (two rounds), 60 + 40 layers (rounds of 48 + 12)
    ("64-layers-one-group", 64, 1, 64, 40, 16, [0] * 64, [0.8], 6),
    ("100-layers-two-groups", 100, 1, 64, 33, 33, [0] * 60 + [1] * 40, [0.5, 1.5], 7),
    # every chunk one token (records hold only heads, no symbols)
    ("one-token-chunks", 2, 2, 64, 9, 1, [0, 1], [0.5, 1.0], 8),
    # the largest layer count the library takes, in one group (22 decode
    # rounds of 48 items per record)
    ("1024-layers", 1024, 1, 64, 6, 4, [0] * 1024, [0.8], 9),
    # head_dim 256: four 64-channel slices per head
    ("d256", 2, 2, 256, 70, 32, [0, 1], [0.3, 1.2], 10),
]


def case_inputs(case):
    name, L, H, D, T, Cc, lg, steps, seed = case
    if name == "tiny-config":
        cfg = synth.CONFIGS["tiny"]
        lv = cfg.levels[0]
        return (cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens,
                list(lv.layer_group), list(lv.steps), synth.generate(cfg), lv.level_id)
    X = synth.random_kv(L, H, D, T, seed, scale=[3.0, 40.0, 300.0][seed % 3])
    return L, H, D, T, Cc, lg, steps, X, 7


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def pair(request):
    U.need_gpu()
    args = case_inputs(request.param)
    print("case", request.param[0], flush=True)
    return args, U.gpu_roundtrip(*args), U.oracle_roundtrip(*args)


def test_tables_bit_exact(pair):
    args, g, o = pair
    fb = len(o["blob"])
    assert g["cd"].format_bytes(g["lv"]) == fb
    got = U.u8(g["tables"])[:fb]
    assert np.array_equal(got[:64], o["blob"][:64])
    assert np.array_equal(got, o["blob"])


def test_stats_exact(pair):
    args, g, o = pair
    assert np.array_equal(g["stats"].cpu().numpy().astype(np.uint64), o["stats"])


def test_records_bit_exact(pair):
    args, g, o = pair
    assert g["st_enc"] == 0
    offs = g["offs"].cpu().numpy().astype(np.uint64)
    assert np.array_equal(offs, o["offs"])
    got = U.u8(g["out"])[:int(offs[-1])]
    assert np.array_equal(got, o["data"])


def test_decode_bit_exact(pair):
    args, g, o = pair
    assert g["st_dec"] == 0
    y = g["y"].cpu().numpy().view(np.uint16)
    assert np.array_equal(y, o["Y"])


def test_paged_decode_bit_exact(pair):
    """The paged decoder over a seeded random block table gives the oracle's
    pool; untouched blocks keep their fill."""
    args, g, o = pair
    L, H, D, T, Cc, lg, steps = args[:7]
    nb = -(-T // 16)
    NB = nb + 3
    bt = np.random.default_rng(11).permutation(NB)[:nb].astype(np.int32)
    pool = U.torch.full((L, 2, NB, H, 16, D), 0x7E00, dtype=U.torch.int16, device="cuda").view(
        g["x"].dtype)
    bt_dev = U.torch.from_numpy(bt).cuda()
    refs, n = g["cd"].refs_for(g["out"], g["offs"])
    g["cd"].decode_paged([g["lv"]], [g["tables"]], refs, n, pool, bt_dev)
    assert g["cd"].read_status() == 0
    want = np.full((L, 2, NB, H, 16, D), 0x7E00, dtype=np.uint16)
    for c in range(len(o["offs"]) - 1):
        rec = o["data"][int(o["offs"][c]):int(o["offs"][c + 1])]
        assert U.O.decode_chunk_paged(o["shp"], o["blob"], rec, want, bt) == U.O.OK
    assert np.array_equal(pool.cpu().view(U.torch.int16).numpy().view(np.uint16), want)
