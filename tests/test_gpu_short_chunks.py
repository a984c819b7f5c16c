"""The decoder's three-chain pipeline on very short chunks, against the oracle
byte by byte (tables, records, contiguous decode, paged decode).

Small shapes normally get one record per decode workgroup (the dispatch plan
minimises the simulated time, and a few workgroups fit the chip at once). With
many KV heads there are enough table sets that the plan puts three records of
a 16-layer group in each workgroup, so every wavefront runs three chains:

- 3-token chunks: one pipelined iteration per chunk, and the last block mixes
  chunk lengths 3, 3 and 2 (the longer chains finish one at a time);
- 2-token chunks: the pipelined loop runs no iteration (prologue and epilogue
  only), then single records;
- 16-token chunks: every chain's page starts at the same offset, so the paged
  decoder advances one page counter for all chains.
"""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [
    # name, L, H, D, T, C
    ("3-token-chunks", 16, 64, 64, 35, 3),
    ("2-token-chunks", 16, 64, 64, 26, 2),
    ("16-token-chunks", 16, 32, 64, 181, 16),
]


@pytest.mark.parametrize("name,L,H,D,T,Cc", CASES, ids=[c[0] for c in CASES])
def test_short_chunks_match_oracle(name, L, H, D, T, Cc):
    U.need_gpu()
    torch = U.torch
    O = U.O
    print("case", name, flush=True)
    X = synth.random_kv(L, H, D, T, 91, scale=40.0, rho=0.8)
    lg, steps = [0] * L, [0.45]
    # the case is only meaningful with three records per decode workgroup
    rpb, _, _ = U.C.cg_decode_plan(U.C.shape(L, H, D, T, Cc), [U.C.Level(6, lg, steps)], -(-T // Cc))
    assert rpb == 3
    g = U.gpu_roundtrip(L, H, D, T, Cc, lg, steps, X, 6)
    o = U.oracle_roundtrip(L, H, D, T, Cc, lg, steps, X, 6)
    assert g["st_enc"] == 0 and g["st_dec"] == 0
    assert np.array_equal(U.u8(g["tables"])[:len(o["blob"])], o["blob"])
    assert np.array_equal(g["offs"].cpu().numpy().astype(np.uint64), o["offs"])
    assert np.array_equal(U.u8(g["out"])[:int(o["offs"][-1])], o["data"])
    assert np.array_equal(g["y"].cpu().view(torch.int16).numpy().view(np.uint16), o["Y"])

    n_pages = -(-T // 16)
    nb = n_pages + 5
    bt = np.random.default_rng(92).permutation(nb)[:n_pages].astype(np.int32)
    pool = torch.zeros((L, 2, nb, H, 16, D), dtype=torch.float16, device="cuda")
    cd = g["cd"]
    refs, n = cd.refs_for(g["out"], g["offs"])
    cd.decode_paged([g["lv"]], [g["tables"]], refs, n, pool, torch.from_numpy(bt).to("cuda"))
    assert cd.read_status() == 0
    oshp = O.shape(L, H, D, T, Cc)
    opool = np.zeros((L, 2, nb, H, 16, D), dtype=np.uint16)
    offs, data = o["offs"], o["data"]
    for c in range(len(offs) - 1):
        assert O.decode_chunk_paged(oshp, o["blob"], data[int(offs[c]):int(offs[c + 1])], opool, bt) == O.OK
    assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), opool)
