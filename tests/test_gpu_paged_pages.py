"""Paged decode against the oracle's paged decode, byte by byte, where the
page layout is not the easy case ("vLLM中的PagedAttention优化": K/V in
16-token blocks found through a block table; "CacheGen实战" 2.3: records
decoded straight into the model's cache):

- a chunk length that is not a multiple of the 16-token page, with the
  planner putting three records in a workgroup, so one wavefront's chains
  start at different offsets inside their pages;
- chunks of more than 128 pages, so each chain's window of block-table
  entries moves on inside the chunk: once with a wavefront's chains in step
  (one record, 33 layers: two or three chains per wavefront) and once with
  one chain per wavefront and the chunk length again not a multiple of 16.
"""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [
    # name, L, H, D, T, C
    ("page-offsets-0-8", 16, 8, 128, 1000, 40),
    ("window-in-step", 33, 1, 64, 7680, 2560),
    ("window-one-chain", 16, 1, 64, 7900, 2600),
]


@pytest.mark.parametrize("name,L,H,D,T,Cc", CASES, ids=[c[0] for c in CASES])
def test_paged_decode_matches_oracle(name, L, H, D, T, Cc):
    U.need_gpu()
    torch = U.torch
    O = U.O
    print("case", name, flush=True)
    X = synth.random_kv(L, H, D, T, 77)
    lg, steps = [0] * L, [0.6]
    g = U.gpu_roundtrip(L, H, D, T, Cc, lg, steps, X, 5)
    assert g["st_enc"] == 0 and g["st_dec"] == 0
    oshp = O.shape(L, H, D, T, Cc)
    blob, _ = O.build_tables(oshp, 5, lg, steps, X)
    data, offs = O.encode_all(oshp, blob, X)
    goffs = g["offs"].cpu().numpy().astype(np.uint64)
    assert np.array_equal(goffs, offs)
    assert np.array_equal(U.u8(g["out"])[:int(offs[-1])], data)

    n_pages = -(-T // 16)
    nb = n_pages + 7
    bt = np.random.default_rng(78).permutation(nb)[:n_pages].astype(np.int32)
    pool = torch.zeros((L, 2, nb, H, 16, D), dtype=torch.float16, device="cuda")
    cd = g["cd"]
    refs, n = cd.refs_for(g["out"], g["offs"])
    cd.decode_paged([g["lv"]], [g["tables"]], refs, n, pool, torch.from_numpy(bt).to("cuda"))
    assert cd.read_status() == 0
    opool = np.zeros((L, 2, nb, H, 16, D), dtype=np.uint16)
    for c in range(len(offs) - 1):
        assert O.decode_chunk_paged(oshp, blob, data[int(offs[c]):int(offs[c + 1])], opool, bt) == O.OK
    assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), opool)
