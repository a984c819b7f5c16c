"""The attention consumer of the restored cache on the GPU against the oracle
("CacheGen实战" 2.3: the decoded cache is used by the model unchanged;
"vLLM中的PagedAttention优化": paged K/V through a block table).

Tolerance, per (layer, query head), from the arithmetic: scores are fp32
sums of D exact products, so |dS| <= D 2^-24 sum_d |q_d k_d| (plus one
rounding of the scale); a weight exp(S - max) then carries a relative error
of at most 2 scale |dS| plus the exponential's few ulps, and the fp32
weighted sum over the tokens of a wavefront and the merge of the partials add
a relative error well below 1e-4. The output is a convex combination of the
V rows, so
    |o - o_exact| <= max|V| (4 scale D 2^-24 max_t sum_d |q_d k_td| + 1e-4).
"""
import numpy as np
import pytest

from kv_cache_compression_encode_amd import synth

from tests import gpu_util as U

pytestmark = pytest.mark.gpu

F16, BF16 = 0, 1


def bits_of(a32, dtype):
    t = U.torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(U.torch.bfloat16 if dtype == BF16 else U.torch.float16).view(U.torch.int16).numpy().view(np.uint16)


def f64_of(bits, dtype):
    t = U.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(U.torch.bfloat16 if dtype == BF16 else U.torch.float16).double().numpy()


def bound(q64, pool64, bt, T, scale, G):
    """Per (l, qh) tolerance of the docstring."""
    L, Hq, D = q64.shape
    tol = np.zeros((L, Hq))
    K = np.stack([pool64[:, 0, bt[t // 16], :, t % 16, :] for t in range(T)], axis=1)  # [L][T][H][D]
    V = np.stack([pool64[:, 1, bt[t // 16], :, t % 16, :] for t in range(T)], axis=1)
    for l in range(L):
        for qh in range(Hq):
            h = qh // G
            smax = np.abs(K[l, :, h, :] * q64[l, qh][None, :]).sum(axis=1).max()
            tol[l, qh] = np.abs(V[l, :, h, :]).max() * (4 * scale * D * 2.0**-24 * smax + 1e-4)
    return tol


def run_gpu(L, H, D, T, G, dtype, q_bits, pool_bits, bt, scale):
    torch = U.torch
    shp = U.C.shape(L, H, D, max(T, 1), 64, dtype)
    cd = U.codec.Codec(shp)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float16
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    pool = torch.from_numpy(pool_bits.view(np.int16)).cuda().view(tdt)
    o = cd.attend_paged(q, pool, torch.from_numpy(bt).cuda(), T, scale)
    st = cd.read_status()
    return o.cpu().numpy().astype(np.float64), st


CASES = [
    # L, H, G, D, T, dtype, seed, value scale
    (2, 2, 4, 128, 333, F16, 1, 1.0),
    (1, 1, 1, 64, 16, F16, 2, 1.0),
    (2, 1, 16, 256, 100, BF16, 3, 3.0),
    (3, 2, 8, 128, 1, F16, 4, 1.0),
    (1, 2, 3, 128, 777, F16, 5, 0.5),
    (1, 1, 8, 128, 5000, F16, 6, 2.0),
    (2, 3, 5, 64, 250, BF16, 7, 8.0),
]


@pytest.mark.parametrize("L,H,G,D,T,dtype,seed,vs", CASES, ids=[str(c[:6]) for c in CASES])
def test_attend_matches_oracle(L, H, G, D, T, dtype, seed, vs):
    U.need_gpu()
    print("attend case", L, H, G, D, T, dtype, flush=True)
    rng = np.random.default_rng(seed)
    nbl = -(-T // 16)
    nb = nbl + 5
    bt = rng.permutation(nb)[:nbl].astype(np.int32)
    pool_bits = bits_of(rng.standard_normal((L, 2, nb, H, 16, D)) * vs, dtype)
    q_bits = bits_of(rng.standard_normal((L, H * G, D)), dtype)
    scale = 1.0 / np.sqrt(D)
    got, st = run_gpu(L, H, D, T, G, dtype, q_bits, pool_bits, bt, scale)
    assert st == 0
    ref = U.O.attend_paged(U.O.shape(L, H, D, T, 64, dtype), q_bits, pool_bits, bt, T, float(np.float32(scale)))
    tol = bound(f64_of(q_bits, dtype), f64_of(pool_bits, dtype), bt, T, scale, G)
    err = np.abs(got - ref).max(axis=2)
    assert np.all(err <= tol), (err.max(), tol.min())


def test_bad_block_table_entry_is_reported():
    U.need_gpu()
    rng = np.random.default_rng(8)
    L, H, D, T = 1, 1, 64, 40
    nb = 4
    bt = np.array([0, 7, 2], dtype=np.int32)  # 7 is outside the pool
    pool_bits = bits_of(rng.standard_normal((L, 2, nb, H, 16, D)), F16)
    q_bits = bits_of(rng.standard_normal((L, 2, D)), F16)
    _, st = run_gpu(L, H, D, T, 2, F16, q_bits, pool_bits, bt, 0.125)
    assert st == U.C.CG_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_decode_then_attend(dtype):
    """End to end: records decoded into a paged pool on the GPU, attention on
    the GPU, against the oracle's decode and attention."""
    U.need_gpu()
    torch = U.torch
    L, H, D, T, Cc, G = 3, 2, 128, 700, 256, 4
    X = synth.random_kv(L, H, D, T, 41) if dtype == F16 else synth.random_kv_bf16(L, H, D, T, 41)
    args = (L, H, D, T, Cc, [0, 1, 1], [0.5, 1.5], X, 9)
    g = U.gpu_roundtrip(*args, dtype=dtype)
    o = U.oracle_roundtrip(*args, dtype=dtype)
    assert g["st_enc"] == 0
    nbl = -(-T // 16)
    nb = nbl + 3
    bt = np.random.default_rng(42).permutation(nb)[:nbl].astype(np.int32)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float16
    pool = torch.zeros((L, 2, nb, H, 16, D), dtype=tdt, device="cuda")
    cd = g["cd"]
    refs, n = cd.refs_for(g["out"], g["offs"])
    btd = torch.from_numpy(bt).cuda()
    cd.decode_paged([g["lv"]], [g["tables"]], refs, n, pool, btd)
    assert cd.read_status() == 0
    rng = np.random.default_rng(43)
    q_bits = bits_of(rng.standard_normal((L, H * G, D)), dtype)
    q = torch.from_numpy(q_bits.view(np.int16)).cuda().view(tdt)
    scale = 1.0 / np.sqrt(D)
    got = cd.attend_paged(q, pool, btd, T, scale)
    assert cd.read_status() == 0
    opool = np.zeros((L, 2, nb, H, 16, D), dtype=np.uint16)
    offs = o["offs"]
    for c in range(len(offs) - 1):
        assert U.O.decode_chunk_paged(o["shp"], o["blob"], o["data"][int(offs[c]):int(offs[c + 1])], opool, bt) == 0
    assert np.array_equal(pool.cpu().view(torch.int16).numpy().view(np.uint16), opool)
    ref = U.O.attend_paged(U.O.shape(L, H, D, T, Cc, dtype), q_bits, opool, bt, T, float(np.float32(scale)))
    tol = bound(f64_of(q_bits, dtype), f64_of(opool, dtype), bt, T, scale, G)
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max(axis=2)
    assert np.all(err <= tol), (err.max(), tol.min())


def test_attend_full_size_sampled():
    """The 34B shape (48 layers, 8 kv heads, 64 query heads, 128 dims, 32768
    tokens, pages placed at random) in the launch configuration the bench
    times; sampled (layer, query head) pairs against the oracle."""
    U.need_gpu()
    torch = U.torch
    L, H, G, D, T = 48, 8, 8, 128, 32768
    nbl = T // 16
    gen = torch.Generator(device="cuda").manual_seed(44)
    pool = torch.randn((L, 2, nbl, H, 16, D), generator=gen, device="cuda").to(torch.float16)
    q = torch.randn((L, H * G, D), generator=gen, device="cuda").to(torch.float16)
    bt = np.random.default_rng(45).permutation(nbl).astype(np.int32)
    btd = torch.from_numpy(bt).cuda()
    cd = U.codec.Codec(U.C.shape(L, H, D, T, 1536))
    scale = 1.0 / np.sqrt(D)
    o = cd.attend_paged(q, pool, btd, T, scale)
    assert cd.read_status() == 0
    rng = np.random.default_rng(46)
    ident = np.arange(nbl, dtype=np.int32)
    for _ in range(4):
        l, qh = int(rng.integers(L)), int(rng.integers(H * G))
        h = qh // G
        sub = pool[l][:, btd.long(), h].unsqueeze(0).unsqueeze(3).contiguous()  # [1][2][nbl][1][16][D]
        sub_bits = sub.cpu().view(torch.int16).numpy().view(np.uint16)
        q_bits = q[l, qh].reshape(1, 1, D).cpu().view(torch.int16).numpy().view(np.uint16)
        ref = U.O.attend_paged(U.O.shape(1, 1, D, T, 1536), q_bits, sub_bits, ident, T,
                               float(np.float32(scale)))[0, 0]
        tol = bound(f64_of(q_bits, F16), f64_of(sub_bits, F16), ident, T, scale, 1)[0, 0]
        err = np.abs(o[l, qh].cpu().numpy().astype(np.float64) - ref).max()
        print("sample", l, qh, "err", err, "bound", tol, flush=True)
        assert err <= tol
