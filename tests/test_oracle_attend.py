"""Attention over the restored paged cache: the consumer of the decoded KV
("CacheGen实战" section 2.3: decoded KV is filled into the model's cache and
used unchanged; KV-cache optimisation article, 「vLLM中的PagedAttention优化」:
K/V read from physical blocks through a block table). One new token per
layer, grouped query heads."""
import numpy as np
import pytest

from oracle import oracle as O


def pool_and_table(rng, L, H, D, T, extra=3, dtype=np.float16, scale=1.0):
    nbl = -(-T // 16)
    nb = nbl + extra
    bt = rng.permutation(nb)[:nbl].astype(np.int32)
    pool = (rng.standard_normal((L, 2, nb, H, 16, D)) * scale).astype(dtype)
    return pool, bt


def numpy_attend(q16, pool16, bt, T, scale, G):
    """Independent route: gather K/V by token, numpy matmul + exp in float64."""
    L, Hq, D = q16.shape
    K = np.stack([pool16[:, 0, bt[t // 16], :, t % 16, :] for t in range(T)], axis=1).astype(np.float64)
    V = np.stack([pool16[:, 1, bt[t // 16], :, t % 16, :] for t in range(T)], axis=1).astype(np.float64)
    o = np.zeros((L, Hq, D))
    for l in range(L):
        for qh in range(Hq):
            s = scale * (K[l, :, qh // G, :] @ q16[l, qh].astype(np.float64))
            p = np.exp(s - s.max())
            o[l, qh] = (p @ V[l, :, qh // G, :]) / p.sum()
    return o


@pytest.mark.parametrize("L,H,G,D,T,seed", [(2, 2, 4, 64, 100, 1), (1, 3, 1, 128, 16, 2), (2, 1, 8, 128, 333, 3)])
def test_matches_numpy_route(L, H, G, D, T, seed):
    rng = np.random.default_rng(seed)
    pool, bt = pool_and_table(rng, L, H, D, T)
    q = rng.standard_normal((L, H * G, D)).astype(np.float16)
    shp = O.shape(L, H, D, T, 64)
    sc = 1.0 / np.sqrt(D)
    o = O.attend_paged(shp, q.view(np.uint16), pool.view(np.uint16), bt, T, sc)
    ref = numpy_attend(q, pool, bt, T, sc, G)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(4)
    L, H, D, T = 1, 1, 64, 40
    pool, bt = pool_and_table(rng, L, H, D, T)
    q = rng.standard_normal((L, 2, D)).astype(np.float16)
    shp = O.shape(L, H, D, T, 64)
    # one token: the output is that token's V
    o = O.attend_paged(shp, q.view(np.uint16), pool.view(np.uint16), bt, 1, 0.125)
    assert np.array_equal(o[0, 0], pool[0, 1, bt[0], 0, 0].astype(np.float64))
    # identical keys: uniform weights, the output is the mean of V
    p2 = pool.copy()
    p2[:, 0] = p2[0, 0, bt[0], 0, 0]
    o = O.attend_paged(shp, q.view(np.uint16), p2.view(np.uint16), bt, T, 0.125)
    t = np.arange(T)
    mean_v = p2[0, 1][bt[t // 16], 0, t % 16].astype(np.float64).mean(axis=0)
    assert np.allclose(o[0, 1], mean_v, rtol=1e-13, atol=1e-13)
    # a dominant key: the weight of every other token underflows relative to it
    p3 = pool.copy()
    p3[0, 0, bt[1], 0, 5] = (q[0, 0] * 100).astype(np.float16)
    o = O.attend_paged(shp, q.view(np.uint16), p3.view(np.uint16), bt, T, 1.0)
    assert np.allclose(o[0, 0], p3[0, 1, bt[1], 0, 5].astype(np.float64), rtol=1e-9, atol=1e-9)


def test_block_placement_does_not_matter():
    rng = np.random.default_rng(5)
    L, H, D, T = 1, 2, 64, 70
    pool, bt = pool_and_table(rng, L, H, D, T, extra=6)
    q = rng.standard_normal((L, 4, D)).astype(np.float16)
    shp = O.shape(L, H, D, T, 64)
    o1 = O.attend_paged(shp, q.view(np.uint16), pool.view(np.uint16), bt, T, 0.1)
    # move every logical block to another physical block
    bt2 = np.roll(np.setdiff1d(np.arange(pool.shape[2]), []), 2)[:len(bt)].astype(np.int32)
    pool2 = np.zeros_like(pool)
    pool2[:, :, bt2] = pool[:, :, bt]
    o2 = O.attend_paged(shp, q.view(np.uint16), pool2.view(np.uint16), bt2, T, 0.1)
    assert np.array_equal(o1, o2)


def test_grouped_heads_share_their_kv_head():
    rng = np.random.default_rng(6)
    L, H, D, T, G = 1, 2, 64, 50, 3
    pool, bt = pool_and_table(rng, L, H, D, T)
    q = np.repeat(rng.standard_normal((L, 1, D)).astype(np.float16), H * G, axis=1)
    shp = O.shape(L, H, D, T, 64)
    o = O.attend_paged(shp, q.view(np.uint16), pool.view(np.uint16), bt, T, 0.1)
    assert np.array_equal(o[0, 0], o[0, G - 1]) and np.array_equal(o[0, G], o[0, 2 * G - 1])
    assert not np.array_equal(o[0, 0], o[0, G])


def test_bf16_elements():
    import torch
    rng = np.random.default_rng(7)
    L, H, D, T = 1, 2, 64, 90
    pool32, bt = pool_and_table(rng, L, H, D, T, dtype=np.float32)
    q32 = rng.standard_normal((L, 4, D)).astype(np.float32)
    to_bits = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    to_f64 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    pb, qb = to_bits(pool32), to_bits(q32)
    shp = O.shape(L, H, D, T, 64, O.BF16)
    o = O.attend_paged(shp, qb, pb, bt, T, 0.125)
    ref = numpy_attend(to_f64(qb), to_f64(pb), bt, T, 0.125, 2)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_invalid_arguments():
    rng = np.random.default_rng(8)
    pool, bt = pool_and_table(rng, 1, 1, 64, 20)
    q = np.zeros((1, 1, 64), dtype=np.uint16)
    shp = O.shape(1, 1, 64, 20, 64)
    with pytest.raises(RuntimeError):
        O.attend_paged(shp, q, pool.view(np.uint16), bt, 0, 1.0)
    bad = bt.copy()
    bad[1] = pool.shape[2]
    with pytest.raises(RuntimeError):
        O.attend_paged(shp, q, pool.view(np.uint16), bad, 20, 1.0)
