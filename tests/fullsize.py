"""Sampled parity at the workloads' full sizes: the oracle computes single
tables and single groups one by one; decoded slices are compared with numpy's
dequant(quant(x)). Shared by the GPU tests."""
import numpy as np

from oracle import oracle as O
from tests import npref


def check_tables(cfg, lvd, X, blob_gpu, rng, n=6):
    oshp = O.shape_of(cfg)
    G = len(lvd.steps)
    f = O.table_f(blob_gpu, oshp, G)
    for _ in range(n):
        g = int(rng.integers(G))
        kv, h, d = int(rng.integers(2)), int(rng.integers(cfg.kv_heads)), int(rng.integers(cfg.head_dim))
        counts, _ = O.table_counts(oshp, lvd.layer_group, lvd.steps, X, g, kv, h, d)
        assert np.array_equal(f[g, kv, h, d], O.normalize(counts)), (g, kv, h, d)


def record_group(rec, gpc, gi):
    ds = int(rec[44:48].view(np.uint32)[0])
    go = rec[64:64 + 8 * (gpc + 1)].view(np.uint64)
    nw = rec[64 + 8 * (gpc + 1):64 + 8 * (gpc + 1) + 4 * gpc].view(np.uint32)
    return rec[ds + int(go[gi]):ds + int(go[gi]) + 2 * int(nw[gi])].view(np.uint16)


def check_groups(cfg, X, blob_gpu, out_bytes, offs, rng, n=4, chunks=None):
    oshp = O.shape_of(cfg)
    S = cfg.head_dim // 64
    gpc = cfg.layers * 2 * cfg.kv_heads * S
    chunks = list(range(cfg.n_chunks)) if chunks is None else chunks
    picks = [chunks[-1]] + [chunks[int(rng.integers(len(chunks)))] for _ in range(n - 1)]
    for c in picks:
        l, kv, h, j = (int(rng.integers(cfg.layers)), int(rng.integers(2)),
                       int(rng.integers(cfg.kv_heads)), int(rng.integers(S)))
        w = O.encode_group(oshp, blob_gpu, X, c, l, kv, h, j)
        k = chunks.index(c)
        rec = out_bytes(int(offs[k]), int(offs[k + 1]))
        assert rec[:4].tobytes() == b"CGCK" and int(rec[8:12].view(np.uint32)[0]) == c
        got = record_group(rec, gpc, ((l * 2 + kv) * cfg.kv_heads + h) * S + j)
        assert np.array_equal(got, w), (c, l, kv, h, j)


def check_slices(cfg, layer_steps, X, y_slice, rng, n=4, tokens=None):
    """y_slice(l, kv, h) -> uint16 [T][D] of the decoded cache."""
    for _ in range(n):
        l, kv, h = int(rng.integers(cfg.layers)), int(rng.integers(2)), int(rng.integers(cfg.kv_heads))
        st = layer_steps[l]
        ref = npref.dequantize(npref.quantize(X[l, kv, h], st), st).view(np.uint16)
        got = y_slice(l, kv, h)
        if tokens is not None:
            ref = ref[tokens]
            got = got[tokens]
        assert np.array_equal(got, ref), (l, kv, h, int(np.count_nonzero(got != ref)))
