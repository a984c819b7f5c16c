"""Whole-tensor parity at the workloads' full sizes, shared by the GPU tests.

* tables: the oracle builds the tables of every (layer group, head) slice of
  the tensor on its own (a sub-tensor of that group's layers and that head;
  the tables of a (group, K|V, head, dim) depend on nothing else) and every
  table of the GPU blob is compared with it;
* records: the oracle encodes every chunk with the GPU's tables and every
  byte of every record is compared;
* decoded elements: every element is compared with numpy's dequant(quant(x))
  (tests/npref.py, pinned against the oracle on small shapes).

The oracle is single-threaded C called through ctypes, which releases the
GIL, so independent chunks and slices run on a thread pool sized to the host
share of one GPU (16 cores)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import oracle as O
from tests import npref

WORKERS = max(1, min(16, os.cpu_count() or 1))


def pool_map(fn, items):
    with ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, items))


def layers_of(lvd, g):
    return [l for l in range(len(lvd.layer_group)) if lvd.layer_group[l] == g]


def check_all_tables(cfg, lvd, X, blob_gpu, dtype=O.F16, robust=False, tokens=None):
    """Every table f[g][kv][h][d] of blob_gpu equals the oracle's tables of the
    (layers of g, head h) sub-tensor of X (its first `tokens` tokens)."""
    T = X.shape[3] if tokens is None else tokens
    G = len(lvd.steps)
    oshp = O.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, T, cfg.chunk_tokens, dtype)
    f_gpu = O.table_f(blob_gpu, oshp, G)

    def one(gh):
        g, h = gh
        ls = layers_of(lvd, g)
        if not ls:
            return 0
        sub = np.ascontiguousarray(X[ls][:, :, h:h + 1, :T, :])
        sshp = O.shape(len(ls), 1, cfg.head_dim, T, cfg.chunk_tokens, dtype)
        blob, _ = O.build_tables(sshp, lvd.level_id, [0] * len(ls), [lvd.steps[g]], sub,
                                 flags=O.TABLES_ROBUST if robust else 0)
        want = O.table_f(blob, sshp, 1)[0][:, 0]  # [2][D][256]
        return int(np.count_nonzero(f_gpu[g, :, h] != want))

    bad = pool_map(one, [(g, h) for g in range(G) for h in range(cfg.kv_heads)])
    assert sum(bad) == 0, "tables differ in %d entries" % sum(bad)
    return G * 2 * cfg.kv_heads * cfg.head_dim


def check_all_records(cfg, X, blob_gpu, rec_bytes, chunks, dtype=O.F16):
    """Every byte of the record of each chunk in `chunks` (rec_bytes(k) ->
    uint8 record of chunks[k]) equals the oracle's encoding of that chunk."""
    oshp = O.shape(cfg.layers, cfg.kv_heads, cfg.head_dim, X.shape[3], cfg.chunk_tokens, dtype)
    recs = [rec_bytes(k) for k in range(len(chunks))]

    def one(k):
        want = O.encode_chunk(oshp, blob_gpu, X, chunks[k])
        got = recs[k]
        if len(got) != len(want):
            return (chunks[k], "length %d != %d" % (len(got), len(want)))
        n = int(np.count_nonzero(got != want))
        return (chunks[k], n) if n else None

    bad = [b for b in pool_map(one, range(len(chunks))) if b]
    assert not bad, bad[:4]
    return sum(len(r) for r in recs)


def check_all_decoded(cfg, X, layer_steps, y_layer, dtype=0, token_steps=None):
    """Every element of the decoded cache equals numpy's dequant(quant(x)).
    y_layer(l) -> uint16 [2][H][T][D] of layer l. token_steps (optional):
    list of (token slice, per-layer steps) when chunks use different levels."""
    parts = token_steps or [(slice(None), layer_steps)]

    def one(l):
        got = y_layer(l)
        bad = 0
        for t, steps in parts:
            st = steps[l]
            if dtype == 0:
                ref = npref.dequantize(npref.quantize(X[l][:, :, t], st), st).view(np.uint16)
            else:
                ref = npref.dequantize_bits(npref.quantize_bits(X[l][:, :, t], st, 1), st, 1)
            bad += int(np.count_nonzero(got[:, :, t] != ref))
        return bad

    bad = pool_map(one, range(cfg.layers))
    assert sum(bad) == 0, "decoded elements differ: %d (per layer %s)" % (sum(bad), bad)
    return cfg.layers * sum(X[0][:, :, t].size for t, _ in parts)


def record_group(rec, gpc, gi):
    ds = int(rec[44:48].view(np.uint32)[0])
    go = rec[64:64 + 8 * (gpc + 1)].view(np.uint64)
    nw = rec[64 + 8 * (gpc + 1):64 + 8 * (gpc + 1) + 4 * gpc].view(np.uint32)
    return rec[ds + int(go[gi]):ds + int(go[gi]) + 2 * int(nw[gi])].view(np.uint16)
