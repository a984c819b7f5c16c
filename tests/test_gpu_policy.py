"""Per-chunk level policies end to end on the GPU (the long-context workload
cut to 8 chunks): bandwidth-adaptive record selection streamed into a paged
cache, and recency-based encoding decoded as a level mix. Every decoded
value is compared with numpy's dequant(quant(x)) at its chunk's level, and
every byte of the picked records with the oracle's encoding at that level."""
import dataclasses

import numpy as np
import pytest

from tests import fullsize as F
from tests import gpu_util as U

torch = U.torch
from kv_cache_compression_encode_amd import cg as C  # noqa: E402
from kv_cache_compression_encode_amd import policy as P  # noqa: E402
from kv_cache_compression_encode_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu
TOKENS = 8 * 1536 - 500  # 8 chunks, the last one short


def workload():
    cfg = dataclasses.replace(synth.CONFIGS["long"], tokens=TOKENS)
    return cfg, synth.generate(cfg)


def check_by_chunk(cfg, X, levels, y_layer):
    """Every element of the decoded cache at its chunk's level."""
    token_steps = []
    for c in range(cfg.n_chunks):
        lvd = cfg.levels[int(levels[c])]
        t = slice(c * cfg.chunk_tokens, min((c + 1) * cfg.chunk_tokens, cfg.tokens))
        token_steps.append((t, [lvd.steps[g] for g in lvd.layer_group]))
    F.check_all_decoded(cfg, X, None, y_layer, token_steps=token_steps)


def test_bandwidth_adaptive_stream():
    U.need_gpu()
    cfg, X = workload()
    cd = U.codec.Codec(U.codec.shape_of(cfg))
    x = U.to_dev(X)
    lvs, tabs, conts = [], [], []
    for lvd in cfg.levels:
        lv = U.codec.level_of(lvd)
        tables = cd.build_tables(x, lv)
        out, offs = cd.encode(x, lv, tables)
        assert cd.read_status() == 0
        o = offs.cpu().numpy().astype(np.uint64)
        lvs.append(lv)
        tabs.append(tables)
        conts.append((U.u8(out[:int(o[-1])]), o))
    trace = synth.bandwidth_trace(cfg.n_chunks, seed=31)  # visits all three bands
    levels = P.levels_for_bandwidth(trace)
    print("trace", np.round(trace, 2).tolist(), "levels", levels.tolist(), flush=True)
    assert set(levels.tolist()) == {0, 1, 2}
    recs, offs, tor = P.pick_records(conts, levels)
    bt = synth.block_table(cfg)
    pool = torch.zeros((cfg.layers, 2, len(bt), cfg.kv_heads, 16, cfg.head_dim), dtype=torch.float16,
                       device="cuda")
    copy_stream = torch.cuda.Stream()
    keep = P.stream_into_pool(cd, lvs, tabs, recs, offs, tor, pool, torch.from_numpy(bt).cuda(),
                              copy_stream=copy_stream)
    torch.cuda.synchronize()
    del keep
    assert cd.read_status() == 0
    pool_h = pool.cpu().view(torch.int16).numpy().view(np.uint16)
    del pool
    T, H, D = cfg.tokens, cfg.kv_heads, cfg.head_dim

    def y_layer(l):
        blocks = pool_h[l][:, bt]  # [2][blocks][H][16][D]
        return blocks.transpose(0, 2, 1, 3, 4).reshape(2, H, -1, D)[:, :, :T]

    check_by_chunk(cfg, X, levels, y_layer)
    # the picked records are the oracle's, at each chunk's level
    for k in range(len(cfg.levels)):
        cs = [c for c in range(cfg.n_chunks) if int(levels[c]) == k]
        blob = U.u8(tabs[k][:cd.format_bytes(lvs[k])])
        F.check_all_records(cfg, X, blob, lambda i, cs=cs: recs[int(offs[cs[i]]):int(offs[cs[i] + 1])], cs)
    assert P.transfer_seconds(offs, trace) > 0


def test_recency_levels_mix():
    U.need_gpu()
    cfg, X = workload()
    cd = U.codec.Codec(U.codec.shape_of(cfg))
    x = U.to_dev(X)
    lvs = [U.codec.level_of(lvd) for lvd in cfg.levels]
    tabs = [cd.build_tables(x, lv) for lv in lvs]
    levels = C.cg_recency_levels(cfg.n_chunks, 2, 5)
    assert levels.tolist() == [2, 2, 2, 1, 1, 1, 0, 0]
    segs = P.encode_by_level(cd, x, lvs, tabs, levels)
    assert cd.read_status() == 0
    refs, n = P.refs_for_segments(cd, segs)
    assert n == cfg.n_chunks
    y = cd.decode(lvs, tabs, refs, n)
    assert cd.read_status() == 0
    y_h = y.cpu().view(torch.int16).numpy().view(np.uint16)
    check_by_chunk(cfg, X, levels, lambda l: y_h[l])
    # every segment's records are the oracle's at that level
    for b, e, k, out, offs in segs:
        blob = U.u8(tabs[k][:cd.format_bytes(lvs[k])])
        o = offs.cpu().numpy()
        F.check_all_records(cfg, X, blob, lambda i, out=out, o=o: U.u8(out[int(o[i]):int(o[i + 1])]),
                            list(range(b, e)))
