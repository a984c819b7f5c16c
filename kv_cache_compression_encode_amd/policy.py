"""Per-chunk level policies over the multi-level container, composed from the
C-ABI calls (no codec arithmetic here):

- bandwidth-adaptive selection ("CacheGen实战" 2.2): every chunk is encoded
  at all levels; the sender picks one record per chunk from the bandwidth of
  its transfer (cg_select_level) and the receiver streams the picked records
  into a paged cache (cg_stream_decode_paged);
- recency-based allocation (the CacheGen technical analysis, dynamic bit
  allocation): each chunk is encoded once, at the level its distance from
  the newest chunk selects (cg_recency_levels), and decoded as a level mix.
"""
from __future__ import annotations

import numpy as np
import torch

from . import cg as C
from .codec import Codec


def levels_for_bandwidth(trace_gbps) -> np.ndarray:
    """Level index per chunk from the bandwidth (Gbit/s) of its transfer."""
    return np.array([C.cg_select_level(float(b)) for b in trace_gbps], dtype=np.int32)


def pick_records(containers, levels):
    """containers[k] = (bytes uint8 [N], offsets uint64 [n_chunks + 1]) of level
    k; returns (records uint8, offsets uint64 [n + 1], table_of_record int32)
    with chunk c's record taken from level levels[c]."""
    parts, offs, tor = [], [0], []
    for c, k in enumerate(levels):
        data, o = containers[int(k)]
        rec = data[int(o[c]):int(o[c + 1])]
        parts.append(rec)
        offs.append(offs[-1] + rec.size)
        tor.append(int(k))
    return np.concatenate(parts), np.array(offs, dtype=np.uint64), np.array(tor, dtype=np.int32)


def transfer_seconds(offsets, trace_gbps) -> float:
    """Time to send record c at trace_gbps[c] Gbit/s, summed over chunks."""
    sizes = np.diff(np.asarray(offsets, dtype=np.float64))
    return float(np.sum(sizes * 8.0 / (np.asarray(trace_gbps, dtype=np.float64) * 1e9)))


def stream_into_pool(codec: Codec, levels, tables, records, offsets, table_of_record, pool, block_table,
                     stream=None, copy_stream=None):
    """Streams host records into the paged pool (pinned copy of `records`
    made here); returns when all work is enqueued on `stream`."""
    host = torch.from_numpy(records).pin_memory()
    largest = int(np.diff(offsets).max())
    staging = torch.empty(2 * largest + 512, dtype=torch.uint8, device=codec.device)
    refs = torch.empty(2 * C.REF_BYTES, dtype=torch.uint8, device=codec.device)
    C.cg_stream_decode_paged(codec.shp, levels, tables, host, offsets, table_of_record, len(offsets) - 1,
                             staging, refs, pool, pool.shape[2], block_table, codec.status,
                             stream=stream, copy_stream=copy_stream)
    return host, staging, refs  # keep alive until the stream has run


def recency_segments(levels):
    """Maximal runs of equal level: [(chunk_begin, chunk_end, level)]."""
    segs, b = [], 0
    for c in range(1, len(levels) + 1):
        if c == len(levels) or levels[c] != levels[b]:
            segs.append((b, c, int(levels[b])))
            b = c
    return segs


def encode_by_level(codec: Codec, x, levels_objs, tables, chunk_levels):
    """Encodes each run of chunks at its level; returns the segments as
    (chunk_begin, chunk_end, level, out, offsets)."""
    segs = []
    for b, e, k in recency_segments(chunk_levels):
        out, offs = codec.encode(x, levels_objs[k], tables[k], chunk_begin=b, chunk_end=e)
        segs.append((b, e, k, out, offs))
    return segs


def refs_for_segments(codec: Codec, segs):
    """Device refs of every chunk, in chunk order, each naming its level."""
    parts = [(out, offs, range(e - b), k) for b, e, k, out, offs in segs]
    return codec.make_refs(parts)
