"""Torch-side plumbing around the C ABI: allocates device buffers with torch
and calls the binding. No codec arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import cg as C


def shape_of(cfg, tokens=None, dtype=C.CG_DTYPE_F16) -> C.cg_shape:
    return C.shape(cfg.layers, cfg.kv_heads, cfg.head_dim,
                   cfg.tokens if tokens is None else tokens, cfg.chunk_tokens, dtype)


def torch_dtype(shp) -> torch.dtype:
    return torch.bfloat16 if shp.dtype == C.CG_DTYPE_BF16 else torch.float16


def level_of(lv) -> C.Level:
    return C.Level(lv.level_id, lv.layer_group, lv.steps)


def n_chunks(shp) -> int:
    return -(-shp.tokens // shp.chunk_tokens)


def _bytes(n, device):
    # 256-byte aligned by torch's caching allocator
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


class Codec:
    """Holds one shape and reusable workspaces."""

    def __init__(self, shp: C.cg_shape, device="cuda"):
        self.shp = shp
        self.device = torch.device(device)
        self.status = torch.zeros(4, dtype=torch.int32, device=self.device)
        self._ws = {}

    def _workspace(self, key, nbytes):
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            self._ws.pop(key, None)
            t = _bytes(nbytes, self.device)
            self._ws[key] = t
        return t

    def read_status(self) -> int:
        torch.cuda.current_stream().synchronize()
        return int(self.status[0].item())

    # -- tables -----------------------------------------------------------
    def tables_bytes(self, level: C.Level) -> int:
        return C.cg_tables_bytes(self.shp, level.n_groups)

    def format_bytes(self, level: C.Level) -> int:
        return C.cg_tables_format_bytes(self.shp, level.n_groups)

    def build_tables(self, x: torch.Tensor, level: C.Level, tables=None, stats=None, prof=None, flags=0):
        if tables is None:
            tables = _bytes(self.tables_bytes(level), self.device)
        ws = self._workspace("build", C.cg_build_workspace_bytes(self.shp, level.n_groups))
        C.cg_build_tables(self.shp, level, x, tables, ws, flags, stats, prof)
        return tables

    # -- encode -------------------------------------------------------------
    def encode(self, x, level, tables, chunk_begin=0, chunk_end=None, out=None, offsets=None,
               prof=None):
        """Records of chunks [chunk_begin, chunk_end) -> (out bytes, offsets u64 [n+1])."""
        if chunk_end is None:
            chunk_end = n_chunks(self.shp)
        n = chunk_end - chunk_begin
        if out is None:
            out = _bytes(C.cg_encode_bound(self.shp, chunk_begin, chunk_end), self.device)
        if offsets is None:
            offsets = torch.zeros(n + 1, dtype=torch.int64, device=self.device)
        ws = self._workspace("encode", C.cg_encode_workspace_bytes(self.shp, chunk_begin, chunk_end))
        C.cg_encode(self.shp, level, tables, x, chunk_begin, chunk_end, out, offsets, ws, self.status,
                    prof)
        return out, offsets

    # -- decode -------------------------------------------------------------
    def make_refs(self, parts):
        """parts: list of (container bytes, offsets, chunk indices within it, table index)
        -> device array of cg_chunk_ref, one per listed chunk, in the given order."""
        rows = []
        for base, offsets, idx, table in parts:
            offs = offsets.detach().cpu().numpy().astype(np.uint64)
            for i in idx:
                rows.append((base.data_ptr() + int(offs[i]), int(offs[i + 1] - offs[i]), table))
        arr = np.zeros((len(rows), 3), dtype=np.uint64)
        for k, (p, b, t) in enumerate(rows):
            arr[k] = (p, b, t)
        return torch.from_numpy(arr.view(np.uint8).reshape(-1).copy()).to(self.device), len(rows)

    def refs_for(self, out, offsets, table=0):
        """Device-side refs for every record of one cg_encode call (no host sync)."""
        n = offsets.numel() - 1
        refs = torch.empty(n * C.REF_BYTES, dtype=torch.uint8, device=self.device)
        C.cg_make_refs(out, offsets, n, table, refs)
        return refs, n

    def decode(self, levels, tables, refs, n_refs, y=None, prof=None):
        if y is None:
            y = torch.empty((self.shp.layers, 2, self.shp.kv_heads, self.shp.tokens, self.shp.head_dim),
                            dtype=torch_dtype(self.shp), device=self.device)
        C.cg_decode(self.shp, levels, tables, refs, n_refs, y, self.status, prof)
        return y

    def attend_paged(self, q, pool, block_table, n_tokens, scale, o=None, prof=None):
        """Attention of one new token per layer over the paged cache:
        q [layers][q_heads][head_dim] of the shape's element type -> fp32 o."""
        L, Hq, D = q.shape
        if o is None:
            o = torch.empty((L, Hq, D), dtype=torch.float32, device=self.device)
        ws = self._workspace("attend", C.cg_attend_workspace_bytes(self.shp, Hq, n_tokens))
        C.cg_attend_paged(self.shp, Hq, q, pool, pool.shape[2], block_table, n_tokens, scale, o, ws,
                          self.status, prof)
        return o

    def decode_paged(self, levels, tables, refs, n_refs, pool, block_table, prof=None):
        C.cg_decode_paged(self.shp, levels, tables, refs, n_refs, pool, pool.shape[2], block_table,
                          self.status, prof)
        return pool
