"""ctypes binding of libcg.so: one Python function per C entry point, same
names, argument marshalling only (every step of the codec runs in the HIP
kernels). Tensors are torch device tensors; streams default to torch's
current stream. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcg.so")

CG_OK = 0
CG_ERR_INVALID_ARG = -1
CG_ERR_UNSUPPORTED = -2
CG_ERR_CAPACITY = -3
CG_ERR_HIP = -4
CG_ERR_CORRUPT = -5
CG_ERR_TABLE = -6
CG_DTYPE_F16 = 0
CG_DTYPE_BF16 = 1
CG_TABLES_ROBUST = 1
CG_NOALLOC_SCRATCH_BYTES = 32 << 20


class CgError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %d (%s)" % (fn, code, status_string(code)))


class cg_shape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class cg_level(ctypes.Structure):
    _fields_ = [("level_id", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("layer_group", ctypes.c_void_p), ("step", ctypes.c_void_p)]


class cg_chunk_ref(ctypes.Structure):
    _fields_ = [("record", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("table", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class cg_profile(ctypes.Structure):
    _fields_ = [("main_begin", ctypes.c_void_p), ("main_end", ctypes.c_void_p)]


REF_BYTES = ctypes.sizeof(cg_chunk_ref)  # 24

_hip = None


def hip():
    """The HIP runtime (already loaded by torch), for events only."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip = h
    return _hip


class KernelTimer:
    """Two HIP events a call records around its main kernel (cg_profile)."""

    def __init__(self):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        if hip().hipEventCreate(ctypes.byref(a)) or hip().hipEventCreate(ctypes.byref(b)):
            raise RuntimeError("hipEventCreate failed")
        self.c = cg_profile(a.value, b.value)

    def elapsed_ms(self) -> float:
        hip().hipEventSynchronize(self.c.main_end)
        ms = ctypes.c_float()
        if hip().hipEventElapsedTime(ctypes.byref(ms), self.c.main_begin, self.c.main_end):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            hip().hipEventDestroy(self.c.main_begin)
            hip().hipEventDestroy(self.c.main_end)
        except Exception:
            pass


def _prof(p):
    return ctypes.byref(p.c) if p is not None else None


class Level:
    """A cg_level whose host arrays stay alive with it."""

    def __init__(self, level_id: int, layer_group, steps):
        self.lg = np.ascontiguousarray(layer_group, dtype=np.uint8)
        self.steps = np.ascontiguousarray(steps, dtype=np.float32)
        self.level_id = int(level_id)
        self.n_groups = len(self.steps)
        self.c = cg_level(self.level_id, self.n_groups, self.lg.ctypes.data, self.steps.ctypes.data)


def shape(layers, kv_heads, head_dim, tokens, chunk_tokens, dtype=CG_DTYPE_F16) -> cg_shape:
    return cg_shape(int(layers), int(kv_heads), int(head_dim), int(chunk_tokens), int(tokens), int(dtype), 0)


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError("libcg.so is not built (%s); run python -m kv_cache_compression_encode_amd.build" % LIB)
    L = ctypes.CDLL(LIB)
    P, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    sp, lp = ctypes.POINTER(cg_shape), ctypes.POINTER(cg_level)
    pp = ctypes.POINTER(cg_profile)
    sigs = {
        "cg_version": (i32, []),
        "cg_status_string": (ctypes.c_char_p, [i32]),
        "cg_tables_bytes": (sz, [sp, i32]),
        "cg_tables_format_bytes": (sz, [sp, i32]),
        "cg_build_workspace_bytes": (sz, [sp, i32]),
        "cg_build_tables": (i32, [sp, lp, P, P, P, sz, ctypes.c_uint32, P, pp, P]),
        "cg_build_tables_noalloc": (i32, [sp, lp, P, P, ctypes.c_uint32, P, pp, P]),
        "cg_encode_bound": (sz, [sp, i64, i64]),
        "cg_encode_workspace_bytes": (sz, [sp, i64, i64]),
        "cg_encode": (i32, [sp, lp, P, P, i64, i64, P, u64, P, P, sz, P, pp, P]),
        "cg_make_refs": (i32, [P, P, i32, i32, P, P]),
        "cg_decode": (i32, [sp, i32, lp, P, P, i32, P, P, pp, P]),
        "cg_decode_paged": (i32, [sp, i32, lp, P, P, i32, P, i64, P, P, pp, P]),
        "cg_decode_plan": (i32, [sp, i32, lp, i32, i32, P]),
        "cg_copy": (i32, [P, P, u64, P]),
        "cg_select_level": (i32, [ctypes.c_double]),
        "cg_recency_levels": (i32, [i64, i64, i64, P]),
        "cg_stream_decode_paged": (i32, [sp, i32, lp, P, P, P, P, i32, P, u64, P, P, i64, P, P, P, P]),
        "cg_attend_workspace_bytes": (sz, [sp, i32, i64]),
        "cg_attend_paged": (i32, [sp, i32, P, P, i64, P, i64, ctypes.c_float, P, P, sz, P, pp, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


EXPORTS = ("cg_version", "cg_status_string", "cg_tables_bytes", "cg_tables_format_bytes",
           "cg_build_workspace_bytes", "cg_build_tables", "cg_build_tables_noalloc", "cg_encode_bound",
           "cg_encode_workspace_bytes", "cg_encode", "cg_make_refs", "cg_decode",
           "cg_decode_paged", "cg_decode_plan", "cg_stream_decode_paged", "cg_copy", "cg_select_level",
           "cg_recency_levels", "cg_attend_workspace_bytes", "cg_attend_paged")


def status_string(code: int) -> str:
    try:
        return lib().cg_status_string(int(code)).decode()
    except ImportError:
        return "?"


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, rc):
    if rc != CG_OK:
        raise CgError(fn, rc)


# ---- one wrapper per entry point -------------------------------------------
def cg_version() -> int:
    return lib().cg_version()


def cg_status_string(code: int) -> str:
    return status_string(code)


def cg_tables_bytes(shp: cg_shape, n_groups: int) -> int:
    return lib().cg_tables_bytes(ctypes.byref(shp), n_groups)


def cg_tables_format_bytes(shp: cg_shape, n_groups: int) -> int:
    return lib().cg_tables_format_bytes(ctypes.byref(shp), n_groups)


def cg_build_workspace_bytes(shp: cg_shape, n_groups: int) -> int:
    return lib().cg_build_workspace_bytes(ctypes.byref(shp), n_groups)


def cg_build_tables(shp, level: Level, x, tables, ws, flags=0, stats=None, prof=None, stream=None):
    rc = lib().cg_build_tables(ctypes.byref(shp), ctypes.byref(level.c), _ptr(x), _ptr(tables),
                               _ptr(ws), ws.numel() * ws.element_size(), int(flags), _ptr(stats),
                               _prof(prof), _stream(stream))
    _check("cg_build_tables", rc)


def cg_build_tables_noalloc(shp, level: Level, x, tables, flags=0, stats=None, prof=None, stream=None):
    rc = lib().cg_build_tables_noalloc(ctypes.byref(shp), ctypes.byref(level.c), _ptr(x), _ptr(tables),
                                       int(flags), _ptr(stats), _prof(prof), _stream(stream))
    _check("cg_build_tables_noalloc", rc)


def cg_encode_bound(shp, chunk_begin, chunk_end) -> int:
    return lib().cg_encode_bound(ctypes.byref(shp), chunk_begin, chunk_end)


def cg_encode_workspace_bytes(shp, chunk_begin, chunk_end) -> int:
    return lib().cg_encode_workspace_bytes(ctypes.byref(shp), chunk_begin, chunk_end)


def cg_encode(shp, level: Level, tables, x, chunk_begin, chunk_end, out, chunk_offsets, ws, status,
              prof=None, stream=None):
    rc = lib().cg_encode(ctypes.byref(shp), ctypes.byref(level.c), _ptr(tables), _ptr(x),
                         chunk_begin, chunk_end, _ptr(out), out.numel() * out.element_size(),
                         _ptr(chunk_offsets), _ptr(ws), ws.numel() * ws.element_size(), _ptr(status),
                         _prof(prof), _stream(stream))
    _check("cg_encode", rc)


def cg_make_refs(base, offsets, n, table, refs, stream=None):
    rc = lib().cg_make_refs(_ptr(base), _ptr(offsets), int(n), int(table), _ptr(refs), _stream(stream))
    _check("cg_make_refs", rc)


def _levels_and_tables(levels, tables):
    arr = (cg_level * len(levels))(*[lv.c for lv in levels])
    tp = (ctypes.c_void_p * len(tables))(*[_ptr(t) for t in tables])
    return arr, tp


def cg_decode(shp, levels, tables, refs, n_refs, y, status, prof=None, stream=None):
    arr, tp = _levels_and_tables(levels, tables)
    rc = lib().cg_decode(ctypes.byref(shp), len(levels), arr, tp, _ptr(refs), int(n_refs), _ptr(y),
                         _ptr(status), _prof(prof), _stream(stream))
    _check("cg_decode", rc)


def cg_decode_paged(shp, levels, tables, refs, n_refs, pool, num_blocks, block_table, status,
                    prof=None, stream=None):
    arr, tp = _levels_and_tables(levels, tables)
    rc = lib().cg_decode_paged(ctypes.byref(shp), len(levels), arr, tp, _ptr(refs), int(n_refs),
                               _ptr(pool), int(num_blocks), _ptr(block_table), _ptr(status),
                               _prof(prof), _stream(stream))
    _check("cg_decode_paged", rc)


def cg_decode_plan(shp, levels, n_refs, compute_units=0):
    """(records_per_block, split, records_per_block2) of the decode dispatch
    over compute_units compute units (0: the current device's)."""
    arr = (cg_level * len(levels))(*[lv.c for lv in levels])
    out = np.zeros(3, dtype=np.int32)
    _check("cg_decode_plan", lib().cg_decode_plan(ctypes.byref(shp), len(levels), arr, int(n_refs),
                                                  int(compute_units), out.ctypes.data))
    return int(out[0]), int(out[1]), int(out[2])


def cg_attend_workspace_bytes(shp, q_heads, n_tokens) -> int:
    return lib().cg_attend_workspace_bytes(ctypes.byref(shp), int(q_heads), int(n_tokens))


def cg_attend_paged(shp, q_heads, q, pool, num_blocks, block_table, n_tokens, scale, o, ws, status,
                    prof=None, stream=None):
    rc = lib().cg_attend_paged(ctypes.byref(shp), int(q_heads), _ptr(q), _ptr(pool), int(num_blocks),
                               _ptr(block_table), int(n_tokens), float(scale), _ptr(o), _ptr(ws),
                               ws.numel() * ws.element_size(), _ptr(status), _prof(prof), _stream(stream))
    _check("cg_attend_paged", rc)


def cg_stream_decode_paged(shp, levels, tables, records_host, offsets_host, table_of_record, n_records,
                           staging, refs, pool, num_blocks, block_table, status, stream=None,
                           copy_stream=None):
    """records_host: pinned torch uint8 tensor; offsets_host: numpy uint64 [n+1];
    table_of_record: numpy int32 [n] or None."""
    arr, tp = _levels_and_tables(levels, tables)
    offs = np.ascontiguousarray(offsets_host, dtype=np.uint64)
    tor = None if table_of_record is None else np.ascontiguousarray(table_of_record, dtype=np.int32)
    rc = lib().cg_stream_decode_paged(
        ctypes.byref(shp), len(levels), arr, tp, _ptr(records_host), offs.ctypes.data,
        None if tor is None else tor.ctypes.data, int(n_records), _ptr(staging),
        staging.numel() * staging.element_size(), _ptr(refs), _ptr(pool), int(num_blocks),
        _ptr(block_table), _ptr(status), _stream(stream), _stream(copy_stream))
    _check("cg_stream_decode_paged", rc)


def cg_copy(dst, src, nbytes, stream=None):
    _check("cg_copy", lib().cg_copy(_ptr(dst), _ptr(src), int(nbytes), _stream(stream)))


def cg_select_level(bandwidth_gbps: float) -> int:
    return lib().cg_select_level(float(bandwidth_gbps))


def cg_recency_levels(n_chunks: int, near_chunks: int, far_chunks: int) -> np.ndarray:
    out = np.zeros(max(int(n_chunks), 1), dtype=np.int32)
    _check("cg_recency_levels", lib().cg_recency_levels(int(n_chunks), int(near_chunks), int(far_chunks),
                                                        out.ctypes.data))
    return out[:int(n_chunks)]
