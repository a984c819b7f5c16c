"""ctypes binding of the plain C oracle (cg_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the GPU smoke check and the CPU
baseline of bench.py. The product path (the HIP library and its binding)
never imports this module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_CORRUPT, ERR_TABLE = 0, -1, -2, -3, -5, -6
F16, BF16 = 0, 1          # element types
TABLES_ROBUST = 1         # cgo_build_tables flag

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, no SIMD intrinsics)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


class Shape(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        sp = ctypes.POINTER(Shape)
        L.cgo_half_to_float.argtypes = [ctypes.c_uint16]
        L.cgo_half_to_float.restype = ctypes.c_float
        L.cgo_float_to_half.argtypes = [ctypes.c_float]
        L.cgo_float_to_half.restype = ctypes.c_uint16
        L.cgo_quantize.argtypes = [ctypes.c_uint16, ctypes.c_float, P, P]
        L.cgo_quantize.restype = i32
        L.cgo_dequantize.argtypes = [i32, ctypes.c_float]
        L.cgo_dequantize.restype = ctypes.c_uint16
        L.cgo_quantize_dt.argtypes = [ctypes.c_int, ctypes.c_uint16, ctypes.c_float, P, P]
        L.cgo_quantize_dt.restype = i32
        L.cgo_dequantize_dt.argtypes = [ctypes.c_int, i32, ctypes.c_float]
        L.cgo_dequantize_dt.restype = ctypes.c_uint16
        L.cgo_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.cgo_bf16_to_float.restype = ctypes.c_float
        L.cgo_float_to_bf16.argtypes = [ctypes.c_float]
        L.cgo_float_to_bf16.restype = ctypes.c_uint16
        L.cgo_wrap16.argtypes = [i32]
        L.cgo_wrap16.restype = i32
        L.cgo_normalize.argtypes = [P, P]
        L.cgo_normalize.restype = None
        L.cgo_normalize_robust.argtypes = [P, P]
        L.cgo_normalize_robust.restype = None
        L.cgo_table_counts.argtypes = [sp, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, P, P]
        L.cgo_table_counts.restype = None
        L.cgo_tables_f_offset.argtypes = [sp, i32]
        L.cgo_tables_f_offset.restype = u64
        L.cgo_tables_format_bytes.argtypes = [sp, i32]
        L.cgo_tables_format_bytes.restype = u64
        L.cgo_build_tables.argtypes = [sp, i32, i32, P, P, P, ctypes.c_uint32, P, u64, P]
        L.cgo_build_tables.restype = ctypes.c_int
        L.cgo_group_word_bound.argtypes = [i64]
        L.cgo_group_word_bound.restype = i64
        L.cgo_encode_group_q.argtypes = [P, i64, P, ctypes.c_int, P, i64]
        L.cgo_encode_group_q.restype = i64
        L.cgo_decode_group_q.argtypes = [P, i64, i64, P, P]
        L.cgo_decode_group_q.restype = ctypes.c_int
        L.cgo_encode_group.argtypes = [sp, P, P, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, P, i64]
        L.cgo_encode_group.restype = i64
        L.cgo_record_data_start.argtypes = [sp]
        L.cgo_record_data_start.restype = u64
        L.cgo_record_bound.argtypes = [sp, i64]
        L.cgo_record_bound.restype = u64
        L.cgo_encode_chunk.argtypes = [sp, P, P, i64, P, u64]
        L.cgo_encode_chunk.restype = i64
        L.cgo_decode_chunk.argtypes = [sp, P, P, u64, P]
        L.cgo_decode_chunk.restype = ctypes.c_int
        L.cgo_decode_chunk_paged.argtypes = [sp, P, P, u64, P, i64, P]
        L.cgo_decode_chunk_paged.restype = ctypes.c_int
        L.cgo_attend_paged.argtypes = [sp, i32, P, P, i64, P, i64, ctypes.c_double, P]
        L.cgo_attend_paged.restype = ctypes.c_int
        L.cgo_half_to_float_array.argtypes = [P, i64, P]
        L.cgo_float_to_half_array.argtypes = [P, i64, P]
        L.cgo_quantize_array.argtypes = [P, i64, ctypes.c_float, P]
        L.cgo_dequantize_array.argtypes = [P, i64, ctypes.c_float, P]
        L.cgo_bf16_to_float_array.argtypes = [P, i64, P]
        L.cgo_float_to_bf16_array.argtypes = [P, i64, P]
        L.cgo_quantize_array_dt.argtypes = [ctypes.c_int, P, i64, ctypes.c_float, P]
        L.cgo_dequantize_array_dt.argtypes = [ctypes.c_int, P, i64, ctypes.c_float, P]
        for fn in ("cgo_half_to_float_array", "cgo_float_to_half_array", "cgo_quantize_array",
                   "cgo_dequantize_array", "cgo_bf16_to_float_array", "cgo_float_to_bf16_array",
                   "cgo_quantize_array_dt", "cgo_dequantize_array_dt"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def shape(L, H, D, T, C, dtype=F16) -> Shape:
    return Shape(int(L), int(H), int(D), int(C), int(T), int(dtype), 0)


def shape_of(cfg) -> Shape:
    return shape(cfg.layers, cfg.kv_heads, cfg.head_dim, cfg.tokens, cfg.chunk_tokens,
                 getattr(cfg, "dtype", F16))


# ---- scalar helpers ------------------------------------------------------
def half_to_float(h: int) -> float:
    return lib().cgo_half_to_float(int(h))


def float_to_half(f: float) -> int:
    return lib().cgo_float_to_half(float(f))


def quantize(h: int, step: float):
    sat, nan_ = ctypes.c_int(0), ctypes.c_int(0)
    q = lib().cgo_quantize(int(h), float(step), ctypes.byref(sat), ctypes.byref(nan_))
    return q, sat.value, nan_.value


def dequantize(q: int, step: float) -> int:
    return lib().cgo_dequantize(int(q), float(step))


def quantize_dt(dtype: int, h: int, step: float):
    sat, nan_ = ctypes.c_int(0), ctypes.c_int(0)
    q = lib().cgo_quantize_dt(int(dtype), int(h), float(step), ctypes.byref(sat), ctypes.byref(nan_))
    return q, sat.value, nan_.value


def dequantize_dt(dtype: int, q: int, step: float) -> int:
    return lib().cgo_dequantize_dt(int(dtype), int(q), float(step))


def bf16_to_float(h: int) -> float:
    return lib().cgo_bf16_to_float(int(h))


def float_to_bf16(f: float) -> int:
    return lib().cgo_float_to_bf16(float(f))


def bf16_to_float_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().cgo_bf16_to_float_array(_p(h), h.size, _p(out))
    return out


def float_to_bf16_array(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().cgo_float_to_bf16_array(_p(f), f.size, _p(out))
    return out


def half_to_float_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().cgo_half_to_float_array(_p(h), h.size, _p(out))
    return out


def float_to_half_array(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().cgo_float_to_half_array(_p(f), f.size, _p(out))
    return out


def quantize_array(xh: np.ndarray, step: float, dtype: int = F16) -> np.ndarray:
    xh = np.ascontiguousarray(xh).view(np.uint16)
    out = np.empty(xh.shape, dtype=np.int32)
    lib().cgo_quantize_array_dt(int(dtype), _p(xh), xh.size, float(step), _p(out))
    return out


def dequantize_array(q: np.ndarray, step: float, dtype: int = F16) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int32)
    out = np.empty(q.shape, dtype=np.uint16)
    lib().cgo_dequantize_array_dt(int(dtype), _p(q), q.size, float(step), _p(out))
    return out


def wrap16(v: int) -> int:
    return lib().cgo_wrap16(int(v))


def normalize(counts, robust: bool = False) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    assert c.shape == (256,)
    f = np.zeros(256, dtype=np.uint16)
    (lib().cgo_normalize_robust if robust else lib().cgo_normalize)(_p(c), _p(f))
    return f


# ---- tables ---------------------------------------------------------------
def tables_format_bytes(shp: Shape, n_groups: int) -> int:
    return lib().cgo_tables_format_bytes(ctypes.byref(shp), n_groups)


def tables_f_offset(shp: Shape, n_groups: int) -> int:
    return lib().cgo_tables_f_offset(ctypes.byref(shp), n_groups)


def build_tables(shp: Shape, level_id: int, layer_group, steps, X: np.ndarray, flags: int = 0):
    lg = np.ascontiguousarray(layer_group, dtype=np.uint8)
    st = np.ascontiguousarray(steps, dtype=np.float32)
    G = len(st)
    n = tables_format_bytes(shp, G)
    blob = np.zeros(n, dtype=np.uint8)
    stats = np.zeros(4, dtype=np.uint64)
    rc = lib().cgo_build_tables(ctypes.byref(shp), level_id, G, _p(lg), _p(st),
                                _p(np.ascontiguousarray(X).view(np.uint16)), int(flags), _p(blob), n,
                                _p(stats))
    if rc != OK:
        raise RuntimeError("cgo_build_tables failed: %d" % rc)
    return blob, stats


def table_f(blob: np.ndarray, shp: Shape, n_groups: int) -> np.ndarray:
    """u16 f[G][2][H][D][256] view of a blob."""
    off = tables_f_offset(shp, n_groups)
    cnt = n_groups * 2 * shp.kv_heads * shp.head_dim * 256
    return blob[off:off + 2 * cnt].view(np.uint16).reshape(n_groups, 2, shp.kv_heads, shp.head_dim, 256)


def table_counts(shp: Shape, layer_group, steps, X, g, kv, h, d):
    lg = np.ascontiguousarray(layer_group, dtype=np.uint8)
    st = np.ascontiguousarray(steps, dtype=np.float32)
    counts = np.zeros(256, dtype=np.uint64)
    stats = np.zeros(4, dtype=np.uint64)
    lib().cgo_table_counts(ctypes.byref(shp), _p(lg), _p(st), _p(np.ascontiguousarray(X).view(np.uint16)),
                           g, kv, h, d, _p(counts), _p(stats))
    return counts, stats


# ---- groups ---------------------------------------------------------------
def _lane_ptrs(f_lane: np.ndarray):
    f_lane = np.ascontiguousarray(f_lane, dtype=np.uint16)
    assert f_lane.shape == (64, 256)
    arr = (ctypes.c_void_p * 64)(*[f_lane.ctypes.data + 512 * k for k in range(64)])
    return f_lane, arr


def encode_group_q(q: np.ndarray, f_lane: np.ndarray, robust: bool = False) -> np.ndarray:
    """q: int32 [64][n]; f_lane: u16 [64][256]. Returns the u16 word stream
    (robust: symbols of frequency 0 are coded as escapes)."""
    q = np.ascontiguousarray(q, dtype=np.int32)
    n = q.shape[1]
    cap = lib().cgo_group_word_bound(n)
    out = np.zeros(cap, dtype=np.uint16)
    keep, arr = _lane_ptrs(f_lane)
    m = lib().cgo_encode_group_q(_p(q), n, arr, int(bool(robust)), _p(out), cap)
    if m < 0:
        raise RuntimeError("cgo_encode_group_q failed: %d" % m)
    return out[:m].copy()


def decode_group_q(words: np.ndarray, n: int, f_lane: np.ndarray):
    w = np.ascontiguousarray(words, dtype=np.uint16)
    q = np.zeros((64, n), dtype=np.int32)
    keep, arr = _lane_ptrs(f_lane)
    rc = lib().cgo_decode_group_q(_p(w) if len(w) else None, len(w), n, arr, _p(q))
    return rc, q


def encode_group(shp: Shape, blob: np.ndarray, X: np.ndarray, c, l, kv, h, j) -> np.ndarray:
    n = min(shp.chunk_tokens, shp.tokens - c * shp.chunk_tokens)
    cap = lib().cgo_group_word_bound(n)
    out = np.zeros(cap, dtype=np.uint16)
    m = lib().cgo_encode_group(ctypes.byref(shp), _p(blob), _p(np.ascontiguousarray(X).view(np.uint16)),
                               c, l, kv, h, j, _p(out), cap)
    if m < 0:
        raise RuntimeError("cgo_encode_group failed: %d" % m)
    return out[:m].copy()


# ---- chunk records --------------------------------------------------------
def record_data_start(shp: Shape) -> int:
    return lib().cgo_record_data_start(ctypes.byref(shp))


def encode_chunk(shp: Shape, blob: np.ndarray, X: np.ndarray, c: int) -> np.ndarray:
    cap = lib().cgo_record_bound(ctypes.byref(shp), c)
    out = np.zeros(cap, dtype=np.uint8)
    n = lib().cgo_encode_chunk(ctypes.byref(shp), _p(blob), _p(np.ascontiguousarray(X).view(np.uint16)),
                               c, _p(out), cap)
    if n < 0:
        raise RuntimeError("cgo_encode_chunk failed: %d" % n)
    return out[:n].copy()


def decode_chunk(shp: Shape, blob: np.ndarray, rec: np.ndarray, Y: np.ndarray) -> int:
    assert Y.dtype in (np.uint16, np.float16) and Y.flags["C_CONTIGUOUS"]
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    return lib().cgo_decode_chunk(ctypes.byref(shp), _p(blob), _p(rec), len(rec), _p(Y))


def decode_chunk_paged(shp: Shape, blob, rec, pool: np.ndarray, block_table: np.ndarray) -> int:
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    return lib().cgo_decode_chunk_paged(ctypes.byref(shp), _p(blob), _p(rec), len(rec), _p(pool),
                                        pool.shape[2], _p(bt))


def encode_all(shp: Shape, blob, X):
    """All chunk records of a tensor, concatenated; returns (bytes, offsets)."""
    nch = -(-shp.tokens // shp.chunk_tokens)
    recs = [encode_chunk(shp, blob, X, c) for c in range(nch)]
    offs = np.zeros(nch + 1, dtype=np.uint64)
    for c, r in enumerate(recs):
        offs[c + 1] = offs[c] + len(r)
    return np.concatenate(recs), offs


def decode_all(shp: Shape, blob, data, offs, Y=None):
    if Y is None:
        Y = np.zeros((shp.layers, 2, shp.kv_heads, shp.tokens, shp.head_dim), dtype=np.uint16)
    for c in range(len(offs) - 1):
        rc = decode_chunk(shp, blob, data[int(offs[c]):int(offs[c + 1])], Y)
        if rc != OK:
            raise RuntimeError("cgo_decode_chunk failed on chunk %d: %d" % (c, rc))
    return Y


# ---- attention over the restored (paged) cache ------------------------------
def attend_paged(shp: Shape, q_bits: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                 n_tokens: int, scale: float) -> np.ndarray:
    """q_bits: element bits [L][Hq][D]; pool [L][2][NB][H][16][D] element bits.
    Returns binary64 o [L][Hq][D]."""
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    pl = np.ascontiguousarray(pool).view(np.uint16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    L, Hq, D = q.shape
    o = np.zeros((L, Hq, D), dtype=np.float64)
    rc = lib().cgo_attend_paged(ctypes.byref(shp), Hq, _p(q), _p(pl), pl.shape[2], _p(bt), int(n_tokens),
                                float(scale), _p(o))
    if rc != OK:
        raise RuntimeError("cgo_attend_paged failed: %d" % rc)
    return o
