"""The C ABI library loads and exports every entry point include/cg.h declares
(no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cg.h")
LIB = os.path.join(ROOT, "kv_cache_compression_encode_amd", "libcg.so")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cg_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared()
    for fn in ("cg_build_tables", "cg_encode", "cg_decode", "cg_decode_paged"):
        assert fn in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared():
        assert hasattr(lib, name), name


@pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")
def test_host_only_queries():
    from kv_cache_compression_encode_amd import cg as C
    assert C.cg_version() == 1
    assert C.cg_status_string(C.CG_ERR_CORRUPT) == "corrupt record or stream"
    shp = C.shape(4, 2, 64, 1024, 256)
    assert C.cg_tables_format_bytes(shp, 3) > 0
    assert C.cg_tables_bytes(shp, 3) > C.cg_tables_format_bytes(shp, 3)
    assert C.cg_tables_bytes(C.shape(4, 2, 65, 1024, 256), 3) == 0      # head_dim % 64
    assert C.cg_encode_bound(shp, 0, 4) > 0 and C.cg_encode_bound(shp, 0, 5) == 0
    assert C.cg_encode_workspace_bytes(shp, 1, 2) > 0


def test_binding_names_match_header():
    from kv_cache_compression_encode_amd import cg as C
    for name in declared():
        assert hasattr(C, name), name
    assert set(C.EXPORTS) == set(declared())


@pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")
def test_argument_checks_before_any_launch():
    """Calls that fail validation return before touching the GPU, so these
    run without one: bad shapes, element types, flags and attention limits."""
    from kv_cache_compression_encode_amd import cg as C
    ok = C.shape(4, 2, 64, 1024, 256)
    assert C.cg_tables_bytes(C.shape(4, 2, 64, 0, 256), 3) == 0                 # no tokens
    assert C.cg_tables_bytes(C.shape(4, 2, 64, 1024, 256, dtype=2), 3) == 0     # unknown element type
    bad = C.shape(4, 2, 64, 1024, 256)
    bad.reserved = 1
    assert C.cg_tables_bytes(bad, 3) == 0
    assert C.cg_tables_bytes(ok, 0) == 0 and C.cg_tables_bytes(ok, 256) == 0    # group count
    # attention: q_heads a multiple of kv_heads, at most 16 per kv head, D in {64, 128, 256}
    assert C.cg_attend_workspace_bytes(ok, 4, 100) > 0
    assert C.cg_attend_workspace_bytes(ok, 3, 100) == 0
    assert C.cg_attend_workspace_bytes(ok, 34, 100) == 0
    assert C.cg_attend_workspace_bytes(ok, 4, 0) == 0
    assert C.cg_attend_workspace_bytes(C.shape(4, 2, 192, 1024, 256), 4, 100) == 0
    # unknown table flags are refused before the first launch
    lv = C.Level(0, [0, 0, 1, 1], [0.5, 1.0])
    L = C.lib()
    rc = L.cg_build_tables(C.ctypes.byref(ok), C.ctypes.byref(lv.c), 256, 256, 256, 1 << 20, 2, None, None, None)
    assert rc == C.CG_ERR_INVALID_ARG
    # decoders: no levels
    rc = L.cg_decode(C.ctypes.byref(ok), 0, None, None, None, 1, None, None, None, None)
    assert rc == C.CG_ERR_INVALID_ARG
