"""The C-ABI library loads on the host and exports every entry point that
include/tbe.h declares; host-side argument errors come back as status codes
without touching the GPU (no compute call runs here)."""
import ctypes as C
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(tbe_[a-z0-9_]+)\s*\(",
                            src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tbe_forward", "tbe_preprocess", "tbe_backward_rowwise_adagrad"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import table_embedding_amd as te
    L = te.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(te.EXPORTS)


def test_every_entry_point_has_declared_argument_types():
    """Without argtypes ctypes passes Python ints as C int, masked to 32 bits:
    a device pointer would reach the library truncated."""
    import table_embedding_amd as te
    L = te.lib()
    for n in te.EXPORTS:
        assert getattr(L, n).argtypes is not None, n


def test_status_strings():
    import table_embedding_amd as te
    assert te.tbe_status_string(0) == "ok"
    for code in range(-7, 0):
        assert te.tbe_status_string(code) not in ("ok", "unknown status")


def test_host_argument_errors_need_no_gpu():
    import table_embedding_amd as te
    L = te.lib()
    h = C.c_void_p()
    rows = (C.c_int64 * 1)(10)
    dims = (C.c_int32 * 1)(6)   # not a multiple of 4
    pool = (C.c_int32 * 1)(0)
    w = (C.c_void_p * 1)(0x1000)
    m = (C.c_void_p * 1)(0x2000)
    assert L.tbe_plan_create(None, 1, rows, dims, pool, 1, w, m) == te.TBE_E_ARG
    assert L.tbe_plan_create(C.byref(h), 0, rows, dims, pool, 1, w, m) == te.TBE_E_ARG
    assert L.tbe_plan_create(C.byref(h), 1, rows, dims, pool, 7, w, m) == te.TBE_E_ARG
    assert L.tbe_plan_create(C.byref(h), 1, rows, dims, pool, 1, w, m) == te.TBE_E_UNSUPPORTED
    w_bad = (C.c_void_p * 1)(0x1002)
    dims[0] = 8
    assert L.tbe_plan_create(C.byref(h), 1, rows, dims, pool, 1, w_bad, m) == te.TBE_E_ARG
    big = (C.c_int64 * 2)(1 << 31, 1 << 31)
    d2 = (C.c_int32 * 2)(8, 8)
    p2 = (C.c_int32 * 2)(0, 0)
    w2 = (C.c_void_p * 2)(0x1000, 0x1000)
    m2 = (C.c_void_p * 2)(0x2000, 0x2000)
    assert L.tbe_plan_create(C.byref(h), 2, big, d2, p2, 1, w2, m2) == te.TBE_E_RANGE
    n = C.c_size_t()
    assert L.tbe_workspace_size(None, 1, 1, C.byref(n)) == te.TBE_E_ARG
    assert L.tbe_forward(None, 1, 0, None, None, 0, None, None, 0, None) == te.TBE_E_ARG
    assert L.tbe_forward_preprocess(None, 1, 0, None, None, 0, None, None, 0, None, 0,
                                    None) == te.TBE_E_ARG
    assert L.tbe_plan_destroy(None) == te.TBE_OK
