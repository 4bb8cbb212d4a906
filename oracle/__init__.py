"""CPU oracle of the TBE hot path (ctypes wrapper around tbe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package.  The HIP library and its Python
binding never import it and share no code with it.

The oracle is plain single-threaded C computing in double precision; see the
header of tbe_oracle.c for the definitions and the passages they follow.
All arrays handed in and out are host numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tbe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_tbe.so")

F32, F16, BF16 = 0, 1, 2
I32, I64 = 0, 1
WD = {"f32": F32, "f16": F16, "bf16": BF16}
IT = {"i32": I32, "i64": I64}
LONG_RUN = 256
CHUNK = 256


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99, -O2, one thread)."""
    if force or not os.path.exists(_LIB):
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall",
                               "-Wno-unused-function", "-o", _LIB, _SRC, "-lm"])
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.oracle_round.argtypes = [i32, C.c_double]
        L.oracle_round.restype = C.c_double
        L.oracle_decode.argtypes = [i32, vp, i64]
        L.oracle_decode.restype = C.c_double
        L.oracle_store.argtypes = [i32, vp, i64, C.c_double]
        L.oracle_store.restype = None
        L.oracle_forward.argtypes = [i32, vp, vp, vp, i32, vp, i64, i32, vp, vp, vp, vp, i64]
        L.oracle_forward.restype = C.c_int
        L.oracle_preprocess.argtypes = [i32, vp, i64, i32, vp, vp] + [vp] * 12
        L.oracle_preprocess.restype = C.c_int
        L.oracle_backward_rowwise_adagrad.argtypes = (
            [i32, vp, vp, vp, i32, vp, vp, i64, i32, vp, vp, vp, vp, i64, C.c_float, C.c_float])
        L.oracle_backward_rowwise_adagrad.restype = C.c_int
        L.oracle_backward.argtypes = (
            [i32, vp, vp, vp, i32, vp, vp, i64, i32, vp, vp, vp, vp, i64, i32, C.c_float,
             C.c_float])
        L.oracle_backward.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _ptr_array(arrs):
    return (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _storage(wdtype):
    return np.float32 if wdtype == "f32" else np.uint16


def round_to(wdtype: str, x: float) -> float:
    return lib().oracle_round(WD[wdtype], float(x))


def encode(wdtype: str, values: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float64 values into the storage format (raw bits for 16-bit)."""
    v = np.ascontiguousarray(values, dtype=np.float64).ravel()
    out = np.zeros(v.size, dtype=_storage(wdtype))
    L = lib()
    for i in range(v.size):
        L.oracle_store(WD[wdtype], out.ctypes.data, i, float(v[i]))
    return out.reshape(np.shape(values))


def decode(wdtype: str, stored: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(stored)
    flat = s.ravel()
    L = lib()
    return np.array([L.oracle_decode(WD[wdtype], flat.ctypes.data, i) for i in range(flat.size)],
                    dtype=np.float64).reshape(s.shape)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (code {rc})")


def forward(rows, dims, pooling, wdtype, weights, B, itype, indices, offsets, psw=None,
            out=None, out_stride=None):
    """Pooled output [B, Dtot] float32.  weights: list of storage arrays [R_t, D_t]."""
    T = len(rows)
    rows_a = np.asarray(rows, np.int64)
    dims_a = np.asarray(dims, np.int32)
    pool_a = np.asarray(pooling, np.int32)
    ws = [np.ascontiguousarray(w) for w in weights]
    assert all(w.dtype == _storage(wdtype) for w in ws)
    dtot = int(dims_a.sum())
    if out is None:
        out = np.zeros((B, dtot), np.float32)
    stride = out_stride if out_stride is not None else out.shape[-1]
    psw_a = None if psw is None else np.ascontiguousarray(psw, np.float32)
    rc = lib().oracle_forward(T, _p(rows_a), _p(dims_a), _p(pool_a), WD[wdtype], _ptr_array(ws),
                              B, IT[itype], _p(np.ascontiguousarray(indices)),
                              _p(np.ascontiguousarray(offsets)), _p(psw_a), _p(out), stride)
    _check(rc, "forward")
    return out


def preprocess(rows, B, itype, indices, offsets):
    """Transposition, stable sort, run-length encoding and classification.

    Returns a dict of int64/uint64 arrays trimmed to their counts."""
    T = len(rows)
    rows_a = np.asarray(rows, np.int64)
    offsets = np.ascontiguousarray(offsets)
    N = int(offsets[-1])
    n1 = max(N, 1)
    key = np.zeros(n1, np.uint64)
    bag = np.zeros(n1, np.int64)
    skey = np.zeros(n1, np.uint64)
    spos = np.zeros(n1, np.int64)
    rstart = np.zeros(n1 + 1, np.int64)
    rkey = np.zeros(n1, np.uint64)
    sl = np.zeros(n1, np.int64)
    ll = np.zeros(n1, np.int64)
    cl = np.zeros(n1 + 1, np.int64)
    cs = np.zeros(n1 + 1, np.int64)
    cn = np.zeros(n1 + 1, np.int64)
    counts = np.zeros(4, np.int64)
    rc = lib().oracle_preprocess(T, _p(rows_a), B, IT[itype], _p(np.ascontiguousarray(indices)),
                                 _p(offsets), _p(key), _p(bag), _p(skey), _p(spos), _p(rstart),
                                 _p(rkey), _p(sl), _p(ll), _p(cl), _p(cs), _p(cn), _p(counts))
    _check(rc, "preprocess")
    U, ns, nl, nc = (int(c) for c in counts)
    return dict(key=key[:N], bag=bag[:N], sorted_key=skey[:N], sorted_pos=spos[:N],
                run_start=rstart[:U + 1], run_key=rkey[:U], short_list=sl[:ns],
                long_list=ll[:nl], chunk_long=cl[:nc], chunk_start=cs[:nc], chunk_len=cn[:nc],
                U=U, n_short=ns, n_long=nl, n_chunks=nc)


OPTIMIZERS = {"rowwise_adagrad": 0, "adagrad": 1, "sgd": 2}


def backward(rows, dims, pooling, wdtype, weights, state, B, itype, indices, offsets, psw, grad,
             lr, eps, optimizer="rowwise_adagrad", grad_stride=None):
    """Updates weights (storage arrays) and the optimizer state in place:
    rowwise_adagrad: state[t] float32 [R_t]; adagrad (element-wise): float32
    [R_t, D_t]; sgd: state ignored (None)."""
    T = len(rows)
    rows_a = np.asarray(rows, np.int64)
    dims_a = np.asarray(dims, np.int32)
    pool_a = np.asarray(pooling, np.int32)
    for a in weights:
        assert a.flags["C_CONTIGUOUS"] and a.dtype == _storage(wdtype)
    opt = OPTIMIZERS[optimizer]
    if opt == 2:
        state = [np.zeros(1, np.float32) for _ in range(T)]
    for t, a in enumerate(state):
        assert a.flags["C_CONTIGUOUS"] and a.dtype == np.float32
        need = rows[t] * (dims[t] if opt == 1 else 1) if opt != 2 else 0
        assert a.size >= need
    grad = np.ascontiguousarray(grad, np.float32)
    stride = grad_stride if grad_stride is not None else grad.shape[-1]
    psw_a = None if psw is None else np.ascontiguousarray(psw, np.float32)
    rc = lib().oracle_backward(
        T, _p(rows_a), _p(dims_a), _p(pool_a), WD[wdtype], _ptr_array(weights),
        _ptr_array(state), B, IT[itype], _p(np.ascontiguousarray(indices)),
        _p(np.ascontiguousarray(offsets)), _p(psw_a), _p(grad), stride, opt,
        C.c_float(lr), C.c_float(eps))
    _check(rc, "backward")


def backward_rowwise_adagrad(rows, dims, pooling, wdtype, weights, momentum, B, itype, indices,
                             offsets, psw, grad, lr, eps, grad_stride=None):
    """Updates weights (storage arrays) and momentum (float32 arrays) in place."""
    T = len(rows)
    rows_a = np.asarray(rows, np.int64)
    dims_a = np.asarray(dims, np.int32)
    pool_a = np.asarray(pooling, np.int32)
    for a in weights:
        assert a.flags["C_CONTIGUOUS"] and a.dtype == _storage(wdtype)
    for a in momentum:
        assert a.flags["C_CONTIGUOUS"] and a.dtype == np.float32
    grad = np.ascontiguousarray(grad, np.float32)
    stride = grad_stride if grad_stride is not None else grad.shape[-1]
    psw_a = None if psw is None else np.ascontiguousarray(psw, np.float32)
    rc = lib().oracle_backward_rowwise_adagrad(
        T, _p(rows_a), _p(dims_a), _p(pool_a), WD[wdtype], _ptr_array(weights),
        _ptr_array(momentum), B, IT[itype], _p(np.ascontiguousarray(indices)),
        _p(np.ascontiguousarray(offsets)), _p(psw_a), _p(grad), stride,
        C.c_float(lr), C.c_float(eps))
    _check(rc, "backward")
