"""ctypes binding of libtbe_hip.so (include/tbe.h), argument marshalling only.

Each function has the name of the C entry point it calls, takes torch device
tensors (or None where the C argument is nullable), checks dtype, device and
contiguity, and passes raw pointers plus the current HIP stream.  Every step
of the hot path runs in the HIP kernels; there is no fallback: if the library
is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtbe_hip.so")

# include/tbe.h constants
TBE_OK, TBE_E_ARG, TBE_E_UNSUPPORTED, TBE_E_WORKSPACE, TBE_E_RANGE, TBE_E_HIP, TBE_E_ALLOC = (
    0, -1, -2, -3, -4, -5, -6)
TBE_E_TOO_LARGE = -7
TBE_STATIC_WS_BYTES = 256 << 20
TBE_F32, TBE_F16, TBE_BF16 = 0, 1, 2
TBE_I32, TBE_I64 = 0, 1
TBE_SUM, TBE_MEAN = 0, 1
TBE_FWD_NO_HIST, TBE_FWD_REQUIRE_HIST, TBE_FWD_BALANCE, TBE_FWD_NO_BALANCE = 0x1, 0x2, 0x4, 0x8
TBE_FWD_SAVE_HIST = 0x10
TBE_BWD_PREPROCESSED, TBE_BWD_FUSED_LONG, TBE_BWD_CONCURRENT = 0x1, 0x2, 0x4
TBE_BWD_ORDER_CHUNKS, TBE_BWD_NO_ORDER_CHUNKS = 0x8, 0x10
TBE_BWD_HIST = 0x20
TBE_BWD_CONCURRENT_AUTO = 0x40

EXPORTS = ("tbe_plan_create", "tbe_plan_destroy", "tbe_plan_key_bases", "tbe_workspace_size",
           "tbe_workspace_views", "tbe_forward", "tbe_forward_checked", "tbe_forward_preprocess",
           "tbe_preprocess",
           "tbe_backward_rowwise_adagrad", "tbe_backward_rowwise_adagrad_noalloc",
           "tbe_backward", "tbe_validate", "tbe_prof_enable",
           "tbe_prof_read", "tbe_prof_calibrate", "tbe_test_knob", "tbe_status_string")
TBE_PROF_NAME_LEN = 32

# debug_row_updates: one uint32 word per linear key
_U32 = torch.uint32

WDTYPE_OF_TORCH = {torch.float32: TBE_F32, torch.float16: TBE_F16, torch.bfloat16: TBE_BF16}
ITYPE_OF_TORCH = {torch.int32: TBE_I32, torch.int64: TBE_I64}


class TBEError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {tbe_status_string(code)} ({code})")
        self.code = code


class WsViews(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("sorted_key", "sorted_bag",
                                           "sorted_scale", "run_start", "run_key", "single_task", "tiny_task",
                                           "medium_task", "long_task", "long_cbeg",
                                           "chunk_task", "chunk_perm", "counters", "prep_error",
                                           "hist_counts", "long_flag", "dense_rows", "dense_count",
                                           "total")] + [
        ("num_buckets", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run table_embedding_amd/build.py "
                              "(or __graft_entry__.build()) first")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
        L.tbe_plan_create.argtypes = [C.POINTER(vp), i32, vp, vp, vp, i32, vp, vp]
        L.tbe_plan_destroy.argtypes = [vp]
        L.tbe_plan_key_bases.argtypes = [vp, vp]
        L.tbe_workspace_size.argtypes = [vp, i64, i64, C.POINTER(C.c_size_t)]
        L.tbe_workspace_views.argtypes = [vp, i64, i64, C.POINTER(WsViews)]
        L.tbe_forward.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, u32, vp]
        L.tbe_forward_checked.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, u32, vp, vp]
        L.tbe_preprocess.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, C.c_size_t, vp]
        L.tbe_forward_preprocess.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, u32, vp,
                                             C.c_size_t, vp]
        L.tbe_backward_rowwise_adagrad.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp,
                                                   C.c_float, C.c_float, vp, C.c_size_t, u32,
                                                   vp, vp]
        L.tbe_backward_rowwise_adagrad_noalloc.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp,
                                                           C.c_float, C.c_float, u32, vp, vp]
        L.tbe_validate.argtypes = [vp, i64, i32, vp, vp, i64, vp, u32, vp]
        L.tbe_backward.argtypes = [vp, i64, i32, vp, vp, i64, vp, vp, i32, C.c_float, C.c_float,
                                   vp, C.c_size_t, u32, vp, vp]
        L.tbe_prof_enable.argtypes = [C.c_int]
        L.tbe_prof_read.argtypes = [i32, vp, vp, vp, C.POINTER(i32)]
        L.tbe_prof_calibrate.argtypes = [i32, vp]
        L.tbe_test_knob.argtypes = [i32, i64]
        L.tbe_status_string.argtypes = [C.c_int]
        L.tbe_status_string.restype = C.c_char_p
        for n in EXPORTS[:-1]:  # every entry point but the status text returns a status
            getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def tbe_status_string(code: int) -> str:
    return lib().tbe_status_string(int(code)).decode()


def _check(fn, rc):
    if rc != TBE_OK:
        raise TBEError(fn, rc)


def _dptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _itype(indices, offsets):
    if offsets.dtype not in ITYPE_OF_TORCH:
        raise TypeError("offsets must be int32 or int64")
    if indices is not None and indices.numel() and indices.dtype != offsets.dtype:
        raise TypeError("indices and offsets must share one integer type")
    return ITYPE_OF_TORCH[offsets.dtype]


def tbe_plan_create(rows: Sequence[int], dims: Sequence[int], pooling: Sequence[int],
                    weights: Sequence[torch.Tensor], momentum: Sequence[torch.Tensor]):
    T = len(rows)
    if not (len(dims) == len(pooling) == len(weights) == len(momentum) == T):
        raise ValueError("per-table lists must have one entry per table")
    wd = weights[0].dtype
    if wd not in WDTYPE_OF_TORCH:
        raise TypeError("weights must be float32, float16 or bfloat16")
    for t in range(T):
        if weights[t].dtype != wd:
            raise TypeError("all tables must share one weight dtype")
        if tuple(weights[t].shape) != (int(rows[t]), int(dims[t])):
            raise ValueError(f"weights[{t}] must be [{rows[t]}, {dims[t]}]")
        if tuple(momentum[t].shape) not in ((int(rows[t]),), (int(rows[t]), int(dims[t]))):
            # [R_t] for row-wise Adagrad (and SGD), [R_t, D_t] for element-wise Adagrad
            raise ValueError(f"momentum[{t}] must be [{rows[t]}] or [{rows[t]}, {dims[t]}]")
    rows_a = (C.c_int64 * T)(*[int(r) for r in rows])
    dims_a = (C.c_int32 * T)(*[int(d) for d in dims])
    pool_a = (C.c_int32 * T)(*[int(p) for p in pooling])
    w_a = (C.c_void_p * T)(*[_dptr(w, wd, "weights") for w in weights])
    m_a = (C.c_void_p * T)(*[_dptr(m, torch.float32, "momentum") for m in momentum])
    h = C.c_void_p()
    _check("tbe_plan_create", lib().tbe_plan_create(C.byref(h), T, rows_a, dims_a, pool_a,
                                                    WDTYPE_OF_TORCH[wd], w_a, m_a))
    return h


def tbe_plan_destroy(plan) -> None:
    _check("tbe_plan_destroy", lib().tbe_plan_destroy(plan))


def tbe_plan_key_bases(plan, T: int):
    a = (C.c_int64 * T)()
    _check("tbe_plan_key_bases", lib().tbe_plan_key_bases(plan, a))
    return [int(x) for x in a]


def tbe_workspace_size(plan, B: int, num_lookups: int) -> int:
    n = C.c_size_t()
    _check("tbe_workspace_size", lib().tbe_workspace_size(plan, int(B), int(num_lookups),
                                                          C.byref(n)))
    return int(n.value)


def tbe_workspace_views(plan, B: int, num_lookups: int) -> dict:
    v = WsViews()
    _check("tbe_workspace_views", lib().tbe_workspace_views(plan, int(B), int(num_lookups),
                                                            C.byref(v)))
    return {n: getattr(v, n) for n, _ in WsViews._fields_}


def tbe_forward(plan, B: int, indices, offsets, num_lookups: int, per_sample_weights,
                out: torch.Tensor, flags: int = 0, stream=None) -> None:
    it = _itype(indices, offsets)
    rc = lib().tbe_forward(plan, int(B), it, _dptr(indices, None, "indices"),
                           _dptr(offsets, None, "offsets"), int(num_lookups),
                           _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
                           _dptr(out, torch.float32, "out"), int(flags), _stream(stream))
    _check("tbe_forward", rc)


def tbe_forward_checked(plan, B: int, indices, offsets, num_lookups: int, per_sample_weights,
                        out: torch.Tensor, err: torch.Tensor, flags: int = 0,
                        stream=None) -> None:
    """tbe_forward with the offsets and indices checked as they are read; err:
    device uint32 tensor of TBE_VALIDATE_WORDS words (tbe_validate's layout)."""
    it = _itype(indices, offsets)
    if err.numel() < TBE_VALIDATE_WORDS:
        raise ValueError("err needs TBE_VALIDATE_WORDS words")
    rc = lib().tbe_forward_checked(plan, int(B), it, _dptr(indices, None, "indices"),
                                   _dptr(offsets, None, "offsets"), int(num_lookups),
                                   _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
                                   _dptr(out, torch.float32, "out"), int(flags),
                                   _dptr(err, (torch.uint32, torch.int32), "err"),
                                   _stream(stream))
    _check("tbe_forward_checked", rc)


TBE_VALIDATE_REPAIR = 0x1
TBE_VALIDATE_WORDS = 4
TBE_INVALID_OFFSET_START, TBE_INVALID_OFFSET_END, TBE_INVALID_OFFSET_ORDER = 0x1, 0x2, 0x4
TBE_INVALID_OFFSET_RANGE, TBE_INVALID_INDEX = 0x8, 0x10


def tbe_validate(plan, B: int, indices, offsets, num_lookups: int, err: torch.Tensor,
                 flags: int = 0, stream=None) -> None:
    """Check (and with TBE_VALIDATE_REPAIR repair in place) the lookup
    contract; err: device int32 tensor of TBE_VALIDATE_WORDS words."""
    it = _itype(indices, offsets)
    if err.numel() < TBE_VALIDATE_WORDS:
        raise ValueError("err needs TBE_VALIDATE_WORDS words")
    rc = lib().tbe_validate(plan, int(B), it, _dptr(indices, None, "indices"),
                            _dptr(offsets, None, "offsets"), int(num_lookups),
                            _dptr(err, None, "err"), int(flags), _stream(stream))
    _check("tbe_validate", rc)


def tbe_forward_preprocess(plan, B: int, indices, offsets, num_lookups: int,
                           per_sample_weights, out: torch.Tensor, ws: torch.Tensor,
                           flags: int = 0, stream=None) -> None:
    """tbe_forward on `stream` and tbe_preprocess into ws on a side stream of the
    plan, forked from and joined into `stream` (one native call)."""
    it = _itype(indices, offsets)
    rc = lib().tbe_forward_preprocess(plan, int(B), it, _dptr(indices, None, "indices"),
                                      _dptr(offsets, None, "offsets"), int(num_lookups),
                                      _dptr(per_sample_weights, torch.float32,
                                            "per_sample_weights"),
                                      _dptr(out, torch.float32, "out"), int(flags),
                                      _dptr(ws, None, "ws"), ws.numel() * ws.element_size(),
                                      _stream(stream))
    _check("tbe_forward_preprocess", rc)


def tbe_preprocess(plan, B: int, indices, offsets, num_lookups: int, per_sample_weights,
                   ws: torch.Tensor, stream=None) -> None:
    it = _itype(indices, offsets)
    rc = lib().tbe_preprocess(plan, int(B), it, _dptr(indices, None, "indices"),
                              _dptr(offsets, None, "offsets"), int(num_lookups),
                              _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
                              _dptr(ws, None, "ws"), ws.numel() * ws.element_size(),
                              _stream(stream))
    _check("tbe_preprocess", rc)


def tbe_backward_rowwise_adagrad(plan, B: int, indices, offsets, num_lookups: int,
                                 per_sample_weights, grad_out: torch.Tensor, lr: float,
                                 eps: float, ws: torch.Tensor, flags: int = 0,
                                 debug_row_updates: Optional[torch.Tensor] = None,
                                 stream=None) -> None:
    it = _itype(indices, offsets)
    rc = lib().tbe_backward_rowwise_adagrad(
        plan, int(B), it, _dptr(indices, None, "indices"), _dptr(offsets, None, "offsets"),
        int(num_lookups), _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
        _dptr(grad_out, torch.float32, "grad_out"), float(lr), float(eps),
        _dptr(ws, None, "ws"), ws.numel() * ws.element_size(), int(flags),
        _dptr(debug_row_updates, _U32, "debug_row_updates"), _stream(stream))
    _check("tbe_backward_rowwise_adagrad", rc)


def tbe_backward_rowwise_adagrad_noalloc(plan, B: int, indices, offsets, num_lookups: int,
                                         per_sample_weights, grad_out: torch.Tensor, lr: float,
                                         eps: float, flags: int = 0,
                                         debug_row_updates: Optional[torch.Tensor] = None,
                                         stream=None) -> None:
    """tbe_backward_rowwise_adagrad with the library's static workspace (no
    workspace argument; the call allocates nothing)."""
    it = _itype(indices, offsets)
    rc = lib().tbe_backward_rowwise_adagrad_noalloc(
        plan, int(B), it, _dptr(indices, None, "indices"), _dptr(offsets, None, "offsets"),
        int(num_lookups), _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
        _dptr(grad_out, torch.float32, "grad_out"), float(lr), float(eps), int(flags),
        _dptr(debug_row_updates, _U32, "debug_row_updates"), _stream(stream))
    _check("tbe_backward_rowwise_adagrad_noalloc", rc)


TBE_OPT_ROWWISE_ADAGRAD, TBE_OPT_ADAGRAD, TBE_OPT_SGD = 0, 1, 2

TBE_KNOB_RLE_DEEP_LOOKUPS, TBE_KNOB_BWD_DEEP_LOOKUPS = 1, 2
TBE_KNOB_BWD_STREAM_LOOKUPS, TBE_KNOB_WAIT_POLLS = 3, 4
TBE_KNOB_DENSE_LOOKUPS = 5


def tbe_test_knob(knob: int, value: int) -> None:
    """Test-only override of a variant threshold or the look-back poll limit
    (value < 0 restores the default)."""
    _check("tbe_test_knob", lib().tbe_test_knob(int(knob), int(value)))


def tbe_backward(plan, B: int, indices, offsets, num_lookups: int, per_sample_weights,
                 grad_out: torch.Tensor, optimizer: int, lr: float, eps: float,
                 ws: torch.Tensor, flags: int = 0,
                 debug_row_updates: Optional[torch.Tensor] = None, stream=None) -> None:
    it = _itype(indices, offsets)
    rc = lib().tbe_backward(
        plan, int(B), it, _dptr(indices, None, "indices"), _dptr(offsets, None, "offsets"),
        int(num_lookups), _dptr(per_sample_weights, torch.float32, "per_sample_weights"),
        _dptr(grad_out, torch.float32, "grad_out"), int(optimizer), float(lr), float(eps),
        _dptr(ws, None, "ws"), ws.numel() * ws.element_size(), int(flags),
        _dptr(debug_row_updates, _U32, "debug_row_updates"), _stream(stream))
    _check("tbe_backward", rc)


def tbe_prof_enable(enable: bool) -> None:
    _check("tbe_prof_enable", lib().tbe_prof_enable(1 if enable else 0))


def tbe_prof_calibrate(launches: int, stream=None) -> None:
    _check("tbe_prof_calibrate", lib().tbe_prof_calibrate(int(launches), _stream(stream)))


def tbe_prof_read(max_kernels: int = 64) -> dict:
    """{kernel family: (launches, total milliseconds)}; clears the records."""
    names = C.create_string_buffer(max_kernels * TBE_PROF_NAME_LEN)
    n = (C.c_int64 * max_kernels)()
    ms = (C.c_double * max_kernels)()
    cnt = C.c_int32()
    _check("tbe_prof_read", lib().tbe_prof_read(max_kernels, names, n, ms, C.byref(cnt)))
    out = {}
    for k in range(min(cnt.value, max_kernels)):
        raw = names.raw[k * TBE_PROF_NAME_LEN:(k + 1) * TBE_PROF_NAME_LEN]
        out[raw.split(b"\0", 1)[0].decode()] = (int(n[k]), float(ms[k]))
    return out
