"""MI355X-native Table Batched Embedding (TBE) hot path.

The work runs in libtbe_hip.so (hand-written HIP for gfx950, C ABI in
include/tbe.h).  This package holds its ctypes binding (`_lib`, same names
as the C entry points) and `TBE`, a small owner of one plan, its tables'
tensors and a workspace.  PyTorch provides device memory and streams only.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, TBE_BF16, TBE_BWD_CONCURRENT, TBE_BWD_CONCURRENT_AUTO, TBE_BWD_FUSED_LONG,
    TBE_BWD_NO_ORDER_CHUNKS,
    TBE_BWD_HIST, TBE_BWD_ORDER_CHUNKS, TBE_BWD_PREPROCESSED,
    TBE_E_ALLOC,
    TBE_E_ARG, TBE_E_HIP, TBE_E_RANGE, TBE_E_UNSUPPORTED, TBE_E_WORKSPACE, TBE_F16, TBE_F32,
    TBE_FWD_BALANCE, TBE_FWD_NO_BALANCE, TBE_FWD_NO_HIST, TBE_FWD_REQUIRE_HIST, TBE_I32, TBE_I64, TBE_MEAN, TBE_OK, TBE_SUM,
    TBEError, lib, tbe_backward_rowwise_adagrad, tbe_forward, tbe_forward_preprocess,
    tbe_plan_create,
    tbe_plan_destroy, tbe_plan_key_bases, tbe_preprocess, tbe_prof_calibrate, tbe_prof_enable,
    tbe_prof_read,
    tbe_status_string, tbe_validate, TBE_VALIDATE_REPAIR, TBE_VALIDATE_WORDS,
    tbe_backward, TBE_OPT_ROWWISE_ADAGRAD, TBE_OPT_ADAGRAD, TBE_OPT_SGD,
    TBE_INVALID_OFFSET_START, TBE_INVALID_OFFSET_END, TBE_INVALID_OFFSET_ORDER,
    TBE_INVALID_OFFSET_RANGE, TBE_INVALID_INDEX,
    tbe_workspace_size, tbe_workspace_views, tbe_test_knob, TBE_KNOB_RLE_DEEP_LOOKUPS,
    TBE_KNOB_BWD_DEEP_LOOKUPS, TBE_KNOB_BWD_STREAM_LOOKUPS, TBE_KNOB_WAIT_POLLS,
    tbe_backward_rowwise_adagrad_noalloc, TBE_E_TOO_LARGE, TBE_STATIC_WS_BYTES,
    tbe_forward_checked, TBE_FWD_SAVE_HIST, TBE_KNOB_DENSE_LOOKUPS)


class TBE:
    """One plan over caller-owned tables plus a reusable workspace.

    weights[t]: device [R_t, D_t] float32/float16/bfloat16; momentum[t]: device
    float32 optimizer state, [R_t] (row-wise Adagrad, SGD) or [R_t, D_t]
    (element-wise Adagrad).  Both are updated in place by `backward`.
    """

    def __init__(self, rows: Sequence[int], dims: Sequence[int], pooling: Sequence[int],
                 weights: Sequence[torch.Tensor], momentum: Sequence[torch.Tensor]):
        self.rows = [int(r) for r in rows]
        self.dims = [int(d) for d in dims]
        self.pooling = [int(p) for p in pooling]
        self.weights = list(weights)
        self.momentum = list(momentum)
        self.T = len(self.rows)
        self.dtot = sum(self.dims)
        self.plan = tbe_plan_create(self.rows, self.dims, self.pooling, self.weights,
                                    self.momentum)
        self._ws: Optional[torch.Tensor] = None

    def close(self):
        if self.plan is not None:
            tbe_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def key_bases(self):
        return tbe_plan_key_bases(self.plan, self.T)

    def workspace(self, B: int, num_lookups: int) -> torch.Tensor:
        """A workspace large enough for B bags and num_lookups lookups (grown on demand)."""
        need = tbe_workspace_size(self.plan, B, num_lookups)
        if self._ws is None or self._ws.numel() < need:
            dev = self.weights[0].device
            self._ws = torch.empty(need, dtype=torch.uint8, device=dev)
        return self._ws

    def forward(self, B: int, indices: torch.Tensor, offsets: torch.Tensor,
                per_sample_weights: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
        if out is None:
            out = torch.empty((B, self.dtot), dtype=torch.float32, device=offsets.device)
        tbe_forward(self.plan, B, indices, offsets, indices.numel(), per_sample_weights, out,
                    flags)
        return out

    def forward_and_preprocess(self, B: int, indices: torch.Tensor, offsets: torch.Tensor,
                               per_sample_weights: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, flags: int = 0
                               ) -> torch.Tensor:
        """tbe_forward_preprocess: the forward on the current stream and, at the same
        time, tbe_preprocess of the same lookups on a side stream of the plan (default
        priority); the current stream then waits for both.  A later backward(...,
        flags=TBE_BWD_PREPROCESSED) on the current stream reuses the workspace (FBTriton
        page, "Backward": the preprocessing can move into forward).  Only the order of
        launches differs from forward() then preprocess()."""
        if out is None:
            out = torch.empty((B, self.dtot), dtype=torch.float32, device=offsets.device)
        ws = self.workspace(B, indices.numel())
        tbe_forward_preprocess(self.plan, B, indices, offsets, indices.numel(),
                               per_sample_weights, out, ws, flags)
        return out

    def preprocess(self, B: int, indices: torch.Tensor, offsets: torch.Tensor,
                   per_sample_weights: Optional[torch.Tensor] = None) -> torch.Tensor:
        ws = self.workspace(B, indices.numel())
        tbe_preprocess(self.plan, B, indices, offsets, indices.numel(), per_sample_weights, ws)
        return ws

    def backward(self, B: int, indices: torch.Tensor, offsets: torch.Tensor,
                 per_sample_weights: Optional[torch.Tensor], grad_out: torch.Tensor,
                 lr: float, eps: float, flags: int = 0,
                 debug_row_updates: Optional[torch.Tensor] = None,
                 optimizer: int = TBE_OPT_ROWWISE_ADAGRAD) -> None:
        """optimizer: TBE_OPT_ROWWISE_ADAGRAD (momentum[t] of R_t floats),
        TBE_OPT_ADAGRAD (element-wise: momentum[t] of R_t x D_t floats) or
        TBE_OPT_SGD (momentum untouched)."""
        ws = self.workspace(B, indices.numel())
        if optimizer == TBE_OPT_ROWWISE_ADAGRAD:
            tbe_backward_rowwise_adagrad(self.plan, B, indices, offsets, indices.numel(),
                                         per_sample_weights, grad_out, lr, eps, ws, flags,
                                         debug_row_updates)
        else:
            tbe_backward(self.plan, B, indices, offsets, indices.numel(), per_sample_weights,
                         grad_out, optimizer, lr, eps, ws, flags, debug_row_updates)
