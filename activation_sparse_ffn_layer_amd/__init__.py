"""Neuron-aware sparse FFN (PowerInfer's hot path) for AMD MI355X.

The compute lives in libpi.so (hand-written HIP for gfx950, C ABI in
include/pi.h). This package is its Python face: :class:`Context` and
:class:`Ffn` wrap the handles, and the functions below pass torch tensors'
device pointers through. torch supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
from ctypes import c_double, c_int32, c_void_p
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import ACT, KERNEL_CLASSES, MASK_MODE, PI_OK, WTYPE, FfnDesc, PiError, StackDump, _ptr, lib

__all__ = ["Context", "Ffn", "PiError", "predict", "sparse_ffn", "layer", "layer_noalloc", "q4_dequant", "compact", "glue", "stack_run",
           "stack_run_dump", "stack_profile", "KERNEL_CLASSES",
           "hot_first_order", "permute_rows", "lib"]


class Context:
    """A pi_ctx: a stream of one device plus scratch sized for the largest layer and batch."""

    def __init__(self, max_batch: int, max_d: int, max_ffn: int, max_rank: int, device: int = 0,
                 stream: Optional[torch.cuda.Stream] = None):
        self.device = device
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        h = c_void_p()
        st = lib().pi_ctx_create(device, c_void_p(self.stream.cuda_stream), max_batch, max_d, max_ffn, max_rank,
                                 ctypes.byref(h))
        if st != PI_OK:
            raise PiError(st, "pi_ctx_create failed")
        self.handle = h
        self.max_batch, self.max_d, self.max_ffn, self.max_rank = max_batch, max_d, max_ffn, max_rank

    def set_mask_mode(self, mode: str):
        """Masking of batches: "union" (default) or "per_token" (pi_ctx_set_mask_mode)."""
        self.check(lib().pi_ctx_set_mask_mode(self.handle, MASK_MODE[mode]))

    def check(self, status: int):
        if status != PI_OK:
            raise PiError(status, lib().pi_last_error(self.handle).decode())

    def close(self):
        if getattr(self, "handle", None):
            lib().pi_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _desc(layer, neuron_table=None) -> FfnDesc:
    """The C descriptor of a layer object (see :class:`Ffn`)."""
    return FfnDesc(
        d=layer.d, ffn=layer.ffn, rank=layer.rank, act=ACT[layer.act], wtype=WTYPE[layer.wtype],
        threshold=float(layer.threshold),
        w_up=_ptr(layer.w_up), w_gate=_ptr(layer.w_gate), w_down_t=_ptr(layer.w_down_t),
        s_up=_ptr(layer.s_up), s_gate=_ptr(layer.s_gate), s_down=_ptr(layer.s_down),
        b=_ptr(layer.b), p_w1=_ptr(layer.p_w1), p_w2=_ptr(layer.p_w2), p_b=_ptr(layer.p_b),
        neuron_table=_ptr(neuron_table), hot_prefix=int(getattr(layer, "hot_prefix", 0) or 0),
        y_center=_ptr(getattr(layer, "glue_center", None)))


class Ffn:
    """A pi_ffn: a layer description over borrowed device tensors.

    ``layer`` is any object with the fields of a layer (d, ffn, rank, act, wtype,
    threshold, w_up, w_gate, w_down_t, s_up, s_gate, s_down, b, p_w1, p_w2, p_b, and
    optionally hot_prefix and glue_center); its tensors must stay alive as long as this
    object."""

    def __init__(self, ctx: Context, layer, neuron_table: Optional[torch.Tensor] = None):
        self.ctx = ctx
        self.layer = layer
        self.neuron_table = neuron_table
        desc = _desc(layer, neuron_table)
        h = c_void_p()
        ctx.check(lib().pi_ffn_create(ctx.handle, ctypes.byref(desc), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            lib().pi_ffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def predict(ctx: Context, ffn: Ffn, x: torch.Tensor, mask: torch.Tensor, idx: torch.Tensor, n_active: torch.Tensor,
            logits: Optional[torch.Tensor] = None):
    ctx.check(lib().pi_predict(ctx.handle, ffn.handle, _ptr(x), x.shape[0], _ptr(mask), _ptr(idx), _ptr(n_active),
                               _ptr(logits)))


def sparse_ffn(ctx: Context, ffn: Ffn, x: torch.Tensor, idx: torch.Tensor, n_active: torch.Tensor, y: torch.Tensor):
    ctx.check(lib().pi_sparse_ffn(ctx.handle, ffn.handle, _ptr(x), x.shape[0], _ptr(idx), _ptr(n_active), _ptr(y)))


def layer(ctx: Context, ffn: Ffn, x: torch.Tensor, y: torch.Tensor, mask: Optional[torch.Tensor] = None,
          idx: Optional[torch.Tensor] = None, n_active: Optional[torch.Tensor] = None):
    ctx.check(lib().pi_layer(ctx.handle, ffn.handle, _ptr(x), x.shape[0], _ptr(y), _ptr(mask), _ptr(idx),
                             _ptr(n_active)))


def layer_noalloc(layer, x: torch.Tensor, y: torch.Tensor, mask: Optional[torch.Tensor] = None,
                  idx: Optional[torch.Tensor] = None, n_active: Optional[torch.Tensor] = None,
                  device: int = 0, stream: Optional[torch.cuda.Stream] = None):
    """pi_layer_noalloc: one layer with no context and no device allocation (the library's fixed
    scratch array). Raises PiError with the status on failure."""
    st = stream if stream is not None else torch.cuda.current_stream(device)
    desc = _desc(layer)
    status = lib().pi_layer_noalloc(device, c_void_p(st.cuda_stream), ctypes.byref(desc), _ptr(x), x.shape[0],
                                    _ptr(y), _ptr(mask), _ptr(idx), _ptr(n_active))
    if status != PI_OK:
        raise PiError(status, "pi_layer_noalloc failed")


def q4_dequant(ctx: Context, codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor):
    """pi_q4_dequant: Q4_0 rows (codes [rows][d/2] uint8, scales [rows][d/32] fp16 bits) to
    out [rows][d] fp32 on the context's stream."""
    rows, d = out.shape
    ctx.check(lib().pi_q4_dequant(ctx.handle, _ptr(codes), _ptr(scales), rows, d, _ptr(out)))


def compact(ctx: Context, v: torch.Tensor, threshold: float, mask: torch.Tensor, idx: torch.Tensor,
            n_active: torch.Tensor):
    ctx.check(lib().pi_compact(ctx.handle, _ptr(v), v.shape[0], v.shape[1], float(threshold), _ptr(mask), _ptr(idx),
                               _ptr(n_active)))


def glue(ctx: Context, y: torch.Tensor, x_prev: torch.Tensor, x_out: torch.Tensor,
         center: Optional[torch.Tensor] = None):
    ctx.check(lib().pi_glue(ctx.handle, _ptr(y), _ptr(center), _ptr(x_prev), y.shape[0], y.shape[1],
                            int(x_prev.dtype == torch.float32), _ptr(x_out)))


def stack_run(ctx: Context, ffns: Sequence[Ffn], x_tokens: torch.Tensor, batch: int, y_out: torch.Tensor,
              n_active_log: Optional[torch.Tensor] = None, use_graph: bool = True):
    arr = (c_void_p * len(ffns))(*[f.handle.value for f in ffns])
    ctx.check(lib().pi_stack_run(ctx.handle, arr, len(ffns), _ptr(x_tokens), x_tokens.shape[0], batch, _ptr(y_out),
                                 _ptr(n_active_log), int(bool(use_graph))))


def stack_run_dump(ctx: Context, ffns: Sequence[Ffn], x_tokens: torch.Tensor, batch: int, y_out: torch.Tensor,
                   n_active_log: Optional[torch.Tensor] = None, x: Optional[torch.Tensor] = None,
                   mask: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                   n: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, ffn_stride: int = 0):
    """stack_run recording every (step, layer): x [S][L][B][d], mask [S][L][B][stride/64] int64,
    idx [S][L][stride] int32, n [S][L] int32, y [S][L][B][d] fp32 (each optional)."""
    arr = (c_void_p * len(ffns))(*[f.handle.value for f in ffns])
    stride = ffn_stride or max(f.layer.ffn for f in ffns)
    dump = StackDump(x=_ptr(x), mask=_ptr(mask), idx=_ptr(idx), n=_ptr(n), y=_ptr(y), ffn_stride=stride)
    ctx.check(lib().pi_stack_run_dump(ctx.handle, arr, len(ffns), _ptr(x_tokens), x_tokens.shape[0], batch,
                                      _ptr(y_out), _ptr(n_active_log), ctypes.byref(dump)))


def stack_profile(ctx: Context, ffns: Sequence[Ffn], x_tokens: torch.Tensor, batch: int, y_out: torch.Tensor,
                  n_active_log: Optional[torch.Tensor] = None):
    """Eager stack run with a HIP event pair around every kernel launch (blocks until done).

    Returns {kernel class: (total ms, launches)}."""
    arr = (c_void_p * len(ffns))(*[f.handle.value for f in ffns])
    ms = (ctypes.c_double * len(KERNEL_CLASSES))()
    cnt = (ctypes.c_int64 * len(KERNEL_CLASSES))()
    ctx.check(lib().pi_stack_profile(ctx.handle, arr, len(ffns), _ptr(x_tokens), x_tokens.shape[0], batch,
                                     _ptr(y_out), _ptr(n_active_log), ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}


def hot_first_order(p: np.ndarray) -> np.ndarray:
    """Host call: neuron table ordering neurons by descending activation probability."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    out = np.empty(p.size, dtype=np.int32)
    st = lib().pi_hot_first_order(p.ctypes.data_as(ctypes.POINTER(c_double)), p.size,
                                  out.ctypes.data_as(ctypes.POINTER(c_int32)))
    if st != PI_OK:
        raise PiError(st, "pi_hot_first_order failed")
    return out


def permute_rows(ctx: Context, src: torch.Tensor, dst: torch.Tensor, perm: torch.Tensor):
    rows = src.shape[0]
    row_bytes = src[0].numel() * src.element_size() if rows else 0
    ctx.check(lib().pi_permute_rows(ctx.handle, _ptr(src), _ptr(dst), _ptr(perm), rows, row_bytes))
