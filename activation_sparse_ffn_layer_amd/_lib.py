"""ctypes binding of libpi.so (include/pi.h), argument marshalling only.

Every function here forwards device pointers of torch tensors to the C ABI; all
arithmetic happens in the library's HIP kernels. There is no fallback: if
libpi.so is missing or fails to load, :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int32, c_int64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpi.so")

PI_OK, PI_ERR_INVALID, PI_ERR_UNSUPPORTED, PI_ERR_OOM, PI_ERR_HIP = range(5)
KERNEL_CLASSES = ("stage1", "stage2", "truemask", "up", "down", "reduce")
ACT = {"relu": 0, "reglu": 1, "sqrelu": 2}
WTYPE = {"f32": 0, "f16": 1, "q4_0": 2}
MASK_MODE = {"union": 0, "per_token": 1}


class FfnDesc(ctypes.Structure):
    _fields_ = [
        ("d", c_int32), ("ffn", c_int32), ("rank", c_int32), ("act", c_int32), ("wtype", c_int32),
        ("threshold", c_float),
        ("w_up", c_void_p), ("w_gate", c_void_p), ("w_down_t", c_void_p),
        ("s_up", c_void_p), ("s_gate", c_void_p), ("s_down", c_void_p),
        ("b", c_void_p), ("p_w1", c_void_p), ("p_w2", c_void_p), ("p_b", c_void_p),
        ("neuron_table", c_void_p), ("hot_prefix", c_int32), ("y_center", c_void_p),
    ]


class StackDump(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("mask", c_void_p), ("idx", c_void_p), ("n", c_void_p), ("y", c_void_p),
                ("ffn_stride", c_int32)]


_SIGS = {
    "pi_abi_version": (c_int32, []),
    "pi_status_str": (ctypes.c_char_p, [c_int32]),
    "pi_last_error": (ctypes.c_char_p, [c_void_p]),
    "pi_ctx_create": (c_int32, [c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32, POINTER(c_void_p)]),
    "pi_ctx_destroy": (None, [c_void_p]),
    "pi_ctx_set_stream": (c_int32, [c_void_p, c_void_p]),
    "pi_ctx_set_mask_mode": (c_int32, [c_void_p, c_int32]),
    "pi_ffn_create": (c_int32, [c_void_p, POINTER(FfnDesc), POINTER(c_void_p)]),
    "pi_ffn_destroy": (None, [c_void_p]),
    "pi_predict": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "pi_sparse_ffn": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "pi_layer": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "pi_layer_noalloc": (c_int32, [c_int32, c_void_p, POINTER(FfnDesc), c_void_p, c_int32, c_void_p, c_void_p,
                                   c_void_p, c_void_p]),
    "pi_q4_dequant": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p]),
    "pi_compact": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p]),
    "pi_glue": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    "pi_stack_run": (c_int32, [c_void_p, POINTER(c_void_p), c_int32, c_void_p, c_int32, c_int32, c_void_p,
                               c_void_p, c_int32]),
    "pi_stack_run_dump": (c_int32, [c_void_p, POINTER(c_void_p), c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                    c_void_p, POINTER(StackDump)]),
    "pi_stack_profile": (c_int32, [c_void_p, POINTER(c_void_p), c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                   c_void_p, POINTER(c_double), POINTER(c_int64)]),
    "pi_hot_first_order": (c_int32, [POINTER(c_double), c_int32, POINTER(c_int32)]),
    "pi_permute_rows": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int64]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if libpi.so has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m activation_sparse_ffn_layer_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class PiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{lib().pi_status_str(status).decode()}: {msg}")
        self.status = status


def _ptr(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    return c_void_p(t.data_ptr())
