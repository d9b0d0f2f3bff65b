"""ctypes binding of libsage_attn.so (include/sage_attn.h).

Argument marshalling only: every step of the path runs in the HIP kernels.
PyTorch supplies device memory and the current stream. There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage_attn.so")
SAGE_BLOCK = 64
SAGE_OK, SAGE_ERR_INVALID_ARG, SAGE_ERR_UNSUPPORTED, SAGE_ERR_WORKSPACE, SAGE_ERR_HIP = 0, -1, -2, -3, -4
(SAGE_KERNEL_AUTO, SAGE_KERNEL_FUSED, SAGE_KERNEL_SPLIT, SAGE_KERNEL_PERSISTENT, SAGE_KERNEL_WIDE,
 SAGE_KERNEL_ENTRY) = 0, 1, 2, 3, 4, 5

_lock = threading.Lock()
_lib = None


class SageError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library {LIB_PATH} is not built; run "
                    "`python -m quantized_exact_attention_smooth_amd.build` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            F = ctypes.c_float
            L.sage_status_str.argtypes = [I]
            L.sage_status_str.restype = ctypes.c_char_p
            for n in ("sage_prep_scratch_bytes", "sage_workspace_bytes"):
                getattr(L, n).argtypes = [I, I, I, I, I, ctypes.POINTER(Z)]
                getattr(L, n).restype = I
            L.sage_quant_prep.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
            L.sage_quant_prep.restype = I
            L.sage_quant_prep_noalloc.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P]
            L.sage_quant_prep_noalloc.restype = I
            L.sage_attn_fwd_prepped.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P]
            L.sage_attn_fwd_prepped.restype = I
            L.sage_attn_fwd_prepped_kernel.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
            L.sage_attn_fwd_prepped_kernel.restype = I
            L.sage_attn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, Z, P]
            L.sage_attn_fwd.restype = I
            L.sage_attn_fwd_kernel.argtypes = [P, P, P, P, I, I, I, I, I, I, F, I, P, Z, P]
            L.sage_attn_fwd_kernel.restype = I
            L.sage_quant_prep_kv.argtypes = [P, P, I, I, I, I, P, P, P, P, P, P, Z, P]
            L.sage_quant_prep_kv.restype = I
            L.sage_attn_fwd_kv_prepped.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, P]
            L.sage_attn_fwd_kv_prepped.restype = I
            L.sage_auto_design.argtypes = [I, I, I, I, I, I, ctypes.POINTER(I)]
            L.sage_auto_design.restype = I
            L.sage_debug_qk_int32.argtypes = [P, P, I, I, I, I, I, P, I, P, P]
            L.sage_debug_qk_int32.restype = I
            L.sage_debug_codecs.argtypes = [P, I, P, P, P]
            L.sage_debug_codecs.restype = I
            L.sage_debug_epoch_trace.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, I, P, P, P, P,
                                                 P]
            L.sage_debug_epoch_trace.restype = I
            L.sage_debug_epoch_trace_kv.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P, P, P, P, P]
            L.sage_debug_epoch_trace_kv.restype = I
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().sage_status_str(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != SAGE_OK:
        raise SageError(fn, status)
