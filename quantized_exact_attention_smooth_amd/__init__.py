"""MI355X (gfx950) SageAttention2-style quantized exact attention with K smoothing.

Python face of the C ABI in include/sage_attn.h (same names, torch tensors in
place of raw pointers). Inputs are bf16 CUDA tensors [B, H, L, D] with D in
{64, 128}; outputs are allocated with torch on the same device; calls run on
torch's current stream.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (LIB_PATH, SAGE_BLOCK, SAGE_KERNEL_AUTO, SAGE_KERNEL_ENTRY, SAGE_KERNEL_FUSED,  # noqa: F401
                   SAGE_KERNEL_PERSISTENT, SAGE_KERNEL_SPLIT, SAGE_KERNEL_WIDE, SageError, check, lib,
                   status_str)

__all__ = ["workspace_bytes", "prep_scratch_bytes", "quant_prep", "attn_fwd_prepped", "attn_fwd", "quant_prep_kv",
           "attn_fwd_kv_prepped", "auto_design",
           "debug_qk_int32", "debug_codecs", "debug_epoch_trace", "debug_epoch_trace_kv", "SageError", "status_str", "LIB_PATH",
           "SAGE_KERNEL_AUTO", "SAGE_KERNEL_FUSED", "SAGE_KERNEL_SPLIT", "SAGE_KERNEL_PERSISTENT", "SAGE_KERNEL_WIDE",
           "SAGE_KERNEL_ENTRY"]


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t.data_ptr()


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, H, Lq, D = q.shape
    Lkv = k.shape[2]
    if tuple(k.shape) != (B, H, Lkv, D):
        raise ValueError("k must be [B, H, Lkv, D] matching q")
    return B, H, Lq, Lkv, D


def workspace_bytes(B: int, H: int, Lq: int, Lkv: int, D: int) -> int:
    n = ctypes.c_size_t(0)
    check("sage_workspace_bytes", lib().sage_workspace_bytes(B, H, Lq, Lkv, D, ctypes.byref(n)))
    return n.value


def prep_scratch_bytes(B: int, H: int, Lq: int, Lkv: int, D: int) -> int:
    n = ctypes.c_size_t(0)
    check("sage_prep_scratch_bytes", lib().sage_prep_scratch_bytes(B, H, Lq, Lkv, D, ctypes.byref(n)))
    return n.value


def quant_prep(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, stream=None) -> dict:
    """sage_quant_prep. Returns dict of q_i8, q_scale, k_i8, k_scale, k_mean,
    v_fp8 ([B, H, NKB, D, 64] uint8), v_scale and the shape."""
    B, H, Lq, Lkv, D = _dims(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must match k")
    nqb, nkb = -(-Lq // SAGE_BLOCK), -(-Lkv // SAGE_BLOCK)
    dev = q.device
    r = dict(q_i8=torch.empty((B, H, nqb * SAGE_BLOCK, D), dtype=torch.int8, device=dev),
             q_scale=torch.empty((B, H, nqb), dtype=torch.float32, device=dev),
             k_i8=torch.empty((B, H, nkb * SAGE_BLOCK, D), dtype=torch.int8, device=dev),
             k_scale=torch.empty((B, H, nkb), dtype=torch.float32, device=dev),
             k_mean=torch.empty((B, H, D), dtype=torch.float32, device=dev),
             v_fp8=torch.empty((B, H, nkb, D, SAGE_BLOCK), dtype=torch.uint8, device=dev),
             v_scale=torch.empty((B, H, D), dtype=torch.float32, device=dev))
    nbytes = prep_scratch_bytes(B, H, Lq, Lkv, D)
    scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sage_quant_prep(_dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"),
                               _dev(v, torch.bfloat16, "v"), B, H, Lq, Lkv, D,
                               r["q_i8"].data_ptr(), r["q_scale"].data_ptr(), r["k_i8"].data_ptr(),
                               r["k_scale"].data_ptr(), r["k_mean"].data_ptr(), r["v_fp8"].data_ptr(),
                               r["v_scale"].data_ptr(), scratch.data_ptr(), nbytes, _stream(stream))
    check("sage_quant_prep", st)
    r["_scratch"] = scratch  # keep alive until the stream is done with it
    r["shape"] = (B, H, Lq, Lkv, D)
    return r


def quant_prep_kv(k: torch.Tensor, v: torch.Tensor, stream=None) -> dict:
    """sage_quant_prep_kv: the K/V half of quant_prep. Returns dict of k_i8,
    k_scale, k_mean, v_fp8 ([B, H, NKB, D, 64] uint8), v_scale and
    kv_shape (B, H, Lkv, D)."""
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, H, Lkv, D] of one shape")
    B, H, Lkv, D = k.shape
    nkb = -(-Lkv // SAGE_BLOCK)
    dev = k.device
    r = dict(k_i8=torch.empty((B, H, nkb * SAGE_BLOCK, D), dtype=torch.int8, device=dev),
             k_scale=torch.empty((B, H, nkb), dtype=torch.float32, device=dev),
             k_mean=torch.empty((B, H, D), dtype=torch.float32, device=dev),
             v_fp8=torch.empty((B, H, nkb, D, SAGE_BLOCK), dtype=torch.uint8, device=dev),
             v_scale=torch.empty((B, H, D), dtype=torch.float32, device=dev))
    nbytes = prep_scratch_bytes(B, H, 1, Lkv, D)
    scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sage_quant_prep_kv(_dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"), B, H, Lkv, D,
                                  r["k_i8"].data_ptr(), r["k_scale"].data_ptr(), r["k_mean"].data_ptr(),
                                  r["v_fp8"].data_ptr(), r["v_scale"].data_ptr(), scratch.data_ptr(), nbytes,
                                  _stream(stream))
    check("sage_quant_prep_kv", st)
    r["_scratch"] = scratch
    r["kv_shape"] = (B, H, Lkv, D)
    return r


def attn_fwd_kv_prepped(q: torch.Tensor, kv: dict, causal: bool, sm_scale: float = None,
                        out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """sage_attn_fwd_kv_prepped: bf16 q [B, H, Lq, D] against the K/V operands
    of quant_prep_kv (or quant_prep), Q coded inside the main loop."""
    B, H, Lkv, D = kv["kv_shape"] if "kv_shape" in kv else (*kv["shape"][:2], *kv["shape"][3:])
    if q.dim() != 4 or q.shape[0] != B or q.shape[1] != H or q.shape[3] != D:
        raise ValueError("q must be [B, H, Lq, D] matching the prepared K/V")
    Lq = q.shape[2]
    if out is None:
        out = torch.empty((B, H, Lq, D), dtype=torch.bfloat16, device=q.device)
    st = lib().sage_attn_fwd_kv_prepped(
        _dev(q, torch.bfloat16, "q"), _dev(kv["k_i8"], torch.int8, "k_i8"),
        _dev(kv["k_scale"], torch.float32, "k_scale"), _dev(kv["v_fp8"], torch.uint8, "v_fp8"),
        _dev(kv["v_scale"], torch.float32, "v_scale"), _dev(out, torch.bfloat16, "out"), B, H, Lq, Lkv, D,
        int(bool(causal)), float(sm_scale) if sm_scale else 0.0, _stream(stream))
    check("sage_attn_fwd_kv_prepped", st)
    return out


def auto_design(B: int, H: int, Lq: int, Lkv: int, D: int, whole_path: bool = True) -> int:
    """sage_auto_design: the SAGE_KERNEL_* value SAGE_KERNEL_AUTO selects."""
    d = ctypes.c_int(-1)
    check("sage_auto_design", lib().sage_auto_design(B, H, Lq, Lkv, D, int(bool(whole_path)), ctypes.byref(d)))
    return d.value


def attn_fwd_prepped(prep: dict, causal: bool, sm_scale: float = None, out: torch.Tensor = None,
                     stream=None, kernel: int = SAGE_KERNEL_AUTO) -> torch.Tensor:
    """sage_attn_fwd_prepped_kernel on the dict quant_prep returns (kernel:
    SAGE_KERNEL_AUTO, _FUSED, _SPLIT, _PERSISTENT or _WIDE; _ENTRY needs bf16
    Q and is refused)."""
    B, H, Lq, Lkv, D = prep["shape"]
    if out is None:
        out = torch.empty((B, H, Lq, D), dtype=torch.bfloat16, device=prep["q_i8"].device)
    st = lib().sage_attn_fwd_prepped_kernel(
        _dev(prep["q_i8"], torch.int8, "q_i8"), _dev(prep["q_scale"], torch.float32, "q_scale"),
        _dev(prep["k_i8"], torch.int8, "k_i8"), _dev(prep["k_scale"], torch.float32, "k_scale"),
        _dev(prep["v_fp8"], torch.uint8, "v_fp8"), _dev(prep["v_scale"], torch.float32, "v_scale"),
        _dev(out, torch.bfloat16, "out"), B, H, Lq, Lkv, D, int(bool(causal)),
        float(sm_scale) if sm_scale else 0.0, int(kernel), _stream(stream))
    check("sage_attn_fwd_prepped_kernel", st)
    return out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool, sm_scale: float = None,
             out: torch.Tensor = None, workspace: torch.Tensor = None, stream=None,
             kernel: int = SAGE_KERNEL_AUTO) -> torch.Tensor:
    """sage_attn_fwd (kernel SAGE_KERNEL_AUTO) or sage_attn_fwd_kernel (any
    other design, SAGE_KERNEL_ENTRY included): preparation and main loop.
    workspace (uint8, optional) is reused when large enough."""
    B, H, Lq, Lkv, D = _dims(q, k)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v must match k")
    nbytes = workspace_bytes(B, H, Lq, Lkv, D)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, H, Lq, D), dtype=torch.bfloat16, device=q.device)
    args = (_dev(q, torch.bfloat16, "q"), _dev(k, torch.bfloat16, "k"), _dev(v, torch.bfloat16, "v"),
            _dev(out, torch.bfloat16, "out"), B, H, Lq, Lkv, D, int(bool(causal)),
            float(sm_scale) if sm_scale else 0.0)
    ws = (_dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    if kernel == SAGE_KERNEL_AUTO:
        check("sage_attn_fwd", lib().sage_attn_fwd(*args, *ws))
    else:
        check("sage_attn_fwd_kernel", lib().sage_attn_fwd_kernel(*args, int(kernel), *ws))
    return out


def debug_epoch_trace(prep: dict, b: int, h: int, row0: int, causal: bool, sm_scale: float = None,
                      stream=None, kernel: int = SAGE_KERNEL_AUTO) -> dict:
    """sage_debug_epoch_trace: per-epoch checkpoints of rows row0 .. row0+31 of
    head (b, h). Returns stats [32, NKB+1, 4] (NaN where not written), p8
    [32, NKB, 64] uint8 (0xFF where not written), pv and ro [32, NKB, D] and
    out."""
    B, H, Lq, Lkv, D = prep["shape"]
    nkb = -(-Lkv // SAGE_BLOCK)
    dev = prep["q_i8"].device
    stats = torch.full((32, nkb + 1, 4), float("nan"), dtype=torch.float32, device=dev)
    p8 = torch.full((32, nkb, SAGE_BLOCK), 0xFF, dtype=torch.uint8, device=dev)
    pv = torch.full((32, nkb, D), float("nan"), dtype=torch.float32, device=dev)
    ro = torch.full((32, nkb, D), float("nan"), dtype=torch.float32, device=dev)
    out = torch.zeros((B, H, Lq, D), dtype=torch.bfloat16, device=dev)
    st = lib().sage_debug_epoch_trace(
        _dev(prep["q_i8"], torch.int8, "q_i8"), _dev(prep["q_scale"], torch.float32, "q_scale"),
        _dev(prep["k_i8"], torch.int8, "k_i8"), _dev(prep["k_scale"], torch.float32, "k_scale"),
        _dev(prep["v_fp8"], torch.uint8, "v_fp8"), _dev(prep["v_scale"], torch.float32, "v_scale"),
        _dev(out, torch.bfloat16, "out"), B, H, Lq, Lkv, D, int(bool(causal)),
        float(sm_scale) if sm_scale else 0.0, int(kernel), int(b), int(h), int(row0), stats.data_ptr(),
        p8.data_ptr(), pv.data_ptr(), ro.data_ptr(), _stream(stream))
    check("sage_debug_epoch_trace", st)
    return dict(stats=stats, p8=p8, pv=pv, ro=ro, out=out)


def debug_epoch_trace_kv(q: torch.Tensor, kv: dict, b: int, h: int, row0: int, causal: bool,
                         sm_scale: float = None, stream=None) -> dict:
    """sage_debug_epoch_trace_kv: the checkpoints of debug_epoch_trace for the
    entry design's main loop (bf16 q against the K/V operands of
    quant_prep_kv or quant_prep)."""
    B, H, Lkv, D = kv["kv_shape"] if "kv_shape" in kv else (*kv["shape"][:2], *kv["shape"][3:])
    Lq = q.shape[2]
    nkb = -(-Lkv // SAGE_BLOCK)
    dev = q.device
    stats = torch.full((32, nkb + 1, 4), float("nan"), dtype=torch.float32, device=dev)
    p8 = torch.full((32, nkb, SAGE_BLOCK), 0xFF, dtype=torch.uint8, device=dev)
    pv = torch.full((32, nkb, D), float("nan"), dtype=torch.float32, device=dev)
    ro = torch.full((32, nkb, D), float("nan"), dtype=torch.float32, device=dev)
    out = torch.zeros((B, H, Lq, D), dtype=torch.bfloat16, device=dev)
    st = lib().sage_debug_epoch_trace_kv(
        _dev(q, torch.bfloat16, "q"), _dev(kv["k_i8"], torch.int8, "k_i8"),
        _dev(kv["k_scale"], torch.float32, "k_scale"), _dev(kv["v_fp8"], torch.uint8, "v_fp8"),
        _dev(kv["v_scale"], torch.float32, "v_scale"), _dev(out, torch.bfloat16, "out"), B, H, Lq, Lkv, D,
        int(bool(causal)), float(sm_scale) if sm_scale else 0.0, int(b), int(h), int(row0), stats.data_ptr(),
        p8.data_ptr(), pv.data_ptr(), ro.data_ptr(), _stream(stream))
    check("sage_debug_epoch_trace_kv", st)
    return dict(stats=stats, p8=p8, pv=pv, ro=ro, out=out)


def debug_qk_int32(prep: dict, tiles, stream=None) -> torch.Tensor:
    """sage_debug_qk_int32: int32 [n, 64, 64] QK tiles for (b, h, qb, kb) records."""
    B, H, Lq, Lkv, D = prep["shape"]
    arr = (ctypes.c_int * (4 * len(tiles)))(*[int(x) for t in tiles for x in t])
    acc = torch.empty((max(len(tiles), 1), SAGE_BLOCK, SAGE_BLOCK), dtype=torch.int32,
                      device=prep["q_i8"].device)
    st = lib().sage_debug_qk_int32(_dev(prep["q_i8"], torch.int8, "q_i8"), _dev(prep["k_i8"], torch.int8, "k_i8"),
                                   B, H, Lq, Lkv, D, ctypes.cast(arr, ctypes.c_void_p), len(tiles),
                                   acc.data_ptr(), _stream(stream))
    check("sage_debug_qk_int32", st)
    return acc[:len(tiles)]


def debug_codecs(x: torch.Tensor, stream=None):
    """sage_debug_codecs: (E4M3FN codes, bf16 bits as int16) of fp32 values."""
    n = x.numel()
    p8 = torch.empty(n, dtype=torch.uint8, device=x.device)
    bf = torch.empty(n, dtype=torch.int16, device=x.device)
    st = lib().sage_debug_codecs(_dev(x, torch.float32, "x"), n, p8.data_ptr(), bf.data_ptr(), _stream(stream))
    check("sage_debug_codecs", st)
    return p8, bf


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
