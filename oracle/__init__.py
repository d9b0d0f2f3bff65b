"""Python binding of the CPU oracle (oracle/sage_oracle.c).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package. The HIP library never does, and this
package imports nothing from the HIP library's package.

The C library is compiled with gcc on first use (or by build()); the
functions below marshal numpy arrays and run independent heads or row ranges
on a thread pool (the C calls release the GIL).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
BLOCK = 64

_lock = threading.Lock()
_lib = None


# ORACLE_SANITIZE=1 selects a build with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only; the process must preload the
# sanitizer runtimes, e.g. LD_PRELOAD="$(gcc -print-file-name=libasan.so)
# $(gcc -print-file-name=libubsan.so)" ASAN_OPTIONS=detect_leaks=0).
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _sanitize() -> bool:
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def build(force: bool = False, sanitize: bool = None) -> str:
    """Compile liboracle.so with gcc (plain C11, -O2, no FMA contraction);
    with sanitize (default: ORACLE_SANITIZE=1) the instrumented variant."""
    sanitize = _sanitize() if sanitize is None else sanitize
    lib = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", *(_SAN_FLAGS if sanitize else []), "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P = ctypes.c_void_p
            I = ctypes.c_int
            L = ctypes.c_long
            lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_to_f32.restype = ctypes.c_float
            lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
            lib.orc_f32_to_bf16.restype = ctypes.c_uint16
            lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_decode.restype = ctypes.c_double
            lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
            lib.orc_e4m3_encode.restype = ctypes.c_uint8
            for name in ("orc_bf16_round_array", "orc_e4m3_encode_array", "orc_e4m3_decode_array"):
                getattr(lib, name).argtypes = [P, P, L]
                getattr(lib, name).restype = None
            lib.orc_prep_head.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, P, P]
            lib.orc_prep_head.restype = I
            lib.orc_attn_rows.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_float, I, I, P]
            lib.orc_attn_rows.restype = I
            lib.orc_attn_row_trace.argtypes = [P, P, P, P, P, P, I, I, I, I, ctypes.c_float, I, P, P, P, P, P]
            lib.orc_attn_row_trace.restype = I
            for name in ("orc_attn_unquant_rows", "orc_attn_ref_rows"):
                getattr(lib, name).argtypes = [P, P, P, I, I, I, I, ctypes.c_double, I, I, P]
                getattr(lib, name).restype = I
            lib.orc_sage_head.argtypes = [P, P, P, I, I, I, I, ctypes.c_float, P]
            lib.orc_sage_head.restype = I
            _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    """Cores this process may use, capped by OMP_NUM_THREADS when it is set
    (the machine's share can be smaller than what the kernel reports)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


# ----------------------------------------------------------------- codecs

def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 values -> bf16 bits (uint16), nearest-even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_round_array(_p(x), _p(out), x.size)
    return out


def e4m3_encode(x) -> np.ndarray:
    """float32 values -> E4M3FN bytes (nearest-even, saturating)."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_e4m3_encode_array(_p(x), _p(out), x.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_array(_p(c), _p(out), c.size)
    return out


# ----------------------------------------------------------- preparation

def prep_head(q_bits, k_bits, v_bits, smooth: bool = True) -> dict:
    """One head: q [Lq, D], k/v [Lkv, D] bf16 bits -> prepared operands.

    Returns dict(q8 [nqb*64, D] int8, q_scale [nqb] f32, k8, k_scale, k_mean [D],
    v8 [nkb*64, D] uint8 token-major, v_scale [D], exact_mean bool).
    """
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    Lq, D = q.shape
    Lkv = k.shape[0]
    nqb, nkb = -(-Lq // BLOCK), -(-Lkv // BLOCK)
    r = dict(q8=np.empty((nqb * BLOCK, D), np.int8), q_scale=np.empty(nqb, np.float32),
             k8=np.empty((nkb * BLOCK, D), np.int8), k_scale=np.empty(nkb, np.float32),
             k_mean=np.empty(D, np.float32), v8=np.empty((nkb * BLOCK, D), np.uint8),
             v_scale=np.empty(D, np.float32))
    st = _load().orc_prep_head(_p(q), _p(k), _p(v), Lq, Lkv, D, int(bool(smooth)), _p(r["q8"]),
                               _p(r["q_scale"]), _p(r["k8"]), _p(r["k_scale"]), _p(r["k_mean"]),
                               _p(r["v8"]), _p(r["v_scale"]))
    if st < 0:
        raise MemoryError("oracle prep allocation failed")
    r["exact_mean"] = (st == 0)
    r["Lq"], r["Lkv"], r["D"] = Lq, Lkv, D
    return r


def attn_rows(prep: dict, causal: bool, sm_scale: float, r0: int = 0, r1: int = None) -> np.ndarray:
    """Quantized epoch loop for rows [r0, r1); returns bf16 bits [r1-r0, D]."""
    Lq, Lkv, D = prep["Lq"], prep["Lkv"], prep["D"]
    r1 = Lq if r1 is None else r1
    out = np.zeros((Lq, D), np.uint16)
    st = _load().orc_attn_rows(_p(prep["q8"]), _p(prep["q_scale"]), _p(prep["k8"]), _p(prep["k_scale"]),
                               _p(prep["v8"]), _p(prep["v_scale"]), Lq, Lkv, D, int(bool(causal)),
                               float(sm_scale), int(r0), int(r1), _p(out))
    if st == 2:
        raise ArithmeticError("INT8 dot product outside the int32-exact range")
    if st < 0:
        raise MemoryError("oracle allocation failed")
    return out[r0:r1]


def attn_row_trace(prep: dict, causal: bool, sm_scale: float, i: int) -> dict:
    """Per-epoch checkpoints of query row i of the quantized epoch loop:
    stats [NKB+1, 4] (m, l, alpha, 0 after each epoch; r, l at the end),
    p8 [NKB, 64] uint8, pv and ro [NKB, D] float32, out [D] bf16 bits."""
    Lq, Lkv, D = prep["Lq"], prep["Lkv"], prep["D"]
    nkb = -(-Lkv // BLOCK)
    stats = np.zeros((nkb + 1, 4), np.float32)
    p8 = np.zeros((nkb, BLOCK), np.uint8)
    pv = np.zeros((nkb, D), np.float32)
    ro = np.zeros((nkb, D), np.float32)
    out = np.zeros(D, np.uint16)
    st = _load().orc_attn_row_trace(_p(prep["q8"]), _p(prep["q_scale"]), _p(prep["k8"]), _p(prep["k_scale"]),
                                    _p(prep["v8"]), _p(prep["v_scale"]), Lq, Lkv, D, int(bool(causal)),
                                    float(sm_scale), int(i), _p(out), _p(stats), _p(p8), _p(pv), _p(ro))
    if st == 2:
        raise ArithmeticError("INT8 dot product outside the int32-exact range")
    if st < 0:
        raise MemoryError("oracle allocation failed")
    return dict(stats=stats, p8=p8, pv=pv, ro=ro, out=out)


def attn_rows_parallel(prep: dict, causal: bool, sm_scale: float, r0: int = 0, r1: int = None,
                       threads: int = None, chunk: int = BLOCK) -> np.ndarray:
    Lq = prep["Lq"]
    r1 = Lq if r1 is None else r1
    threads = threads or default_threads()
    spans = [(a, min(a + chunk, r1)) for a in range(r0, r1, chunk)]
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda s: attn_rows(prep, causal, sm_scale, s[0], s[1]), spans))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, prep["D"]), np.uint16)


def sage_head(q_bits, k_bits, v_bits, causal: bool, sm_scale: float) -> np.ndarray:
    """The whole path for one head in one C call: bf16 bits in, bf16 bits out."""
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    Lq, D = q.shape
    out = np.zeros((Lq, D), np.uint16)
    st = _load().orc_sage_head(_p(q), _p(k), _p(v), Lq, k.shape[0], D, int(bool(causal)),
                               float(sm_scale), _p(out))
    if st != 0:
        raise RuntimeError(f"oracle head failed with status {st}")
    return out


# ------------------------------------------------- fp64 references (ii), (iii)

def _fp64_call(name, q, k, v, causal, sm_scale, r0, r1):
    q = _c(q, np.float64)
    k = _c(k, np.float64)
    v = _c(v, np.float64)
    Lq, D = q.shape
    r1 = Lq if r1 is None else r1
    out = np.zeros((Lq, D), np.float64)
    st = getattr(_load(), name)(_p(q), _p(k), _p(v), Lq, k.shape[0], D, int(bool(causal)), float(sm_scale),
                                int(r0), int(r1), _p(out))
    if st != 0:
        raise MemoryError("oracle allocation failed")
    return out[r0:r1]


def attn_unquant(q, k, v, causal: bool, sm_scale: float, r0: int = 0, r1: int = None) -> np.ndarray:
    """(ii): the 64-key epoch loop in fp64 with identity quantizers."""
    return _fp64_call("orc_attn_unquant_rows", q, k, v, causal, sm_scale, r0, r1)


def attn_ref(q, k, v, causal: bool, sm_scale: float, r0: int = 0, r1: int = None) -> np.ndarray:
    """(iii): brute-force fp64 softmax attention."""
    return _fp64_call("orc_attn_ref_rows", q, k, v, causal, sm_scale, r0, r1)


def attn_ref_parallel(q, k, v, causal, sm_scale, r0=0, r1=None, threads=None, chunk=BLOCK):
    r1 = q.shape[0] if r1 is None else r1
    threads = threads or default_threads()
    spans = [(a, min(a + chunk, r1)) for a in range(r0, r1, chunk)]
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda s: attn_ref(q, k, v, causal, sm_scale, s[0], s[1]), spans))
    return np.concatenate(parts, axis=0)


def run_heads(fn, items, threads: int = None):
    """Map fn over independent items (heads, blocks) on a thread pool."""
    threads = threads or default_threads()
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))
