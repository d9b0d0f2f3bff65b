"""The C-ABI library loads, exports every entry point include/sage_attn.h
declares, and rejects bad arguments before any GPU call (CPU only: no
compute call is made; the pointers passed are never dereferenced on the
error paths tested)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")


@pytest.fixture(scope="module")
def lib():
    from quantized_exact_attention_smooth_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from quantized_exact_attention_smooth_amd import build
        build.build()
    return _lib.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s*(sage_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("sage_quant_prep", "sage_quant_prep_noalloc", "sage_attn_fwd", "sage_attn_fwd_prepped",
              "sage_attn_fwd_prepped_kernel", "sage_attn_fwd_kernel", "sage_quant_prep_kv",
              "sage_attn_fwd_kv_prepped", "sage_auto_design", "sage_debug_epoch_trace_kv",
              "sage_workspace_bytes",
              "sage_prep_scratch_bytes", "sage_debug_qk_int32", "sage_debug_codecs", "sage_debug_epoch_trace",
              "sage_status_str"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from quantized_exact_attention_smooth_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(sage_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code, name in [(0, "SAGE_OK"), (-1, "SAGE_ERR_INVALID_ARG"), (-2, "SAGE_ERR_UNSUPPORTED"),
                       (-3, "SAGE_ERR_WORKSPACE"), (-4, "SAGE_ERR_HIP"), (7, "SAGE_ERR_UNKNOWN")]:
        assert lib.sage_status_str(code).decode() == name


def _ws(lib, *dims):
    n = ctypes.c_size_t(0)
    return lib.sage_workspace_bytes(*dims, ctypes.byref(n)), n.value


def test_size_queries_validate_shapes(lib):
    assert _ws(lib, 2, 32, 4096, 4096, 128)[0] == 0
    assert _ws(lib, 0, 1, 64, 64, 64)[0] == -1
    assert _ws(lib, 1, 1, 0, 64, 64)[0] == -1
    assert _ws(lib, 1, 1, 64, -5, 64)[0] == -1
    assert _ws(lib, 1, 1, 64, 64, 96)[0] == -2
    assert _ws(lib, 1, 1, 64, 64, 256)[0] == -2
    assert _ws(lib, 1 << 20, 1 << 10, 1 << 12, 1 << 12, 128)[0] == -1  # overflow guard
    # one head's K codes must stay below 2 GiB (32-bit buffer offsets)
    assert _ws(lib, 1, 1, 64, (1 << 24) - 64, 128)[0] == 0
    assert _ws(lib, 1, 1, 64, (1 << 24) - 63, 128)[0] == -1
    assert _ws(lib, 1, 1, 64, 1 << 25, 64)[0] == -1
    # the preparation pass launches B*H*(NQB + 2*NKB) workgroups in one dimension
    assert _ws(lib, 1 << 14, 1 << 15, 1, 1, 64)[0] == 0
    assert _ws(lib, 1 << 15, 1 << 15, 1, 1, 64)[0] == -1
    assert lib.sage_workspace_bytes(1, 1, 64, 64, 64, None) == -1


def test_workspace_size_covers_every_part(lib):
    B, H, L, D = 2, 32, 4096, 128
    st, n = _ws(lib, B, H, L, L, D)
    codes = 3 * B * H * L * D
    assert st == 0 and n >= codes and n < codes * 1.2
    st, n1 = _ws(lib, 1, 1, 1000, 1000, 64)
    assert st == 0 and n1 >= 3 * 1024 * 64


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced on these paths


def test_attn_fwd_rejects_bad_arguments_without_touching_the_gpu(lib):
    _, need = _ws(lib, 1, 2, 128, 128, 128)
    f = lib.sage_attn_fwd
    assert f(None, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, FAKE, need, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 96, 0, 0.0, FAKE, need, None) == -2
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, FAKE, need - 1, None) == -3
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 2, 0.0, FAKE, need, None) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, float("nan"), FAKE, need, None) == -1
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, odd, need, None) == -1
    assert f(FAKE, FAKE, FAKE, odd, 1, 2, 128, 128, 128, 0, 0.0, FAKE, need, None) == -1
    g = lib.sage_attn_fwd_kernel  # every design value and argument checked before any launch
    for design in (-1, 6):
        assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, design, FAKE, need, None) == -1
    for design in range(6):
        assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, design, FAKE, need - 1, None) == -3
        assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 2, 0.0, design, FAKE, need, None) == -1
        assert g(odd, FAKE, FAKE, FAKE, 1, 2, 128, 128, 128, 0, 0.0, design, FAKE, need, None) == -1
        assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 128, 128, 96, 0, 0.0, design, FAKE, need, None) == -2


def test_prep_and_prepped_reject_bad_arguments(lib):
    n = ctypes.c_size_t(0)
    assert lib.sage_prep_scratch_bytes(1, 1, 64, 64, 64, ctypes.byref(n)) == 0
    p = lib.sage_quant_prep
    args = [FAKE] * 3 + [1, 1, 64, 64, 64] + [FAKE] * 8 + [n.value, None]
    assert p(*args[:8], None, *args[9:]) == -1
    short = list(args)
    short[16] = n.value - 1
    assert p(*short) == -3
    odd = list(args)
    odd[8] = ctypes.c_void_p((1 << 20) + 1)
    assert p(*odd) == -1
    na = lib.sage_quant_prep_noalloc  # checks shapes, pointers and its 16 MiB scratch bound before any GPU call
    assert na(FAKE, FAKE, FAKE, 1, 64, 64, 65536, 128, *([FAKE] * 7), None) == -3
    assert na(None, FAKE, FAKE, 1, 1, 64, 64, 128, *([FAKE] * 7), None) == -1
    assert na(FAKE, FAKE, FAKE, 1, 1, 64, 64, 96, *([FAKE] * 7), None) == -2
    a = lib.sage_attn_fwd_prepped
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 64, 64, 0, 0.0, None) == -1
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 32, 0, 0.0, None) == -2
    assert a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 3, 0.0, None) == -1
    k = lib.sage_attn_fwd_prepped_kernel
    assert k(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 0, 0.0, 5, None) == -1   # entry: bf16 Q
    assert k(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 0, 0.0, 6, None) == -1   # unknown design
    assert k(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 0, 0.0, -1, None) == -1
    assert k(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 64, 64, 0, 0.0, 2, None) == -1
    assert k(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 32, 0, 0.0, 1, None) == -2


def test_kv_prep_and_kv_prepped_reject_bad_arguments(lib):
    n = ctypes.c_size_t(0)
    assert lib.sage_prep_scratch_bytes(1, 1, 1, 64, 64, ctypes.byref(n)) == 0
    p = lib.sage_quant_prep_kv
    args = [FAKE, FAKE, 1, 1, 64, 64] + [FAKE] * 6 + [n.value, None]
    assert p(*args[:6], None, *args[7:]) == -1                  # missing k_i8
    short = list(args)
    short[12] = n.value - 1
    assert p(*short) == -3
    assert p(FAKE, FAKE, 1, 1, 64, 96, *args[6:]) == -2          # unsupported D
    odd = list(args)
    odd[0] = ctypes.c_void_p((1 << 20) + 8)
    assert p(*odd) == -1                                         # k not 16-byte aligned
    a = lib.sage_attn_fwd_kv_prepped
    ok = [FAKE] * 6 + [1, 1, 64, 64, 64, 0, 0.0, None]
    assert a(*ok[:0], None, *ok[1:]) == -1                       # missing q
    assert a(ctypes.c_void_p((1 << 20) + 2), *ok[1:]) == -1      # q not 16-byte aligned
    assert a(*ok[:5], None, *ok[6:]) == -1                       # missing out
    assert a(*ok[:10], 32, *ok[11:]) == -2                       # unsupported D
    assert a(*ok[:11], 3, *ok[12:]) == -1                        # causal not 0/1


def test_auto_design_reports_the_choice(lib):
    d = ctypes.c_int(-1)
    for shape, whole, want in [((2, 32, 4096, 4096, 128), 1, 5), ((2, 32, 4096, 4096, 128), 0, 1),
                               ((1, 8, 1000, 1000, 128), 1, 2), ((1, 1, 128, 192, 128), 0, 2),
                               ((4, 16, 8192, 8192, 64), 1, 5), ((1, 24, 32760, 32760, 128), 0, 1)]:
        assert lib.sage_auto_design(*shape, whole, ctypes.byref(d)) == 0 and d.value == want, (shape, whole)
    assert lib.sage_auto_design(1, 1, 64, 64, 96, 1, ctypes.byref(d)) == -2
    assert lib.sage_auto_design(1, 1, 64, 64, 64, 2, ctypes.byref(d)) == -1
    assert lib.sage_auto_design(1, 1, 64, 64, 64, 1, None) == -1


def test_debug_qk_rejects_out_of_range_tiles(lib):
    bad = (ctypes.c_int * 4)(0, 0, 2, 0)  # query block 2 of a 128-row head does not exist
    assert lib.sage_debug_qk_int32(FAKE, FAKE, 1, 1, 128, 128, 64, bad, 1, FAKE, None) == -1
    neg = (ctypes.c_int * 4)(0, -1, 0, 0)
    assert lib.sage_debug_qk_int32(FAKE, FAKE, 1, 1, 128, 128, 64, neg, 1, FAKE, None) == -1
    assert lib.sage_debug_codecs(None, 4, FAKE, FAKE, None) == -1
    t = lib.sage_debug_epoch_trace
    ok = [FAKE] * 7 + [2, 3, 128, 128, 64, 1, 0.0]
    assert t(*ok, 1, 2, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1       # b out of range
    assert t(*ok, 1, 0, 3, 0, FAKE, FAKE, FAKE, FAKE, None) == -1       # h out of range
    assert t(*ok, 2, 0, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == -1      # row0 not a multiple of 32
    assert t(*ok, 1, 0, 0, 128, FAKE, FAKE, FAKE, FAKE, None) == -1     # row0 >= Lq
    assert t(*ok, 1, 0, 0, 0, None, FAKE, FAKE, FAKE, None) == -1       # missing stats
    assert t(*ok, 2, 0, 0, 0, FAKE, FAKE, None, FAKE, None) == -1       # missing pv
    assert t(*ok, 5, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1       # entry design: not traced
    assert t(*ok, 6, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1       # unknown design
    tk = lib.sage_debug_epoch_trace_kv
    okk = [FAKE] * 6 + [2, 3, 128, 128, 64, 1, 0.0]
    assert tk(None, *okk[1:], 0, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1      # missing q
    assert tk(*okk, 2, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == -1                # b out of range
    assert tk(*okk, 0, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == -1               # row0 not a multiple of 32
    assert tk(*okk, 0, 0, 0, FAKE, FAKE, None, FAKE, None) == -1                # missing pv
    assert lib.sage_debug_codecs(FAKE, 0, FAKE, FAKE, None) == 0
