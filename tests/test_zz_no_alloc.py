"""sage_quant_prep_noalloc, the preparation entry point that allocates
nothing (its scratch is a static device array in the library), against
sage_quant_prep: bit-identical outputs on two calls in a row, the second on
a smaller input, so that the second call runs on the array the first one
left behind. The prepared operands of both then give the same attention
output."""
import ctypes

import numpy as np
import pytest
import torch

import seeded_inputs as si
import quantized_exact_attention_smooth_amd as sage
from quantized_exact_attention_smooth_amd import _lib

pytestmark = pytest.mark.gpu

NAMES = ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_fp8", "v_scale")


def _noalloc(q, k, v):
    B, H, Lq, D = q.shape
    Lkv = k.shape[2]
    nqb, nkb = -(-Lq // 64), -(-Lkv // 64)
    dev = q.device
    # outputs allocated by the caller (here, before the call)
    o = dict(q_i8=torch.full((B, H, nqb * 64, D), 0x55, dtype=torch.int8, device=dev),
             q_scale=torch.full((B, H, nqb), float("nan"), dtype=torch.float32, device=dev),
             k_i8=torch.full((B, H, nkb * 64, D), 0x55, dtype=torch.int8, device=dev),
             k_scale=torch.full((B, H, nkb), float("nan"), dtype=torch.float32, device=dev),
             k_mean=torch.full((B, H, D), float("nan"), dtype=torch.float32, device=dev),
             v_fp8=torch.full((B, H, nkb, D, 64), 0x55, dtype=torch.uint8, device=dev),
             v_scale=torch.full((B, H, D), float("nan"), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    st = _lib.lib().sage_quant_prep_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Lq, Lkv, D,
                                            *(o[n].data_ptr() for n in NAMES),
                                            torch.cuda.current_stream().cuda_stream)
    _lib.check("sage_quant_prep_noalloc", st)
    o["shape"] = (B, H, Lq, Lkv, D)
    return o


def _bits(t):
    a = t.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a


# The second call of each pair is smaller than the first. In the first two
# pairs both calls take the two-pass preparation, which uses the scratch
# (the second call's is a finalize launch, or the finalize folded into the
# quantization pass: at most 4 splits). The third pair's second call is a
# short key set, prepared in one launch without the scratch.
@pytest.mark.parametrize("first,second", [((2, 3, 1000, 1300, 128, "normal"), (1, 2, 1000, 1100, 64, "normal")),
                                          ((1, 4, 4096, 4096, 128, "normal"),
                                           (1, 4, 500, 1000, 128, "student_t_outlier")),
                                          ((1, 2, 2000, 2100, 128, "normal"),
                                           (1, 1, 65, 130, 128, "student_t_outlier"))])
def test_noalloc_prep_equals_prep_on_two_calls(first, second, gpu_device):
    for i, (B, H, Lq, Lkv, D, dist) in enumerate((first, second)):
        print(f"noalloc prep call {i}: shape {(B, H, Lq, Lkv, D)} {dist}", flush=True)
        q, k, v = (t.to(gpu_device) for t in si.make_qkv(B, H, Lq, Lkv, D, dist, 3.0, seed=40 + i))
        ref = sage.quant_prep(q, k, v)
        got = _noalloc(q, k, v)
        torch.cuda.synchronize()
        for n in NAMES:
            assert np.array_equal(_bits(got[n]), _bits(ref[n])), (i, n)
        a = sage.attn_fwd_prepped(ref, True, None)
        b = sage.attn_fwd_prepped(got, True, None)
        torch.cuda.synchronize()
        assert np.array_equal(si.bf16_bits(a), si.bf16_bits(b)), i


def test_noalloc_prep_rejects_scratch_beyond_its_array(gpu_device):
    """A shape whose preparation scratch exceeds the 16 MiB array is refused
    before any GPU work (no pointer is dereferenced)."""
    fake = ctypes.c_void_p(1 << 20)
    n = ctypes.c_size_t(0)
    _lib.check("sage_prep_scratch_bytes", _lib.lib().sage_prep_scratch_bytes(1, 64, 64, 65536, 128, ctypes.byref(n)))
    assert n.value > 16 << 20
    st = _lib.lib().sage_quant_prep_noalloc(fake, fake, fake, 1, 64, 64, 65536, 128, *([fake] * 7), None)
    assert st == _lib.SAGE_ERR_WORKSPACE
