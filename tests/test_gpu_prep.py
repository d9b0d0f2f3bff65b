"""sage_quant_prep against the oracle, bit for bit: K channel means, INT8 codes
and scales of Q and K, E4M3 codes and scales of V, on every head of every
named workload at full size and on ragged and degenerate shapes."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import quantized_exact_attention_smooth_amd as sage
from _parity import assert_prep_equal, gpu_prep_numpy, oracle_preps, say

pytestmark = pytest.mark.gpu


def _run(q, k, v, dev):
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    p = sage.quant_prep(qg, kg, vg)
    torch.cuda.synchronize()
    g = gpu_prep_numpy(p)
    del p, qg, kg, vg
    return g


@pytest.mark.parametrize("idx", range(len(si.WORKLOADS)))
def test_prep_bit_exact_on_workload(idx, gpu_device):
    w = si.WORKLOADS[idx]
    say(f"prep parity: {w.name}")
    q, k, v = si.workload_qkv(w)
    g = _run(q, k, v, gpu_device)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    # all heads, in groups to bound host memory
    for i in range(0, len(heads), 16):
        orc = oracle_preps(q, k, v, heads[i:i + 16])
        for (b, h), o in orc.items():
            assert o["exact_mean"]
            assert_prep_equal(g, o, b, h)


# Lkv = 1024 and 1025 sit on either side of the largest key count whose
# statistics splits the quantization workgroups reduce themselves (four splits
# of 256 keys); longer keys take the separate finalize launch.
SHAPES = [(1, 1, 1, 1, 64), (1, 2, 63, 65, 128), (2, 1, 64, 64, 64), (1, 1, 65, 1, 128), (1, 3, 1000, 129, 64),
          (1, 1, 129, 1000, 128), (1, 1, 255, 257, 128), (2, 2, 300, 511, 64), (1, 2, 100, 1024, 128),
          (1, 2, 100, 1025, 64)]


@pytest.mark.parametrize("B,H,Lq,Lkv,D", SHAPES)
def test_prep_bit_exact_on_ragged_shapes(B, H, Lq, Lkv, D, gpu_device):
    say(f"prep parity: shape {(B, H, Lq, Lkv, D)}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", 3.0, seed=Lq + 7 * Lkv + D)
    g = _run(q, k, v, gpu_device)
    for (b, h), o in oracle_preps(q, k, v, [(b, h) for b in range(B) for h in range(H)]).items():
        assert_prep_equal(g, o, b, h)
    nqb, nkb = -(-Lq // 64), -(-Lkv // 64)
    assert np.all(g["q_i8"][:, :, Lq:] == 0) and np.all(g["k_i8"][:, :, Lkv:] == 0)
    assert np.all(g["v8"][:, :, Lkv:] == 0)
    assert g["q_scale"].shape == (B, H, nqb) and g["k_scale"].shape == (B, H, nkb)


def test_prep_degenerate_blocks(gpu_device):
    """Zero Q blocks, K constant per channel (smoothed to exactly zero), a
    zero V channel, and outlier values: scales 0 and codes 0 where the block
    or channel is zero."""
    B, H, L, D = 1, 2, 200, 64
    q, k, v = si.make_qkv(B, H, L, L, D, "normal", 0.0, seed=5)
    q[:, 0, :64] = 0
    k[:, 1] = torch.linspace(-5, 5, D).to(torch.bfloat16)[None, None, :]
    v[:, 0, :, 3] = 0
    k[0, 0, 17, 5] = 3000.0
    say("prep parity: degenerate blocks")
    g = _run(q, k, v, gpu_device)
    for (b, h), o in oracle_preps(q, k, v, [(0, 0), (0, 1)]).items():
        assert_prep_equal(g, o, b, h)
    assert g["q_scale"][0, 0, 0] == 0 and np.all(g["q_i8"][0, 0, :64] == 0)
    assert np.all(g["k_scale"][0, 1] == 0) and np.all(g["k_i8"][0, 1] == 0)
    assert g["v_scale"][0, 0, 3] == 0 and np.all(g["v8"][0, 0, :, 3] == 0)


def test_prep_tiny_and_subnormal_scales(gpu_device):
    """Blocks and channels whose scale is below 2^-60, where the quotients
    are taken by division rather than from the reciprocal, and subnormal bf16
    inputs (scales that are fp32 subnormals): codes and scales bit-exact
    against the oracle's IEEE single divisions."""
    B, H, L, D = 1, 2, 260, 128
    q, k, v = si.make_qkv(B, H, L, L, D, "normal", 1.0, seed=6)
    q, k, v = q.clone(), k.clone(), v.clone()
    q[:, 0, :64] *= 1e-30
    q[:, 0, 64:128] *= 1e-39
    q[:, 1, 192:] *= 1e-25
    k[:, 0] *= 1e-30           # every K block of head 0 after smoothing
    k[:, 1, :, :40] *= 1e-39   # subnormal channels of head 1
    v[:, 0, :, 5] *= 1e-30     # one V channel below the fast path
    v[:, 1, :, :16] *= 1e-39
    say("prep parity: tiny and subnormal scales")
    g = _run(q, k, v, gpu_device)
    for (b, h), o in oracle_preps(q, k, v, [(0, 0), (0, 1)]).items():
        assert_prep_equal(g, o, b, h)
    assert 0 < g["q_scale"][0, 0, 1] < 2.0 ** -126  # a subnormal scale was produced and kept


def test_prep_is_deterministic(gpu_device):
    w = si.WORKLOADS[1]
    q, k, v = (t.to(gpu_device) for t in si.workload_qkv(w))
    say("prep determinism x20")
    first = gpu_prep_numpy(sage.quant_prep(q, k, v))
    for _ in range(20):
        again = gpu_prep_numpy(sage.quant_prep(q, k, v))
        for n in first:
            assert np.array_equal(first[n].view(np.uint8), again[n].view(np.uint8)), n
