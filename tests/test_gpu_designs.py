"""The other main-loop designs against the oracle and against the fused
design: the wave-specialised one (SAGE_KERNEL_SPLIT), the persistent one
(SAGE_KERNEL_PERSISTENT, fused waves in workgroups fed by a work counter),
the wide one (SAGE_KERNEL_WIDE, 8-wave workgroups) and the entry one
(SAGE_KERNEL_ENTRY, whole-path calls only: the main loop codes Q from bf16
itself, with the preparation pass's arithmetic, so the codes and therefore
the outputs are the same bits).

Every design runs the same per-epoch arithmetic in the same order (the same
P bytes, the same rescale and matrix-core accumulation of RO, the same
epilogue), so their outputs must agree bit for bit on every shape; each is
also checked against the oracle directly, to the output bar (max-abs 2e-2,
mean-abs 2e-3 per head or block).
"""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as si
import quantized_exact_attention_smooth_amd as sage
from _parity import assert_out_close, oracle_preps, oracle_rows, say

pytestmark = pytest.mark.gpu

FUSED = sage.SAGE_KERNEL_FUSED
ENTRY = sage.SAGE_KERNEL_ENTRY
DESIGNS = {"split": sage.SAGE_KERNEL_SPLIT, "persistent": sage.SAGE_KERNEL_PERSISTENT, "wide": sage.SAGE_KERNEL_WIDE,
           "entry": ENTRY}


@pytest.fixture(params=sorted(DESIGNS))
def design(request):
    return DESIGNS[request.param]


def _both(q, k, v, causal, sm_scale, dev, design):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if design == ENTRY:  # a whole-path design: both sides start from the bf16 inputs
        a = sage.attn_fwd(qd, kd, vd, causal, sm_scale, kernel=FUSED)
        b = sage.attn_fwd(qd, kd, vd, causal, sm_scale, kernel=ENTRY)
    else:
        pr = sage.quant_prep(qd, kd, vd)
        a = sage.attn_fwd_prepped(pr, causal, sm_scale, kernel=FUSED)
        b = sage.attn_fwd_prepped(pr, causal, sm_scale, kernel=design)
    torch.cuda.synchronize()
    return si.bf16_bits(a), si.bf16_bits(b)


SHAPES = [(1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True), (1, 2, 63, 63, 64, True), (1, 1, 64, 64, 128, False),
          (1, 1, 65, 65, 128, True), (1, 2, 127, 129, 64, False), (1, 1, 129, 127, 128, True),
          (2, 3, 200, 333, 128, True), (1, 1, 1000, 64, 64, True), (1, 1, 64, 1000, 128, True),
          (1, 1, 191, 193, 64, False), (1, 2, 300, 300, 128, True), (1, 1, 257, 1, 128, False),
          (1, 1, 384, 384, 64, True), (1, 1, 130, 190, 128, False), (1, 1, 200, 64, 128, True),
          # non-causal with B*H a multiple of 8: the head-grouped tile order
          (1, 8, 300, 200, 128, False), (2, 8, 129, 500, 64, False)]


@pytest.mark.parametrize("B,H,Lq,Lkv,D,causal", SHAPES)
def test_design_equals_fused_and_oracle_on_edge_shapes(B, H, Lq, Lkv, D, causal, design, gpu_device):
    say(f"design {design} vs fused vs oracle: shape {(B, H, Lq, Lkv, D, causal)}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=Lq * 5 + Lkv + D)
    sc = 1 / math.sqrt(D)
    fused, split = _both(q, k, v, causal, sc, gpu_device, design)
    assert np.array_equal(fused, split)
    for (b, h), o in oracle_preps(q, k, v, [(b, h) for b in range(B) for h in range(H)]).items():
        assert_out_close(split[b, h], oracle_rows(o, causal, sc, 0, Lq), f"designs: edge shapes head {(b, h)}")


@pytest.mark.parametrize("idx", [0, 1])
def test_design_small_workloads_against_oracle(idx, design, gpu_device):
    w = si.WORKLOADS[idx]
    say(f"design {design} vs oracle (all rows): {w.name}")
    q, k, v = si.workload_qkv(w)
    fused, split = _both(q, k, v, w.causal, w.sm_scale, gpu_device, design)
    assert np.array_equal(fused, split)
    for (b, h), o in oracle_preps(q, k, v, si.oracle_heads(w)).items():
        assert_out_close(split[b, h], oracle_rows(o, w.causal, w.sm_scale, 0, w.Lq), f"designs: {w.name} head {(b, h)}")


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_design_equals_fused_on_full_size_workloads(idx, design, gpu_device):
    """Bit-identical to the fused design at full size (whose oracle parity on
    the seeded subsets is tested in test_gpu_attn); one seeded block is also
    checked against the oracle directly."""
    w = si.WORKLOADS[idx]
    say(f"design {design} vs fused (full size): {w.name}")
    q, k, v = si.workload_qkv(w)
    fused, split = _both(q, k, v, w.causal, w.sm_scale, gpu_device, design)
    assert np.array_equal(fused, split)
    b, h, qb = si.oracle_blocks(w)[-1] if w.oracle_subset[0] == "blocks" else (*si.oracle_heads(w)[0], w.Lq // 64 - 1)
    r0, r1 = 64 * qb, min(w.Lq, 64 * qb + 64)
    o = oracle_preps(q, k, v, [(b, h)])[(b, h)]
    assert_out_close(split[b, h, r0:r1], oracle_rows(o, w.causal, w.sm_scale, r0, r1), f"designs: {w.name} {(b, h, qb)}")


@pytest.mark.parametrize("seed", range(6))
def test_design_equals_fused_on_seeded_random_shapes(seed, design, gpu_device):
    r = np.random.default_rng(1000 + seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    Lq, Lkv = int(r.integers(1, 700)), int(r.integers(1, 700))
    D = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    dist = "student_t_outlier" if seed % 3 == 2 else "normal"
    say(f"design {design} vs fused: seed {seed} shape {(B, H, Lq, Lkv, D, causal)} {dist}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, dist, 3.0, seed=77 + seed)
    fused, split = _both(q, k, v, causal, 1 / math.sqrt(D), gpu_device, design)
    assert np.array_equal(fused, split)


def test_design_repeated_launches_are_bit_identical(design, gpu_device):
    w = si.WORKLOADS[2]
    q, k, v = (t.to(gpu_device) for t in si.workload_qkv(w))
    out = torch.empty((w.B, w.H, w.Lq, w.D), dtype=torch.bfloat16, device=gpu_device)
    if design == ENTRY:
        ws = torch.empty(sage.workspace_bytes(w.B, w.H, w.Lq, w.Lkv, w.D), dtype=torch.uint8, device=gpu_device)
        run = lambda o: sage.attn_fwd(q, k, v, w.causal, w.sm_scale, out=o, workspace=ws, kernel=ENTRY)  # noqa: E731
    else:
        pr = sage.quant_prep(q, k, v)
        run = lambda o: sage.attn_fwd_prepped(pr, w.causal, w.sm_scale, out=o, kernel=design)  # noqa: E731
    first = si.bf16_bits(run(None))
    for i in range(50):
        run(out)
    torch.cuda.synchronize()
    assert np.array_equal(si.bf16_bits(out), first)


def test_entry_codes_q_blocks_at_the_scale_edges(gpu_device):
    """Q blocks that reach the corners of the INT8 step: an all-zero block
    (scale 0, every code 0), a block whose scale is below 2^-60 (the quotient
    is taken by division), one of subnormal bf16 values, one of very large
    values, and blocks whose second 32-row half lies past Lq (the absmax of
    the rows below Lq alone sets the scale). The entry design must give the
    fused design's bits, and both the oracle's values."""
    B, H, D = 1, 2, 128
    sc = 1 / math.sqrt(D)
    for Lq in (33, 64 * 7 + 20):
        q, k, v = si.make_qkv(B, H, Lq, 300, D, "normal", 2.0, seed=4000 + Lq)
        q = q.clone()
        if Lq > 64:
            q[:, :, 0:64] = 0.0                  # block 0: all zero
            q[:, :, 64:128] *= 1e-30             # block 1: scale ~ 1e-30 / 127 < 2^-60
            q[:, :, 128:192] *= 1e-39            # block 2: subnormal bf16 values
            q[:, 0, 192:256] *= 1e30             # block 3: very large values (scores stay finite)
            q[:, :, 256:320, ::3] = 0.0
        for causal in (False, True):
            say(f"entry vs fused at the Q scale edges: Lq {Lq} causal {causal}")
            fused, entry = _both(q, k, v, causal, sc, gpu_device, ENTRY)
            assert np.array_equal(fused, entry), (Lq, causal)
            for (b, h), o in oracle_preps(q, k, v, [(0, 0), (0, 1)]).items():
                assert_out_close(entry[b, h], oracle_rows(o, causal, sc, 0, Lq), f"entry: scale edges {(b, h)}")
    # The largest bf16 magnitudes code to +-127 with a scale near 2.7e36; the
    # scores then overflow fp32, so only the two designs are compared.
    q, k, v = si.make_qkv(1, 1, 100, 100, D, "normal", 2.0, seed=4100)
    q = q.clone()
    q[:, :, :64] = torch.finfo(torch.bfloat16).max * torch.sign(q[:, :, :64])
    fused, entry = _both(q, k, v, True, sc, gpu_device, ENTRY)
    assert np.array_equal(fused, entry)


KV_SHAPES = [(1, 1, 1, 1, 64, False), (1, 2, 65, 63, 128, True), (2, 3, 200, 333, 128, True),
             (1, 1, 1000, 64, 64, True), (1, 8, 300, 200, 128, False), (1, 1, 257, 1000, 64, False)]


@pytest.mark.parametrize("B,H,Lq,Lkv,D,causal", KV_SHAPES)
def test_kv_prep_and_kv_prepped_equal_the_full_preparation_path(B, H, Lq, Lkv, D, causal, gpu_device):
    """sage_quant_prep_kv writes the K/V operands of sage_quant_prep bit for
    bit, and sage_attn_fwd_kv_prepped on them (bf16 Q coded in the main loop)
    gives the fused design's output on sage_quant_prep's operands."""
    say(f"kv prep + kv-prepped main loop vs full prep + fused: shape {(B, H, Lq, Lkv, D, causal)}")
    q, k, v = (t.to(gpu_device) for t in si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=3 * Lq + Lkv))
    full = sage.quant_prep(q, k, v)
    kv = sage.quant_prep_kv(k, v)
    torch.cuda.synchronize()
    for n in ("k_i8", "k_scale", "k_mean", "v_fp8", "v_scale"):
        assert torch.equal(full[n].view(torch.uint8) if full[n].dtype != torch.float32 else full[n].view(torch.int32),
                           kv[n].view(torch.uint8) if kv[n].dtype != torch.float32 else kv[n].view(torch.int32)), n
    sc = 1 / math.sqrt(D)
    a = si.bf16_bits(sage.attn_fwd_prepped(full, causal, sc, kernel=FUSED))
    b = si.bf16_bits(sage.attn_fwd_kv_prepped(q, kv, causal, sc))
    c = si.bf16_bits(sage.attn_fwd_kv_prepped(q, full, causal, sc))  # K/V of the full preparation pass
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_whole_path_auto_uses_the_reported_design(gpu_device):
    """sage_attn_fwd (automatic design) equals the design sage_auto_design
    reports, run explicitly, and the fused design, bit for bit."""
    for B, H, Lq, Lkv, D, causal in [(2, 32, 512, 512, 128, True), (1, 2, 300, 300, 64, False)]:
        q, k, v = (t.to(gpu_device) for t in si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=Lq + D))
        d = sage.auto_design(B, H, Lq, Lkv, D)
        auto = si.bf16_bits(sage.attn_fwd(q, k, v, causal))
        expl = si.bf16_bits(sage.attn_fwd(q, k, v, causal, kernel=d))
        fused = si.bf16_bits(sage.attn_fwd(q, k, v, causal, kernel=FUSED))
        torch.cuda.synchronize()
        assert np.array_equal(auto, expl) and np.array_equal(auto, fused), (B, H, Lq, d)


def test_persistent_counter_returns_to_zero_across_streams_and_shapes(gpu_device):
    """Launches of the persistent design alternate shapes (grids smaller than,
    equal to and larger than the resident workgroup count) and two streams;
    each must leave its stream's counter at 0 for the next, so every output
    equals the fused design's."""
    s2 = torch.cuda.Stream()
    cases = [(1, 1, 128, 192, 128, False), (2, 32, 4096, 4096, 128, True), (1, 2, 1000, 700, 64, True),
             (4, 16, 2048, 2048, 64, True)]
    preps, refs = [], []
    for i, (B, H, Lq, Lkv, D, causal) in enumerate(cases):
        q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=300 + i)
        pr = sage.quant_prep(q.to(gpu_device), k.to(gpu_device), v.to(gpu_device))
        preps.append((pr, causal))
        refs.append(si.bf16_bits(sage.attn_fwd_prepped(pr, causal, None, kernel=FUSED)))
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (pr, causal) in enumerate(preps):
            st = s2 if (i + rep) % 2 else torch.cuda.current_stream()
            with torch.cuda.stream(st):
                o = sage.attn_fwd_prepped(pr, causal, None, kernel=sage.SAGE_KERNEL_PERSISTENT)
            st.synchronize()
            assert np.array_equal(si.bf16_bits(o), refs[i]), (rep, i)
