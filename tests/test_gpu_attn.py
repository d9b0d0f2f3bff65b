"""The fused main loop and the whole path against the oracle.

Bar: per checked head or block, max-abs <= 2e-2 and mean-abs <= 2e-3 of the
bf16 output against the oracle's bf16 output from the same bf16 inputs
(P bytes, exp and summation order differ between the two, so outputs are
not expected to be bit-identical). Exact expectations where the math fixes
the result (zero Q with constant V, one-hot keys). Full-size workloads run
in the same launch configuration the benchmark times and are checked on
their seeded oracle subsets.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import quantized_exact_attention_smooth_amd as sage
from _parity import assert_out_close, assert_prep_equal, gpu_prep_numpy, oracle_preps, oracle_rows, say

pytestmark = pytest.mark.gpu


def _gpu_out(q, k, v, causal, sm_scale, dev, end_to_end=False):
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    if end_to_end:
        o = sage.attn_fwd(qg, kg, vg, causal, sm_scale)
    else:
        o = sage.attn_fwd_prepped(sage.quant_prep(qg, kg, vg), causal, sm_scale)
    torch.cuda.synchronize()
    return si.bf16_bits(o)


@pytest.mark.parametrize("idx", [0, 1])
def test_small_workloads_all_rows(idx, gpu_device):
    w = si.WORKLOADS[idx]
    say(f"attn parity (all rows): {w.name}")
    q, k, v = si.workload_qkv(w)
    out = _gpu_out(q, k, v, w.causal, w.sm_scale, gpu_device)
    for (b, h), o in oracle_preps(q, k, v, si.oracle_heads(w)).items():
        ref = oracle_rows(o, w.causal, w.sm_scale, 0, w.Lq)
        assert_out_close(out[b, h], ref, f"{w.name} head {(b, h)}")


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_full_size_workloads_on_oracle_subset(idx, gpu_device):
    """Both calls at full size against the oracle on the seeded subset: the
    prepared-operand main loop and the whole path (sage_attn_fwd, the step
    the benchmark times; on these full grids it runs the entry design)."""
    w = si.WORKLOADS[idx]
    say(f"attn parity (oracle subset): {w.name}")
    q, k, v = si.workload_qkv(w)
    outs = {"prepped": _gpu_out(q, k, v, w.causal, w.sm_scale, gpu_device),
            "whole path": _gpu_out(q, k, v, w.causal, w.sm_scale, gpu_device, end_to_end=True)}
    if w.oracle_subset[0] == "blocks":
        items = [(b, h, qb * 64, min(w.Lq, qb * 64 + 64)) for (b, h, qb) in si.oracle_blocks(w)]
    else:
        items = [(b, h, 0, w.Lq) for (b, h) in si.oracle_heads(w)]
    preps = oracle_preps(q, k, v, sorted({(b, h) for (b, h, _, _) in items}))
    worst = (0.0, 0.0)
    for (b, h, r0, r1) in items:
        ref = oracle_rows(preps[(b, h)], w.causal, w.sm_scale, r0, r1)
        for path, out in outs.items():
            mx, mean = assert_out_close(out[b, h, r0:r1], ref, f"{w.name} {(b, h, r0, r1)} {path}")
            worst = (max(worst[0], mx), max(worst[1], mean))
    say(f"  worst max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e}")


SHAPES = [(1, 1, 1, 1, 64, False), (1, 1, 1, 1, 128, True), (1, 2, 63, 63, 64, True), (1, 1, 64, 64, 128, False),
          (1, 1, 65, 65, 128, True), (1, 2, 127, 129, 64, False), (1, 1, 129, 127, 128, True),
          (2, 3, 200, 333, 128, True), (1, 1, 1000, 64, 64, True), (1, 1, 64, 1000, 128, True),
          (1, 1, 191, 193, 64, False), (1, 2, 300, 300, 128, True), (1, 1, 257, 1, 128, False),
          (1, 1, 384, 384, 64, True),
          # a few query rows against many keys (decode-like): 64 epochs in one workgroup per head
          (1, 4, 16, 4096, 128, False), (1, 2, 1, 4096, 64, True), (2, 2, 33, 4000, 128, True)]


@pytest.mark.parametrize("B,H,Lq,Lkv,D,causal", SHAPES)
def test_ragged_and_edge_shapes(B, H, Lq, Lkv, D, causal, gpu_device):
    say(f"attn parity: shape {(B, H, Lq, Lkv, D, causal)}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=Lq * 5 + Lkv + D)
    sc = 1 / math.sqrt(D)
    out = _gpu_out(q, k, v, causal, sc, gpu_device)
    for (b, h), o in oracle_preps(q, k, v, [(b, h) for b in range(B) for h in range(H)]).items():
        ref = oracle_rows(o, causal, sc, 0, Lq)
        assert_out_close(out[b, h], ref, f"edge and ragged shapes head {(b, h)}")
        if causal and Lq > Lkv:
            assert np.all(out[b, h, :Lq - Lkv] == 0)


E2E_SHAPES = [(1, 1, 1, 1, 64, True), (1, 2, 63, 65, 128, False), (2, 1, 65, 1, 128, True),
              (1, 3, 1000, 129, 64, True), (1, 1, 129, 1000, 128, True), (1, 2, 300, 300, 128, False),
              (2, 2, 200, 511, 64, False)]


def test_end_to_end_equals_prep_then_main(gpu_device):
    # sage_attn_fwd runs the preparation pass into its workspace and then the
    # main loop: the output equals the two public calls bit for bit.
    w = si.WORKLOADS[1]
    q, k, v = si.workload_qkv(w)
    say("attn_fwd == quant_prep + attn_fwd_prepped")
    a = _gpu_out(q, k, v, True, w.sm_scale, gpu_device, end_to_end=True)
    b = _gpu_out(q, k, v, True, w.sm_scale, gpu_device)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("shape", E2E_SHAPES)
def test_end_to_end_equals_prep_then_main_on_edges(shape, gpu_device):
    B, H, Lq, Lkv, D, causal = shape
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", 2.0, seed=31)
    if Lq > 64:
        q[:, :, 64:128] = 0  # an all-zero Q block (scale 0, codes 0)
    say(f"attn_fwd == prep + prepped on {shape}")
    sm = 1.0 / math.sqrt(D)
    a = _gpu_out(q, k, v, causal, sm, gpu_device, end_to_end=True)
    b = _gpu_out(q, k, v, causal, sm, gpu_device)
    assert np.array_equal(a, b)


def test_default_scale_is_one_over_sqrt_d(gpu_device):
    q, k, v = si.make_qkv(1, 2, 150, 150, 64, "normal", 1.0, seed=9)
    say("sm_scale <= 0 selects 1/sqrt(D)")
    a = _gpu_out(q, k, v, True, 0.0, gpu_device)
    b = _gpu_out(q, k, v, True, 0.125, gpu_device)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("L,D,causal", [(192, 128, False), (300, 64, True), (1000, 128, True)])
def test_zero_q_constant_v_is_exact(L, D, causal, gpu_device):
    _, k, _ = si.make_qkv(1, 1, L, L, D, "normal", 2.0, seed=L)
    vc = torch.from_numpy(np.random.default_rng(L).normal(0, 2, D).astype(np.float32)).to(torch.bfloat16)
    v = vc.reshape(1, 1, 1, D).expand(1, 1, L, D).contiguous()
    q = torch.zeros((1, 1, L, D), dtype=torch.bfloat16)
    say(f"zero Q, constant V: {(L, D, causal)}")
    out = _gpu_out(q, k, v, causal, 1 / math.sqrt(D), gpu_device)
    want = np.broadcast_to(si.bf16_bits(vc), (L, D))
    assert np.array_equal(out[0, 0], want)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_scale", [1.0, 2.0 ** 100])
def test_one_hot_keys_exact(D, causal, q_scale, gpu_device):
    """Query i matches key i only, so out[i] is exactly the dequantized V row
    i; with Q times 2^100 the scores reach about 2^108 (the large-score
    exponent path) and the result must be the same."""
    L = D
    rng = np.random.default_rng(D + causal)
    perm = rng.permutation(D)
    qk = np.zeros((L, D), np.float32)
    qk[np.arange(L), perm] = 16.0
    vv = (rng.uniform(0.5, 1.0, (L, D)) * rng.choice([-1, 1], (L, D))).astype(np.float32)
    vv[0, :] = 1.0
    t = lambda x: torch.from_numpy(x).to(torch.bfloat16).reshape(1, 1, L, D)
    qq = qk * np.float32(q_scale)
    say(f"one-hot keys: D={D} causal={causal} Q scale {q_scale}")
    out = _gpu_out(t(qq), t(qk), t(vv), causal, 1 / math.sqrt(D), gpu_device)
    p = oracle.prep_head(si.bf16_bits(t(qq))[0, 0], si.bf16_bits(t(qk))[0, 0], si.bf16_bits(t(vv))[0, 0])
    dec = oracle.e4m3_decode(p["v8"][:L]).astype(np.float32)
    want = oracle.bf16_round(dec * p["v_scale"][None, :])
    assert np.array_equal(out[0, 0], want)


def test_repeated_launches_are_bit_identical(gpu_device):
    """Fixed reduction order and no atomics in the main loop: 1000 launches
    of the 128x192 workload and 50 of the ragged causal one repeat exactly."""
    for idx, reps in ((0, 1000), (1, 50)):
        w = si.WORKLOADS[idx]
        q, k, v = (t.to(gpu_device) for t in si.workload_qkv(w))
        p = sage.quant_prep(q, k, v)
        first = sage.attn_fwd_prepped(p, w.causal, w.sm_scale).clone()
        say(f"repetition x{reps}: {w.name}")
        outs = torch.empty((reps,) + tuple(first.shape), dtype=first.dtype, device=gpu_device) if reps <= 64 else None
        for i in range(reps):
            o = sage.attn_fwd_prepped(p, w.causal, w.sm_scale)
            if outs is not None:
                outs[i] = o
            else:
                assert torch.equal(o.view(torch.int16), first.view(torch.int16)), i
        if outs is not None:
            assert torch.equal(outs.view(torch.int16), first.view(torch.int16).expand_as(outs))
        torch.cuda.synchronize()


def test_oracle_accuracy_holds_for_gpu_output(gpu_device):
    """GPU output against brute-force fp64 attention: cosine >= 0.995 on the
    ragged causal workload (all heads)."""
    w = si.WORKLOADS[1]
    q, k, v = si.workload_qkv(w)
    say("gpu vs fp64 cosine")
    out = _gpu_out(q, k, v, w.causal, w.sm_scale, gpu_device)
    for h in range(w.H):
        qf, kf, vf = (oracle.bf16_to_f32(si.bf16_bits(t[0, h])).astype(np.float64) for t in (q, k, v))
        ref = oracle.attn_ref_parallel(qf, kf, vf, w.causal, w.sm_scale)
        a = oracle.bf16_to_f32(out[0, h]).astype(np.float64).ravel()
        cos = a @ ref.ravel() / math.sqrt((a @ a) * (ref.ravel() @ ref.ravel()))
        assert cos >= 0.995, (h, cos)


def test_more_heads_than_a_grid_dimension_holds(gpu_device):
    # B*H = 72000 heads (> 2^16, the largest y extent of a launch grid): 17
    # seeded heads repeated, a period chosen so that a head index that wrapped
    # at 2^16 would pick different data. The last heads are checked against
    # the oracle, prepared operands bit for bit and outputs to the tolerance.
    B, H, L, D, period = 2, 36000, 64, 64, 17
    q0, k0, v0 = si.make_qkv(1, period, L, L, D, "normal", 2.0, seed=31)
    idx = torch.arange(B * H) % period
    dev = gpu_device
    qg, kg, vg = (t[0].to(dev)[idx].reshape(B, H, L, D).contiguous() for t in (q0, k0, v0))
    say(f"{B}x{H} heads, L={L} D={D} causal")
    p = sage.quant_prep(qg, kg, vg)
    out = si.bf16_bits(sage.attn_fwd_prepped(p, True, 0.125))
    torch.cuda.synchronize()
    g = {n: p[n][:, -2:].cpu().numpy() for n in ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_scale")}
    vv = p["v_fp8"][:, -2:].cpu().numpy()
    g["v8"] = vv.transpose(0, 1, 2, 4, 3).reshape(B, 2, -1, D)
    del p, qg, kg, vg
    for b in range(B):
        for j, h in enumerate((H - 2, H - 1)):
            src = (b * H + h) % period
            o = oracle.prep_head(si.bf16_bits(q0[0, src]), si.bf16_bits(k0[0, src]), si.bf16_bits(v0[0, src]))
            assert_prep_equal(g, o, b, j)
            assert_out_close(out[b, h], oracle.attn_rows(o, True, 0.125), f"many heads (B*H beyond a grid dimension): head ({b},{h})")


def _random_shapes(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 700)),
                    int(rng.integers(1, 700)), D, bool(rng.integers(0, 2)),
                    str(rng.choice(["normal", "student_t_outlier"])), float(rng.choice([0.0, 2.0, 4.0])), i))
    return out


@pytest.mark.parametrize("B,H,Lq,Lkv,D,causal,dist,sigma,seed", _random_shapes())
def test_seeded_random_shapes(B, H, Lq, Lkv, D, causal, dist, sigma, seed, gpu_device):
    # Shapes, masks and value distributions drawn from a fixed seed: every
    # head against the oracle, prepared operands bit for bit and outputs to
    # the tolerance.
    say(f"random shape {seed}: {(B, H, Lq, Lkv, D, causal, dist, sigma)}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, dist, sigma, seed=1000 + seed)
    sc = 1 / math.sqrt(D)
    qg, kg, vg = q.to(gpu_device), k.to(gpu_device), v.to(gpu_device)
    p = sage.quant_prep(qg, kg, vg)
    out = si.bf16_bits(sage.attn_fwd_prepped(p, causal, sc))
    torch.cuda.synchronize()
    g = gpu_prep_numpy(p)
    for (b, h), o in oracle_preps(q, k, v, [(b, h) for b in range(B) for h in range(H)]).items():
        assert_prep_equal(g, o, b, h)
        assert_out_close(out[b, h], oracle_rows(o, causal, sc, 0, Lq), f"seeded random shapes head {(b, h)}")


def _times_pow2(t: torch.Tensor, e: int) -> torch.Tensor:
    """2^e times a bf16 tensor (exact for these values: all stay normal)."""
    return (t.float() * 2.0 ** e).to(torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
def test_power_of_two_scalings_act_exactly(causal, gpu_device):
    """The oracle's metamorphic pins, on the GPU path bit for bit: V times 2^5
    scales the output by exactly 2^5; K times 2^-7 with sm_scale times 2^7,
    and Q times 2^3 with sm_scale times 2^-3, leave it unchanged (every scale
    the kernels form is a product or quotient that a power of two passes
    through exactly: means, block and channel scales, reciprocals, the
    folded log2-domain factor)."""
    B, H, L, D = 1, 2, 333, 128
    say(f"attn parity: power-of-two scalings, causal={causal}")
    q, k, v = si.make_qkv(B, H, L, L, D, "normal", 2.0, seed=77)
    sc = 1 / math.sqrt(D)
    out = _gpu_out(q, k, v, causal, sc, gpu_device, end_to_end=True)
    out_f = oracle.bf16_to_f32(out).astype(np.float64)
    got_v = _gpu_out(q, k, _times_pow2(v, 5), causal, sc, gpu_device, end_to_end=True)
    np.testing.assert_array_equal(oracle.bf16_to_f32(got_v).astype(np.float64), out_f * 2.0 ** 5)
    got_k = _gpu_out(q, _times_pow2(k, -7), v, causal, sc * 2.0 ** 7, gpu_device, end_to_end=True)
    np.testing.assert_array_equal(got_k, out)
    got_q = _gpu_out(_times_pow2(q, 3), k, v, causal, sc * 2.0 ** -3, gpu_device, end_to_end=True)
    np.testing.assert_array_equal(got_q, out)


@pytest.mark.parametrize("causal", [False, True])
def test_large_scores_stay_finite_and_match_the_oracle(causal, gpu_device):
    """Rows whose running max reaches 2^12 in the log2 domain take their
    exponents relative to the row's integer top score. Head 1 has Q times
    3000 (row maxima 1e4 to 2.3e4 log2 units, where the oracle's own fp32
    score rounding stays near 2^-9 of a unit) and must meet the output bar;
    head 2 has Q times 1e30 (scores near 1e31, where fp32 arithmetic leaves
    only the top keys with p > 0) and must give the oracle's values too.
    Every output is finite."""
    B, H, L, D = 1, 3, 333, 128
    q, k, v = si.make_qkv(B, H, L, L, D, "normal", 2.0, seed=91)
    q = q.clone()
    q[:, 1] *= 3000.0
    q[:, 2] *= 1e30
    sc = 1 / math.sqrt(D)
    say(f"attn parity: large scores, causal={causal}")
    out = _gpu_out(q, k, v, causal, sc, gpu_device)
    assert np.all(np.isfinite(oracle.bf16_to_f32(out)))
    for (b, h), o in oracle_preps(q, k, v, [(0, 0), (0, 1), (0, 2)]).items():
        assert_out_close(out[b, h], oracle_rows(o, causal, sc, 0, L), f"attn: large scores head {h}")


CONCURRENT_CASES = {
    # small grids: the split design
    "split": [((1, 4, 777, 777, 128), True, 11), ((2, 2, 300, 1025, 64), False, 12)],
    # full grids (at least 256 tiles): the entry design, beside a small one
    "entry": [((2, 32, 512, 512, 128), True, 13), ((1, 64, 512, 700, 64), False, 14),
              ((1, 2, 300, 300, 128), True, 15)],
}


@pytest.mark.parametrize("which", sorted(CONCURRENT_CASES))
def test_concurrent_calls_on_two_streams_match_sequential(which, gpu_device):
    """Calls keep no state between them: host threads, each on its own
    stream (default priority), run different shapes at the same time, and
    every output equals the one from a sequential run bit for bit."""
    import threading
    say(f"attn parity: concurrent calls on separate streams ({which})")
    cases = CONCURRENT_CASES[which]
    inputs = [tuple(t.to(gpu_device) for t in si.make_qkv(*shape, "normal", 2.0, seed))
              for shape, _, seed in cases]
    seq = []
    for (shape, causal, _), (q, k, v) in zip(cases, inputs):
        seq.append(si.bf16_bits(sage.attn_fwd(q, k, v, causal, 1 / math.sqrt(shape[4]))))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=gpu_device) for _ in cases]
    results = [None] * len(cases)
    errors = []

    def run(i):
        try:
            (shape, causal, _), (q, k, v) = cases[i], inputs[i]
            with torch.cuda.stream(streams[i]):
                outs = [sage.attn_fwd(q, k, v, causal, 1 / math.sqrt(shape[4])) for _ in range(3)]
            streams[i].synchronize()
            results[i] = [si.bf16_bits(o) for o in outs]
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(len(cases)):
        for got in results[i]:
            np.testing.assert_array_equal(got, seq[i])


@pytest.mark.parametrize("B,H,L,D,causal", [(1, 3, 500, 128, True), (2, 32, 512, 128, True)])
def test_graph_replays_match_eager_runs(B, H, L, D, causal, gpu_device):
    """sage_attn_fwd allocates nothing and issues no memset or host
    synchronisation, so a captured HIP graph of it replays correctly: four
    replays, with eager work and synchronisation between them and new input
    values copied in before some, each equal bit for bit to an eager call on
    the same inputs. The small shape runs the split design, the full grid the
    entry design."""
    say(f"attn parity: HIP graph replays, shape {(B, H, L, D, causal)}")
    sc = 1 / math.sqrt(D)
    q, k, v = (t.to(gpu_device) for t in si.make_qkv(B, H, L, L, D, "normal", 2.0, seed=21))
    ws = torch.empty(sage.workspace_bytes(B, H, L, L, D), dtype=torch.uint8, device=gpu_device)
    out = torch.empty_like(q)
    side = torch.cuda.Stream(device=gpu_device)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sage.attn_fwd(q, k, v, causal, sc, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sage.attn_fwd(q, k, v, causal, sc, out=out, workspace=ws)
    for r in range(4):
        if r % 2 == 1:  # new input values in the captured buffers
            nq, nk, nv = si.make_qkv(B, H, L, L, D, "normal", 2.0, seed=100 + r)
            q.copy_(nq.to(gpu_device)), k.copy_(nk.to(gpu_device)), v.copy_(nv.to(gpu_device))
        expect = si.bf16_bits(sage.attn_fwd(q, k, v, causal, sc))
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(si.bf16_bits(out), expect)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_largest_key_count_zero_q_constant_v_is_exact(D, causal, gpu_device):
    """The largest key count the library admits: one head's K and V codes
    fill 2^31 - 64 D bytes, the limit of the main loop's 32-bit buffer
    offsets (2^24 - 64 keys at D = 128, 2^25 - 64 at D = 64; 262,143 or
    524,287 epochs and 65,536 or 131,072 statistics splits). With Q = 0 every score
    is 0, so p = 1 for each visible key and every V code is +-448. RO's
    partial sums, multiples of 64 * 448 = 7 * 2^12 over at most 2^19 epochs,
    are exact in fp32, and so is each lane half's share of the key count
    (< 2^24); their total is within 2^-25 of the count. The output is
    therefore bf16(v_c) in every row, whatever K holds (the fp32 errors are
    far below half a bf16 ulp)."""
    B, H, Lq = 1, 1, 256
    Lkv = (1 << 31) // D - 64
    say(f"zero Q, constant V at the largest key count: Lq={Lq} Lkv={Lkv} causal={causal}")
    gen = torch.Generator(device=gpu_device)
    gen.manual_seed(2024 + causal)
    k = torch.randn((B, H, Lkv, D), generator=gen, device=gpu_device, dtype=torch.float32).to(torch.bfloat16)
    vc = torch.from_numpy(np.random.default_rng(9).normal(0, 2, D).astype(np.float32)).to(torch.bfloat16)
    v = vc.to(gpu_device).reshape(1, 1, 1, D).expand(B, H, Lkv, D).contiguous()
    q = torch.zeros((B, H, Lq, D), dtype=torch.bfloat16, device=gpu_device)
    out = sage.attn_fwd(q, k, v, causal, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    got = si.bf16_bits(out)[0, 0]
    del k, v, out
    torch.cuda.empty_cache()
    np.testing.assert_array_equal(got, np.broadcast_to(si.bf16_bits(vc), (Lq, D)))


@pytest.mark.parametrize("causal", [False, True])
def test_largest_query_count_zero_q_constant_v_is_exact(causal, gpu_device):
    """2^24 - 64 query rows against 200 keys (D = 128; 131,072 main-loop
    workgroups, 4 GiB of output). Zero Q and constant V give bf16(v_c) in
    every row that sees a key; causal (bottom-right) rows above the last
    Lkv see none and output 0. Compared on the GPU."""
    B, H, D, Lkv = 1, 1, 128, 200
    Lq = (1 << 24) - 64
    say(f"zero Q, constant V at the largest query count: Lq={Lq} Lkv={Lkv} causal={causal}")
    k = si.make_qkv(B, H, 1, Lkv, D, "normal", 2.0, seed=5)[1].to(gpu_device)
    vc = torch.from_numpy(np.random.default_rng(10).normal(0, 2, D).astype(np.float32)).to(torch.bfloat16)
    v = vc.to(gpu_device).reshape(1, 1, 1, D).expand(B, H, Lkv, D).contiguous()
    q = torch.zeros((B, H, Lq, D), dtype=torch.bfloat16, device=gpu_device)
    out = sage.attn_fwd(q, k, v, causal, 1 / math.sqrt(D))
    vcd = vc.to(gpu_device).view(torch.int16)
    got = out.view(torch.int16)[0, 0]
    first = Lq - Lkv if causal else 0  # rows before this one see no key
    assert bool((got[first:] == vcd).all())
    assert bool((got[:first] == 0).all())
    del q, out, got
    torch.cuda.empty_cache()
