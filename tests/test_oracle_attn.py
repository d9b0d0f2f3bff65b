"""Pins for the oracle's attention: the 64-key epoch loop, masks, online
rescaling and the quantized contract.

  * (ii) unquantized epoch loop == (iii) brute-force softmax attention, fp64,
    over ragged and causal sweeps: pins tiling, masks, epoch skipping and the
    online rescale independently of any quantizer;
  * smoothing invariance of exact attention;
  * closed forms of the quantized path: zero Q (uniform weights), constant V,
    one-hot keys;
  * accuracy of the quantized path against fp64 attention (cosine >= 0.995)
    and an ablation showing what K smoothing buys.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import seeded_inputs as si

SWEEP_L = [1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193]


def _f64_head(Lq, Lkv, D, seed, sigma=0.0):
    q, k, v = si.make_qkv(1, 1, Lq, Lkv, D, "normal", sigma, seed)
    return [oracle.bf16_to_f32(si.bf16_bits(t)[0, 0]).astype(np.float64) for t in (q, k, v)]


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L", SWEEP_L)
def test_unquantized_epoch_loop_equals_bruteforce(L, causal, D):
    q, k, v = _f64_head(L, L, D, seed=L * 10 + D + causal)
    sc = 1 / math.sqrt(D)
    assert _rel(oracle.attn_unquant(q, k, v, causal, sc), oracle.attn_ref(q, k, v, causal, sc)) <= 1e-12


@pytest.mark.parametrize("Lq,Lkv", [(65, 193), (193, 65), (200, 64), (1, 129), (1000, 1000), (64, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_unquantized_epoch_loop_equals_bruteforce_rectangular(Lq, Lkv, causal):
    D = 64
    q, k, v = _f64_head(Lq, Lkv, D, seed=Lq + 3 * Lkv)
    sc = 0.125
    a = oracle.attn_unquant(q, k, v, causal, sc)
    b = oracle.attn_ref(q, k, v, causal, sc)
    assert _rel(a, b) <= 1e-12
    if causal and Lq > Lkv:  # rows that see no key output 0
        assert np.all(a[:Lq - Lkv] == 0)


def test_bruteforce_matches_numpy_softmax_definition():
    q, k, v = _f64_head(70, 70, 64, seed=1)
    sc = 0.125
    s = q @ k.T * sc
    s = np.where(np.tril(np.ones((70, 70), bool)), s, -np.inf)
    w = np.exp(s - s.max(1, keepdims=True))
    ref = (w / w.sum(1, keepdims=True)) @ v
    assert _rel(oracle.attn_ref(q, k, v, True, sc), ref) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_smoothing_invariance_of_exact_attention(causal):
    q, k, v = _f64_head(150, 150, 128, seed=21)
    off = np.random.default_rng(2).normal(0, 4, 128)
    sc = 1 / math.sqrt(128)
    for fn in (oracle.attn_unquant, oracle.attn_ref):
        assert _rel(fn(q, k + off[None, :], v, causal, sc), fn(q, k, v, causal, sc)) <= 1e-12


# ---------------------------------------------------------- quantized closed forms

def _bits(x):
    return oracle.bf16_round(np.asarray(x, np.float32))


def _bf16_ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("L,D,causal", [(192, 128, False), (1000, 128, True), (129, 64, True), (65, 64, False)])
def test_zero_q_gives_mean_of_dequantized_v(L, D, causal):
    """Q = 0: every score is 0, so each visible key has weight 1/n_i and the
    output is the exact mean of dec(V8)*sv over the visible keys (up to the
    fp32 accumulation and the final bf16 rounding)."""
    _, k, v = _f64_head(L, L, D, seed=L + D, sigma=2.0)
    q = np.zeros((L, D), np.float32)
    p = oracle.prep_head(_bits(q), _bits(k), _bits(v))
    out = oracle.bf16_to_f32(oracle.attn_rows(p, causal, 1 / math.sqrt(D))).astype(np.float64)
    dec = oracle.e4m3_decode(p["v8"][:L])
    sv = p["v_scale"].astype(np.float64)
    rows = range(0, L, max(1, L // 40))
    for i in rows:
        n = i + 1 if causal else L
        exact = np.array([float(sum(Fraction(x) for x in dec[:n, c]) / n) for c in range(D)]) * sv
        tol = _bf16_ulp(exact) + n * 2.0 ** -23 * 448 * sv
        assert np.all(np.abs(out[i] - exact) <= tol), i


@pytest.mark.parametrize("L,D,causal", [(192, 128, False), (300, 64, True)])
def test_zero_q_constant_v_is_exact(L, D, causal):
    _, k, _ = _f64_head(L, L, D, seed=5, sigma=2.0)
    vc = oracle.bf16_to_f32(_bits(np.random.default_rng(4).normal(0, 2, D)))
    v = np.tile(vc, (L, 1))
    p = oracle.prep_head(_bits(np.zeros((L, D))), _bits(k), _bits(v))
    assert np.all(np.abs(oracle.e4m3_decode(p["v8"][:L])) == 448.0)
    out = oracle.attn_rows(p, causal, 1 / math.sqrt(D))
    np.testing.assert_array_equal(out, np.tile(_bits(vc), (L, 1)))


def test_constant_v_random_q_within_fp8_bound():
    """V constant per channel: out/v_c = sum dec(P8) / sum p. Each P8 is within
    2^-4 relative or 2^-10 absolute of p, and l >= the fp64 denominator's
    order of magnitude, which bounds the ratio."""
    L, D = 192, 128
    q, k, _ = _f64_head(L, L, D, seed=8, sigma=2.0)
    vc = oracle.bf16_to_f32(_bits(np.random.default_rng(6).uniform(0.5, 2, D) * np.sign(np.arange(D) - 60.5)))
    v = np.tile(vc, (L, 1)).astype(np.float64)
    p = oracle.prep_head(_bits(q), _bits(k), _bits(v))
    sc = 1 / math.sqrt(D)
    out = oracle.bf16_to_f32(oracle.attn_rows(p, False, sc)).astype(np.float64)
    s = q @ k.T * sc
    lref = np.exp(s - s.max(1, keepdims=True)).sum(1)
    bound = 2.0 ** -4 + L * 2.0 ** -10 / (0.5 * lref) + 2.0 ** -7
    ratio = np.abs(out / vc[None, :] - 1)
    assert np.all(ratio <= bound[:, None])
    assert np.median(ratio) < 0.01


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_one_hot_keys_select_one_value_row(D, causal):
    """Q[i] = K[i] = 16 e_pi(i): query i matches key i only; every other key's
    weight is below e^-22 and flushes to 0 in FP8, so out[i] is exactly the
    dequantized V row i (V magnitudes in [0.5, 1] keep dec(V8) >= 224, so the
    remnants of earlier epochs, rescaled by alpha ~ 1e-10, vanish in fp32)."""
    L = D
    rng = np.random.default_rng(D + causal)
    perm = rng.permutation(D)
    qk = np.zeros((L, D), np.float32)
    qk[np.arange(L), perm] = 16.0
    v = rng.uniform(0.5, 1.0, (L, D)) * rng.choice([-1, 1], (L, D))
    v[0, :] = 1.0
    p = oracle.prep_head(_bits(qk), _bits(qk), _bits(v))
    out = oracle.attn_rows(p, causal, 1 / math.sqrt(D))
    dec = oracle.e4m3_decode(p["v8"][:L]).astype(np.float32)
    assert np.all(np.abs(dec) >= 224)
    expect = _bits(dec * p["v_scale"][None, :])
    np.testing.assert_array_equal(out, expect)


@pytest.mark.parametrize("D", [64, 128])
def test_one_hot_keys_at_huge_scores_stay_exact(D):
    """The same one-hot rows with Q scaled by 2^100 (exact in bf16): scores
    reach about 2^108, every other key (negative after smoothing) is below the
    top by a comparable amount, and p = exp(z - m) is 1 for the top key and 0
    for the rest, so the output is again exactly the dequantized V row and
    finite (the reading for very large scores: every p <= 1)."""
    L = D
    rng = np.random.default_rng(3 * D)
    perm = rng.permutation(D)
    k = np.zeros((L, D), np.float32)
    k[np.arange(L), perm] = 16.0
    q = k * np.float32(2.0 ** 100)
    v = rng.uniform(0.5, 1.0, (L, D)) * rng.choice([-1, 1], (L, D))
    p = oracle.prep_head(_bits(q), _bits(k), _bits(v))
    assert float(p["q_scale"][0]) > 2.0 ** 90
    for causal in (False, True):
        out = oracle.attn_rows(p, causal, 1 / math.sqrt(D))
        dec = oracle.e4m3_decode(p["v8"][:L]).astype(np.float32)
        np.testing.assert_array_equal(out, _bits(dec * p["v_scale"][None, :]))


def test_rows_without_visible_keys_output_zero():
    Lq, Lkv, D = 130, 64, 64
    q, k, v = _f64_head(Lq, Lkv, D, seed=3)
    p = oracle.prep_head(_bits(q), _bits(k), _bits(v))
    out = oracle.bf16_to_f32(oracle.attn_rows(p, True, 0.125))
    assert np.all(out[:Lq - Lkv] == 0)
    assert np.any(out[Lq - Lkv:] != 0)


# ---------------------------------------------------------- accuracy vs fp64

def _cos(a, b):
    a = a.ravel().astype(np.float64)
    b = b.ravel().astype(np.float64)
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def _quant_vs_fp64(w, heads, rows_per_head=None, smooth=True, seed=None):
    q, k, v = si.workload_qkv(w, seed)
    res = []
    for (b, h) in heads:
        qb, kb, vb = (si.bf16_bits(t[b, h]) for t in (q, k, v))
        p = oracle.prep_head(qb, kb, vb, smooth=smooth)
        r0, r1 = rows_per_head if rows_per_head else (0, w.Lq)
        out = oracle.bf16_to_f32(oracle.attn_rows_parallel(p, w.causal, w.sm_scale, r0, r1))
        qf, kf, vf = (oracle.bf16_to_f32(x).astype(np.float64) for x in (qb, kb, vb))
        ref = oracle.attn_ref_parallel(qf, kf, vf, w.causal, w.sm_scale, r0, r1)
        res.append(_cos(out, ref))
    return res


def test_quantized_accuracy_q128_kv192():
    w = si.WORKLOADS[0]
    assert min(_quant_vs_fp64(w, si.oracle_heads(w))) >= 0.995


def test_quantized_accuracy_ragged_causal_l1000():
    w = si.WORKLOADS[1]
    assert min(_quant_vs_fp64(w, si.oracle_heads(w))) >= 0.995


def test_quantized_accuracy_small_outlier_distribution():
    """The student-t / x20 outlier-channel distribution at a reduced length.

    Measured here: cosine 0.9918 and 0.9939. The loss comes from the 64-row
    INT8 blocks themselves (Q's heavy t(3) tail sets a coarse block step; the
    K outlier channels do the same for K): fp64 attention on the dequantized
    operands reaches the same cosine (next test). The 0.995 bound is therefore
    not met on this distribution by the block contract, and this test records
    the measured level instead of loosening the contract."""
    w = si.Workload("outlier_small", 1, 2, 1024, 1024, 64, True, "student_t_outlier", 0.0)
    assert min(_quant_vs_fp64(w, [(0, 0), (0, 1)], seed=4)) >= 0.99


@pytest.mark.parametrize("dist,D,sigma", [("student_t_outlier", 64, 0.0), ("normal", 128, 4.0)])
def test_epoch_loop_matches_fp64_attention_of_dequantized_operands(dist, D, sigma):
    """Q, K and V replaced by their dequantized codes (K + mean): fp64 attention
    on those differs from the contract only by the online FP8 rounding of P
    and fp32 accumulation, which must be small."""
    L = 512
    q, k, v = si.make_qkv(1, 1, L, L, D, dist, sigma, seed=31)
    qb, kb, vb = (si.bf16_bits(t[0, 0]) for t in (q, k, v))
    p = oracle.prep_head(qb, kb, vb)
    qd = p["q8"][:L].astype(np.float64) * np.repeat(p["q_scale"], 64)[:L, None]
    kd = p["k8"][:L].astype(np.float64) * np.repeat(p["k_scale"], 64)[:L, None] + p["k_mean"][None, :]
    vd = oracle.e4m3_decode(p["v8"][:L]) * p["v_scale"][None, :]
    sc = 1 / math.sqrt(D)
    ref = oracle.attn_ref_parallel(qd, kd, vd, True, sc)
    out = oracle.bf16_to_f32(oracle.attn_rows_parallel(p, True, sc))
    assert _cos(out, ref) >= 0.9995


def test_smoothing_ablation_large_k_offset():
    """With a per-channel K offset of sigma 4 the smoothed path stays accurate;
    without smoothing the per-block INT8 step grows and the error rises."""
    w = si.Workload("offset_small", 1, 2, 512, 512, 128, True, "normal", 4.0)
    with_s = _quant_vs_fp64(w, [(0, 0), (0, 1)], seed=2)
    without = _quant_vs_fp64(w, [(0, 0), (0, 1)], smooth=False, seed=2)
    assert min(with_s) >= 0.995
    for a, b in zip(with_s, without):
        assert (1 - b) > 1.5 * (1 - a)


def _scaled_bits(bits: np.ndarray, e: int) -> np.ndarray:
    """bf16 bits of 2^e times the bf16 values (exact: no value leaves the
    normal range in these tests)."""
    x = oracle.bf16_to_f32(bits).astype(np.float64) * 2.0 ** e
    assert np.all((x == 0) | ((np.abs(x) >= 2.0 ** -126) & (np.abs(x) < 2.0 ** 127)))
    return _bits(x)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("e", [-9, 6])
def test_power_of_two_scalings_act_exactly(causal, e):
    """Metamorphic pins of where each scale enters, bit for bit: every scale
    of the contract is a quotient or product that a power of two passes
    through exactly. V times 2^e: the channel scales gain 2^e, the E4M3 codes
    stay, and the output is 2^e times the original. K times 2^e with sm_scale
    times 2^-e: the K means and block scales gain 2^e, the codes stay, and the
    scores and output are unchanged (likewise for Q). A scale applied twice
    or dropped, or sm_scale applied to the wrong factor, fails one of these."""
    L, D = 200, 64
    q, k, v = si.make_qkv(1, 1, L, L, D, "normal", 2.0, seed=31 + e)
    qb, kb, vb = (si.bf16_bits(t)[0, 0] for t in (q, k, v))
    sc = 1 / math.sqrt(D)
    base = oracle.prep_head(qb, kb, vb)
    out = oracle.attn_rows(base, causal, sc)

    pv = oracle.prep_head(qb, kb, _scaled_bits(vb, e))
    np.testing.assert_array_equal(pv["v8"], base["v8"])
    np.testing.assert_array_equal(pv["v_scale"], base["v_scale"] * np.float32(2.0 ** e))
    np.testing.assert_array_equal(oracle.attn_rows(pv, causal, sc), _scaled_bits(out, e))

    pk = oracle.prep_head(qb, _scaled_bits(kb, e), vb)
    np.testing.assert_array_equal(pk["k8"], base["k8"])
    np.testing.assert_array_equal(pk["k_scale"], base["k_scale"] * np.float32(2.0 ** e))
    np.testing.assert_array_equal(pk["k_mean"], base["k_mean"] * np.float32(2.0 ** e))
    np.testing.assert_array_equal(oracle.attn_rows(pk, causal, sc * 2.0 ** -e), out)

    pq = oracle.prep_head(_scaled_bits(qb, e), kb, vb)
    np.testing.assert_array_equal(pq["q8"], base["q8"])
    np.testing.assert_array_equal(oracle.attn_rows(pq, causal, sc * 2.0 ** -e), out)


# ---------------------------------------------------------------------------
# Reading R9: the denominator l sums the fp32 probabilities p before their
# FP8 rounding ("d" and "FP8 probability" are separate checkpoints in the
# Experiment Log's Phase 2B prototype). The two tests below fail if l summed
# the decoded FP8 probabilities instead.

def _bf16(x):
    import torch
    return torch.tensor(np.float32(x)).to(torch.bfloat16).view(torch.int16).item() & 0xFFFF


def test_denominator_of_two_keys_sums_fp32_probabilities():
    """One query, two keys, hand-computed. Q row = 127 e_0 gives s_q = 1 and
    code 127; K rows +-127 e_0 have channel mean 0, s_k = 1 and codes +-127,
    so the scores are z = +-(16129 * sm_scale) rounded to fp32. With sm_scale
    chosen so that p_2 = exp(z_2 - z_1) is near 0.3: l = 1 + p_2 in fp32,
    while the FP8 probability of key 2 is 0.3125 (E4M3 spacing 2^-5 there),
    so a denominator of decoded FP8 values would be 1.3125."""
    D = 64
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 127.0
    k = np.zeros((2, D), np.float32)
    k[0, 0], k[1, 0] = 127.0, -127.0
    v = np.ones((2, D), np.float32)  # constant V: V8 = 448 and sv = RN(1/448)
    p = oracle.prep_head(oracle.bf16_round(q), oracle.bf16_round(k), oracle.bf16_round(v))
    assert p["q_scale"][0] == 1 and p["k_scale"][0] == 1 and p["q8"][0, 0] == 127 and p["k8"][1, 0] == -127
    sm = np.float32(math.log(1 / 0.3) / 32258.0)
    z1 = np.float32(np.float32(16129.0) * sm)  # (acc * (sq * sk)) * sm with sq * sk = 1
    p2 = np.float32(math.exp(-2.0 * float(z1)))
    l_hand = np.float32(np.float32(1.0) + p2)
    assert abs(p2 - 0.3) < 1e-6 and oracle.e4m3_decode(oracle.e4m3_encode([p2]))[0] == 0.3125
    t = oracle.attn_row_trace(p, False, float(sm), 0)
    assert t["stats"][0, 1] == l_hand and t["stats"][1, 1] == l_hand
    assert list(t["p8"][0, :2]) == [0x38, int(oracle.e4m3_encode([p2])[0])]
    r = np.float32(np.float32(1.0) / l_hand)
    assert t["stats"][1, 0] == r
    # RO = 448 * 1 + 448 * 0.3125 = 588 exactly; out = bf16((RO * r) * sv)
    sv = np.float32(np.float32(1.0) / np.float32(448.0))
    want = _bf16(np.float32(np.float32(np.float32(588.0) * r) * sv))
    assert t["out"][0] == want and want != _bf16(1.0)


def test_constant_v_output_reflects_fp32_denominator():
    """V constant per channel: every V code is +-448, so out / v_c is
    sum dec(P8) / sum p up to fp32 rounding. With the fp32 denominator this
    ratio differs from 1 by the FP8 rounding of the weights and a sizeable
    share of outputs leave bf16(v_c) (measured 22-38 % of the elements on
    these shapes); with a denominator of decoded FP8 values every output
    would be exactly bf16(v_c)."""
    for L, D, causal in [(192, 128, False), (300, 64, True)]:
        q, k, _ = _f64_head(L, L, D, seed=8, sigma=2.0)
        vc = oracle.bf16_to_f32(oracle.bf16_round(np.random.default_rng(6).uniform(0.5, 2, D)
                                                  * np.sign(np.arange(D) - 60.5)))
        v = np.tile(vc, (L, 1))
        p = oracle.prep_head(oracle.bf16_round(q), oracle.bf16_round(k), oracle.bf16_round(v))
        out = oracle.attn_rows(p, causal, 1 / math.sqrt(D))
        share = float(np.mean(out != np.tile(oracle.bf16_round(vc), (L, 1))))
        assert share >= 0.15, (L, D, share)
