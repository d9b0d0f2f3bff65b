"""Pins for the oracle's preparation pass: K channel mean, K smoothing, INT8
block quantization of Q and K, and per-channel FP8 quantization of V.

Checks are stated against exact arithmetic (math.fsum, fp64 quotients), the
format's properties and hand-built special cases, never by re-running the
oracle's own formula.
"""
import math

import numpy as np
import torch
import pytest

import oracle
import seeded_inputs as si


def _head(Lq, Lkv, D, seed, sigma=2.0, dist="normal"):
    q, k, v = si.make_qkv(1, 1, Lq, Lkv, D, dist, sigma, seed)
    return [si.bf16_bits(t)[0, 0] for t in (q, k, v)]


SHAPES = [(1, 1, 64), (63, 65, 64), (128, 192, 128), (200, 129, 128), (1000, 1000, 128), (257, 300, 64)]


@pytest.mark.parametrize("Lq,Lkv,D", SHAPES)
def test_k_mean_is_the_exactly_rounded_mean(Lq, Lkv, D):
    qb, kb, vb = _head(Lq, Lkv, D, seed=Lq + Lkv)
    p = oracle.prep_head(qb, kb, vb)
    assert p["exact_mean"]
    kf = oracle.bf16_to_f32(kb).astype(np.float64)
    for c in range(D):
        exact = math.fsum(kf[:, c])  # exact sum, one rounding to double
        assert p["k_mean"][c] == np.float32(exact / Lkv)


def test_inexact_fp64_channel_sum_is_flagged():
    D, L = 64, 64
    k = np.zeros((L, D), np.float32)
    k[0, :] = 1.0  # lost going forward (1 + 2^60 - 2^60 = 0), kept going backward
    k[1, :] = 2.0 ** 60
    k[2, :] = -(2.0 ** 60)
    kb = oracle.bf16_round(k)
    p = oracle.prep_head(kb, kb, kb)
    assert not p["exact_mean"]


def _check_int8_blocks(x, codes, scales, L):
    """x: the fp32 values that were quantized ([L, D]); codes [nb*64, D]."""
    D = x.shape[1]
    nb = scales.shape[0]
    assert nb == -(-L // 64)
    assert np.all(codes[L:] == 0), "padded rows must be 0"
    for b in range(nb):
        blk = x[b * 64:min(L, b * 64 + 64)].astype(np.float64)
        cb = codes[b * 64:min(L, b * 64 + 64)].astype(np.int64)
        a = np.abs(blk).max()
        assert scales[b] == np.float32(np.float32(a) / np.float32(127.0))
        if a == 0:
            assert np.all(cb == 0)
            continue
        s = float(scales[b])
        assert np.all(np.abs(cb) <= 127)
        # nearest integer to the exact quotient (a half-integer tie may go either way)
        assert np.all(np.abs(blk / s - cb) <= 0.5 + 1e-5)
        # the absmax element codes to +-127
        i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        assert abs(cb[i, j]) == 127
        # reconstruction error within half a step
        assert np.all(np.abs(cb * s - blk) <= 0.5 * s * (1 + 1e-5))


@pytest.mark.parametrize("Lq,Lkv,D", SHAPES)
def test_q_and_smoothed_k_codes_are_nearest_block_codes(Lq, Lkv, D):
    qb, kb, vb = _head(Lq, Lkv, D, seed=3 * Lq + Lkv, sigma=4.0)
    p = oracle.prep_head(qb, kb, vb)
    qf = oracle.bf16_to_f32(qb)
    kf = oracle.bf16_to_f32(kb)
    ks = (kf - p["k_mean"][None, :]).astype(np.float32)  # one fp32 subtraction per element
    _check_int8_blocks(qf, p["q8"], p["q_scale"], Lq)
    _check_int8_blocks(ks, p["k8"], p["k_scale"], Lkv)


def test_smoothing_removes_the_channel_offset():
    """K = K0 + offset: smoothed codes of K equal those of K0 - mean(K0) when
    the offset is exactly representable and does not change rounding."""
    D, L = 64, 128
    rng = np.random.default_rng(5)
    k0 = oracle.bf16_to_f32(oracle.bf16_round(rng.integers(-8, 9, (L, D)).astype(np.float32) / 8))
    off = rng.integers(-16, 17, D).astype(np.float32)
    k1 = k0 + off[None, :]  # exact: small dyadic values
    p0 = oracle.prep_head(oracle.bf16_round(k0), oracle.bf16_round(k0), oracle.bf16_round(k0))
    p1 = oracle.prep_head(oracle.bf16_round(k0), oracle.bf16_round(k1), oracle.bf16_round(k0))
    np.testing.assert_array_equal(p1["k_mean"], p0["k_mean"] + off)
    np.testing.assert_array_equal(p1["k8"], p0["k8"])
    np.testing.assert_array_equal(p1["k_scale"], p0["k_scale"])


def test_zero_blocks_have_zero_scale_and_codes():
    D, L = 64, 130
    q = np.zeros((L, D), np.float32)
    q[70:, :] = 1.5
    k = np.tile(np.linspace(-3, 3, D, dtype=np.float32), (L, 1))  # constant per channel
    p = oracle.prep_head(oracle.bf16_round(q), oracle.bf16_round(k), oracle.bf16_round(q))
    assert p["q_scale"][0] == 0 and np.all(p["q8"][:64] == 0)
    assert p["q_scale"][1] > 0
    assert np.all(p["k_scale"] == 0) and np.all(p["k8"] == 0)


@pytest.mark.parametrize("Lq,Lkv,D", SHAPES)
def test_v_fp8_codes(Lq, Lkv, D):
    qb, kb, vb = _head(Lq, Lkv, D, seed=Lq * 7 + Lkv)
    p = oracle.prep_head(qb, kb, vb)
    vf = oracle.bf16_to_f32(vb).astype(np.float64)
    sv = p["v_scale"].astype(np.float64)
    a = np.abs(vf).max(axis=0)
    np.testing.assert_array_equal(p["v_scale"], (a.astype(np.float32) / np.float32(448.0)))
    v8 = p["v8"]
    assert np.all(v8[Lkv:] == 0)
    dec = oracle.e4m3_decode(v8[:Lkv])
    assert np.all(np.abs(dec) <= 448)
    # the channel absmax maps to +-448
    for c in range(D):
        t = np.argmax(np.abs(vf[:, c]))
        assert abs(dec[t, c]) == 448.0
    # relative error of a normal E4M3 value <= 2^-4, absolute <= 2^-10 in the subnormal range
    y = vf / sv[None, :]
    err = np.abs(dec - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))


def test_dequantized_scores_track_fp32_scores():
    """q8 . k8 * sq * sk approximates Q . (K - mean) within the INT8 step bound."""
    qb, kb, vb = _head(64, 64, 128, seed=99, sigma=2.0)
    p = oracle.prep_head(qb, kb, vb)
    qf = oracle.bf16_to_f32(qb).astype(np.float64)
    ks = (oracle.bf16_to_f32(kb) - p["k_mean"]).astype(np.float64)
    acc = p["q8"][:64].astype(np.int64) @ p["k8"][:64].astype(np.int64).T
    approx = acc * float(p["q_scale"][0]) * float(p["k_scale"][0])
    exact = qf @ ks.T
    sq, sk = float(p["q_scale"][0]), float(p["k_scale"][0])
    bound = 0.5 * sk * np.abs(qf).sum(1)[:, None] + 0.5 * sq * np.abs(ks).sum(1)[None, :] + 0.25 * 128 * sq * sk
    assert np.all(np.abs(approx - exact) <= bound * (1 + 1e-6))


# ---------------------------------------------------------------------------
# Rounding rule and quotient of the codes, pinned on constructed blocks
# (BASELINE workload contract: scale = absmax/127, round half to even, clamp;
# V scale = absmax/448 with E4M3FN nearest-even codes). Each case below tells
# the contract's rule apart from a plausible slip: rounding ties away from
# zero, or multiplying by a rounded reciprocal of the scale instead of
# dividing by it.

def _bits(x):
    """bf16 bits of float32 values that are already bf16 numbers (exact)."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def _all_positive_bf16():
    b = np.arange(0x0001, 0x7F80, dtype=np.uint32)  # every positive finite bf16
    return (b << 16).view(np.float32)


# half-integers with their round-half-to-even integers (hand table)
_TIES = [(0.5, 0), (1.5, 2), (2.5, 2), (3.5, 4), (4.5, 4), (63.5, 64), (64.5, 64), (125.5, 126), (126.5, 126)]


def test_int8_ties_round_half_to_even():
    """Absmax 127 makes the block scale exactly 1, so every half-integer is a
    tie: the contract's codes are the even neighbours (rint), where rounding
    half away from zero would give 1, 3, 5, 65, 127 for some of them."""
    D = 64
    q = np.zeros((64, D), np.float32)
    q[0, 0] = 127.0
    for i, (x, _) in enumerate(_TIES):
        q[1, i], q[2, i] = x, -x
    # K: rows in (+, -) pairs, so every channel sums to zero and the mean is
    # exactly 0: the smoothed values are the raw ones.
    k = np.zeros((64, D), np.float32)
    k[:3] = q[:3]
    k[3:6] = -q[:3]
    p = oracle.prep_head(_bits(q), _bits(k), _bits(q))
    assert p["q_scale"][0] == 1.0 and p["k_scale"][0] == 1.0 and np.all(p["k_mean"] == 0)
    for i, (x, code) in enumerate(_TIES):
        assert p["q8"][1, i] == code and p["q8"][2, i] == -code, (x, p["q8"][1, i])
        assert p["k8"][1, i] == code and p["k8"][4, i] == -code, (x, p["k8"][1, i])


def test_v_ties_round_to_even_code():
    """V channel absmax 448 makes its scale exactly 1: the V codes are the
    E4M3FN codes of the values themselves. Values halfway between two E4M3
    neighbours take the neighbour with the even code (OCP FP8 rounding)."""
    # (value, expected code): 1.0625 lies between 1.0 (0x38) and 1.125 (0x39),
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A), 2.125 between 2.0 (0x40)
    # and 2.25 (0x41), 12.5 between 12 (0x54) and 13 (0x55), 0.0029296875
    # (3 * 2^-10) between the subnormals 2^-9 (0x01) and 2^-8 (0x02).
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.125, 0x40), (12.5, 0x54), (3 * 2.0 ** -10, 0x02)]
    D, L = 64, 64
    v = np.zeros((L, D), np.float32)
    v[0, :len(cases)] = 448.0
    for i, (x, _) in enumerate(cases):
        v[1, i], v[2, i] = x, -x
    z = np.zeros((L, D), np.float32)
    p = oracle.prep_head(_bits(z), _bits(z), _bits(v))
    for i, (x, code) in enumerate(cases):
        assert p["v_scale"][i] == 1.0
        assert p["v8"][1, i] == code and p["v8"][2, i] == code | 0x80, (x, hex(p["v8"][1, i]))


def _straddles_int8():
    """(a, x): block absmax a and a value x whose code from the IEEE quotient
    RN(x / s), s = RN(a / 127), differs from the code from RN(x * RN(1 / s)).
    Exhaustive over bf16 x <= a for every bf16 a in [1, 2)."""
    allv = _all_positive_bf16()
    out = []
    for a in allv[(allv >= 1.0) & (allv < 2.0)]:
        s = np.float32(a) / np.float32(127.0)
        xs = allv[allv <= a]
        ieee = np.rint(xs / s)
        alt = np.rint(xs * (np.float32(1.0) / s))
        for x in xs[ieee != alt]:
            out.append((np.float32(a), np.float32(x)))
    return out


def test_int8_codes_follow_the_ieee_quotient():
    cases = _straddles_int8()
    assert len(cases) >= 10
    D = 64
    n = len(cases)
    q = np.zeros((64 * n, D), np.float32)
    k = np.zeros((64 * n, D), np.float32)
    for b, (a, x) in enumerate(cases):
        r = 64 * b
        q[r, 0], q[r + 1, 1], q[r + 1, 2] = a, x, -x
        # K block: (+, -) row pairs, so the channel means are exactly 0
        k[r, 0], k[r + 1, 0], k[r + 2, 1], k[r + 3, 1] = a, -a, x, -x
    p = oracle.prep_head(_bits(q), _bits(k), _bits(q))
    assert np.all(p["k_mean"] == 0)
    for b, (a, x) in enumerate(cases):
        s = a / np.float32(127.0)
        want = int(np.rint(x / s))            # numpy float32 division: IEEE quotient
        slip = int(np.rint(x * (np.float32(1.0) / s)))
        assert want != slip
        assert p["q_scale"][b] == s and p["k_scale"][b] == s
        r = 64 * b
        assert (p["q8"][r + 1, 1], p["q8"][r + 1, 2]) == (want, -want), (a, x, p["q8"][r + 1, 1], want)
        assert (p["k8"][r + 2, 1], p["k8"][r + 3, 1]) == (want, -want), (a, x, p["k8"][r + 2, 1], want)


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_v_codes_follow_the_ieee_quotient():
    """Values whose E4M3 code from the IEEE quotient RN(v / sv), sv =
    RN(a / 448), differs from the code from RN(v * RN(1 / sv)); exhaustive
    over bf16 v in [a 2^-9, a] for every bf16 channel absmax a in [1, 2).
    Expected codes: torch's E4M3FN cast of numpy's float32 quotient."""
    allv = _all_positive_bf16()
    chans = []
    for a in allv[(allv >= 1.0) & (allv < 2.0)]:
        sv = np.float32(a) / np.float32(448.0)
        xs = allv[(allv <= a) & (allv >= a * 2.0 ** -9)]
        d = _torch_e4m3(xs / sv) != _torch_e4m3(xs * (np.float32(1.0) / sv))
        if d.any():
            chans.append((np.float32(a), xs[d]))
    assert len(chans) >= 3 and sum(len(x) for _, x in chans) >= 20
    D = 64
    assert len(chans) <= D
    L = 1 + 2 * max(len(x) for _, x in chans)
    v = np.zeros((L, D), np.float32)
    for c, (a, xs) in enumerate(chans):
        v[0, c] = a
        v[1:1 + len(xs), c] = xs
        v[1 + len(xs):1 + 2 * len(xs), c] = -xs
    z = np.zeros((L, D), np.float32)
    p = oracle.prep_head(_bits(z), _bits(z), _bits(v))
    for c, (a, xs) in enumerate(chans):
        sv = a / np.float32(448.0)
        assert p["v_scale"][c] == sv
        want = _torch_e4m3(np.concatenate([xs, -xs]) / sv)
        got = p["v8"][1:1 + 2 * len(xs), c]
        assert np.array_equal(got, want), (a, got, want)
