"""Pins for the oracle's preparation pass: K channel mean, K smoothing, INT8
block quantization of Q and K, and per-channel FP8 quantization of V.

Checks are stated against exact arithmetic (math.fsum, fp64 quotients), the
format's properties and hand-built special cases, never by re-running the
oracle's own formula.
"""
import math

import numpy as np
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
