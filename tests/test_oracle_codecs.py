"""Pins for the oracle's number codecs (bf16 and FP8 E4M3FN).

Each check is independent of the oracle's code: printed format values
(tests/golden/e4m3fn_points.txt, OCP FP8 specification), torch's own casts,
and brute-force nearest-value search in numpy.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_points.txt")


def _golden_points():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                pts.append((int(c, 16), float(v)))
    return pts


def test_e4m3_decode_matches_printed_format_values():
    for code, value in _golden_points():
        got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        if np.isnan(value):
            assert np.isnan(got), hex(code)
        else:
            assert got == value and np.signbit(got) == np.signbit(value), hex(code)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))
    assert np.isnan(got).sum() == 2


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def _nearest_even_bruteforce(x):
    """Nearest finite E4M3 value by exhaustive search; ties to the even code;
    magnitudes beyond 448 saturate."""
    pos = np.arange(127, dtype=np.uint8)
    table = torch.from_numpy(pos).view(torch.float8_e4m3fn).double().numpy()
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates take the even code
    idx = np.where(cand & (pos[None, :] % 2 == 0), pos[None, :], 255).min(axis=1)
    only = np.where(cand, pos[None, :], 255).min(axis=1)
    code = np.where(cand.sum(axis=1) > 1, idx, only).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def test_e4m3_encode_is_nearest_even_on_dense_sweep():
    rng = np.random.default_rng(7)
    pos = np.arange(126, dtype=np.uint8)
    table = torch.from_numpy(pos).view(torch.float8_e4m3fn).float().numpy()
    mids = ((table[:-1].astype(np.float64) + table[1:]) / 2).astype(np.float32)  # exact ties
    sweep = np.concatenate([
        rng.uniform(0, 1, 20000), rng.uniform(0, 448, 20000), 2.0 ** rng.uniform(-14, 9, 20000),
        mids, np.nextafter(mids, 0), np.nextafter(mids, 1000), table,
        [0.0, 2 ** -10, 3 * 2 ** -11, 448.0, 449.0, 464.0, 470.0, 1e6, np.inf]]).astype(np.float32)
    sweep = np.concatenate([sweep, -sweep])
    got = oracle.e4m3_encode(sweep)
    assert np.array_equal(got, _nearest_even_bruteforce(sweep))


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000) * 50, rng.uniform(-1, 1, 50000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


def test_e4m3_encode_saturates_instead_of_nan():
    x = np.array([448.0, 463.9, 464.0, 500.0, 1e30, np.inf, -464.0, -np.inf], np.float32)
    assert list(oracle.e4m3_encode(x)) == [0x7E] * 6 + [0xFE] * 2
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_small_values_flush_and_keep_sign():
    x = np.array([2 ** -10, 2 ** -11, -2 ** -11, 1.5 * 2 ** -10, 0.0, -0.0], np.float32)
    assert list(oracle.e4m3_encode(x)) == [0x00, 0x00, 0x80, 0x01, 0x00, 0x80]


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(10000) * 1e30).astype(np.float32),
                        (rng.standard_normal(10000) * 1e-30).astype(np.float32)])
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    # exact ties: low 16 bits == 0x8000
    ties = ((rng.integers(0, 2 ** 16, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, y, ties[np.isfinite(ties)], np.array([3.3895314e38, -3.3895314e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(x), ref)


def test_bf16_to_f32_is_exact_widening():
    b = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_to_f32(b)
    ok = (np.isnan(ref) & np.isnan(got)) | (ref == got)
    assert np.all(ok)
