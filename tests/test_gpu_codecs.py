"""GPU conversions against the oracle's codecs, bit for bit.

  * sage_debug_codecs runs the FP8 packing the main loop applies to P and the
    bf16 conversion of its epilogue on chosen fp32 values;
  * the preparation pass's E4M3 encoder is driven exhaustively: a V channel
    whose absmax is 448 has scale exactly 1, so every bf16 value in
    [-448, 448] placed in that channel is encoded as itself.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_exact_attention_smooth_amd as sage
from _parity import say

pytestmark = pytest.mark.gpu


def _sweep():
    rng = np.random.default_rng(0)
    pos = np.arange(127, dtype=np.uint8)
    table = oracle.e4m3_decode(pos)
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    x = np.concatenate([
        np.linspace(0, 1, 200001, dtype=np.float32), 2.0 ** rng.uniform(-24, 0, 100000).astype(np.float32),
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000)), table.astype(np.float32),
        rng.uniform(-448, 448, 100000).astype(np.float32),
        np.array([0.0, -0.0, 2 ** -10, 3 * 2 ** -11, 2 ** -9, 2 ** -6, 1.0, 448.0], np.float32)])
    return x.astype(np.float32)


def test_p8_packing_matches_oracle_encoder(gpu_device):
    x = _sweep()
    x = x[np.abs(x) <= 448]
    say(f"debug_codecs on {x.size} values")
    p8, bf = sage.debug_codecs(torch.from_numpy(x).to(gpu_device))
    torch.cuda.synchronize()
    got = p8.cpu().numpy()
    want = oracle.e4m3_encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} FP8 codes differ, e.g. x={x[bad[:5]]} gpu={got[bad[:5]]} oracle={want[bad[:5]]}"


def test_bf16_conversion_matches_oracle(gpu_device):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 3,
                        ((rng.integers(0, 2 ** 16, 50000).astype(np.uint32) << 16) | 0x8000).view(np.float32)])
    x = x[np.isfinite(x)]
    say(f"debug_codecs bf16 on {x.size} values")
    _, bf = sage.debug_codecs(torch.from_numpy(x).to(gpu_device))
    torch.cuda.synchronize()
    got = bf.cpu().numpy().view(np.uint16)
    want = oracle.bf16_round(x)
    assert np.array_equal(got, want)


def test_prep_v_encoder_is_exhaustive_over_bf16(gpu_device):
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f32(all_bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    bits = all_bits[keep]
    D = 128
    L = -(-(bits.size) // D) + 1
    col = np.zeros((L, D), np.uint16)
    flat = np.concatenate([bits, np.zeros(L * D - D - bits.size, np.uint16)])
    col[1:] = flat.reshape(L - 1, D)
    col[0] = oracle.bf16_round(np.full(D, 448.0, np.float32))  # channel absmax 448 -> scale 1
    t = torch.from_numpy(col.view(np.int16)).view(torch.bfloat16).reshape(1, 1, L, D)
    say(f"prep over {bits.size} bf16 values, L={L}")
    p = sage.quant_prep(t.to(gpu_device), t.to(gpu_device), t.to(gpu_device))
    torch.cuda.synchronize()
    assert np.all(p["v_scale"].cpu().numpy() == 1.0)
    v = p["v_fp8"].cpu().numpy()[0, 0]  # [NKB, D, 64]
    got = v.transpose(0, 2, 1).reshape(-1, D)[:L]
    want = oracle.e4m3_encode(oracle.bf16_to_f32(col))
    assert np.array_equal(got, want)
