"""The INT8 QK scores of the main loop's matrix-core code, bit for bit: the
int32 tiles of sage_debug_qk_int32 equal the exact integer product of the
oracle's codes (which the preparation tests show equal the GPU's)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import quantized_exact_attention_smooth_amd as sage
from _parity import oracle_preps, say

pytestmark = pytest.mark.gpu


def _tiles_for(B, H, nqb, nkb, n, seed):
    rng = np.random.default_rng(seed)
    t = {(0, 0, 0, 0), (B - 1, H - 1, nqb - 1, nkb - 1), (0, H - 1, nqb - 1, 0), (B - 1, 0, 0, nkb - 1)}
    while len(t) < n:
        t.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nqb)), int(rng.integers(nkb))))
    return sorted(t)


@pytest.mark.parametrize("B,H,Lq,Lkv,D,sigma", [(1, 1, 128, 192, 128, 2.0), (1, 8, 1000, 1000, 128, 2.0),
                                                (2, 3, 333, 130, 64, 4.0), (1, 2, 65, 1, 64, 1.0),
                                                (2, 4, 2048, 2048, 128, 4.0)])
def test_qk_int32_tiles_exact(B, H, Lq, Lkv, D, sigma, gpu_device):
    say(f"qk int32 parity: {(B, H, Lq, Lkv, D)}")
    q, k, v = si.make_qkv(B, H, Lq, Lkv, D, "normal", sigma, seed=Lq * 3 + Lkv)
    p = sage.quant_prep(q.to(gpu_device), k.to(gpu_device), v.to(gpu_device))
    nqb, nkb = -(-Lq // 64), -(-Lkv // 64)
    tiles = _tiles_for(B, H, nqb, nkb, min(96, B * H * nqb * nkb), seed=D)
    acc = sage.debug_qk_int32(p, tiles)
    torch.cuda.synchronize()
    acc = acc.cpu().numpy()
    orc = oracle_preps(q, k, v, sorted({(b, h) for (b, h, _, _) in tiles}))
    for i, (b, h, qb, kb) in enumerate(tiles):
        o = orc[(b, h)]
        qc = o["q8"][qb * 64:qb * 64 + 64].astype(np.int64)
        kc = o["k8"][kb * 64:kb * 64 + 64].astype(np.int64)
        want = qc @ kc.T
        assert np.abs(want).max() < 2 ** 24
        assert np.array_equal(acc[i], want), f"tile {(b, h, qb, kb)}"


def test_qk_int32_extreme_codes(gpu_device):
    """All codes +-127 (largest products): the int32 path stays exact."""
    B, H, L, D = 1, 1, 128, 128
    rng = np.random.default_rng(3)
    sign = rng.choice([-1.0, 1.0], (B, H, L, D)).astype(np.float32)
    t = torch.from_numpy(sign).to(torch.bfloat16)
    p = sage.quant_prep(t.to(gpu_device), t.to(gpu_device), t.to(gpu_device))
    assert int(p["q_i8"].abs().min()) == 127
    tiles = [(0, 0, a, b) for a in range(2) for b in range(2)]
    say("qk int32 parity: extreme codes")
    acc = sage.debug_qk_int32(p, tiles).cpu().numpy()
    qc = p["q_i8"].cpu().numpy()[0, 0].astype(np.int64)
    kc = p["k_i8"].cpu().numpy()[0, 0].astype(np.int64)
    for i, (_, _, a, b) in enumerate(tiles):
        assert np.array_equal(acc[i], qc[a * 64:a * 64 + 64] @ kc[b * 64:b * 64 + 64].T)
