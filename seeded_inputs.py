"""Seeded synthetic inputs for the quantized-attention workloads.

This module only draws random numbers and rounds them to bf16 storage. It holds
none of the attention method's arithmetic, so both the CPU oracle and the HIP
library can take their inputs from it without sharing any computation.

Workloads (shapes, masks and value distributions) stand in for the private,
fixed fixture the Experiment Log measures on (Phase 2A "canonical Q/K/V/output
fixtures" and Phase 2B "Q128 x KV192 x D128"); no public dataset is involved.

Recipe
  * generator: numpy PCG64 seeded with SeedSequence([seed, stream]); one
    stream per tensor: Q=1, K=2, V=3, K offset=4, outlier channels=5,
    oracle sample choice=6.
  * "normal": Q, K, V ~ N(0, 1) drawn as float32; K gets a per-(b, h, channel)
    offset ~ N(0, sigma) (sigma is a standard deviation) added in float32.
  * "student_t_outlier": Q, K = 0.5 * t(nu=3); 4 seeded K channels (the same
    for every head) multiplied by 20; V ~ N(0, 1).
  * storage: float32 -> bf16 by torch's round-to-nearest-even cast, layout
    [B, H, L, D] with D contiguous.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np
import torch

STREAM_Q, STREAM_K, STREAM_V, STREAM_OFFSET, STREAM_OUTLIER, STREAM_SAMPLE = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Lq: int
    Lkv: int
    D: int
    causal: bool
    dist: str = "normal"
    k_offset_sigma: float = 0.0
    # what the oracle checks in full at this size: "all" heads, n seeded
    # (b, h) "heads", or n seeded 64-row query "blocks"
    oracle_subset: Tuple[str, int] = ("all", 0)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def metric_ops(self) -> float:
        """4*B*H*Lq*Lkv*D, halved when causal (the throughput convention)."""
        ops = 4.0 * self.B * self.H * self.Lq * self.Lkv * self.D
        return ops / 2 if self.causal else ops


WORKLOADS: List[Workload] = [
    Workload("q128_kv192_d128", 1, 1, 128, 192, 128, False, "normal", 2.0, ("all", 0)),
    Workload("ragged_causal_b1_h8_l1000_d128", 1, 8, 1000, 1000, 128, True, "normal", 2.0, ("all", 0)),
    Workload("causal_b2_h32_l4096_d128", 2, 32, 4096, 4096, 128, True, "normal", 4.0, ("heads", 8)),
    Workload("long_b1_h24_l32760_d128", 1, 24, 32760, 32760, 128, False, "normal", 2.0, ("blocks", 16)),
    Workload("outlier_causal_b4_h16_l8192_d64", 4, 16, 8192, 8192, 64, True, "student_t_outlier", 0.0,
             ("blocks", 16)),
]
HEADLINE = 2


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 array -> bf16 tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (CPU or GPU) -> uint16 numpy array of its storage bits."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def draw_qkv_f32(B, H, Lq, Lkv, D, dist="normal", k_offset_sigma=0.0, seed=0):
    """The float32 draws before bf16 rounding (see module docstring)."""
    if dist == "normal":
        q = _rng(seed, STREAM_Q).standard_normal((B, H, Lq, D), dtype=np.float32)
        k = _rng(seed, STREAM_K).standard_normal((B, H, Lkv, D), dtype=np.float32)
        v = _rng(seed, STREAM_V).standard_normal((B, H, Lkv, D), dtype=np.float32)
        if k_offset_sigma:
            off = _rng(seed, STREAM_OFFSET).normal(0.0, k_offset_sigma, (B, H, 1, D)).astype(np.float32)
            k += off
    elif dist == "student_t_outlier":
        q = (0.5 * _rng(seed, STREAM_Q).standard_t(3.0, (B, H, Lq, D))).astype(np.float32)
        k = (0.5 * _rng(seed, STREAM_K).standard_t(3.0, (B, H, Lkv, D))).astype(np.float32)
        ch = _rng(seed, STREAM_OUTLIER).choice(D, size=4, replace=False)
        k[..., ch] *= np.float32(20.0)
        v = _rng(seed, STREAM_V).standard_normal((B, H, Lkv, D), dtype=np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return q, k, v


def make_qkv(B, H, Lq, Lkv, D, dist="normal", k_offset_sigma=0.0, seed=0):
    """bf16 CPU tensors q [B,H,Lq,D], k and v [B,H,Lkv,D]."""
    q, k, v = draw_qkv_f32(B, H, Lq, Lkv, D, dist, k_offset_sigma, seed)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def workload_qkv(w: Workload, seed: int = None):
    """Inputs of a named workload; the default seed is its index in WORKLOADS."""
    if seed is None:
        seed = WORKLOADS.index(w)
    return make_qkv(w.B, w.H, w.Lq, w.Lkv, w.D, w.dist, w.k_offset_sigma, seed)


def oracle_heads(w: Workload, seed: int = None) -> List[Tuple[int, int]]:
    """(b, h) pairs the oracle checks in full."""
    if seed is None:
        seed = WORKLOADS.index(w)
    all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    kind, n = w.oracle_subset
    if kind == "all" or n >= len(all_heads):
        return all_heads
    if kind == "heads":
        idx = _rng(seed, STREAM_SAMPLE).choice(len(all_heads), size=n, replace=False)
        return [all_heads[i] for i in sorted(idx)]
    return sorted({(b, h) for (b, h, _) in oracle_blocks(w, seed)})


def oracle_blocks(w: Workload, seed: int = None) -> List[Tuple[int, int, int]]:
    """(b, h, query block) triples (64 rows each) the oracle checks; always
    includes the first and the last (possibly ragged) query block."""
    if seed is None:
        seed = WORKLOADS.index(w)
    nqb = (w.Lq + 63) // 64
    kind, n = w.oracle_subset
    if kind != "blocks":
        return [(b, h, qb) for (b, h) in oracle_heads(w, seed) for qb in range(nqb)]
    r = _rng(seed, STREAM_SAMPLE)
    picks = {(0, 0, 0), (w.B - 1, w.H - 1, nqb - 1)}
    while len(picks) < n:
        picks.add((int(r.integers(w.B)), int(r.integers(w.H)), int(r.integers(nqb))))
    return sorted(picks)
