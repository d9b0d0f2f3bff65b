"""Helpers shared by the GPU parity tests: run the oracle on chosen heads or
rows and compare with the HIP library's outputs."""
import math
import sys

import numpy as np
import torch

import oracle
import seeded_inputs as si

MAX_ABS = 2e-2   # bf16 output vs the oracle, per checked head or block
MEAN_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def head_bits(t, b, h):
    return si.bf16_bits(t[b, h])


def oracle_preps(q, k, v, heads, threads=None):
    """{(b, h): oracle prep dict} computed on a thread pool."""
    def one(bh):
        b, h = bh
        return bh, oracle.prep_head(head_bits(q, b, h), head_bits(k, b, h), head_bits(v, b, h))
    return dict(oracle.run_heads(one, list(heads), threads))


def gpu_prep_numpy(p):
    """GPU prep outputs as numpy, V codes re-laid token-major [B, H, NKB*64, D]."""
    r = {n: p[n].cpu().numpy() for n in ("q_i8", "q_scale", "k_i8", "k_scale", "k_mean", "v_scale")}
    v = p["v_fp8"].cpu().numpy()  # [B, H, NKB, D, 64]
    B, H, nkb, D, _ = v.shape
    r["v8"] = v.transpose(0, 1, 2, 4, 3).reshape(B, H, nkb * 64, D)
    return r


def assert_prep_equal(g, o, b, h):
    """Bit-exact comparison of one head's prepared operands."""
    for gk, ok in (("q_i8", "q8"), ("k_i8", "k8"), ("v8", "v8")):
        a, e = g[gk][b, h], o[ok]
        if not np.array_equal(a, e):
            bad = np.argwhere(a != e)
            raise AssertionError(f"{gk} head ({b},{h}): {len(bad)} codes differ, first at {bad[0].tolist()}: "
                                 f"gpu {a[tuple(bad[0])]} oracle {e[tuple(bad[0])]}")
    for gk, ok in (("q_scale", "q_scale"), ("k_scale", "k_scale"), ("k_mean", "k_mean"), ("v_scale", "v_scale")):
        a, e = g[gk][b, h], o[ok]
        if not np.array_equal(a.view(np.uint32), e.view(np.uint32)):
            bad = np.argwhere(a.view(np.uint32) != e.view(np.uint32))
            raise AssertionError(f"{gk} head ({b},{h}): {len(bad)} values differ, first {bad[0].tolist()}: "
                                 f"gpu {a[tuple(bad[0])]!r} oracle {e[tuple(bad[0])]!r}")


def out_errors(gpu_bits, orc_bits):
    a = oracle.bf16_to_f32(gpu_bits).astype(np.float64)
    e = oracle.bf16_to_f32(orc_bits).astype(np.float64)
    d = np.abs(a - e)
    return float(d.max()), float(d.mean())


# Worst output margins seen per comparison label in this session (label ->
# [max-abs, mean-abs, comparisons]); conftest prints them at the end.
MARGINS = {}


def _label(what):
    """Group comparisons by their workload or shape (drop head/row indices)."""
    return what.split(" (")[0].split(" head")[0].strip() or "unlabelled"


def assert_out_close(gpu_bits, orc_bits, what=""):
    mx, mean = out_errors(gpu_bits, orc_bits)
    m = MARGINS.setdefault(_label(what), [0.0, 0.0, 0])
    m[0], m[1], m[2] = max(m[0], mx), max(m[1], mean), m[2] + 1
    assert np.all(np.isfinite(oracle.bf16_to_f32(gpu_bits))), f"{what}: non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def oracle_rows(prep, causal, sm_scale, r0, r1):
    """Oracle output rows [r0, r1) (bf16 bits), split over the cores."""
    return oracle.attn_rows_parallel(prep, causal, sm_scale, r0, r1, chunk=64)


def cosine(a_bits, ref):
    a = oracle.bf16_to_f32(a_bits).astype(np.float64).ravel()
    b = np.asarray(ref, np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def to_gpu(*ts):
    return [t.cuda() for t in ts]
