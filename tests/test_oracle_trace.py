"""The oracle's per-epoch checkpoints (m, l, alpha, P8, PV, RO, r) are its own
epoch loop copied out: they reproduce the row output bit for bit, replay the
outer PV level RO = RO * alpha + PV exactly in fp32, and keep the online
softmax invariants (Experiment Log, "Phase 2B Fixed Aligned Numerical
Prototype": the checkpoint list; "Phase 1 State-Ownership Decision": strict
tile order, per-tile RO rescaling)."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si

E4M3_ONE = 0x38  # the code of 1.0


def _prep(Lq, Lkv, D, seed):
    q, k, v = si.make_qkv(1, 1, Lq, Lkv, D, "normal", 2.0, seed)
    return oracle.prep_head(*(si.bf16_bits(t[0, 0]) for t in (q, k, v)))


@pytest.mark.parametrize("Lq,Lkv,D,causal", [(128, 192, 128, False), (200, 200, 64, True), (65, 130, 128, True)])
def test_trace_reproduces_rows_and_replays_the_outer_level(Lq, Lkv, D, causal):
    p = _prep(Lq, Lkv, D, seed=11)
    sm = 1.0 / np.sqrt(D)
    rows = oracle.attn_rows(p, causal, sm)
    nkb = -(-Lkv // 64)
    for i in sorted({0, 1, 63, 64, Lq // 2, Lq - 1}):
        t = oracle.attn_row_trace(p, causal, sm, i)
        assert np.array_equal(t["out"], rows[i]), i
        st, ro, pv = t["stats"], t["ro"], t["pv"]
        prev = np.zeros(D, np.float32)
        m_prev = -np.inf
        for e in range(nkb):
            m, l, alpha = st[e, 0], st[e, 1], st[e, 2]
            want = (prev * np.float32(alpha) + pv[e]).astype(np.float32)
            assert np.array_equal(ro[e], want), (i, e)
            assert m >= m_prev and 0.0 <= alpha <= 1.0
            assert t["p8"][e].max() <= E4M3_ONE  # p <= 1
            if m_prev == -np.inf and np.isfinite(m):
                assert alpha == 0.0  # first live epoch
            prev, m_prev = ro[e], m
        l_end, r = st[nkb, 1], st[nkb, 0]
        assert l_end == st[nkb - 1, 1]
        assert r == (np.float32(1.0) / np.float32(l_end) if l_end > 0 else 0.0)
        want_out = oracle.bf16_round((ro[nkb - 1] * r).astype(np.float32) * p["v_scale"])
        assert np.array_equal(t["out"], want_out)


def test_trace_of_masked_epochs_carries_the_state():
    # causal with Lq = Lkv: row 5 sees only epoch 0; later epochs keep its state
    p = _prep(192, 192, 64, seed=12)
    t = oracle.attn_row_trace(p, True, 0.125, 5)
    st = t["stats"]
    for e in (1, 2):
        assert st[e, 0] == st[0, 0] and st[e, 1] == st[0, 1] and st[e, 2] == 1.0
        assert np.array_equal(t["ro"][e], t["ro"][0]) and not t["p8"][e].any()
    assert not t["p8"][0][6:].any()  # keys 6.. of epoch 0 are masked
    assert t["p8"][0][:6].all() or t["p8"][0][:6].max() > 0
