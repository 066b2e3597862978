"""The compact-oracle helper of the full-size GPU tests (tests.common.TailCase) against the
full-problem oracle: with only the last rows of each sequence live (every other row has
softmaxSum = 0, so p = 0 there), the sub-problem must give the same dQ, dK, dKRope and dV, and
the full-size operator inputs it builds must match the full oracle's forward on the live rows."""

import numpy as np
import pytest

from sparse_mla_flash_amd import inputs
from tests.common import Case, TailCase


@pytest.mark.parametrize("spec,tail,kind", [
    (dict(layout="TND", B=3, seq_q=[30, 45, 20], seq_kv=[40, 45, 60], N1=4, topk=24, sparse_mode=3), [7, 19, 0],
     "uniform"),
    (dict(layout="BSND", B=2, S1=33, S2=70, N1=3, topk=20, sparse_mode=3, seq_q=[33, 25], seq_kv=[70, 50]),
     [9, 4], "uniform"),
    (dict(layout="BSND", B=1, S1=40, S2=300, N1=2, topk=32, sparse_mode=3), [25], "window"),
    (dict(layout="BSND", B=1, S1=16, S2=90, N1=2, topk=5, sparse_mode=0, block=4), [6], "uniform"),
])
def test_tail_case_matches_full_oracle(spec, tail, kind):
    p = inputs.problem(**spec)
    inputs.generate(p, 77, index_kind=kind, window=64)
    t = TailCase(p, tail)
    full = Case(p, fwd_rows=t.live)
    # operator inputs of the live rows (and zeros elsewhere)
    assert np.array_equal(t.out_bits, full.out_bits)
    assert np.array_equal(t.m_full, full.m32)
    assert np.array_equal(t.l_full, full.l32)
    pos = np.arange(len(t.live))
    dq, dqr = t.ref_dq(pos)
    fdq, fdqr = full.ref_dq(rows=t.live)
    np.testing.assert_allclose(dq, fdq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dqr, fdqr, rtol=0, atol=1e-12)
    keys = np.arange(p.keys)
    dk, dkr, dv = t.ref_dkv(keys)
    fdk, fdkr, fdv = full.ref_dkv(keys=keys)
    for a, b in ((dk, fdk), (dkr, fdkr), (dv, fdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    assert np.abs(fdv).max() > 0


def test_keys_from_segments_spans_segments():
    p = inputs.problem(layout="TND", B=2, seq_q=[40, 50], seq_kv=[40, 50], N1=2, topk=30, sparse_mode=3)
    inputs.generate(p, 5)
    t = TailCase(p, [0, 35])
    keys = t.keys_from_segments(np.random.default_rng(0), 10, seg_rows=8, min_segments=3)
    assert len(keys) > 0
    idx = p.idx.reshape(p.rows, -1)
    for j in keys:
        segs = {(r - p.q_offset(1)) // 8 for r in t.live if j - p.k_offset(1) in set(idx[r].tolist())}
        assert len(segs) >= 3
