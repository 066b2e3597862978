"""Host-side checks of the seeded input generators (no GPU, no oracle)."""

import numpy as np
import pytest

from sparse_mla_flash_amd import inputs


def _rows(p):
    """(global row, batch, position) for every active query row."""
    for b in range(p.B):
        for i in range(p.lq(b)):
            yield p.q_offset(b) + i, b, i


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-5, 1.0 + 2 ** -8], np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert back[5] == 1.0
    assert back[0] == 1.0 and back[3] == -2.5
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)


@pytest.mark.parametrize("mode", [0, 3])
def test_uniform_indices_are_distinct_valid_and_padded(mode):
    p = inputs.problem("BSND", B=2, S1=40, S2=50, N1=2, topk=16, sparse_mode=mode, seq_q=[40, 33],
                       seq_kv=[50, 20])
    inputs.generate(p, 3)
    idx = p.idx.reshape(p.rows, p.topk)
    for g, b, i in _rows(p):
        hi = min(i + p.lkv(b) - p.lq(b), p.lkv(b) - 1) if mode == 3 else p.lkv(b) - 1
        row = idx[g]
        valid = row[row >= 0]
        assert len(set(valid.tolist())) == len(valid)
        assert valid.min(initial=0) >= 0 and valid.max(initial=0) <= max(hi, 0)
        assert len(valid) == min(p.topk, max(hi + 1, 0))
        # padding sits at the tail
        assert (row[len(valid):] == -1).all()
    # padded query rows of batch 1 hold no selections
    assert (idx[p.q_offset(1) + 33:] == -1).all()


@pytest.mark.parametrize("mode", [0, 3])
def test_block_indices_are_distinct_reachable_blocks(mode):
    """Block selection: distinct block indices, each holding at least one reachable key; rows
    whose range spans at most topk blocks take all of them."""
    p = inputs.problem("BSND", B=2, S1=30, S2=70, N1=2, topk=6, sparse_mode=mode, seq_q=[30, 25],
                       seq_kv=[70, 33], block=8)
    inputs.generate(p, 5)
    idx = p.idx.reshape(p.rows, p.topk)
    for g, b, i in _rows(p):
        hi = min(i + p.lkv(b) - p.lq(b), p.lkv(b) - 1) if mode == 3 else p.lkv(b) - 1
        row = idx[g]
        valid = row[row >= 0]
        assert len(set(valid.tolist())) == len(valid)
        assert (valid * p.block <= hi).all()
        assert len(valid) == min(p.topk, max(hi // p.block + 1, 0) if hi >= 0 else 0)


def test_bench_valid_pair_count_with_blocks():
    """bench.py's valid-pair bookkeeping (the flop count of the metric) against a per-key
    brute-force count, with blocks cut by the key length and the causal bound."""
    import bench
    p = inputs.problem("BSND", B=2, S1=12, S2=30, N1=1, topk=5, sparse_mode=3, seq_q=[12, 9],
                       seq_kv=[30, 17], block=4)
    inputs.generate(p, 9)
    p.idx.reshape(p.rows, p.topk)[0, 0] = -1                  # a skipped block
    got = bench.valid_per_row(p)
    idx = p.idx.reshape(p.rows, p.topk)
    for g, b, i in _rows(p):
        hi = min(i + p.lkv(b) - p.lq(b), p.lkv(b) - 1)
        keys = [j * p.block + r for j in idx[g] if j >= 0 for r in range(p.block)]
        assert got[g] == sum(1 for k in keys if 0 <= k <= hi)


def test_window_indices_half_local():
    p = inputs.problem("BSND", B=1, S1=64, S2=4096, N1=1, topk=64, sparse_mode=3)
    inputs.generate(p, 4, index_kind="window", window=256)
    idx = p.idx.reshape(p.rows, p.topk)
    for g, b, i in _rows(p):
        pos = i + 4096 - 64
        row = idx[g]
        assert len(set(row.tolist())) == 64 and row.min() >= 0 and row.max() <= pos
        assert (row >= pos - 255).sum() >= 32


def test_hot_cold_indices():
    p = inputs.problem("BSND", B=2, S1=8, S2=200, N1=1, topk=60, sparse_mode=0)
    inputs.generate(p, 5, index_kind="hot_cold")
    idx = p.idx.reshape(p.rows, p.topk)
    for b in range(2):
        rows = idx[b * 8:(b + 1) * 8]
        counts = np.bincount(rows.reshape(-1), minlength=200)
        hot = np.nonzero(counts == 8)[0]
        assert len(hot) >= 20                     # the 20 hot keys are in every row
        for r in rows:
            assert len(set(r.tolist())) == 60 and r.min() >= 0


def test_generation_is_seeded():
    a = inputs.generate(inputs.problem("TND", B=2, seq_q=[5, 7], seq_kv=[9, 7], N1=2, topk=8), 11)
    b = inputs.generate(inputs.problem("TND", B=2, seq_q=[5, 7], seq_kv=[9, 7], N1=2, topk=8), 11)
    c = inputs.generate(inputs.problem("TND", B=2, seq_q=[5, 7], seq_kv=[9, 7], N1=2, topk=8), 12)
    for name in ("q", "k", "qr", "kr", "dout", "idx"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.q, c.q)
    assert np.array_equal(a.k, a.v) and a.k is not a.v
    assert a.q.shape == (12, 2, 512) and a.k.shape == (16, 1, 512) and a.idx.shape == (12, 1, 8)


def test_fp16_rounding_is_nearest_even_and_generation_matches_bf16_draws():
    x = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -2.5, 6.0e-8, 70000.0], np.float32)
    back = inputs.f16_bits_to_f64(inputs.f32_to_f16_bits(x))
    assert back[1] == 1.0                           # tie between 1 and 1 + 2^-10 goes to even
    assert back[2] == 1.0 + 2 ** -9                 # tie between 1 + 2^-10 and 1 + 2^-9: even is 2^-9
    assert back[3] == -2.5 and back[4] == 2.0 ** -24 and np.isinf(back[5])
    # the same seed draws the same fp32 normals for both element types: only the rounding differs
    pb = inputs.problem("BSND", B=1, S1=8, S2=32, N1=4, topk=8)
    ph = inputs.problem("BSND", B=1, S1=8, S2=32, N1=4, topk=8, dtype="fp16")
    inputs.generate(pb, 11)
    inputs.generate(ph, 11)
    a, b = inputs.bits_to_f64(pb.q, "bf16"), inputs.bits_to_f64(ph.q, "fp16")
    assert np.all(np.abs(a - b) <= 2 ** -8 * np.abs(b) + 1e-7)
    assert not np.array_equal(a, b)
    assert (pb.idx == ph.idx).all()
    with pytest.raises(ValueError):
        inputs.problem("BSND", dtype="fp32")
