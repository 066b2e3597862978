"""Pins of the fp64 oracle against things other than itself.

Each test ties one part of what the SparseFlashAttentionGrad README ("function
description" section) defines to an independent fact:
  - central finite differences of the loss sum(dO * out) (all five gradients,
    gather semantics with duplicates, skipped slots);
  - torch fp64 autograd of dense masked attention when topk covers every valid
    key (the dense FlashAttention backward of the FA-grad page, "function
    description": dV = P^T dY, dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d)),
    which also pins the logits (rope part included), the bottom-right causal
    geometry, varlen offsets and the softmaxMax / softmaxSum layout;
  - closed forms: all-ones inputs, a single valid slot, two valid slots,
    identical key rows (sum of dS over a row is zero);
  - invariants: column sums of dK / dKRope / dV, slot-permutation and padding
    invariance, invalid indices behaving as -1;
  - block selection (sparseBlockSize > 1): every block selected equals dense
    attention, finite differences with repeated / cut / invalid blocks, and a
    brute-force single-row forward.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import Geometry


def rnd_inputs(g: Geometry, seed: int):
    r = np.random.default_rng(seed)
    q = r.standard_normal((g.rows, g.N1, g.D))
    qr = r.standard_normal((g.rows, g.N1, g.Dr))
    k = r.standard_normal((g.keys, g.D))
    kr = r.standard_normal((g.keys, g.Dr))
    v = r.standard_normal((g.keys, g.D))
    dout = r.standard_normal((g.rows, g.N1, g.D))
    return q, k, v, qr, kr, dout


def row_info(g: Geometry):
    """(batch, position, Lq, Lkv, key offset) for every global query row."""
    out = []
    for b in range(g.B):
        lq = g.S1 if g.seq_q is None else int(g.seq_q[b])
        lkv = g.S2 if g.seq_kv is None else int(g.seq_kv[b])
        if g.layout == "BSND":
            qoff, koff, nrow = b * g.S1, b * g.S2, g.S1
        else:
            qoff, koff, nrow = int(g.seq_q[:b].sum()), int(g.seq_kv[:b].sum()), lq
        for i in range(nrow):
            out.append((b, i, lq, lkv, koff))
    return out


def causal_hi(g, i, lq, lkv):
    return min(i + lkv - lq, lkv - 1) if g.sparse_mode == 3 else lkv - 1


def dense_indices(g: Geometry, rng=None, pad=-1):
    """Every valid key of each row (then padding), optionally shuffled."""
    idx = np.full((g.rows, g.topk), pad, dtype=np.int32)
    for t, (b, i, lq, lkv, koff) in enumerate(row_info(g)):
        if i >= lq:
            continue
        hi = causal_hi(g, i, lq, lkv)
        keys = np.arange(0, hi + 1)
        if rng is not None:
            keys = rng.permutation(keys)
        assert len(keys) <= g.topk
        idx[t, : len(keys)] = keys
    return idx


def messy_indices(g: Geometry, seed: int):
    """Random indices with duplicates, -1, out-of-range and causally masked entries."""
    r = np.random.default_rng(seed)
    idx = r.integers(-2, g.S2 + 3 if g.layout == "BSND" else max(g.seq_kv) + 3, size=(g.rows, g.topk))
    return idx.astype(np.int32)


def loss(g, q, k, v, qr, kr, idx, dout):
    out, _, _ = oracle.forward(g, q, k, v, qr, kr, idx)
    return float((out * dout).sum())


# ---------------------------------------------------------------------------
# finite differences
# ---------------------------------------------------------------------------

FD_CASES = [
    dict(layout="BSND", B=2, S1=4, S2=6, N1=2, D=5, Dr=3, topk=5, sparse_mode=3, seq_q=None, seq_kv=None),
    dict(layout="BSND", B=1, S1=5, S2=4, N1=3, D=4, Dr=2, topk=6, sparse_mode=0, seq_q=None, seq_kv=None),
    dict(layout="BSND", B=2, S1=4, S2=5, N1=2, D=4, Dr=2, topk=4, sparse_mode=3, seq_q=[3, 4], seq_kv=[5, 2]),
    dict(layout="TND", B=2, S1=0, S2=0, N1=2, D=4, Dr=3, topk=5, sparse_mode=3, seq_q=[3, 2], seq_kv=[4, 3]),
]


def geo(c, scale=0.37):
    c = dict(c)
    if c["layout"] == "TND":
        c["S1"], c["S2"] = sum(c["seq_q"]), sum(c["seq_kv"])
    return Geometry(c["layout"], c["B"], c["S1"], c["S2"], c["N1"], c["D"], c["Dr"], c["topk"],
                    c["sparse_mode"], c["seq_q"], c["seq_kv"], scale)


@pytest.mark.parametrize("case", range(len(FD_CASES)))
def test_finite_differences_all_gradients(case):
    g = geo(FD_CASES[case])
    q, k, v, qr, kr, dout = rnd_inputs(g, 10 + case)
    idx = messy_indices(g, 20 + case)
    # force a duplicated valid key in the first active row so gather semantics are exercised
    idx[0, :2] = 0
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    h = 1e-6
    args = dict(q=q, k=k, v=v, qr=qr, kr=kr)
    grads = dict(q=dq.reshape(q.shape), k=dk, v=dv, qr=dqr.reshape(qr.shape), kr=dkr)
    for name, base in args.items():
        fd = np.zeros_like(base)
        flat = base.reshape(-1)
        for e in range(flat.size):
            old = flat[e]
            flat[e] = old + h
            lp = loss(g, args["q"], args["k"], args["v"], args["qr"], args["kr"], idx, dout)
            flat[e] = old - h
            lm = loss(g, args["q"], args["k"], args["v"], args["qr"], args["kr"], idx, dout)
            flat[e] = old
            fd.reshape(-1)[e] = (lp - lm) / (2 * h)
        err = np.abs(fd - grads[name]).max()
        assert err < 1e-6 * max(1.0, np.abs(fd).max()), (name, err)


def test_finite_differences_full_width():
    """Same check once at the operator's real widths D=512, Dr=64 (sampled elements)."""
    g = Geometry("BSND", 1, 3, 5, 2, 512, 64, 4, 3, None, None, 1 / 24)
    q, k, v, qr, kr, dout = rnd_inputs(g, 3)
    idx = np.array([[0, 2, -1, 4], [1, 0, 3, 2], [4, 2, 0, 1]], dtype=np.int32)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    r = np.random.default_rng(0)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("qr", qr, dqr), ("kr", kr, dkr)):
        flat, gflat = arr.reshape(-1), grad.reshape(-1)
        for e in r.choice(flat.size, 12, replace=False):
            old = flat[e]
            flat[e] = old + h
            lp = loss(g, q, k, v, qr, kr, idx, dout)
            flat[e] = old - h
            lm = loss(g, q, k, v, qr, kr, idx, dout)
            flat[e] = old
            assert abs((lp - lm) / (2 * h) - gflat[e]) < 2e-6, (name, e)


# ---------------------------------------------------------------------------
# dense reduction against torch autograd
# ---------------------------------------------------------------------------

def torch_dense(g: Geometry, q, k, v, qr, kr, dout):
    """Dense masked attention per batch/head with torch fp64 autograd.

    Returns out, max, sum (stats in the documented head-major layout) and the
    five gradients, built without any oracle code."""
    T = torch.float64
    Q = torch.tensor(q, dtype=T, requires_grad=True)
    QR = torch.tensor(qr, dtype=T, requires_grad=True)
    K = torch.tensor(k, dtype=T, requires_grad=True)
    KR = torch.tensor(kr, dtype=T, requires_grad=True)
    V = torch.tensor(v, dtype=T, requires_grad=True)
    DO = torch.tensor(dout, dtype=T)
    outs = torch.zeros(g.rows, g.N1, g.D, dtype=T)
    smax = np.zeros(g.stat_shape())
    ssum = np.zeros(g.stat_shape())
    total = torch.zeros((), dtype=T)
    for b in range(g.B):
        lq = g.S1 if g.seq_q is None else int(g.seq_q[b])
        lkv = g.S2 if g.seq_kv is None else int(g.seq_kv[b])
        if g.layout == "BSND":
            qoff, koff = b * g.S1, b * g.S2
        else:
            qoff, koff = int(g.seq_q[:b].sum()), int(g.seq_kv[:b].sum())
        if lq == 0:
            continue
        Qb, QRb = Q[qoff:qoff + lq], QR[qoff:qoff + lq]            # [lq,N,D]
        Kb, KRb, Vb = K[koff:koff + lkv], KR[koff:koff + lkv], V[koff:koff + lkv]
        Z = g.scale * (torch.einsum("ihd,jd->hij", Qb, Kb) + torch.einsum("ihd,jd->hij", QRb, KRb))
        i = torch.arange(lq)[:, None]
        j = torch.arange(lkv)[None, :]
        mask = (j <= i + lkv - lq) if g.sparse_mode == 3 else torch.ones(lq, lkv, dtype=torch.bool)
        has = mask.any(dim=1)                                      # rows with a valid key
        Zm = Z.masked_fill(~mask, -math.inf)
        Zs = Zm[:, has]
        P = torch.softmax(Zs, dim=-1)
        O = torch.einsum("hij,jd->ihd", P, Vb)                     # [rows,N,D]
        rows_idx = torch.nonzero(has).flatten()
        total = total + (O * DO[qoff + rows_idx]).sum()
        with torch.no_grad():
            outs[qoff + rows_idx] = O
            mz = Zs.max(dim=-1).values                             # [N, rows]
            lz = torch.exp(Zs - mz[..., None]).sum(-1)
            for h in range(g.N1):
                for a, r_ in enumerate(rows_idx.tolist()):
                    if g.layout == "BSND":
                        smax[b, h, r_] = mz[h, a]
                        ssum[b, h, r_] = lz[h, a]
                    else:
                        smax[h, qoff + r_] = mz[h, a]
                        ssum[h, qoff + r_] = lz[h, a]
    total.backward()
    z = lambda t: np.zeros(t.shape) if t.grad is None else t.grad.numpy()
    return outs.detach().numpy(), smax, ssum, z(Q), z(K), z(V), z(QR), z(KR)


DENSE_CASES = [
    ("BSND", 2, 6, 9, 3, 3, None, None),     # causal, S1 < S2
    ("BSND", 1, 7, 7, 4, 0, None, None),     # no mask
    ("BSND", 1, 8, 5, 2, 3, None, None),     # causal, S1 > S2: early rows empty
    ("BSND", 2, 6, 8, 2, 3, [4, 6], [8, 3]), # padded batches
    ("TND", 3, 0, 0, 2, 3, [3, 5, 1], [6, 5, 4]),
    ("TND", 2, 0, 0, 3, 0, [4, 2], [3, 5]),
]


@pytest.mark.parametrize("case", range(len(DENSE_CASES)))
def test_dense_reduction_matches_torch_autograd(case):
    layout, B, S1, S2, N1, mode, sq, skv = DENSE_CASES[case]
    if layout == "TND":
        S1, S2 = sum(sq), sum(skv)
    topk = (S2 if layout == "BSND" else max(skv)) + 2
    g = Geometry(layout, B, S1, S2, N1, 512, 64, topk, mode, sq, skv, 1 / 24)
    q, k, v, qr, kr, dout = rnd_inputs(g, 100 + case)
    idx = dense_indices(g, np.random.default_rng(case))
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    t_out, t_m, t_l, t_dq, t_dk, t_dv, t_dqr, t_dkr = torch_dense(g, q, k, v, qr, kr, dout)
    np.testing.assert_allclose(out, t_out, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(m, t_m, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(l, t_l, atol=1e-12, rtol=1e-10)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    for a, b_ in ((dq, t_dq), (dk, t_dk), (dv, t_dv), (dqr, t_dqr), (dkr, t_dkr)):
        np.testing.assert_allclose(a, b_, atol=1e-11, rtol=1e-9)


# ---------------------------------------------------------------------------
# block selection (sparseBlockSize > 1)
# ---------------------------------------------------------------------------

BLOCK_DENSE_CASES = [
    ("BSND", 1, 6, 11, 2, 3, None, None, 4),     # causal; the last block is cut by the key length
    ("BSND", 2, 5, 8, 3, 0, None, [7, 5], 3),    # no mask; padded key lengths cut the last blocks
    ("BSND", 1, 9, 6, 2, 3, None, None, 5),      # causal, S1 > S2: early rows empty
    ("TND", 2, 0, 0, 2, 3, [4, 3], [9, 5], 2),   # varlen, causal
]


@pytest.mark.parametrize("case", range(len(BLOCK_DENSE_CASES)))
def test_every_block_selected_matches_dense_autograd(case):
    """Indices naming every block of the sequence once (shuffled, with a -1 among them) select
    every key once, so the result is dense masked attention (torch fp64 autograd).  Pins the
    block -> key expansion (block j covers keys j*bs .. j*bs + bs - 1), the per-key length and
    causal checks inside a block, and a -1 skipping only its own block."""
    layout, B, S1, S2, N1, mode, sq, skv, bs = BLOCK_DENSE_CASES[case]
    if layout == "TND":
        S1, S2 = sum(sq), sum(skv)
    maxkv = S2 if layout == "BSND" else max(skv)
    nblk = -(-maxkv // bs)
    g = Geometry(layout, B, S1, S2, N1, 16, 8, nblk + 2, mode, sq, skv, 0.3, block=bs)
    q, k, v, qr, kr, dout = rnd_inputs(g, 200 + case)
    r = np.random.default_rng(case)
    idx = np.full((g.rows, g.topk), -1, dtype=np.int32)
    for t, (b, i, lq, lkv, koff) in enumerate(row_info(g)):
        row = np.concatenate([np.arange(-(-lkv // bs)), [-1]])
        idx[t, :len(row)] = r.permutation(row)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    t_out, t_m, t_l, t_dq, t_dk, t_dv, t_dqr, t_dkr = torch_dense(g, q, k, v, qr, kr, dout)
    np.testing.assert_allclose(out, t_out, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(m, t_m, atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(l, t_l, atol=1e-12, rtol=1e-10)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    for a, b_ in ((dq, t_dq), (dk, t_dk), (dv, t_dv), (dqr, t_dqr), (dkr, t_dkr)):
        np.testing.assert_allclose(a, b_, atol=1e-11, rtol=1e-9)


def test_finite_differences_block_selection():
    """All five gradients of sum(dO * out) by central differences with block selection:
    repeated blocks (their keys count twice), a block cut by the key length, out-of-range and
    negative block indices."""
    g = Geometry("BSND", 2, 4, 7, 2, 5, 3, 3, 3, None, None, 0.37, block=3)
    q, k, v, qr, kr, dout = rnd_inputs(g, 31)
    idx = np.array([[0, 2, 0], [1, -1, 5], [2, 1, 1], [-3, 0, 2],
                    [0, 1, 2], [1, 1, -1], [2, 0, 9], [0, 2, 1]], dtype=np.int32)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    h = 1e-6
    args = dict(q=q, k=k, v=v, qr=qr, kr=kr)
    grads = dict(q=dq.reshape(q.shape), k=dk, v=dv, qr=dqr.reshape(qr.shape), kr=dkr)
    for name, base in args.items():
        fd = np.zeros_like(base)
        flat = base.reshape(-1)
        for e in range(flat.size):
            old = flat[e]
            flat[e] = old + h
            lp = loss(g, args["q"], args["k"], args["v"], args["qr"], args["kr"], idx, dout)
            flat[e] = old - h
            lm = loss(g, args["q"], args["k"], args["v"], args["qr"], args["kr"], idx, dout)
            flat[e] = old
            fd.reshape(-1)[e] = (lp - lm) / (2 * h)
        err = np.abs(fd - grads[name]).max()
        assert err < 1e-6 * max(1.0, np.abs(fd).max()), (name, err)


def test_block_selection_brute_force_single_row():
    """One query row, brute force in plain numpy: the keys of the selected blocks (cut at the
    key length and at the causal bound), softmax over them, out = P V."""
    g = Geometry("BSND", 1, 3, 10, 1, 4, 2, 2, 3, None, None, 0.5, block=4)
    q, k, v, qr, kr, dout = rnd_inputs(g, 41)
    idx = np.array([[2, 0], [1, 2], [0, -1]], dtype=np.int32)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    for t in range(3):
        pos = t + 10 - 3
        keys = [jb * 4 + r for jb in idx[t] if jb >= 0 for r in range(4) if jb * 4 + r < 10 and jb * 4 + r <= pos]
        z = np.array([0.5 * (q[t, 0] @ k[j] + qr[t, 0] @ kr[j]) for j in keys])
        p_ = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
        np.testing.assert_allclose(out[t, 0], p_ @ v[keys], atol=1e-12)
        assert abs(m[0, 0, t] - z.max()) < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_identical_key_rows_give_zero_dq():
    """sum over slots of dS is 0 per (row, head): with all key rows equal to one
    vector c, dQ = scale * (sum dS) * c must vanish although dK, dV do not."""
    g = Geometry("BSND", 1, 6, 10, 3, 16, 4, 7, 0, None, None, 0.3)
    q, k, v, qr, kr, dout = rnd_inputs(g, 5)
    k[:] = k[0]
    kr[:] = kr[0]
    idx = np.stack([np.random.default_rng(i).choice(10, 7, replace=False) for i in range(6)]).astype(np.int32)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    assert np.abs(dq).max() < 1e-12 and np.abs(dqr).max() < 1e-12
    assert np.abs(dk).max() > 1e-3 and np.abs(dv).max() > 1e-3


def test_single_valid_slot():
    """One valid slot: p = 1, dS = 0, so dQ = dK = 0 and dV[j] collects dO."""
    g = Geometry("BSND", 1, 5, 8, 3, 12, 4, 4, 3, None, None, 0.25)
    q, k, v, qr, kr, dout = rnd_inputs(g, 6)
    idx = np.full((5, 4), -1, np.int32)
    sel = [3, 0, 5, 3, 7]
    for t, j in enumerate(sel):
        idx[t, t % 4] = j
    idx[0, 3] = 7                   # causally masked for row 0 (pos 3): still one valid slot
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12 and np.abs(dkr).max() < 1e-12
    expect = np.zeros((8, 12))
    for t, j in enumerate(sel):
        expect[j] += dout[t].sum(axis=0)
    np.testing.assert_allclose(dv, expect, atol=1e-12)


def test_two_valid_slots_closed_form():
    """Two slots: dQ = scale * p1 p2 (dO.(v1 - v2)) (k1 - k2) per head."""
    g = Geometry("BSND", 1, 1, 2, 2, 8, 3, 2, 0, None, None, 0.4)
    q, k, v, qr, kr, dout = rnd_inputs(g, 7)
    idx = np.array([[0, 1]], np.int32)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    for h in range(2):
        z = [0.4 * (q[0, h] @ k[s] + qr[0, h] @ kr[s]) for s in range(2)]
        p1 = 1 / (1 + math.exp(z[1] - z[0]))
        p2 = 1 - p1
        ds1 = p1 * p2 * (dout[0, h] @ (v[0] - v[1]))
        np.testing.assert_allclose(dq[0, h], 0.4 * ds1 * (k[0] - k[1]), atol=1e-13)
        np.testing.assert_allclose(dqr[0, h], 0.4 * ds1 * (kr[0] - kr[1]), atol=1e-13)
    # dK rows are opposite: dK[0] + dK[1] = scale * (ds1 + ds2) q = 0
    np.testing.assert_allclose(dk[0] + dk[1], 0, atol=1e-13)


def test_all_ones_given_out_gives_exact_zero_gradients():
    """All-ones q, k, v, qRope, kRope, dO and out = 1 (bf16-exact): dP = D exactly,
    so dS, dQ, dK vanish bit-exactly and dV[j] = sum over selecting rows of N1/n."""
    g = Geometry("BSND", 1, 9, 12, 4, 512, 64, 6, 3, None, None, 1 / 24)
    ones_q = np.ones((9, 4, 512))
    idx = np.stack([np.random.default_rng(i).permutation(12)[:6] for i in range(9)]).astype(np.int32)
    out, m, l = oracle.forward(g, ones_q, np.ones((12, 512)), np.ones((12, 512)), np.ones((9, 4, 64)),
                               np.ones((12, 64)), idx)
    out_given = np.ones_like(out)
    dq, dk, dv, dqr, dkr = oracle.backward(g, ones_q, np.ones((12, 512)), np.ones((12, 512)),
                                           np.ones((9, 4, 64)), np.ones((12, 64)), idx, ones_q,
                                           out_given, m, l)
    assert not dq.any() and not dk.any() and not dqr.any() and not dkr.any()
    expect = np.zeros(12)
    for t in range(9):
        valid = [j for j in idx[t] if j <= t + 3]
        for j in valid:
            expect[j] += 4 * (1.0 / len(valid))
    np.testing.assert_allclose(dv, np.repeat(expect[:, None], 512, axis=1), rtol=1e-15)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_column_sums():
    """sum_j dK[j] = 0, sum_j dKRope[j] = 0 and sum_j dV[j] = sum of dO over rows with a valid key."""
    g = Geometry("TND", 3, 16, 23, 3, 32, 8, 9, 3, [5, 7, 4], [8, 6, 9], 0.2)
    q, k, v, qr, kr, dout = rnd_inputs(g, 8)
    idx = messy_indices(g, 9)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    np.testing.assert_allclose(dk.sum(0), 0, atol=1e-12)
    np.testing.assert_allclose(dkr.sum(0), 0, atol=1e-12)
    has = (l.T > 0)                                   # [rows, N1] rows/heads with a valid key
    np.testing.assert_allclose(dv.sum(0), (dout * has[..., None]).sum((0, 1)), atol=1e-12)


def test_slot_permutation_and_padding_invariance():
    g = Geometry("BSND", 2, 5, 9, 2, 24, 8, 8, 3, None, None, 0.3)
    q, k, v, qr, kr, dout = rnd_inputs(g, 11)
    idx = messy_indices(g, 12)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    ref = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    r = np.random.default_rng(1)
    perm = np.stack([r.permutation(8) for _ in range(10)])
    idx2 = np.take_along_axis(idx, perm, axis=1)
    out2, m2, l2 = oracle.forward(g, q, k, v, qr, kr, idx2)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    got = oracle.backward(g, q, k, v, qr, kr, idx2, dout, out, m, l)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_invalid_indices_act_as_skipped():
    """Negative, out-of-range and causally masked indices behave exactly like -1."""
    g = Geometry("BSND", 2, 5, 7, 2, 16, 8, 6, 3, [5, 3], [7, 6], 0.3)
    q, k, v, qr, kr, dout = rnd_inputs(g, 13)
    idx = messy_indices(g, 14)
    clean = idx.copy()
    for t, (b, i, lq, lkv, koff) in enumerate(row_info(g)):
        for s in range(g.topk):
            j = clean[t, s]
            if i >= lq or j < 0 or j >= lkv or j > i + lkv - lq:
                clean[t, s] = -1
    assert (clean != idx).any()
    a = oracle.forward(g, q, k, v, qr, kr, idx)
    b = oracle.forward(g, q, k, v, qr, kr, clean)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ga = oracle.backward(g, q, k, v, qr, kr, idx, dout, *a)
    gb = oracle.backward(g, q, k, v, qr, kr, clean, dout, *a)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)
    # padded query rows of batch 1 (rows 3, 4) have zero dQ and zero out
    assert not a[0][5 + 3:].any() and not ga[0][5 + 3:].any()


def test_sampled_backward_matches_full():
    """The row-list / key-list entry points equal slices of the full backward."""
    g = Geometry("BSND", 1, 12, 20, 2, 16, 8, 9, 3, None, None, 0.3)
    q, k, v, qr, kr, dout = rnd_inputs(g, 15)
    idx = messy_indices(g, 16)
    out, m, l = oracle.forward(g, q, k, v, qr, kr, idx)
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, k, v, qr, kr, idx, dout, out, m, l)
    rows = np.array([11, 0, 5])
    sdq, sdqr = oracle.backward_dq(g, q, k, v, qr, kr, idx, dout, out, m, l, rows=rows)
    np.testing.assert_array_equal(sdq, dq[rows])
    np.testing.assert_array_equal(sdqr, dqr[rows])
    keys = np.array([19, 3, 4])
    sdk, sdkr, sdv = oracle.backward_dkv(g, q, k, v, qr, kr, idx, dout, out, m, l, keys=keys)
    np.testing.assert_array_equal(sdk, dk[keys])
    np.testing.assert_array_equal(sdv, dv[keys])
    # a row range splits the key sums additively
    lo = oracle.backward_dkv(g, q, k, v, qr, kr, idx, dout, out, m, l, keys=keys, row_lo=0, row_hi=6)
    hi = oracle.backward_dkv(g, q, k, v, qr, kr, idx, dout, out, m, l, keys=keys, row_lo=6, row_hi=12)
    np.testing.assert_allclose(lo[0] + hi[0], sdk, atol=1e-13)
    # forward on a row list reproduces those rows
    o2, m2, l2 = oracle.forward(g, q, k, v, qr, kr, idx, rows=rows)
    np.testing.assert_array_equal(o2[rows], out[rows])
    np.testing.assert_array_equal(m2[0][:, rows], m[0][:, rows])


def test_page_sample_all_ones_with_given_statistics():
    """The dense FA-grad page's sample program (tests/golden/fa_grad_all_ones_sample.json):
    all-ones inputs with softmaxMax = softmaxSum = 3.0 given (not consistent with
    the inputs).  Every key selected, no mask.  p = exp(scale*D - 3)/3 for every
    slot, dP = FlashSoftmaxGrad = D exactly, so dQ = dK = 0 and
    dV[j] = T * N * p.  Pins the use of the given statistics in P."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fa_grad_all_ones_sample.json")))
    T, N, D = fx["T"], fx["N"], fx["D"]
    g = Geometry("TND", 1, T, T, N, D, 0, T, fx["sparse_mode"], fx["actual_seq_len_q"],
                 fx["actual_seq_len_kv"], fx["scale_value"])
    one = fx["fill_value"]
    q = np.full((T, N, D), one)
    kv = np.full((T, D), one)
    empty_q = np.zeros((T, N, 0))
    empty_k = np.zeros((T, 0))
    idx = np.tile(np.arange(T, dtype=np.int32), (T, 1))
    m = np.full((N, T), fx["softmax_max"])
    l = np.full((N, T), fx["softmax_sum"])
    dq, dk, dv, dqr, dkr = oracle.backward(g, q, kv, kv, empty_q, empty_k, idx, q, q, m, l)
    assert not dq.any() and not dk.any()
    p = math.exp(fx["scale_value"] * D - fx["softmax_max"]) / fx["softmax_sum"]
    np.testing.assert_allclose(dv, T * N * p, rtol=1e-13)
