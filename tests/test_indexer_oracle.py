"""Pins of the lightning-indexer oracle (oracle/indexer.py) to things other than itself.

- torch fp64 autograd of the loss written from the definitions (KL of the head-summed main
  attention softmax against log_softmax of W . ReLU(q~ K~^T)), with every softmax and statistic
  computed by torch, not by the oracle: pins the loss and all three gradients, the target
  distribution, the masks and the layouts (DenseLightningIndexerGradKLLoss README, "function
  description");
- central finite differences of the oracle's own loss (fed exact statistics) against its
  gradients;
- closed forms: W = 0 (uniform Softmax(I)), one admitted key (loss and gradients zero);
- the forward statistics the tests feed in (main and index) against torch's;
- invariants: KL >= 0 on every case;
- planted mistakes in a copy of the oracle's source, each caught by one of the pins above.
"""

import math
import os
import types

import numpy as np
import pytest

from oracle import indexer as ix


def make(layout="BSND", B=1, S1=9, S2=12, N1=4, G=3, Di=8, seq_q=None, seq_kv=None, mode=3, seed=0,
         D=16, Dr=4):
    rng = np.random.default_rng(seed)
    geo = ix.IndexerGeometry(layout, B, S1, S2, N1, G, Di=Di, D=D, Dr=Dr, seq_q=seq_q, seq_kv=seq_kv,
                             sparse_mode=mode, scale=1.0 / math.sqrt(D + Dr))
    if layout == "TND":
        geo.S1, geo.S2 = sum(seq_q), sum(seq_kv)
    t = dict(q=rng.standard_normal((geo.rows, N1, D)), qr=rng.standard_normal((geo.rows, N1, Dr)),
             k=rng.standard_normal((geo.keys, 1, D)), kr=rng.standard_normal((geo.keys, 1, Dr)),
             qi=rng.standard_normal((geo.rows, G, Di)), ki=rng.standard_normal((geo.keys, 1, Di)),
             w=rng.standard_normal((geo.rows, G)))
    return geo, t


def torch_reference(geo, t):
    """Loss and gradients by torch fp64 autograd, statistics by torch (independent of the oracle)."""
    import torch
    qi = torch.tensor(t["qi"], requires_grad=True)
    ki = torch.tensor(t["ki"], requires_grad=True)
    w = torch.tensor(t["w"], requires_grad=True)
    q, qr = torch.tensor(t["q"]), torch.tensor(t["qr"])
    k, kr = torch.tensor(t["k"])[:, 0], torch.tensor(t["kr"])[:, 0]
    smax = np.zeros(geo.B * geo.N1 * geo.S1)
    ssum = np.zeros_like(smax)
    loss = torch.zeros((), dtype=torch.float64)
    for row in range(geo.rows):
        b, i = geo.token(row)
        hi = geo.hi(b, i)
        if hi < 0:
            continue
        k0 = geo.k0(b)
        z = geo.scale * (q[row] @ k[k0:k0 + hi + 1].T + qr[row] @ kr[k0:k0 + hi + 1].T)   # [N1, n]
        for h in range(geo.N1):
            j = geo.stat_index(b, i, h)
            smax[j] = float(z[h].max())
            ssum[j] = float(torch.exp(z[h] - z[h].max()).sum())
        p = torch.softmax(z, dim=1).sum(0)
        p = p / p.sum()
        S = qi[row] @ ki[k0:k0 + hi + 1, 0].T                       # [G, n]
        I = w[row] @ torch.relu(S)
        logq = torch.log_softmax(I, dim=0)
        loss = loss + torch.sum(torch.where(p > 0, p * (torch.log(p) - logq), torch.zeros_like(p)))
    loss.backward()
    stats_i = ix.index_stats(geo, t["qi"], t["ki"], t["w"])
    return dict(loss=float(loss.detach()), dqi=qi.grad.numpy(), dki=ki.grad.numpy()[:, 0], dw=w.grad.numpy(),
                smax=smax, ssum=ssum, stats_i=stats_i)


def torch_index_stats(geo, t):
    """The index statistics by torch (max and sum of exp(I - max)), for the independence check."""
    import torch
    m, s = np.zeros(geo.rows), np.zeros(geo.rows)
    for row in range(geo.rows):
        b, i = geo.token(row)
        hi = geo.hi(b, i)
        if hi < 0:
            continue
        k0 = geo.k0(b)
        S = torch.tensor(t["qi"][row]) @ torch.tensor(t["ki"][k0:k0 + hi + 1, 0]).T
        I = torch.tensor(t["w"][row]) @ torch.relu(S)
        m[row] = float(I.max())
        s[row] = float(torch.exp(I - I.max()).sum())
    return m, s


def run_oracle(geo, t, ref, mod=ix):
    mi, si = torch_index_stats(geo, t)
    return mod.indexer_grad(geo, t["q"], t["k"], t["qr"], t["kr"], ref["smax"], ref["ssum"], t["qi"], t["ki"],
                            t["w"], mi, si)


CASES = {
    "bsnd_causal": dict(),
    "bsnd_nomask_b2": dict(B=2, S1=6, S2=10, mode=0, seed=1),
    "bsnd_s1_gt_s2": dict(S1=12, S2=7, seed=2),
    "tnd_varlen_empty": dict(layout="TND", B=3, seq_q=[5, 0, 7], seq_kv=[8, 3, 7], seed=3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_matches_torch_autograd(name):
    geo, t = make(**CASES[name])
    ref = torch_reference(geo, t)
    loss, _, dqi, dki, dw = run_oracle(geo, t, ref)
    assert abs(loss - ref["loss"]) <= 1e-10 * max(1.0, abs(ref["loss"]))
    np.testing.assert_allclose(dqi, ref["dqi"], atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(dki, ref["dki"], atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(dw, ref["dw"], atol=1e-11, rtol=1e-9)
    assert loss > 0


def test_main_stats_match_torch():
    for name in ("bsnd_nomask_b2", "tnd_varlen_empty"):
        geo, t = make(**CASES[name])
        ref = torch_reference(geo, t)
        m, l = ix.main_stats(geo, t["q"], t["k"], t["qr"], t["kr"])
        n = len(m)
        np.testing.assert_allclose(m, ref["smax"][:n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l, ref["ssum"][:n], rtol=1e-12, atol=1e-12)


def test_index_stats_match_torch():
    geo, t = make(**CASES["tnd_varlen_empty"])
    m, s = ix.index_stats(geo, t["qi"], t["ki"], t["w"])
    mt, st = torch_index_stats(geo, t)
    np.testing.assert_allclose(m, mt, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, st, rtol=1e-12, atol=1e-12)


def test_finite_differences_of_the_loss():
    geo, t = make(S1=5, S2=7, N1=2, G=2, Di=4, seed=7)
    ref = torch_reference(geo, t)
    loss0, _, dqi, dki, dw = run_oracle(geo, t, ref)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, grad in (("qi", dqi), ("ki", dki[:, None, :]), ("w", dw)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in t[name].shape)
            vals = []
            for sgn in (1, -1):
                t2 = {kk: v.copy() for kk, v in t.items()}
                t2[name][idx] += sgn * eps
                mi, si = torch_index_stats(geo, t2)          # statistics follow the perturbed scores
                vals.append(ix.indexer_grad(geo, t2["q"], t2["k"], t2["qr"], t2["kr"], ref["smax"], ref["ssum"],
                                            t2["qi"], t2["ki"], t2["w"], mi, si)[0])
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_zero_weights_give_the_uniform_closed_form():
    geo, t = make(seed=11)
    t["w"][:] = 0.0
    ref = torch_reference(geo, t)
    loss, rows, dqi, dki, dw = run_oracle(geo, t, ref)
    assert np.all(dqi == 0) and np.all(dki == 0)
    for row in range(geo.rows):
        b, i = geo.token(row)
        n = geo.hi(b, i) + 1
        if n <= 0:
            continue
        p = ix.target(geo, t["q"], t["k"], t["qr"], t["kr"], ref["smax"], ref["ssum"], row)
        S, _ = ix.index_scores(geo, t["qi"], t["ki"], t["w"], row)
        assert abs(rows[row] - float(np.sum(p * np.log(p * n)))) <= 1e-12
        np.testing.assert_allclose(dw[row], np.maximum(S, 0) @ (1.0 / n - p), atol=1e-13)


def test_single_admitted_key_gives_zero_loss_and_gradients():
    geo, t = make(S1=4, S2=4, seed=5)            # causal: row 0 admits key 0 only
    ref = torch_reference(geo, t)
    _, rows, dqi, dki, dw = run_oracle(geo, t, ref)
    assert rows[0] == 0.0 and np.all(dqi[0] == 0) and np.all(dw[0] == 0)


def test_target_is_the_head_average_of_the_main_softmax():
    import torch
    geo, t = make(N1=5, seed=4)
    ref = torch_reference(geo, t)
    for row in range(geo.rows):
        b, i = geo.token(row)
        hi = geo.hi(b, i)
        p = ix.target(geo, t["q"], t["k"], t["qr"], t["kr"], ref["smax"], ref["ssum"], row)
        z = geo.scale * (torch.tensor(t["q"][row]) @ torch.tensor(t["k"][:hi + 1, 0]).T
                         + torch.tensor(t["qr"][row]) @ torch.tensor(t["kr"][:hi + 1, 0]).T)
        np.testing.assert_allclose(p, torch.softmax(z, 1).mean(0).numpy(), rtol=1e-12, atol=1e-15)
        assert abs(p.sum() - 1.0) < 1e-12


# planted mistakes: each must be caught by the autograd pin on one of the cases
MUTATIONS = [
    ("dS mask dropped", "dS = (S > 0) * wf[row][:, None] * dI[None, :]", "dS = wf[row][:, None] * dI[None, :]"),
    ("dW without ReLU", "relu = np.maximum(S, 0.0)", "relu = S"),
    ("sign of dI", "dI = sm - p", "dI = p - sm"),
    ("target not normalised", "return tot / norm if norm > 0 else tot", "return tot"),
    ("causal offset", "return min(i + lkv - lq, lkv - 1)", "return min(i, lkv - 1)"),
    ("statistics layout", "return (b * self.N1 + h) * self.S1 + i", "return (i * self.N1 + h) + b * self.N1 * self.S1"),
    ("rope term dropped", "z = qh @ ks.T + qrh @ krs.T", "z = qh @ ks.T"),
    ("scale dropped", "tot += np.exp(geo.scale * z[h] - sm[j]) / ss[j]", "tot += np.exp(z[h] - sm[j]) / ss[j]"),
    ("dK~ from the wrong row", "dki[geo.k0(b): geo.k0(b) + n] += dS.T @ qif[row]",
     "dki[geo.k0(b): geo.k0(b) + n] += dS.T @ qif[max(row - 1, 0)]"),
]


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(label, old, new):
    src = open(os.path.join(os.path.dirname(ix.__file__), "indexer.py")).read()
    assert src.count(old) == 1, label
    mod = types.ModuleType("indexer_mutant")
    exec(compile(src.replace(old, new), "indexer_mutant.py", "exec"), mod.__dict__)
    caught = False
    for name in sorted(CASES):
        geo, t = make(**CASES[name])
        geo = mod.IndexerGeometry(geo.layout, geo.B, geo.S1, geo.S2, geo.N1, geo.G, geo.Di, geo.D, geo.Dr,
                                  geo.seq_q, geo.seq_kv, geo.sparse_mode, geo.scale)
        ref = torch_reference(ix.IndexerGeometry(geo.layout, geo.B, geo.S1, geo.S2, geo.N1, geo.G, geo.Di,
                                                 geo.D, geo.Dr, geo.seq_q, geo.seq_kv, geo.sparse_mode,
                                                 geo.scale), t)
        loss, _, dqi, dki, dw = run_oracle(geo, t, ref, mod)
        ok = (abs(loss - ref["loss"]) <= 1e-10 * max(1.0, abs(ref["loss"])) and np.allclose(dqi, ref["dqi"], atol=1e-11)
              and np.allclose(dki, ref["dki"], atol=1e-11) and np.allclose(dw, ref["dw"], atol=1e-11))
        if not ok:
            caught = True
            break
    assert caught, f"planted mistake not caught: {label}"
