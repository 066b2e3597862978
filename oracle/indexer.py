"""fp64 CPU oracle for the lightning-indexer backward with KL loss -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the benchmark's CPU-baseline leg may import this module.  The HIP
library never calls it and shares no code with it.

It follows the DenseLightningIndexerGradKLLoss README ("function description"), step by step,
per query token t over the keys s its mask admits (K_{:t}: keys 0 .. hi(t)):

  1. index scores   S[g, s] = q~[t, g] . K~[s]                (G index heads, one key head)
                    I[s]    = sum_g W[t, g] ReLU(S[g, s])
  2. target         p[s]    = L1-normalised sum over the N1 main heads of the main attention's
                              softmax P_h[s] = exp(scale z_h[s] - softmaxMax_h) / softmaxSum_h,
                              z_h[s] = q_h . k_s + qRope_h . kRope_s  (the SparseFlashAttention
                              logits, rebuilt from the forward's statistics)
  3. loss           KL(p || Softmax(I)) = sum_s p[s] log(p[s] / Softmax(I)[s]),  summed over t;
                    Softmax(I)[s] = exp(I[s] - softmaxMaxIndex) / softmaxSumIndex
  4. gradients      dI = Softmax(I) - p
                    dW[t, g]  = sum_s dI[s] ReLU(S[g, s])
                    dS[g, s]  = dI[s] W[t, g] [S[g, s] > 0]
                    dq~[t, g] = sum_s dS[g, s] K~[s]
                    dK~[s]   += sum_g dS[g, s] q~[t, g]

Readings of what the page leaves open (also listed in the design doc):
  - shapes follow the sparse attention operator's layouts: BSND query side [B, S1, N, W], key
    side [B, S2, 1, W]; TND [T, N, W]; queryIndex [.., G, Di], keyIndex [.., 1, Di], weights
    [.., G]; main statistics [B, N1, S1] / [N1, T1]; index statistics [B, S1] / [T1];
  - the mask is the sparse operator's: sparseMode 3 admits keys s <= t + Lkv - Lq, mode 0 all;
  - "/sqrt(d)" in the main softmax is the scaleValue attribute; the index scores have no scale;
  - the L1 normalisation of the head sum divides by the sum over the admitted keys (N1 when the
    statistics are exact); a token with no admitted key contributes nothing;
  - terms with p[s] = 0 contribute 0 to the loss; the loss is the sum over all query tokens.

Library primitives used as steps: numpy matmul and exp / log on whole vectors.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


class IndexerGeometry:
    """Shapes and masking of one call (the sparse operator's layouts)."""

    def __init__(self, layout: str, B: int, S1: int, S2: int, N1: int, G: int, Di: int = 128, D: int = 512,
                 Dr: int = 64, seq_q: Optional[Sequence[int]] = None, seq_kv: Optional[Sequence[int]] = None,
                 sparse_mode: int = 3, scale: float = 1.0 / 24.0):
        self.layout, self.B, self.S1, self.S2 = layout, B, S1, S2
        self.N1, self.G, self.Di, self.D, self.Dr = N1, G, Di, D, Dr
        self.seq_q = None if seq_q is None else [int(x) for x in seq_q]
        self.seq_kv = None if seq_kv is None else [int(x) for x in seq_kv]
        self.sparse_mode, self.scale = sparse_mode, float(scale)

    @property
    def rows(self) -> int:
        return self.B * self.S1 if self.layout == "BSND" else self.S1

    @property
    def keys(self) -> int:
        return self.B * self.S2 if self.layout == "BSND" else self.S2

    def lq(self, b):
        return self.S1 if self.seq_q is None else self.seq_q[b]

    def lkv(self, b):
        return self.S2 if self.seq_kv is None else self.seq_kv[b]

    def q0(self, b):
        return b * self.S1 if self.layout == "BSND" else sum(self.seq_q[:b])

    def k0(self, b):
        return b * self.S2 if self.layout == "BSND" else sum(self.seq_kv[:b])

    def token(self, row: int):
        """(batch, position) of a global query row; position >= lq(b) is padding."""
        if self.layout == "BSND":
            return row // self.S1, row % self.S1
        b = 0
        while row >= self.q0(b) + self.lq(b):
            b += 1
        return b, row - self.q0(b)

    def hi(self, b: int, i: int) -> int:
        """Last admitted key position of query position i of batch b (-1: none)."""
        lq, lkv = self.lq(b), self.lkv(b)
        if i >= lq:
            return -1
        if self.sparse_mode == 3:
            return min(i + lkv - lq, lkv - 1)
        return lkv - 1

    def stat_index(self, b: int, i: int, h: int) -> int:
        """Flat index of head h's main statistic of token (b, i): [B, N1, S1] / [N1, T1]."""
        if self.layout == "BSND":
            return (b * self.N1 + h) * self.S1 + i
        return h * self.S1 + self.q0(b) + i


def _flat(x, n, w):
    return np.asarray(x, dtype=np.float64).reshape(n, -1, w)


def index_scores(geo: IndexerGeometry, qi, ki, w, row: int):
    """Step 1 for one query row: S [G, keys], I [keys] over the admitted keys (None: no key)."""
    b, i = geo.token(row)
    hi = geo.hi(b, i)
    if hi < 0:
        return None, None
    qi = _flat(qi, geo.rows, geo.Di)[row]                      # [G, Di]
    ks = _flat(ki, geo.keys, geo.Di)[geo.k0(b): geo.k0(b) + hi + 1, 0]   # [n, Di]
    S = qi @ ks.T                                              # [G, n]
    I = np.asarray(w, dtype=np.float64).reshape(geo.rows, geo.G)[row] @ np.maximum(S, 0.0)
    return S, I


def index_stats(geo: IndexerGeometry, qi, ki, w):
    """Max and sum of exp(I - max) per query row (the indexer forward's statistics; input
    preparation for the tests).  Rows without keys get max 0, sum 0."""
    m = np.zeros(geo.rows)
    s = np.zeros(geo.rows)
    for row in range(geo.rows):
        _, I = index_scores(geo, qi, ki, w, row)
        if I is None:
            continue
        m[row] = I.max()
        s[row] = np.exp(I - m[row]).sum()
    return m, s


def main_stats(geo: IndexerGeometry, q, k, qr, kr):
    """The main attention's forward statistics over every admitted key (input preparation for the
    tests): per (token, head) the max of the scaled logits and the sum of exp(logit - max), laid
    out [B, N1, S1] / [N1, T1]; tokens without keys get max 0, sum 0."""
    sm = np.zeros(geo.B * geo.N1 * geo.S1 if geo.layout == "BSND" else geo.N1 * geo.S1)
    ss = np.zeros_like(sm)
    qf, qrf = _flat(q, geo.rows, geo.D), _flat(qr, geo.rows, geo.Dr)
    kf, krf = _flat(k, geo.keys, geo.D)[:, 0], _flat(kr, geo.keys, geo.Dr)[:, 0]
    for row in range(geo.rows):
        b, i = geo.token(row)
        hi = geo.hi(b, i)
        if hi < 0:
            continue
        k0 = geo.k0(b)
        z = geo.scale * (qf[row] @ kf[k0:k0 + hi + 1].T + qrf[row] @ krf[k0:k0 + hi + 1].T)
        for h in range(geo.N1):
            j = geo.stat_index(b, i, h)
            sm[j] = z[h].max()
            ss[j] = np.exp(z[h] - sm[j]).sum()
    return sm, ss


def target(geo: IndexerGeometry, q, k, qr, kr, smax, ssum, row: int):
    """Step 2 for one query row: the L1-normalised head sum of the main attention's softmax."""
    b, i = geo.token(row)
    hi = geo.hi(b, i)
    if hi < 0:
        return None
    qh = _flat(q, geo.rows, geo.D)[row]                        # [N1, D]
    qrh = _flat(qr, geo.rows, geo.Dr)[row]
    ks = _flat(k, geo.keys, geo.D)[geo.k0(b): geo.k0(b) + hi + 1, 0]
    krs = _flat(kr, geo.keys, geo.Dr)[geo.k0(b): geo.k0(b) + hi + 1, 0]
    z = qh @ ks.T + qrh @ krs.T                                # [N1, n]
    sm = np.asarray(smax, dtype=np.float64).reshape(-1)
    ss = np.asarray(ssum, dtype=np.float64).reshape(-1)
    tot = np.zeros(z.shape[1])
    for h in range(geo.N1):
        j = geo.stat_index(b, i, h)
        if ss[j] > 0:
            tot += np.exp(geo.scale * z[h] - sm[j]) / ss[j]
    norm = tot.sum()
    return tot / norm if norm > 0 else tot


def indexer_grad(geo: IndexerGeometry, q, k, qr, kr, smax, ssum, qi, ki, w, smax_i, ssum_i,
                 rows: Optional[Sequence[int]] = None):
    """Steps 1-4.  Returns (loss, loss per row, dqi [rows, G, Di], dki [keys, Di], dw [rows, G]).

    `rows` restricts the sum to those query rows (dqi / dw of other rows stay zero and dki holds
    only their contributions)."""
    G, Di = geo.G, geo.Di
    dqi = np.zeros((geo.rows, G, Di))
    dki = np.zeros((geo.keys, Di))
    dw = np.zeros((geo.rows, G))
    loss_rows = np.zeros(geo.rows)
    qif = _flat(qi, geo.rows, Di)
    kif = _flat(ki, geo.keys, Di)[:, 0]
    wf = np.asarray(w, dtype=np.float64).reshape(geo.rows, G)
    mi = np.asarray(smax_i, dtype=np.float64).reshape(-1)
    si = np.asarray(ssum_i, dtype=np.float64).reshape(-1)
    for row in (range(geo.rows) if rows is None else rows):
        S, I = index_scores(geo, qi, ki, w, row)
        if S is None or si[row] <= 0:
            continue
        p = target(geo, q, k, qr, kr, smax, ssum, row)
        b, _ = geo.token(row)
        n = S.shape[1]
        sm = np.exp(I - mi[row]) / si[row]                      # Softmax(I)
        pos = p > 0
        loss_rows[row] = float(np.sum(p[pos] * (np.log(p[pos]) - np.log(sm[pos]))))
        dI = sm - p
        relu = np.maximum(S, 0.0)
        dw[row] = relu @ dI
        dS = (S > 0) * wf[row][:, None] * dI[None, :]             # [G, n]
        ks = kif[geo.k0(b): geo.k0(b) + n]
        dqi[row] = dS @ ks
        dki[geo.k0(b): geo.k0(b) + n] += dS.T @ qif[row]
    return float(loss_rows.sum()), loss_rows, dqi, dki, dw
