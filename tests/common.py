"""Shared helpers of the GPU parity tests: seeded inputs, oracle references in
"op mode" (the 16-bit out and fp32 statistics the GPU receives), device
transfer and the tolerance check."""

from __future__ import annotations

import numpy as np

import oracle
from sparse_mla_flash_amd import inputs

# tolerance for bf16 outputs computed with fp32 accumulation (per output tensor)
MAX_ABS = 2e-2
REL_L2 = 5e-3


def f64(bits, dtype="bf16"):
    return inputs.bits_to_f64(bits, dtype)


# unit roundoff of the 16-bit element types (half an ulp at 1.0)
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}


def to_dev(bits, dtype="bf16"):
    """uint16 bits of `dtype` ("bf16" / "fp16") or any other array ("raw") to a GPU tensor."""
    import torch
    if dtype in ("bf16", "fp16"):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


class Case:
    """A generated problem plus its oracle forward (op-mode inputs for the backward)."""

    def __init__(self, p: inputs.Problem, fwd_rows=None, rope=True):
        self.p = p
        self.rope = rope                 # False: the call passes no rope inputs (no rope terms)
        self.g = oracle.Geometry.of(p)
        self.dtype = p.dtype
        dt = p.dtype
        self.q, self.k, self.qr, self.kr = f64(p.q, dt), f64(p.k, dt), f64(p.qr, dt), f64(p.kr, dt)
        if not rope:
            self.qr, self.kr = np.zeros_like(self.qr), np.zeros_like(self.kr)
        self.v = f64(p.v, dt)
        self.dout = f64(p.dout, dt)
        self.idx = p.idx
        out64, m64, l64 = oracle.forward(self.g, self.q, self.k, self.v, self.qr, self.kr, self.idx,
                                         rows=fwd_rows)
        self.out64, self.m64, self.l64 = out64, m64, l64
        # the operator's inputs: out in the element type, statistics in fp32
        self.out_bits = inputs.f32_to_bits(out64.astype(np.float32), dt).reshape(p.q_shape(p.D))
        self.m32 = m64.astype(np.float32)
        self.l32 = l64.astype(np.float32)
        self.out_op = f64(self.out_bits, dt)

    # oracle references in op mode
    def ref_dq(self, rows=None):
        return oracle.backward_dq(self.g, self.q, self.k, self.v, self.qr, self.kr, self.idx, self.dout,
                                  self.out_op, self.m32.astype(np.float64), self.l32.astype(np.float64),
                                  rows=rows)

    def ref_dkv(self, keys=None, row_lo=0, row_hi=None):
        return oracle.backward_dkv(self.g, self.q, self.k, self.v, self.qr, self.kr, self.idx, self.dout,
                                   self.out_op, self.m32.astype(np.float64), self.l32.astype(np.float64),
                                   keys=keys, row_lo=row_lo, row_hi=row_hi)

    def device_inputs(self):
        p, dt = self.p, self.dtype
        return dict(query=to_dev(p.q, dt), key=to_dev(p.k, dt), value=to_dev(p.v, dt),
                    sparse_indices=to_dev(p.idx, "raw"), d_out=to_dev(p.dout, dt), out=to_dev(self.out_bits, dt),
                    softmax_max=to_dev(self.m32, "raw"), softmax_sum=to_dev(self.l32, "raw"),
                    query_rope=to_dev(p.qr, dt) if self.rope else None,
                    key_rope=to_dev(p.kr, dt) if self.rope else None)

    def run_gpu(self, deterministic=False, dev=None):
        import sparse_mla_flash_amd as sf
        p = self.p
        d = dev or self.device_inputs()
        return sf.sparse_flash_attention_grad(
            d["query"], d["key"], d["value"], d["sparse_indices"], d["d_out"], d["out"], d["softmax_max"],
            d["softmax_sum"], p.seq_q, p.seq_kv, d["query_rope"], d["key_rope"], scale_value=p.scale,
            sparse_block_size=p.block, layout=p.layout, sparse_mode=p.sparse_mode,
            deterministic=deterministic)


def compare(name, got: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, rel_l2=REL_L2, scaled=True, u=2.0 ** -8):
    """Tolerance check of one output tensor.

    rel-L2 <= 5e-3 always.  The max-abs bar is 2e-2 per element.  With ``scaled`` (the small
    cases) element x of an output row r (a key row of dK / dKRope / dV, a (token, head) row of
    dQ / dQRope: the last axis) may be off by

        2e-2 + 2u |x| + u max_r |ref|,   u = 2^-8 for bf16 (2^-11 for fp16, passed by the caller).

    The second term is one ulp of the element (the output is rounded to the element type).  The
    third comes from the 16-bit MFMA operands: every product of the sum that forms x carries a
    relative rounding error of up to 2u (two operands rounded), so the error of x scales with
    the size of the terms summed, not with x after cancellation, and the largest entry of the
    same row is a lower bound of that size.  The small cases draw few slots per key, so a key
    selected by every row (and with p = 1 by the first one) has entries of 10-35 and cancelled
    neighbours whose error then exceeds 2e-2.  Full-size workload tests pass scaled=False
    (2e-2 flat)."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    diff = np.abs(got - ref)
    if scaled:
        rowmax = np.abs(ref).max(axis=-1, keepdims=True) if ref.ndim and ref.shape[-1] else np.zeros_like(ref)
        bound = max_abs + 2 * u * np.abs(ref) + u * rowmax
    else:
        bound = np.full(ref.shape, max_abs)
    ma = float(diff.max()) if diff.size else 0.0
    excess = float((diff - bound).max()) if diff.size else 0.0
    peak = float(np.abs(ref).max()) if ref.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got - ref))
    worst = int(np.argmax(diff - bound)) if diff.size else 0
    msg = (f"{name}: max abs {ma:.3e}, worst element {worst} off by {diff.reshape(-1)[worst] if diff.size else 0:.3e} "
           f"against a bound of {bound.reshape(-1)[worst] if diff.size else 0:.3e} (max|ref| {peak:.3f}), "
           f"rel-L2 {rel:.3e} (bound {rel_l2})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert excess <= 0.0 and rel <= rel_l2, msg
    print(f"# compare {name}: max abs {ma:.3e}, rel-L2 {rel:.3e}, max|ref| {peak:.3f}")
    return ma, rel


class TailCase:
    """A full-size problem whose only live query rows are the last ``tail[b]`` rows of each batch /
    sequence b, with an oracle that sees just those rows.

    The oracle runs on a compact sub-problem: the same key side, and per sequence a query length
    of tail[b] holding the live rows.  Row i of a sequence of query length Lq keeps its causal
    bound, because i + Lkv - Lq = i' + Lkv - tail[b] for its sub-problem position i' = i - (Lq -
    tail[b]).  The GPU runs the full problem: every other row gets out = 0 and softmaxSum = 0, so
    by the operator's definition (p = 0 when softmaxSum <= 0) it contributes nothing.  No full-size
    fp64 copy of the query-side tensors is ever made."""

    def __init__(self, p: inputs.Problem, tail):
        self.p = p
        self.tail = [int(t) for t in tail]
        assert len(self.tail) == p.B and all(0 <= t <= p.lq(b) for b, t in enumerate(self.tail))
        rows = []
        for b in range(p.B):
            r0 = p.q_offset(b) + p.lq(b) - self.tail[b]
            rows.append(np.arange(r0, r0 + self.tail[b]))
        self.live = np.concatenate(rows) if rows else np.zeros(0, np.int64)   # global rows, batch order
        s1 = max(self.tail)
        lay = p.layout
        if lay == "BSND":
            sub = inputs.problem("BSND", B=p.B, S1=s1, S2=p.S2, N1=p.N1, topk=p.topk,
                                 sparse_mode=p.sparse_mode, seq_q=self.tail,
                                 seq_kv=[p.lkv(b) for b in range(p.B)], scale=p.scale, block=p.block,
                                 dtype=p.dtype)
            # sub row of global live row: batch b, position tail-relative
            self.sub_row = np.concatenate([b * s1 + np.arange(self.tail[b]) for b in range(p.B)])
        else:
            sub = inputs.problem("TND", B=p.B, seq_q=self.tail, seq_kv=list(p.seq_kv), N1=p.N1, topk=p.topk,
                                 sparse_mode=p.sparse_mode, scale=p.scale, block=p.block, dtype=p.dtype)
            self.sub_row = np.arange(len(self.live))
        sub.scale = p.scale
        self.sub = sub
        self.g = oracle.Geometry.of(sub)
        qf = p.q.reshape(p.rows, p.N1, p.D)
        qrf = p.qr.reshape(p.rows, p.N1, p.Dr)
        dof = p.dout.reshape(p.rows, p.N1, p.D)
        idxf = p.idx.reshape(p.rows, -1)
        n = sub.rows
        self.q = np.zeros((n, p.N1, p.D))
        self.qr = np.zeros((n, p.N1, p.Dr))
        self.dout = np.zeros((n, p.N1, p.D))
        self.idx = np.full((n, idxf.shape[1]), -1, np.int32)
        dt = self.dtype = p.dtype
        self.q[self.sub_row] = f64(qf[self.live], dt)
        self.qr[self.sub_row] = f64(qrf[self.live], dt)
        self.dout[self.sub_row] = f64(dof[self.live], dt)
        self.idx[self.sub_row] = idxf[self.live]
        self.k, self.kr = f64(p.k, dt).reshape(p.keys, p.D), f64(p.kr, dt).reshape(p.keys, p.Dr)
        out64, m64, l64 = oracle.forward(self.g, self.q, self.k, self.k, self.qr, self.kr, self.idx)
        self.out_sub_bits = inputs.f32_to_bits(out64.astype(np.float32), dt)
        self.out_op = f64(self.out_sub_bits, dt)
        self.m32 = m64.astype(np.float32)
        self.l32 = l64.astype(np.float32)
        # full-size operator inputs: live rows from the sub-problem, zeros elsewhere
        out_full = np.zeros((p.rows, p.N1, p.D), np.uint16)
        out_full[self.live] = self.out_sub_bits.reshape(n, p.N1, p.D)[self.sub_row]
        self.out_bits = out_full.reshape(p.q_shape(p.D))
        m_full = np.zeros(p.stat_shape(), np.float32)
        l_full = np.zeros(p.stat_shape(), np.float32)
        self._scatter_stats(m_full, self.m32)
        self._scatter_stats(l_full, self.l32)
        self.m_full, self.l_full = m_full, l_full

    def _stat_pos(self, prob, rows):
        """(head-major) statistic indices of the given global rows of `prob`, per head."""
        if prob.layout == "TND":
            return lambda h: h * prob.S1 + rows
        b = rows // prob.S1
        i = rows % prob.S1
        return lambda h: (b * prob.N1 + h) * prob.S1 + i

    def _scatter_stats(self, full, sub):
        ff, sf = full.reshape(-1), sub.reshape(-1)
        pf, ps = self._stat_pos(self.p, self.live), self._stat_pos(self.sub, self.sub_row)
        for h in range(self.p.N1):
            ff[pf(h)] = sf[ps(h)]

    def device_inputs(self):
        p, dt = self.p, self.dtype
        return dict(query=to_dev(p.q, dt), key=to_dev(p.k, dt), value=to_dev(p.v, dt),
                    sparse_indices=to_dev(p.idx, "raw"), d_out=to_dev(p.dout, dt), out=to_dev(self.out_bits, dt),
                    softmax_max=to_dev(self.m_full, "raw"), softmax_sum=to_dev(self.l_full, "raw"),
                    query_rope=to_dev(p.qr, dt), key_rope=to_dev(p.kr, dt))

    def run_gpu(self, dev, deterministic=False):
        import sparse_mla_flash_amd as sf
        p = self.p
        d = dev
        return sf.sparse_flash_attention_grad(
            d["query"], d["key"], d["value"], d["sparse_indices"], d["d_out"], d["out"], d["softmax_max"],
            d["softmax_sum"], p.seq_q, p.seq_kv, d["query_rope"], d["key_rope"], scale_value=p.scale,
            sparse_block_size=p.block, layout=p.layout, sparse_mode=p.sparse_mode, deterministic=deterministic)

    def ref_dq(self, live_positions):
        """dQ / dQRope of live rows self.live[live_positions]."""
        sub_rows = self.sub_row[live_positions]
        m, l = self.m32.astype(np.float64), self.l32.astype(np.float64)
        return oracle.backward_dq(self.g, self.q, self.k, self.k, self.qr, self.kr, self.idx, self.dout,
                                  self.out_op, m, l, rows=sub_rows)

    def ref_dkv(self, keys):
        """dK / dKRope / dV of the given global key rows, summed over every live row (the key
        numbering is the same in the sub-problem: its key side is the full one)."""
        m, l = self.m32.astype(np.float64), self.l32.astype(np.float64)
        return oracle.backward_dkv(self.g, self.q, self.k, self.k, self.qr, self.kr, self.idx, self.dout,
                                   self.out_op, m, l, keys=keys)

    def keys_from_segments(self, rng, n, seg_rows=512, min_segments=2):
        """Up to n keys, each selected by live rows of at least `min_segments` different
        seg_rows-row segments of its sequence (in-sequence row index // seg_rows)."""
        p = self.p
        idxf = p.idx.reshape(p.rows, -1)
        seen = {}
        for grow in self.live:
            b = self._batch_of(grow)
            i = grow - p.q_offset(b)
            hi = min(i + p.lkv(b) - p.lq(b), p.lkv(b) - 1) if p.sparse_mode == 3 else p.lkv(b) - 1
            sel = idxf[grow].astype(np.int64)
            if p.block > 1:
                sel = (sel[sel >= 0][:, None] * p.block + np.arange(p.block)[None, :]).reshape(-1)
            sel = np.unique(sel[(sel >= 0) & (sel <= hi)])
            seg = i // seg_rows
            for j in sel + p.k_offset(b):
                seen.setdefault(int(j), set()).add(seg)
        multi = np.array(sorted(j for j, s in seen.items() if len(s) >= min_segments), dtype=np.int64)
        if len(multi) > n:
            multi = np.sort(rng.choice(multi, n, replace=False))
        return multi

    def _batch_of(self, grow):
        p = self.p
        for b in range(p.B):
            if p.q_offset(b) <= grow < p.q_offset(b) + p.lq(b):
                return b
        raise ValueError(grow)
