"""Seeded synthetic inputs for SparseFlashAttentionGrad workloads.

This module only draws random numbers and lays them out; it holds none of the
operator's arithmetic (no logits, softmax or gradients).  Both the test suite
(for the CPU oracle and the HIP library) and the benchmark take their inputs
from here, so the two sides always see bit-identical tensors.

Tensor layouts follow the operator's parameter list (SparseFlashAttentionGrad
README, "parameters" section): BSND query-side tensors are [B, S1, N1, D], key
side [B, S2, 1, D]; TND packs tokens as [T, N, D].  Floating-point tensors are
returned as 16-bit patterns (uint16) of the problem's element type, bfloat16 or
IEEE half (the two dtypes of the parameter table), drawn as fp32 N(0, 1) and
rounded to nearest-even; sparseIndices are int32 with -1 marking skipped slots.

Random streams: numpy ``SeedSequence(seed).spawn(6)`` in the fixed order
query, key, queryRope, keyRope, dOut, indices.  ``value`` is a separate copy of
``key`` (the operator requires value == key but the library must not assume the
two buffers alias).
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

D_NOPE = 512
D_ROPE = 64


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (nearest, ties to even); returns uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


DTYPES = ("bf16", "fp16")


def f32_to_bits(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return f32_to_f16_bits(x)
    raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


def bits_to_f64(b: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(b)
    if dtype == "fp16":
        return f16_bits_to_f64(b)
    raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


@dataclasses.dataclass
class Problem:
    """One synthetic SparseFlashAttentionGrad workload (shapes + seeded tensors)."""

    layout: str                      # "BSND" or "TND"
    B: int                           # batches (BSND) or sequences (TND)
    S1: int                          # BSND: padded query length; TND: total query tokens
    S2: int                          # BSND: padded key length; TND: total key tokens
    N1: int
    topk: int
    sparse_mode: int                 # 0 or 3
    seq_q: Optional[List[int]]       # per-batch valid query lengths (required for TND)
    seq_kv: Optional[List[int]]
    scale: float                     # fp32 scaleValue
    D: int = D_NOPE
    Dr: int = D_ROPE
    deterministic: bool = False
    name: str = ""
    block: int = 1                   # sparseBlockSize: each index names `block` consecutive keys
    dtype: str = "bf16"              # element type of the 16-bit tensors: "bf16" or "fp16"
    # tensors (filled by generate())
    q: Optional[np.ndarray] = None       # uint16 bits of the element type
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    qr: Optional[np.ndarray] = None
    kr: Optional[np.ndarray] = None
    dout: Optional[np.ndarray] = None
    idx: Optional[np.ndarray] = None     # int32

    # ---- geometry ---------------------------------------------------------
    @property
    def rows(self) -> int:
        """Total query rows (padded rows included for BSND)."""
        return self.B * self.S1 if self.layout == "BSND" else self.S1

    @property
    def keys(self) -> int:
        return self.B * self.S2 if self.layout == "BSND" else self.S2

    def lq(self, b: int) -> int:
        if self.seq_q is None:
            return self.S1
        return int(self.seq_q[b])

    def lkv(self, b: int) -> int:
        if self.seq_kv is None:
            return self.S2
        return int(self.seq_kv[b])

    def q_offset(self, b: int) -> int:
        """First global query row of batch b."""
        if self.layout == "BSND":
            return b * self.S1
        return int(sum(self.seq_q[:b]))

    def k_offset(self, b: int) -> int:
        if self.layout == "BSND":
            return b * self.S2
        return int(sum(self.seq_kv[:b]))

    def q_shape(self, width: int):
        if self.layout == "BSND":
            return (self.B, self.S1, self.N1, width)
        return (self.S1, self.N1, width)

    def k_shape(self, width: int):
        if self.layout == "BSND":
            return (self.B, self.S2, 1, width)
        return (self.S2, 1, width)

    def idx_shape(self):
        if self.layout == "BSND":
            return (self.B, self.S1, 1, self.topk)
        return (self.S1, 1, self.topk)

    def stat_shape(self):
        if self.layout == "BSND":
            return (self.B, self.N1, self.S1)
        return (self.N1, self.S1)


# ---------------------------------------------------------------------------
# index patterns
# ---------------------------------------------------------------------------

def _causal_hi(p: Problem, b: int, i: int) -> int:
    """Largest key position a query at row i of batch b may select (-1: none)."""
    lkv = p.lkv(b)
    if p.sparse_mode == 3:
        return min(i + lkv - p.lq(b), lkv - 1)
    return lkv - 1


def _distinct_rows(rng, n: np.ndarray, k: int, group: int = 32) -> np.ndarray:
    """Row r: k distinct integers uniform over [0, n[r]) (n[r] >= k), in random order.

    The k smallest of n[r] independent uniform sort keys sit at a uniformly random k-subset of
    positions; a second set of keys shuffles them.  Rows are drawn in groups as one matrix."""
    out = np.empty((len(n), k), dtype=np.int64)
    for g0 in range(0, len(n), group):
        ng = n[g0:g0 + group]
        u = rng.random((len(ng), int(ng.max())))
        u[np.arange(u.shape[1])[None, :] >= ng[:, None]] = 2.0      # outside the row's range
        sel = np.argpartition(u, k - 1, axis=1)[:, :k]
        order = np.argsort(rng.random((len(ng), k)), axis=1)
        out[g0:g0 + group] = np.take_along_axis(sel, order, axis=1)
    return out


def _rows_uniform(p: Problem, rng, b: int) -> np.ndarray:
    """Per query row: distinct uniform keys (with block selection: blocks of p.block keys, the
    last one possibly reaching past the valid range) over the valid range; short ranges take all
    candidates in random order; -1 padded."""
    lq = p.lq(b)
    out = np.full((lq, p.topk), -1, dtype=np.int64)
    n = np.array([_causal_hi(p, b, i) // p.block + 1 for i in range(lq)], dtype=np.int64)
    for i in np.nonzero((n > 0) & (n <= p.topk))[0]:
        out[i, :n[i]] = rng.permutation(int(n[i]))
    long_rows = np.nonzero(n > p.topk)[0]
    if len(long_rows):
        out[long_rows] = _distinct_rows(rng, n[long_rows], p.topk)
    return out


def _rows_window(p: Problem, rng, b: int, window: int) -> np.ndarray:
    """Per query row: half the slots distinct uniform from the local window [pos-window+1, pos],
    the other half distinct uniform over the rest of [0, pos]; short ranges take all keys."""
    lq = p.lq(b)
    out = np.full((lq, p.topk), -1, dtype=np.int64)
    hi = np.array([_causal_hi(p, b, i) for i in range(lq)], dtype=np.int64)
    n = hi + 1
    for i in np.nonzero((n > 0) & (n <= p.topk))[0]:
        out[i, :n[i]] = rng.permutation(int(n[i]))
    rows = np.nonzero(n > p.topk)[0]
    if not len(rows):
        return out
    half = p.topk // 2
    wlo = np.maximum(0, hi[rows] - window + 1)
    wn = hi[rows] - wlo + 1
    loc_k = int(min(half, wn.min()))
    loc = _distinct_rows(rng, wn, loc_k) + wlo[:, None]
    for r, i in enumerate(rows):
        need = p.topk - loc_k
        picked = np.empty(0, dtype=np.int64)
        while len(picked) < need:
            cand = rng.integers(0, n[i], size=2 * (need - len(picked)) + 64)
            _, first = np.unique(cand, return_index=True)
            cand = cand[np.sort(first)]                                 # first draws, in draw order
            cand = cand[~np.isin(cand, loc[r]) & ~np.isin(cand, picked)]
            picked = np.concatenate([picked, cand[:need - len(picked)]])
        sel = np.concatenate([loc[r], picked])
        out[i] = sel[rng.permutation(len(sel))]
    return out


def _rows_hot_cold(p: Problem, rng, b: int) -> np.ndarray:
    """Mode-0 rows where every query selects all hot keys plus distinct cold keys.

    Hot keys are 10% of the key range; with topk above that count each query
    takes all of them (the most the skew allows) and fills the rest uniformly
    from the cold keys.  Slot order is shuffled.
    """
    lkv = p.lkv(b)
    nhot = max(1, int(round(0.1 * lkv)))
    perm = rng.permutation(lkv)
    hot, cold = perm[:nhot], perm[nhot:]
    lq = p.lq(b)
    rows = np.full((p.S1 if p.layout == "BSND" else lq, p.topk), -1, dtype=np.int64)
    take_hot = min(nhot, p.topk)
    for i in range(lq):
        h = hot if take_hot == nhot else hot[rng.choice(nhot, take_hot, replace=False)]
        ncold = min(p.topk - take_hot, len(cold))
        c = cold[rng.choice(len(cold), ncold, replace=False)] if ncold > 0 else np.empty(0, np.int64)
        sel = np.concatenate([h, c])
        rows[i, : len(sel)] = sel[rng.permutation(len(sel))]
    return rows


def _indices(p: Problem, rng: np.random.Generator, kind: str, window: int) -> np.ndarray:
    if p.block != 1 and kind != "uniform":
        raise ValueError("block selection inputs are generated with the uniform recipe only")
    idx = np.full((p.rows, p.topk), -1, dtype=np.int64)
    for b in range(p.B):
        base = p.q_offset(b)
        if kind == "hot_cold":
            r = _rows_hot_cold(p, rng, b)
        elif kind == "uniform":
            r = _rows_uniform(p, rng, b)
        elif kind == "window":
            r = _rows_window(p, rng, b, window)
        else:
            raise ValueError(f"unknown index kind {kind!r}")
        idx[base: base + r.shape[0]] = r
    return idx.astype(np.int32)


# ---------------------------------------------------------------------------
# generation
# ---------------------------------------------------------------------------

def _normal_bits(rng: np.random.Generator, shape, dtype: str = "bf16", chunk: int = 1 << 22) -> np.ndarray:
    """N(0, 1) fp32 values rounded to the element type's bits.  The tensor is cut into fixed chunks of
    ``chunk`` elements; chunk c is drawn from its own generator, seeded by child c of a
    SeedSequence whose entropy is one draw from ``rng``.  The values therefore depend only on
    ``rng``'s state (not on the number of threads), and the chunks are drawn in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nchunk = (n + chunk - 1) // chunk
    kids = np.random.SeedSequence(int(rng.integers(0, 2 ** 63 - 1, dtype=np.int64))).spawn(max(nchunk, 1))

    def fill(c: int) -> None:
        s, e = c * chunk, min(n, (c + 1) * chunk)
        out[s:e] = f32_to_bits(np.random.default_rng(kids[c]).standard_normal(e - s, dtype=np.float32), dtype)

    if nchunk <= 1:
        for c in range(nchunk):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=min(16, nchunk)) as ex:
            list(ex.map(fill, range(nchunk)))
    return out.reshape(shape)


def generate(p: Problem, seed: int, index_kind: str = "uniform", window: int = 4096,
             fill: str = "normal") -> Problem:
    """Fill p's tensors from ``seed``.

    fill="normal": N(0,1) values in p.dtype (the benchmark workloads).
    fill="ones": every float tensor is 1.0 (the all-ones sample input of the
    dense FlashAttention-grad page), indices still random.
    """
    ss = np.random.SeedSequence(seed).spawn(6)
    rq, rk, rqr, rkr, rdo, ridx = (np.random.default_rng(s) for s in ss)
    if fill == "normal":
        p.q = _normal_bits(rq, p.q_shape(p.D), p.dtype)
        p.k = _normal_bits(rk, p.k_shape(p.D), p.dtype)
        p.qr = _normal_bits(rqr, p.q_shape(p.Dr), p.dtype)
        p.kr = _normal_bits(rkr, p.k_shape(p.Dr), p.dtype)
        p.dout = _normal_bits(rdo, p.q_shape(p.D), p.dtype)
    elif fill == "ones":
        one = f32_to_bits(np.ones(1, np.float32), p.dtype)[0]
        p.q = np.full(p.q_shape(p.D), one, np.uint16)
        p.k = np.full(p.k_shape(p.D), one, np.uint16)
        p.qr = np.full(p.q_shape(p.Dr), one, np.uint16)
        p.kr = np.full(p.k_shape(p.Dr), one, np.uint16)
        p.dout = np.full(p.q_shape(p.D), one, np.uint16)
    else:
        raise ValueError(fill)
    p.v = p.k.copy()
    p.idx = _indices(p, ridx, index_kind, window).reshape(p.idx_shape())
    return p


def fp32(x: float) -> float:
    return float(np.float32(x))


def problem(layout="BSND", B=1, S1=128, S2=128, N1=8, topk=64, sparse_mode=3, seq_q=None,
            seq_kv=None, scale=None, D=D_NOPE, Dr=D_ROPE, deterministic=False, name="",
            block=1, dtype="bf16") -> Problem:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    if scale is None:
        scale = 1.0 / math.sqrt(D + Dr)
    if layout == "TND":
        assert seq_q is not None and seq_kv is not None
        S1, S2 = int(sum(seq_q)), int(sum(seq_kv))
    return Problem(layout=layout, B=B, S1=S1, S2=S2, N1=N1, topk=topk, sparse_mode=sparse_mode,
                   seq_q=None if seq_q is None else [int(x) for x in seq_q],
                   seq_kv=None if seq_kv is None else [int(x) for x in seq_kv],
                   scale=fp32(scale), D=D, Dr=Dr, deterministic=deterministic, name=name,
                   block=int(block), dtype=dtype)


# The five benchmark workloads (shapes and index structure).  Seed = workload number.
WORKLOADS = {
    1: dict(spec=dict(layout="BSND", B=1, S1=128, S2=4096, N1=8, topk=1024, sparse_mode=3,
                      name="bsnd_s128q_4096k_n8_topk1024_causal"), kind="uniform"),
    2: dict(spec=dict(layout="BSND", B=1, S1=8192, S2=8192, N1=64, topk=2048, sparse_mode=3,
                      name="bsnd_s8192_n64_topk2048_causal"), kind="uniform"),
    3: dict(spec=dict(layout="TND", B=4, seq_q=[2048, 4096, 8192, 16384],
                      seq_kv=[2048, 4096, 8192, 16384], N1=128, topk=2048, sparse_mode=3,
                      name="tnd_varlen_2k-16k_n128_topk2048_causal"), kind="uniform"),
    4: dict(spec=dict(layout="BSND", B=1, S1=16384, S2=131072, N1=128, topk=2048, sparse_mode=3,
                      name="bsnd_s16384q_131072k_n128_topk2048_window_causal"), kind="window"),
    5: dict(spec=dict(layout="BSND", B=2, S1=4096, S2=32768, N1=48, topk=8192, sparse_mode=0,
                      deterministic=True, name="bsnd_b2_s4096q_32768k_n48_topk8192_hotcold_det"),
            kind="hot_cold"),
    # block selection: 32 blocks of 64 consecutive keys per token (2048 keys, as workload 2)
    6: dict(spec=dict(layout="BSND", B=1, S1=8192, S2=8192, N1=64, topk=32, sparse_mode=3, block=64,
                      name="bsnd_s8192_n64_top32x64blocks_causal"), kind="uniform"),
}


def workload(n: int, seed: Optional[int] = None, dtype: str = "bf16") -> Problem:
    w = WORKLOADS[n]
    p = problem(**w["spec"], dtype=dtype)
    return generate(p, n if seed is None else seed, index_kind=w["kind"])


# ---------------------------------------------------------------------------
# lightning-indexer backward inputs
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class IndexerProblem:
    """Shapes and seeded tensors of one lightning-indexer backward call (the sparse operator's
    layouts; index heads G of width Di = 128)."""

    layout: str
    B: int
    S1: int
    S2: int
    N1: int
    G: int
    sparse_mode: int
    seq_q: Optional[List[int]]
    seq_kv: Optional[List[int]]
    scale: float
    Di: int = 128
    D: int = D_NOPE
    Dr: int = D_ROPE
    dtype: str = "bf16"
    name: str = ""
    q: Optional[np.ndarray] = None       # [rows, N1, 512] bits
    qr: Optional[np.ndarray] = None      # [rows, N1, 64]
    k: Optional[np.ndarray] = None       # [keys, 1, 512]
    kr: Optional[np.ndarray] = None      # [keys, 1, 64]
    qi: Optional[np.ndarray] = None      # [rows, G, 128]
    ki: Optional[np.ndarray] = None      # [keys, 1, 128]
    w: Optional[np.ndarray] = None       # [rows, G]

    @property
    def rows(self) -> int:
        return self.B * self.S1 if self.layout == "BSND" else self.S1

    @property
    def keys(self) -> int:
        return self.B * self.S2 if self.layout == "BSND" else self.S2

    def shape(self, n: int, w: int, side: str = "q"):
        """Tensor shape of n heads of width w on the query (or key) side in this layout."""
        if self.layout == "BSND":
            return (self.B, self.S1 if side == "q" else self.S2, n, w)
        return (self.S1 if side == "q" else self.S2, n, w)


def indexer_problem(layout="BSND", B=1, S1=128, S2=128, N1=16, G=16, sparse_mode=3, seq_q=None, seq_kv=None,
                    scale=None, dtype="bf16", name="") -> IndexerProblem:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    if scale is None:
        scale = 1.0 / math.sqrt(D_NOPE + D_ROPE)
    if layout == "TND":
        assert seq_q is not None and seq_kv is not None
        S1, S2 = int(sum(seq_q)), int(sum(seq_kv))
    return IndexerProblem(layout=layout, B=B, S1=S1, S2=S2, N1=N1, G=G, sparse_mode=sparse_mode,
                          seq_q=None if seq_q is None else [int(x) for x in seq_q],
                          seq_kv=None if seq_kv is None else [int(x) for x in seq_kv],
                          scale=fp32(scale), dtype=dtype, name=name)


def indexer_generate(p: IndexerProblem, seed: int) -> IndexerProblem:
    """Fill p from ``seed``: streams in the order query, queryRope, key, keyRope, queryIndex,
    keyIndex, weights.  Every value is N(0, 1) in fp32 rounded to p.dtype, except the weights,
    drawn N(0, 1 / (G Di)) so that the index scores W . ReLU(q~ K~) have a spread of order one."""
    ss = np.random.SeedSequence(seed).spawn(7)
    rq, rqr, rk, rkr, rqi, rki, rw = (np.random.default_rng(s) for s in ss)
    p.q = _normal_bits(rq, p.shape(p.N1, p.D), p.dtype)
    p.qr = _normal_bits(rqr, p.shape(p.N1, p.Dr), p.dtype)
    p.k = _normal_bits(rk, p.shape(1, p.D, "k"), p.dtype)
    p.kr = _normal_bits(rkr, p.shape(1, p.Dr, "k"), p.dtype)
    p.qi = _normal_bits(rqi, p.shape(p.G, p.Di), p.dtype)
    p.ki = _normal_bits(rki, p.shape(1, p.Di, "k"), p.dtype)
    wshape = p.shape(p.G, 1)[:-1]
    p.w = f32_to_bits(rw.standard_normal(int(np.prod(wshape)), dtype=np.float32)
                      / np.float32(math.sqrt(p.G * p.Di)), p.dtype).reshape(wshape)
    return p
