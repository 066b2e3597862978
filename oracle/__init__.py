"""fp64 CPU oracle for SparseFlashAttentionGrad -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with it.

The arithmetic lives in ``sfag_oracle.c`` (plain loops in fp64, one per formula
of the SparseFlashAttentionGrad README's "function description" section); this
module marshals numpy arrays into it with ctypes.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against central finite differences, torch fp64 autograd of dense masked
attention, closed forms and invariants.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sfag_oracle.c")
_LIB = os.path.join(_HERE, "libsfag_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("S1", ctypes.c_int64), ("S2", ctypes.c_int64),
        ("N1", ctypes.c_int64), ("D", ctypes.c_int64), ("Dr", ctypes.c_int64),
        ("topk", ctypes.c_int64), ("layout", ctypes.c_int32), ("sparse_mode", ctypes.c_int32),
        ("seq_q", ctypes.POINTER(ctypes.c_int32)), ("seq_kv", ctypes.POINTER(ctypes.c_int32)),
        ("scale", ctypes.c_double), ("block", ctypes.c_int64),
    ]


def _load(path: str):
    L = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lp = ctypes.POINTER(ctypes.c_int64)
    pp = ctypes.POINTER(_Problem)
    L.sfag_oracle_forward.argtypes = [pp, dp, dp, dp, dp, dp, ip, lp, ctypes.c_int64, dp, dp, dp]
    L.sfag_oracle_backward_dq.argtypes = [pp, dp, dp, dp, dp, dp, ip, dp, dp, dp, dp, lp,
                                          ctypes.c_int64, dp, dp]
    L.sfag_oracle_backward_dkv.argtypes = [pp, dp, dp, dp, dp, dp, ip, dp, dp, dp, dp, lp,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                           dp, dp, dp]
    L.sfag_oracle_num_threads.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _load(_LIB)
    return _lib


def swap_library(path: Optional[str]):
    """Point the wrappers at another build of the oracle source (None: the default).

    Used by the mutation tests, which compile deliberately broken copies of the
    source and check that the pins reject them.  Returns the previous handle."""
    global _lib
    prev = _lib
    _lib = None if path is None else _load(path)
    return prev


def num_threads() -> int:
    return int(lib().sfag_oracle_num_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


class Geometry:
    """Shapes of one problem as the oracle sees it (generic D / Dr allowed)."""

    def __init__(self, layout: str, B: int, S1: int, S2: int, N1: int, D: int, Dr: int,
                 topk: int, sparse_mode: int, seq_q: Optional[Sequence[int]],
                 seq_kv: Optional[Sequence[int]], scale: float, block: int = 1):
        self.layout, self.B, self.S1, self.S2 = layout, B, S1, S2
        self.N1, self.D, self.Dr, self.topk = N1, D, Dr, topk
        self.block = int(block)          # sparseBlockSize: each index names `block` keys
        self.sparse_mode, self.scale = sparse_mode, scale
        self.seq_q = None if seq_q is None else np.ascontiguousarray(seq_q, dtype=np.int32)
        self.seq_kv = None if seq_kv is None else np.ascontiguousarray(seq_kv, dtype=np.int32)
        if layout == "TND":
            assert self.seq_q is not None and self.seq_kv is not None
        self.rows = B * S1 if layout == "BSND" else S1
        self.keys = B * S2 if layout == "BSND" else S2

    @classmethod
    def of(cls, p) -> "Geometry":
        """From a sparse_mla_flash_amd.inputs.Problem (duck-typed)."""
        return cls(p.layout, p.B, p.S1, p.S2, p.N1, p.D, p.Dr, p.topk, p.sparse_mode,
                   p.seq_q, p.seq_kv, p.scale, getattr(p, "block", 1))

    def c(self) -> _Problem:
        s = _Problem(self.B, self.S1, self.S2, self.N1, self.D, self.Dr, self.topk,
                     0 if self.layout == "BSND" else 1, self.sparse_mode, None, None,
                     float(self.scale), self.block)
        if self.seq_q is not None:
            s.seq_q = _ptr(self.seq_q, ctypes.c_int32)
        if self.seq_kv is not None:
            s.seq_kv = _ptr(self.seq_kv, ctypes.c_int32)
        return s

    def stat_shape(self):
        return (self.B, self.N1, self.S1) if self.layout == "BSND" else (self.N1, self.S1)


def forward(g: Geometry, q, k, v, qr, kr, idx, rows=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Sparse forward: out [rows,N1,D], softmaxMax / softmaxSum in the stats layout.

    With ``rows`` only those query rows are computed; the rest stay zero."""
    q, k, v, qr, kr = (_f64(x) for x in (q, k, v, qr, kr))
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.zeros((g.rows, g.N1, g.D))
    smax = np.zeros(g.stat_shape())
    ssum = np.zeros(g.stat_shape())
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    pb = g.c()
    lib().sfag_oracle_forward(ctypes.byref(pb), _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                              _ptr(v, ctypes.c_double), _ptr(qr, ctypes.c_double),
                              _ptr(kr, ctypes.c_double), _ptr(idx, ctypes.c_int32),
                              None if r is None else _ptr(r, ctypes.c_int64),
                              0 if r is None else len(r), _ptr(out, ctypes.c_double),
                              _ptr(smax, ctypes.c_double), _ptr(ssum, ctypes.c_double))
    return out, smax, ssum


def backward_dq(g: Geometry, q, k, v, qr, kr, idx, dout, out, smax, ssum, rows=None):
    """dQ [n,N1,D] and dQRope [n,N1,Dr] for the listed query rows (all when None)."""
    q, k, v, qr, kr, dout, out, smax, ssum = (_f64(x) for x in (q, k, v, qr, kr, dout, out, smax, ssum))
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = g.rows if r is None else len(r)
    dq = np.zeros((n, g.N1, g.D))
    dqr = np.zeros((n, g.N1, g.Dr))
    pb = g.c()
    lib().sfag_oracle_backward_dq(ctypes.byref(pb), *(_ptr(x, ctypes.c_double) for x in (q, k, v, qr, kr)),
                                  _ptr(idx, ctypes.c_int32),
                                  *(_ptr(x, ctypes.c_double) for x in (dout, out, smax, ssum)),
                                  None if r is None else _ptr(r, ctypes.c_int64), n,
                                  _ptr(dq, ctypes.c_double), _ptr(dqr, ctypes.c_double))
    return dq, dqr


def backward_dkv(g: Geometry, q, k, v, qr, kr, idx, dout, out, smax, ssum, keys=None,
                 row_lo: int = 0, row_hi: Optional[int] = None):
    """dK [n,D], dKRope [n,Dr], dV [n,D] for the listed global key rows (all when None),
    counting only query rows in [row_lo, row_hi)."""
    q, k, v, qr, kr, dout, out, smax, ssum = (_f64(x) for x in (q, k, v, qr, kr, dout, out, smax, ssum))
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    kk = None if keys is None else np.ascontiguousarray(keys, dtype=np.int64)
    n = g.keys if kk is None else len(kk)
    dk = np.zeros((n, g.D))
    dkr = np.zeros((n, g.Dr))
    dv = np.zeros((n, g.D))
    pb = g.c()
    lib().sfag_oracle_backward_dkv(ctypes.byref(pb), *(_ptr(x, ctypes.c_double) for x in (q, k, v, qr, kr)),
                                   _ptr(idx, ctypes.c_int32),
                                   *(_ptr(x, ctypes.c_double) for x in (dout, out, smax, ssum)),
                                   None if kk is None else _ptr(kk, ctypes.c_int64), n,
                                   row_lo, g.rows if row_hi is None else row_hi,
                                   _ptr(dk, ctypes.c_double), _ptr(dkr, ctypes.c_double),
                                   _ptr(dv, ctypes.c_double))
    return dk, dkr, dv


def backward(g: Geometry, q, k, v, qr, kr, idx, dout, out, smax, ssum):
    """Full backward: (dq, dk, dv, dqr, dkr) in the input layouts' shapes (flattened rows)."""
    dq, dqr = backward_dq(g, q, k, v, qr, kr, idx, dout, out, smax, ssum)
    dk, dkr, dv = backward_dkv(g, q, k, v, qr, kr, idx, dout, out, smax, ssum)
    return dq, dk, dv, dqr, dkr
