"""MI355X-native SparseFlashAttentionGrad: gfx950 HIP kernels behind a C ABI.

This module is a thin ctypes binding of ``libsfag.so`` (declared in
``include/sfag.h``).  It only checks tensor shapes / dtypes, allocates outputs
and workspace with torch, and passes torch's current HIP stream; every step of
the computation runs in the library's kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.

Entry points (same names as the C ABI):
  sfag_get_workspace_size, sfag_sparse_flash_attention_grad,
  sfag_sparse_flash_attention_forward, sfag_last_error, sfag_version
and the tensor-level wrappers
  sparse_flash_attention_grad(...)    -> (dq, dk, dv, dq_rope, dk_rope)
  sparse_flash_attention_forward(...) -> (out, softmax_max, softmax_sum)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfag.so")

SFAG_OK = 0
SFAG_ERR_PARAM_NULLPTR = 161001
SFAG_ERR_PARAM_INVALID = 161002
SFAG_ERR_UNSUPPORTED = 161901
SFAG_ERR_WORKSPACE = 161902
SFAG_ERR_DEVICE = 161903

NOALLOC_SCRATCH_BYTES = 256 << 20      # SFAG_NOALLOC_SCRATCH_BYTES
SFAG_DTYPE_BF16 = 0
SFAG_DTYPE_FP16 = 1

EXPORTED = ("sfag_get_workspace_size", "sfag_sparse_flash_attention_grad", "sfag_sparse_flash_attention_grad_noalloc",
            "sfag_sparse_flash_attention_forward", "sfag_set_profile_events", "sfag_last_path", "sfag_last_error",
            "sfag_version", "sfag_lightning_indexer_grad_get_workspace_size",
            "sfag_dense_lightning_indexer_grad_kl_loss")


class SfagError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sfag status {status}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S1", ctypes.c_int64), ("S2", ctypes.c_int64),
                ("N1", ctypes.c_int64), ("N2", ctypes.c_int64), ("D", ctypes.c_int64),
                ("Drope", ctypes.c_int64), ("topk", ctypes.c_int64), ("dtype", ctypes.c_int64)]


class IndexerDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S1", ctypes.c_int64), ("S2", ctypes.c_int64), ("N1", ctypes.c_int64),
                ("G", ctypes.c_int64), ("D", ctypes.c_int64), ("Drope", ctypes.c_int64), ("Di", ctypes.c_int64),
                ("dtype", ctypes.c_int64)]


_lib = None


def lib():
    """Load libsfag.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m sparse_mla_flash_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
        L.sfag_get_workspace_size.restype = ctypes.c_int
        L.sfag_get_workspace_size.argtypes = [ctypes.POINTER(Dims), i32p, i32p, ctypes.c_float,
                                              ctypes.c_int64, ctypes.c_char_p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_uint64)]
        L.sfag_sparse_flash_attention_grad.restype = ctypes.c_int
        L.sfag_sparse_flash_attention_grad.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, ctypes.POINTER(Dims),
            ctypes.c_float, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.sfag_sparse_flash_attention_grad_noalloc.restype = ctypes.c_int
        L.sfag_sparse_flash_attention_grad_noalloc.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, ctypes.POINTER(Dims),
            ctypes.c_float, ctypes.c_int64, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp, vp, vp]
        L.sfag_sparse_flash_attention_forward.restype = ctypes.c_int
        L.sfag_sparse_flash_attention_forward.argtypes = [
            vp, vp, vp, vp, i32p, i32p, vp, vp, ctypes.POINTER(Dims), ctypes.c_float,
            ctypes.c_int64, ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            vp, vp, vp, vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.sfag_lightning_indexer_grad_get_workspace_size.restype = ctypes.c_int
        L.sfag_lightning_indexer_grad_get_workspace_size.argtypes = [
            ctypes.POINTER(IndexerDims), i64p, i64p, ctypes.c_char_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)]
        L.sfag_dense_lightning_indexer_grad_kl_loss.restype = ctypes.c_int
        L.sfag_dense_lightning_indexer_grad_kl_loss.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64p, i64p, ctypes.POINTER(IndexerDims), ctypes.c_double,
            ctypes.c_char_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.sfag_set_profile_events.restype = ctypes.c_int
        L.sfag_set_profile_events.argtypes = [vp, vp, vp, vp]
        L.sfag_last_path.restype = ctypes.c_int32
        L.sfag_last_path.argtypes = []
        L.sfag_last_error.restype = ctypes.c_char_p
        L.sfag_last_error.argtypes = []
        L.sfag_version.restype = ctypes.c_char_p
        L.sfag_version.argtypes = []
        _lib = L
    return _lib


def sfag_last_error() -> str:
    return lib().sfag_last_error().decode()


def sfag_version() -> str:
    return lib().sfag_version().decode()


def sfag_set_profile_events(s1_begin=None, s1_end=None, s2_begin=None, s2_end=None) -> int:
    """Record caller-owned hipEvent_t handles around the two main stages of later calls."""
    return lib().sfag_set_profile_events(s1_begin, s1_end, s2_begin, s2_end)


def sfag_last_path() -> int:
    """0: key-major dense path, 1: scatter path, -1: no backward call yet (this thread)."""
    return lib().sfag_last_path()


def _check(status: int) -> None:
    if status != SFAG_OK:
        raise SfagError(status, sfag_last_error())


def _lens(x: Optional[Sequence[int]]):
    if x is None:
        return None, None
    arr = (ctypes.c_int32 * len(x))(*[int(v) for v in x])
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))


def sfag_get_workspace_size(dims: Dims, seq_len_q=None, seq_len_kv=None, scale_value: float = 1.0,
                            sparse_block_size: int = 1, layout: str = "BSND", sparse_mode: int = 3,
                            pre_tokens: int = 2 ** 31 - 1, next_tokens: int = 2 ** 31 - 1,
                            deterministic: bool = False) -> int:
    _, q = _lens(seq_len_q)
    _k, kv = _lens(seq_len_kv)
    _keep = (_, _k)
    out = ctypes.c_uint64(0)
    _check(lib().sfag_get_workspace_size(ctypes.byref(dims), q, kv, float(scale_value), int(sparse_block_size),
                                         layout.encode(), int(sparse_mode), int(pre_tokens), int(next_tokens),
                                         int(bool(deterministic)), ctypes.byref(out)))
    del _keep
    return int(out.value)


def sfag_sparse_flash_attention_grad(query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum,
                                     seq_len_q, seq_len_kv, query_rope, key_rope, dims: Dims, scale_value,
                                     sparse_block_size, layout, sparse_mode, pre_tokens, next_tokens,
                                     deterministic, d_query, d_key, d_value, d_query_rope, d_key_rope,
                                     workspace, workspace_size, stream) -> int:
    """Raw C call: every tensor argument is a device address (int) or None; returns the status."""
    qa, qp = _lens(seq_len_q)
    ka, kp = _lens(seq_len_kv)
    return lib().sfag_sparse_flash_attention_grad(
        query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum, qp, kp, query_rope, key_rope,
        ctypes.byref(dims), float(scale_value), int(sparse_block_size), layout.encode(), int(sparse_mode),
        int(pre_tokens), int(next_tokens), int(bool(deterministic)), d_query, d_key, d_value, d_query_rope,
        d_key_rope, workspace, int(workspace_size), stream)


def sfag_sparse_flash_attention_grad_noalloc(query, key, value, sparse_indices, d_out, out, softmax_max,
                                             softmax_sum, seq_len_q, seq_len_kv, query_rope, key_rope, dims: Dims,
                                             scale_value, sparse_block_size, layout, sparse_mode, pre_tokens,
                                             next_tokens, deterministic, d_query, d_key, d_value, d_query_rope,
                                             d_key_rope, stream) -> int:
    """Raw C call of the no-allocation variant (the library's built-in scratch replaces the
    workspace); every tensor argument is a device address (int) or None; returns the status."""
    qa, qp = _lens(seq_len_q)
    ka, kp = _lens(seq_len_kv)
    return lib().sfag_sparse_flash_attention_grad_noalloc(
        query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum, qp, kp, query_rope, key_rope,
        ctypes.byref(dims), float(scale_value), int(sparse_block_size), layout.encode(), int(sparse_mode),
        int(pre_tokens), int(next_tokens), int(bool(deterministic)), d_query, d_key, d_value, d_query_rope,
        d_key_rope, stream)


def sfag_sparse_flash_attention_forward(query, key, value, sparse_indices, seq_len_q, seq_len_kv, query_rope,
                                        key_rope, dims: Dims, scale_value, sparse_block_size, layout,
                                        sparse_mode, pre_tokens, next_tokens, out, softmax_max, softmax_sum,
                                        stream) -> int:
    qa, qp = _lens(seq_len_q)
    ka, kp = _lens(seq_len_kv)
    return lib().sfag_sparse_flash_attention_forward(
        query, key, value, sparse_indices, qp, kp, query_rope, key_rope, ctypes.byref(dims), float(scale_value),
        int(sparse_block_size), layout.encode(), int(sparse_mode), int(pre_tokens), int(next_tokens), out,
        softmax_max, softmax_sum, stream)


# ---------------------------------------------------------------------------------------------
# tensor-level wrappers (torch for device memory and streams only)
# ---------------------------------------------------------------------------------------------

def _dims_from(query, key, sparse_indices, layout: str, seq_len_q, seq_len_kv, query_rope=None) -> Dims:
    if layout == "BSND":
        if query.dim() != 4 or key.dim() != 4 or sparse_indices.dim() != 4:
            raise ValueError("BSND expects query [B,S1,N1,D], key [B,S2,1,D], sparse_indices [B,S1,1,topk]")
        B, S1, N1, D = query.shape
        _, S2, N2, _ = key.shape
        topk = sparse_indices.shape[-1]
    elif layout == "TND":
        if query.dim() != 3 or key.dim() != 3 or sparse_indices.dim() != 3:
            raise ValueError("TND expects query [T1,N1,D], key [T2,1,D], sparse_indices [T1,1,topk]")
        if seq_len_q is None or seq_len_kv is None:
            raise ValueError("TND needs actual_seq_lengths_query and actual_seq_lengths_kv")
        S1, N1, D = query.shape
        S2, N2, _ = key.shape
        B = len(seq_len_q)
        topk = sparse_indices.shape[-1]
    else:
        raise ValueError(f"layout must be BSND or TND, got {layout!r}")
    # the rope width is fixed at 64 by the operator; rope tensors are checked against it
    return Dims(int(B), int(S1), int(S2), int(N1), int(N2), int(D), 64, int(topk), _dtype_code(query))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SFAG_DTYPE_BF16
    if t.dtype == torch.float16:
        return SFAG_DTYPE_FP16
    raise ValueError(f"query must be bfloat16 or float16, got {t.dtype}")


def _elem_dtype(dims: Dims):
    import torch
    return torch.float16 if dims.dtype == SFAG_DTYPE_FP16 else torch.bfloat16


def _check_shapes(dims: Dims, layout: str, **tensors) -> None:
    """Every tensor's shape against the dims taken from query / key / sparse_indices, so that a
    mis-shaped tensor is rejected here instead of being read out of bounds by a kernel."""
    B, S1, S2, N1, N2, D, Dr, topk = (dims.B, dims.S1, dims.S2, dims.N1, dims.N2, dims.D, dims.Drope,
                                      dims.topk)
    if layout == "BSND":
        want = dict(query=(B, S1, N1, D), key=(B, S2, N2, D), value=(B, S2, N2, D),
                    sparse_indices=(B, S1, N2, topk), d_out=(B, S1, N1, D), out=(B, S1, N1, D),
                    softmax_max=(B, N1, S1), softmax_sum=(B, N1, S1), query_rope=(B, S1, N1, Dr),
                    key_rope=(B, S2, N2, Dr))
    else:
        want = dict(query=(S1, N1, D), key=(S2, N2, D), value=(S2, N2, D), sparse_indices=(S1, N2, topk),
                    d_out=(S1, N1, D), out=(S1, N1, D), softmax_max=(N1, S1), softmax_sum=(N1, S1),
                    query_rope=(S1, N1, Dr), key_rope=(S2, N2, Dr))
    for name, t in tensors.items():
        if t is None:
            continue
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]} for layout {layout}")
    if (tensors.get("query_rope") is None) != (tensors.get("key_rope") is None):
        raise ValueError("query_rope and key_rope must be given together or both omitted")


def _dev(t, name, dtype):
    import torch
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _seq(x):
    if x is None:
        return None
    return [int(v) for v in (x.tolist() if hasattr(x, "tolist") else x)]


def sparse_flash_attention_grad(query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum,
                                actual_seq_lengths_query=None, actual_seq_lengths_kv=None, query_rope=None,
                                key_rope=None, *, scale_value: float, sparse_block_size: int = 1,
                                layout: str = "BSND", sparse_mode: int = 3, pre_tokens: int = 2 ** 31 - 1,
                                next_tokens: int = 2 ** 31 - 1, deterministic: bool = False, workspace=None):
    """Backward of sparse MLA attention; returns (dq, dk, dv, dq_rope, dk_rope) in the inputs'
    element type (bfloat16 or float16: every 16-bit tensor of a call has query's type)."""
    import torch
    sq, skv = _seq(actual_seq_lengths_query), _seq(actual_seq_lengths_kv)
    dims = _dims_from(query, key, sparse_indices, layout, sq, skv, query_rope)
    bf = _elem_dtype(dims)
    _check_shapes(dims, layout, query=query, key=key, value=value, sparse_indices=sparse_indices, d_out=d_out,
                  out=out, softmax_max=softmax_max, softmax_sum=softmax_sum, query_rope=query_rope,
                  key_rope=key_rope)
    ws = sfag_get_workspace_size(dims, sq, skv, scale_value, sparse_block_size, layout, sparse_mode,
                                 pre_tokens, next_tokens, deterministic)
    dq = torch.empty_like(query)
    dk = torch.empty_like(key)
    dv = torch.empty_like(key)
    dqr = torch.empty_like(query_rope) if query_rope is not None else None
    dkr = torch.empty_like(key_rope) if key_rope is not None else None
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    st = sfag_sparse_flash_attention_grad(
        _dev(query, "query", bf), _dev(key, "key", bf), _dev(value, "value", bf),
        _dev(sparse_indices, "sparse_indices", torch.int32), _dev(d_out, "d_out", bf), _dev(out, "out", bf),
        _dev(softmax_max, "softmax_max", torch.float32), _dev(softmax_sum, "softmax_sum", torch.float32),
        sq, skv, _dev(query_rope, "query_rope", bf), _dev(key_rope, "key_rope", bf), dims, scale_value,
        sparse_block_size, layout, sparse_mode, pre_tokens, next_tokens, deterministic,
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), None if dqr is None else dqr.data_ptr(),
        None if dkr is None else dkr.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    _check(st)
    return dq, dk, dv, dqr, dkr


def sparse_flash_attention_forward(query, key, value, sparse_indices, actual_seq_lengths_query=None,
                                   actual_seq_lengths_kv=None, query_rope=None, key_rope=None, *,
                                   scale_value: float, sparse_block_size: int = 1, layout: str = "BSND",
                                   sparse_mode: int = 3, pre_tokens: int = 2 ** 31 - 1,
                                   next_tokens: int = 2 ** 31 - 1):
    """Sparse forward over the same selection; returns (out in query's element type, softmax_max
    fp32, softmax_sum fp32)."""
    import torch
    sq, skv = _seq(actual_seq_lengths_query), _seq(actual_seq_lengths_kv)
    dims = _dims_from(query, key, sparse_indices, layout, sq, skv, query_rope)
    bf = _elem_dtype(dims)
    _check_shapes(dims, layout, query=query, key=key, value=value, sparse_indices=sparse_indices,
                  query_rope=query_rope, key_rope=key_rope)
    out = torch.empty_like(query)
    if layout == "BSND":
        stat_shape = (dims.B, dims.N1, dims.S1)
    else:
        stat_shape = (dims.N1, dims.S1)
    smax = torch.empty(stat_shape, dtype=torch.float32, device=query.device)
    ssum = torch.empty(stat_shape, dtype=torch.float32, device=query.device)
    st = sfag_sparse_flash_attention_forward(
        _dev(query, "query", bf), _dev(key, "key", bf), _dev(value, "value", bf),
        _dev(sparse_indices, "sparse_indices", torch.int32), sq, skv, _dev(query_rope, "query_rope", bf),
        _dev(key_rope, "key_rope", bf), dims, scale_value, sparse_block_size, layout, sparse_mode, pre_tokens,
        next_tokens, out.data_ptr(), smax.data_ptr(), ssum.data_ptr(), _stream())
    _check(st)
    return out, smax, ssum


# ---- lightning-indexer backward with KL loss ------------------------------------------------------

def _lens64(x: Optional[Sequence[int]]):
    if x is None:
        return None, None
    arr = (ctypes.c_int64 * len(x))(*[int(v) for v in x])
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))


def sfag_lightning_indexer_grad_get_workspace_size(dims: IndexerDims, seq_len_q=None, seq_len_kv=None,
                                                   layout: str = "BSND", sparse_mode: int = 3) -> int:
    a, q = _lens64(seq_len_q)
    b, kv = _lens64(seq_len_kv)
    out = ctypes.c_uint64(0)
    _check(lib().sfag_lightning_indexer_grad_get_workspace_size(ctypes.byref(dims), q, kv, layout.encode(),
                                                                int(sparse_mode), ctypes.byref(out)))
    del a, b
    return int(out.value)


def sfag_dense_lightning_indexer_grad_kl_loss(query, key, query_index, key_index, weights, softmax_max,
                                              softmax_sum, softmax_max_index, softmax_sum_index, query_rope,
                                              key_rope, seq_len_q, seq_len_kv, dims: IndexerDims, scale_value,
                                              layout, sparse_mode, pre_tokens, next_tokens, d_query_index,
                                              d_key_index, d_weights, loss, workspace, workspace_size,
                                              stream) -> int:
    """Raw C call: every tensor argument is a device address (int) or None; returns the status."""
    a, q = _lens64(seq_len_q)
    b, kv = _lens64(seq_len_kv)
    st = lib().sfag_dense_lightning_indexer_grad_kl_loss(
        query, key, query_index, key_index, weights, softmax_max, softmax_sum, softmax_max_index,
        softmax_sum_index, query_rope, key_rope, q, kv, ctypes.byref(dims), float(scale_value), layout.encode(),
        int(sparse_mode), int(pre_tokens), int(next_tokens), d_query_index, d_key_index, d_weights, loss,
        workspace, int(workspace_size), stream)
    del a, b
    return st


def _indexer_dims(query, key, query_index, weights, layout: str, seq_len_q) -> IndexerDims:
    if layout == "BSND":
        if query.dim() != 4 or key.dim() != 4 or query_index.dim() != 4 or weights.dim() != 3:
            raise ValueError("BSND expects query [B,S1,N1,512], key [B,S2,1,512], query_index [B,S1,G,128], "
                             "weights [B,S1,G]")
        B, S1, N1, D = query.shape
        S2 = key.shape[1]
        G, Di = query_index.shape[2], query_index.shape[3]
    elif layout == "TND":
        if query.dim() != 3 or key.dim() != 3 or query_index.dim() != 3 or weights.dim() != 2:
            raise ValueError("TND expects query [T1,N1,512], key [T2,1,512], query_index [T1,G,128], weights [T1,G]")
        if seq_len_q is None:
            raise ValueError("TND needs actual_seq_lengths_query and actual_seq_lengths_kv")
        S1, N1, D = query.shape
        S2 = key.shape[0]
        B = len(seq_len_q)
        G, Di = query_index.shape[1], query_index.shape[2]
    else:
        raise ValueError(f"layout must be BSND or TND, got {layout!r}")
    return IndexerDims(int(B), int(S1), int(S2), int(N1), int(G), int(D), 64, int(Di), _dtype_code(query))


def lightning_indexer_grad_kl_loss(query, key, query_index, key_index, weights, softmax_max, softmax_sum,
                                   softmax_max_index, softmax_sum_index, actual_seq_lengths_query=None,
                                   actual_seq_lengths_kv=None, query_rope=None, key_rope=None, *,
                                   scale_value: float, layout: str = "BSND", sparse_mode: int = 3,
                                   pre_tokens: int = 2 ** 31 - 1, next_tokens: int = 2 ** 31 - 1, workspace=None):
    """Backward of the lightning indexer with its KL loss; returns (d_query_index, d_key_index,
    d_weights, loss): gradients in the inputs' element type, loss a one-element fp32 tensor."""
    import torch
    sq, skv = _seq(actual_seq_lengths_query), _seq(actual_seq_lengths_kv)
    dims = _indexer_dims(query, key, query_index, weights, layout, sq)
    B, S1, S2, N1, G = dims.B, dims.S1, dims.S2, dims.N1, dims.G
    if layout == "BSND":
        want = dict(query=(B, S1, N1, 512), key=(B, S2, 1, 512), query_index=(B, S1, G, 128),
                    key_index=(B, S2, 1, 128), weights=(B, S1, G), softmax_max=(B, N1, S1), softmax_sum=(B, N1, S1),
                    softmax_max_index=(B, S1), softmax_sum_index=(B, S1), query_rope=(B, S1, N1, 64),
                    key_rope=(B, S2, 1, 64))
    else:
        want = dict(query=(S1, N1, 512), key=(S2, 1, 512), query_index=(S1, G, 128), key_index=(S2, 1, 128),
                    weights=(S1, G), softmax_max=(N1, S1), softmax_sum=(N1, S1), softmax_max_index=(S1,),
                    softmax_sum_index=(S1,), query_rope=(S1, N1, 64), key_rope=(S2, 1, 64))
    given = dict(query=query, key=key, query_index=query_index, key_index=key_index, weights=weights,
                 softmax_max=softmax_max, softmax_sum=softmax_sum, softmax_max_index=softmax_max_index,
                 softmax_sum_index=softmax_sum_index, query_rope=query_rope, key_rope=key_rope)
    for name, t in given.items():
        if t is not None and tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]} for layout {layout}")
    el = _elem_dtype(dims)
    f32 = torch.float32
    ws = sfag_lightning_indexer_grad_get_workspace_size(dims, sq, skv, layout, sparse_mode)
    if workspace is None or workspace.numel() < ws:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    dqi = torch.empty_like(query_index)
    dki = torch.empty_like(key_index)
    dw = torch.empty_like(weights)
    loss = torch.empty(1, dtype=f32, device=query.device)
    st = sfag_dense_lightning_indexer_grad_kl_loss(
        _dev(query, "query", el), _dev(key, "key", el), _dev(query_index, "query_index", el),
        _dev(key_index, "key_index", el), _dev(weights, "weights", el), _dev(softmax_max, "softmax_max", f32),
        _dev(softmax_sum, "softmax_sum", f32), _dev(softmax_max_index, "softmax_max_index", f32),
        _dev(softmax_sum_index, "softmax_sum_index", f32), _dev(query_rope, "query_rope", el),
        _dev(key_rope, "key_rope", el), sq, skv, dims, scale_value, layout, sparse_mode, pre_tokens, next_tokens,
        dqi.data_ptr(), dki.data_ptr(), dw.data_ptr(), loss.data_ptr(), workspace.data_ptr(), workspace.numel(),
        _stream())
    _check(st)
    return dqi, dki, dw, loss
