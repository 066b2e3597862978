"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments (SparseFlashAttentionGrad README,
"constraints") with the documented status before anything is launched."""

import ctypes
import os
import re

import pytest

import sparse_mla_flash_amd as sf
from sparse_mla_flash_amd import Dims

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sfag.h")

FAKE = 0x10000          # aligned non-NULL address; never dereferenced on the error paths tested


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfag_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(sf.EXPORTED)
    L = sf.lib()
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in sf.sfag_version()


def dims(**kw):
    base = dict(B=1, S1=128, S2=4096, N1=8, N2=1, D=512, Drope=64, topk=1024, dtype=sf.SFAG_DTYPE_BF16)
    base.update(kw)
    return Dims(*[base[k] for k in ("B", "S1", "S2", "N1", "N2", "D", "Drope", "topk", "dtype")])


def ws(d, **kw):
    args = dict(seq_len_q=None, seq_len_kv=None, scale_value=1 / 24, sparse_block_size=1, layout="BSND",
                sparse_mode=3, deterministic=False)
    args.update(kw)
    return sf.sfag_get_workspace_size(d, **args)


def status_of(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except sf.SfagError as e:
        return e.status
    return sf.SFAG_OK


@pytest.mark.parametrize("field,value", [("N2", 2), ("D", 128), ("Drope", 32), ("N1", 5), ("N1", 256),
                                         ("B", 0), ("B", 257), ("S1", 0), ("S2", 131073), ("topk", 0),
                                         ("dtype", 2), ("dtype", -1)])
def test_invalid_shapes(field, value):
    assert status_of(ws, dims(**{field: value})) == sf.SFAG_ERR_PARAM_INVALID
    assert field.lower() in sf.sfag_last_error().lower() or value is not None


def test_invalid_attributes():
    d = dims()
    assert status_of(ws, d, sparse_mode=1) == sf.SFAG_ERR_PARAM_INVALID
    assert status_of(ws, d, layout="BNSD") == sf.SFAG_ERR_PARAM_INVALID
    assert status_of(ws, d, sparse_block_size=0) == sf.SFAG_ERR_PARAM_INVALID
    assert status_of(ws, d, sparse_block_size=64) == sf.SFAG_OK           # 1024 x 64 slots
    assert status_of(ws, d, sparse_block_size=129) == sf.SFAG_ERR_PARAM_INVALID   # > 131072 slots
    assert status_of(ws, d, scale_value=float("nan")) == sf.SFAG_ERR_PARAM_INVALID
    assert status_of(ws, d, seq_len_q=[129]) == sf.SFAG_ERR_PARAM_INVALID
    assert status_of(ws, d, seq_len_kv=[-1]) == sf.SFAG_ERR_PARAM_INVALID


def test_tnd_lengths():
    d = dims(B=2, S1=30, S2=40)
    assert status_of(ws, d, layout="TND") == sf.SFAG_ERR_PARAM_NULLPTR
    assert status_of(ws, d, layout="TND", seq_len_q=[10, 20], seq_len_kv=[15, 25]) == sf.SFAG_OK
    assert status_of(ws, d, layout="TND", seq_len_q=[10, 21], seq_len_kv=[15, 25]) == sf.SFAG_ERR_PARAM_INVALID


def test_accepted_envelope_and_workspace_sizes(monkeypatch):
    for n1 in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 128):
        assert ws(dims(N1=n1)) > 0
    small = ws(dims(S2=1000))
    assert small >= 1000 * 1088 * 4
    # both dK / dV paths are deterministic by construction: same workspace in both modes
    assert ws(dims(), deterministic=True) == ws(dims())
    # the per-pair path keeps the fp32 accumulator of every key row plus the fp32 partials of a
    # chunk of query rows (here all 128 rows fit one chunk)
    monkeypatch.setenv("SFAG_FORCE_PATH", "scatter")
    d = dims()
    assert ws(d, deterministic=True) == ws(d)
    assert ws(d) >= d.S2 * 1088 * 4 + d.S1 * d.topk * 1088 * 4
    monkeypatch.delenv("SFAG_FORCE_PATH")
    # pre/next tokens are accepted and ignored
    assert sf.sfag_get_workspace_size(dims(), None, None, 0.1, 1, "BSND", 0, -5, 7, False) == ws(dims(), sparse_mode=0)


def test_null_out_pointer_for_workspace_size():
    L = sf.lib()
    d = dims()
    st = L.sfag_get_workspace_size(ctypes.byref(d), None, None, 0.1, 1, b"BSND", 3, 0, 0, 0, None)
    assert st == sf.SFAG_ERR_PARAM_NULLPTR
    st = L.sfag_get_workspace_size(None, None, None, 0.1, 1, b"BSND", 3, 0, 0, 0, ctypes.byref(ctypes.c_uint64()))
    assert st == sf.SFAG_ERR_PARAM_NULLPTR


def grad_call(d, **over):
    args = dict(query=FAKE, key=FAKE, value=FAKE, sparse_indices=FAKE, d_out=FAKE, out=FAKE,
                softmax_max=FAKE, softmax_sum=FAKE, seq_len_q=None, seq_len_kv=None, query_rope=FAKE,
                key_rope=FAKE, dims=d, scale_value=1 / 24, sparse_block_size=1, layout="BSND", sparse_mode=3,
                pre_tokens=0, next_tokens=0, deterministic=False, d_query=FAKE, d_key=FAKE, d_value=FAKE,
                d_query_rope=FAKE, d_key_rope=FAKE, workspace=FAKE, workspace_size=0, stream=None)
    args.update(over)
    return sf.sfag_sparse_flash_attention_grad(**args)


@pytest.mark.parametrize("name", ["query", "key", "value", "sparse_indices", "d_out", "out", "softmax_max",
                                  "softmax_sum", "d_query", "d_key", "d_value"])
def test_grad_null_pointers(name):
    assert grad_call(dims(), **{name: None}) == sf.SFAG_ERR_PARAM_NULLPTR
    assert name in sf.sfag_last_error()


def test_grad_misaligned_and_rope_and_workspace():
    d = dims()
    assert grad_call(d, query=FAKE + 2) == sf.SFAG_ERR_PARAM_INVALID
    # rope inputs: both or neither; with them both rope gradients are required
    assert grad_call(d, query_rope=None) == sf.SFAG_ERR_PARAM_NULLPTR
    assert grad_call(d, d_key_rope=None) == sf.SFAG_ERR_PARAM_NULLPTR
    need = ws(d)
    assert grad_call(d, workspace_size=need - 1) == sf.SFAG_ERR_WORKSPACE
    assert grad_call(d, workspace=None, workspace_size=need) == sf.SFAG_ERR_WORKSPACE
    assert grad_call(d, workspace=FAKE + 16, workspace_size=need) == sf.SFAG_ERR_WORKSPACE
    assert grad_call(dims(N1=7), workspace_size=need) == sf.SFAG_ERR_PARAM_INVALID


def test_forward_validation():
    d = dims()
    f = sf.sfag_sparse_flash_attention_forward
    base = dict(query=FAKE, key=FAKE, value=FAKE, sparse_indices=FAKE, seq_len_q=None, seq_len_kv=None,
                query_rope=FAKE, key_rope=FAKE, dims=d, scale_value=0.1, sparse_block_size=1, layout="BSND",
                sparse_mode=3, pre_tokens=0, next_tokens=0, out=FAKE, softmax_max=FAKE, softmax_sum=FAKE,
                stream=None)
    assert f(**{**base, "out": None}) == sf.SFAG_ERR_PARAM_NULLPTR
    assert f(**{**base, "key_rope": None}) == sf.SFAG_ERR_PARAM_NULLPTR
    assert f(**{**base, "sparse_mode": 2}) == sf.SFAG_ERR_PARAM_INVALID
    assert f(**{**base, "dims": dims(D=256)}) == sf.SFAG_ERR_PARAM_INVALID


def test_error_string_clears_on_success():
    status_of(ws, dims(N2=3))
    assert sf.sfag_last_error() != ""
    ws(dims())
    assert sf.sfag_last_error() == ""


def _cpu_call_tensors(layout="BSND"):
    """Correctly shaped CPU tensors of a tiny problem (shapes only matter here)."""
    import torch
    bf = torch.bfloat16
    if layout == "BSND":
        B, S1, S2, N1, topk = 2, 5, 7, 4, 3
        t = dict(query=torch.zeros(B, S1, N1, 512, dtype=bf), key=torch.zeros(B, S2, 1, 512, dtype=bf),
                 value=torch.zeros(B, S2, 1, 512, dtype=bf), sparse_indices=torch.zeros(B, S1, 1, topk, dtype=torch.int32),
                 d_out=torch.zeros(B, S1, N1, 512, dtype=bf), out=torch.zeros(B, S1, N1, 512, dtype=bf),
                 softmax_max=torch.zeros(B, N1, S1), softmax_sum=torch.zeros(B, N1, S1),
                 query_rope=torch.zeros(B, S1, N1, 64, dtype=bf), key_rope=torch.zeros(B, S2, 1, 64, dtype=bf))
        return t, None, None
    T1, T2, N1, topk = 9, 11, 4, 3
    t = dict(query=torch.zeros(T1, N1, 512, dtype=bf), key=torch.zeros(T2, 1, 512, dtype=bf),
             value=torch.zeros(T2, 1, 512, dtype=bf), sparse_indices=torch.zeros(T1, 1, topk, dtype=torch.int32),
             d_out=torch.zeros(T1, N1, 512, dtype=bf), out=torch.zeros(T1, N1, 512, dtype=bf),
             softmax_max=torch.zeros(N1, T1), softmax_sum=torch.zeros(N1, T1),
             query_rope=torch.zeros(T1, N1, 64, dtype=bf), key_rope=torch.zeros(T2, 1, 64, dtype=bf))
    return t, [4, 5], [5, 6]


@pytest.mark.parametrize("layout", ["BSND", "TND"])
@pytest.mark.parametrize("name,cut", [("d_out", 1), ("out", 1), ("softmax_max", 0), ("softmax_sum", -1),
                                      ("query_rope", -1), ("key_rope", 0), ("value", 0), ("key_rope", -1)])
def test_wrapper_rejects_misshaped_tensors(layout, name, cut):
    """The tensor wrapper checks every tensor against the shapes implied by query, key and
    sparse_indices before anything is allocated or launched."""
    import torch
    t, sq, skv = _cpu_call_tensors(layout)
    shape = list(t[name].shape)
    shape[cut] += 1
    t[name] = torch.zeros(shape, dtype=t[name].dtype)
    with pytest.raises(ValueError, match=name):
        sf.sparse_flash_attention_grad(
            t["query"], t["key"], t["value"], t["sparse_indices"], t["d_out"], t["out"], t["softmax_max"],
            t["softmax_sum"], sq, skv, t["query_rope"], t["key_rope"], scale_value=1 / 24, layout=layout)


def test_wrapper_rejects_half_rope_and_accepts_good_shapes():
    import torch
    t, sq, skv = _cpu_call_tensors("BSND")
    with pytest.raises(ValueError, match="rope"):
        sf.sparse_flash_attention_grad(
            t["query"], t["key"], t["value"], t["sparse_indices"], t["d_out"], t["out"], t["softmax_max"],
            t["softmax_sum"], sq, skv, t["query_rope"], None, scale_value=1 / 24)
    # correct shapes pass the shape checks and stop only at the device check (CPU tensors)
    with pytest.raises(ValueError, match="GPU tensor"):
        sf.sparse_flash_attention_grad(
            t["query"], t["key"], t["value"], t["sparse_indices"], t["d_out"], t["out"], t["softmax_max"],
            t["softmax_sum"], sq, skv, t["query_rope"], t["key_rope"], scale_value=1 / 24)


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The no-allocation entry point refuses a problem whose workspace exceeds its built-in
    scratch, before any device call (the pointers below are never dereferenced)."""
    d = dims(S1=8192, S2=8192, N1=64, topk=2048)
    need = ws(d)
    assert need > sf.NOALLOC_SCRATCH_BYTES
    st = sf.sfag_sparse_flash_attention_grad_noalloc(
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, d, 1 / 24, 1, "BSND", 3,
        2 ** 31 - 1, 2 ** 31 - 1, False, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == sf.SFAG_ERR_WORKSPACE
    assert "scratch" in sf.sfag_last_error()
    st = sf.sfag_sparse_flash_attention_grad_noalloc(
        None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, dims(), 1 / 24, 1, "BSND", 3,
        2 ** 31 - 1, 2 ** 31 - 1, False, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == sf.SFAG_ERR_PARAM_NULLPTR


def test_fp16_dims_accepted_and_sized_like_bf16():
    """Both element types of the page's dtype column are accepted; the workspace does not depend
    on the element type (records and copies are 16-bit either way)."""
    for kw in (dict(), dict(S1=8192, S2=8192, N1=64, topk=2048), dict(S1=4096, S2=131072, N1=128, topk=2048)):
        assert ws(dims(dtype=sf.SFAG_DTYPE_FP16, **kw)) == ws(dims(**kw))


def test_wrapper_takes_the_element_type_from_query():
    import torch
    q = torch.zeros(1, 4, 8, 512, dtype=torch.float16)
    k = torch.zeros(1, 16, 1, 512, dtype=torch.float16)
    idx = torch.zeros(1, 4, 1, 8, dtype=torch.int32)
    assert sf._dims_from(q, k, idx, "BSND", None, None).dtype == sf.SFAG_DTYPE_FP16
    assert sf._dims_from(q.bfloat16(), k.bfloat16(), idx, "BSND", None, None).dtype == sf.SFAG_DTYPE_BF16
    with pytest.raises(ValueError):
        sf._dims_from(q.float(), k.float(), idx, "BSND", None, None)


def ix_dims(**kw):
    base = dict(B=1, S1=256, S2=256, N1=64, G=64, D=512, Drope=64, Di=128, dtype=sf.SFAG_DTYPE_BF16)
    base.update(kw)
    return sf.IndexerDims(*[base[k] for k in ("B", "S1", "S2", "N1", "G", "D", "Drope", "Di", "dtype")])


@pytest.mark.parametrize("field,value", [("G", 0), ("G", 65), ("Di", 64), ("N1", 0), ("N1", 129), ("D", 256),
                                         ("Drope", 0), ("B", 257), ("S2", 0), ("S1", 131073), ("dtype", 2)])
def test_indexer_invalid_shapes(field, value):
    assert status_of(sf.sfag_lightning_indexer_grad_get_workspace_size, ix_dims(**{field: value})) == \
        sf.SFAG_ERR_PARAM_INVALID


def test_indexer_workspace_and_attributes():
    ws = sf.sfag_lightning_indexer_grad_get_workspace_size(ix_dims())
    # the head sums of every (row, key) in fp32 are the largest part
    assert ws >= 256 * 256 * 4
    assert sf.sfag_lightning_indexer_grad_get_workspace_size(ix_dims(dtype=sf.SFAG_DTYPE_FP16)) == ws
    assert status_of(sf.sfag_lightning_indexer_grad_get_workspace_size, ix_dims(), layout="BNSD") == \
        sf.SFAG_ERR_PARAM_INVALID
    assert status_of(sf.sfag_lightning_indexer_grad_get_workspace_size, ix_dims(), sparse_mode=2) == \
        sf.SFAG_ERR_PARAM_INVALID
    # TND: lengths must sum to the token counts
    d = ix_dims(B=2, S1=10, S2=12)
    assert sf.sfag_lightning_indexer_grad_get_workspace_size(d, [4, 6], [5, 7], layout="TND") > 0
    assert status_of(sf.sfag_lightning_indexer_grad_get_workspace_size, d, [4, 5], [5, 7], layout="TND") == \
        sf.SFAG_ERR_PARAM_INVALID
    assert status_of(sf.sfag_lightning_indexer_grad_get_workspace_size, d, None, None, layout="TND") == \
        sf.SFAG_ERR_PARAM_NULLPTR


def test_indexer_null_pointers_are_rejected_before_launch():
    d = ix_dims()
    args = dict(query=16, key=16, query_index=16, key_index=16, weights=16, softmax_max=16, softmax_sum=16,
                softmax_max_index=16, softmax_sum_index=16, query_rope=None, key_rope=None, seq_len_q=None,
                seq_len_kv=None, dims=d, scale_value=1 / 24, layout="BSND", sparse_mode=3, pre_tokens=0,
                next_tokens=0, d_query_index=16, d_key_index=16, d_weights=16, loss=16, workspace=None,
                workspace_size=0, stream=None)
    for name in ("query", "key_index", "weights", "softmax_sum_index", "d_weights", "loss"):
        a = dict(args)
        a[name] = None
        assert sf.sfag_dense_lightning_indexer_grad_kl_loss(**a) == sf.SFAG_ERR_PARAM_NULLPTR, name
    a = dict(args)
    a["query_rope"] = 16                          # key_rope missing
    assert sf.sfag_dense_lightning_indexer_grad_kl_loss(**a) == sf.SFAG_ERR_PARAM_INVALID
    assert sf.sfag_dense_lightning_indexer_grad_kl_loss(**args) == sf.SFAG_ERR_WORKSPACE
