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
    base = dict(B=1, S1=128, S2=4096, N1=8, N2=1, D=512, Drope=64, topk=1024)
    base.update(kw)
    return Dims(*[base[k] for k in ("B", "S1", "S2", "N1", "N2", "D", "Drope", "topk")])


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
                                         ("B", 0), ("B", 257), ("S1", 0), ("S2", 131073), ("topk", 0)])
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
    # the key-major path is deterministic by construction: same workspace in both modes
    assert ws(dims(), deterministic=True) == ws(dims())
    # the scatter path keeps per-pair partials and a sort buffer in deterministic mode
    monkeypatch.setenv("SFAG_FORCE_PATH", "scatter")
    assert ws(dims(), deterministic=True) > ws(dims())
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
