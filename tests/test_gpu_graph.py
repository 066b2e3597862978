"""Backward calls captured in a HIP graph and replayed.

The library enqueues only kernel launches on the caller's stream (no allocation, memset, copy or
synchronisation inside a call), so a call can be captured.  Each case: one eager call (the
reference), the same call captured with torch.cuda.graph, then several replays with eager work
and synchronisations between them (the outputs are overwritten with NaN before every replay).
Every replay must reproduce the eager outputs bit for bit: both dK / dV paths sum in a fixed
order.  The no-allocation entry point is captured as well, since graph capture is one of the
settings it serves."""

import pytest

from sparse_mla_flash_amd import inputs
from tests.common import Case

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dq_rope", "dk_rope")


def _call(sf, p, d, dims, outs, ws, noalloc):
    import torch
    args = (d["query"].data_ptr(), d["key"].data_ptr(), d["value"].data_ptr(), d["sparse_indices"].data_ptr(),
            d["d_out"].data_ptr(), d["out"].data_ptr(), d["softmax_max"].data_ptr(), d["softmax_sum"].data_ptr(),
            p.seq_q, p.seq_kv, d["query_rope"].data_ptr(), d["key_rope"].data_ptr(), dims, p.scale, p.block,
            p.layout, p.sparse_mode, 2 ** 31 - 1, 2 ** 31 - 1, False, *(t.data_ptr() for t in outs))
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        return sf.sfag_sparse_flash_attention_grad_noalloc(*args, stream)
    return sf.sfag_sparse_flash_attention_grad(*args, ws.data_ptr(), ws.numel(), stream)


@pytest.mark.parametrize("path,noalloc", [("dense", False), ("scatter", False), ("dense", True)])
def test_graph_replays_match_eager_call(path, noalloc, monkeypatch):
    import torch
    import sparse_mla_flash_amd as sf
    monkeypatch.setenv("SFAG_FORCE_PATH", path)
    p = inputs.problem("BSND", B=1, S1=150, S2=700, N1=64, topk=96, sparse_mode=3, name="graph")
    inputs.generate(p, 61)
    case = Case(p)
    d = case.device_inputs()
    dims = sf._dims_from(d["query"], d["key"], d["sparse_indices"], p.layout, p.seq_q, p.seq_kv)
    ws_bytes = sf.sfag_get_workspace_size(dims, p.seq_q, p.seq_kv, p.scale, p.block, p.layout, p.sparse_mode,
                                          2 ** 31 - 1, 2 ** 31 - 1, False)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(d["query"]), torch.empty_like(d["key"]), torch.empty_like(d["key"]),
            torch.empty_like(d["query_rope"]), torch.empty_like(d["key_rope"])]
    print(f"graph case path={path} noalloc={noalloc}: eager call", flush=True)
    st = _call(sf, p, d, dims, outs, ws, noalloc)
    assert st == sf.SFAG_OK, sf.sfag_last_error()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _call(sf, p, d, dims, outs, ws, noalloc)
    assert st == sf.SFAG_OK, sf.sfag_last_error()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"graph case path={path} noalloc={noalloc}: replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(NAMES, outs, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{path}/noalloc={noalloc}/replay {rep}/{name}"
