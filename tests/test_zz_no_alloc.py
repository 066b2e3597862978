"""The no-allocation entry point (sfag_sparse_flash_attention_grad_noalloc) against the
workspace entry point, through the C ABI: two calls in a row on the same GPU, the second with a
smaller problem (the scratch keeps the first call's contents), on both dK / dV paths, both
values of the deterministic flag: bit-identical to the workspace entry point, and within the
parity bar of the oracle."""

import numpy as np
import pytest

from sparse_mla_flash_amd import inputs
from tests.common import Case, compare, from_dev

pytestmark = pytest.mark.gpu


def _noalloc(case: Case, det: bool):
    import torch
    import sparse_mla_flash_amd as sf
    p = case.p
    d = case.device_inputs()
    dims = sf._dims_from(d["query"], d["key"], d["sparse_indices"], p.layout, p.seq_q, p.seq_kv)
    outs = [torch.full_like(d["query"], float("nan")), torch.full_like(d["key"], float("nan")),
            torch.full_like(d["key"], float("nan")), torch.full_like(d["query_rope"], float("nan")),
            torch.full_like(d["key_rope"], float("nan"))]
    st = sf.sfag_sparse_flash_attention_grad_noalloc(
        d["query"].data_ptr(), d["key"].data_ptr(), d["value"].data_ptr(), d["sparse_indices"].data_ptr(),
        d["d_out"].data_ptr(), d["out"].data_ptr(), d["softmax_max"].data_ptr(), d["softmax_sum"].data_ptr(),
        p.seq_q, p.seq_kv, d["query_rope"].data_ptr(), d["key_rope"].data_ptr(), dims, p.scale, p.block, p.layout,
        p.sparse_mode, 2 ** 31 - 1, 2 ** 31 - 1, det, *(t.data_ptr() for t in outs),
        torch.cuda.current_stream().cuda_stream)
    assert st == sf.SFAG_OK, sf.sfag_last_error()
    torch.cuda.synchronize()
    return outs, d


@pytest.mark.parametrize("path,det", [("dense", False), ("scatter", True), ("scatter", False)])
def test_noalloc_matches_workspace_entry_point(path, det, monkeypatch):
    import torch
    monkeypatch.setenv("SFAG_FORCE_PATH", path)
    big = inputs.problem("BSND", B=1, S1=150, S2=700, N1=64, topk=96, sparse_mode=3, name="noalloc_a")
    inputs.generate(big, 41)
    small = inputs.problem("TND", B=2, seq_q=[20, 13], seq_kv=[40, 30], N1=8, topk=24, sparse_mode=3,
                           name="noalloc_b")
    inputs.generate(small, 42)
    for p in (big, small):                       # second call: smaller problem, same scratch
        case = Case(p)
        got, dev = _noalloc(case, det)
        ref = case.run_gpu(deterministic=det, dev=dev)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dq_rope", "dk_rope"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{p.name}/{path}/det={det}/{name}"
        # and against the oracle
        rdq, rdqr = case.ref_dq()
        rdk, rdkr, rdv = case.ref_dkv()
        for name, a, r in zip(("dq", "dk", "dv", "dq_rope", "dk_rope"), got, (rdq, rdk, rdv, rdqr, rdkr)):
            compare(f"{p.name}/{path}/oracle/{name}", from_dev(a), r)
