"""GPU backward / forward vs the fp64 oracle on the same seeded inputs.

Every output tensor must satisfy max abs error <= 2e-2 and relative L2 error
<= 5e-3 against the oracle evaluated on the operator's own inputs (bf16 out,
fp32 statistics).  Sizes are small enough for the oracle to finish in seconds
while spanning several 32-key chunks, several 16-head tiles and a ragged tail;
edge cases cover padding, empty rows, invalid / duplicate indices, varlen TND
with an empty sequence, S1 > S2 under the causal mode, every head-group
shape the kernels special-case (N1 < 16, N1 not a multiple of 16, N1 = 128),
B = 256, block selection (sparseBlockSize 4, 16, 64) and fp16 tensors.
"""

import numpy as np
import pytest

from sparse_mla_flash_amd import inputs
from tests.common import Case, compare, from_dev

pytestmark = pytest.mark.gpu

CASES = {
    # name: (problem kwargs, index kind, seed)
    "bsnd_n8_causal_tail": (dict(layout="BSND", B=1, S1=40, S2=600, N1=8, topk=100, sparse_mode=3), "uniform", 1),
    "bsnd_n64_short_prefix": (dict(layout="BSND", B=1, S1=150, S2=150, N1=64, topk=64, sparse_mode=3), "uniform", 2),
    "bsnd_n128_nomask": (dict(layout="BSND", B=1, S1=24, S2=300, N1=128, topk=72, sparse_mode=0), "uniform", 3),
    "bsnd_n48_padded_batches": (dict(layout="BSND", B=2, S1=40, S2=90, N1=48, topk=40, sparse_mode=3,
                                     seq_q=[40, 17], seq_kv=[90, 31]), "uniform", 4),
    "bsnd_n3": (dict(layout="BSND", B=1, S1=20, S2=100, N1=3, topk=33, sparse_mode=0), "uniform", 5),
    "bsnd_n12_s1_gt_s2": (dict(layout="BSND", B=1, S1=70, S2=50, N1=12, topk=48, sparse_mode=3), "uniform", 6),
    "tnd_n16_varlen_empty_seq": (dict(layout="TND", B=4, seq_q=[37, 0, 70, 5], seq_kv=[50, 3, 70, 9], N1=16,
                                      topk=48, sparse_mode=3), "uniform", 7),
    "tnd_n128_varlen": (dict(layout="TND", B=3, seq_q=[20, 33, 9], seq_kv=[64, 33, 40], N1=128, topk=40,
                             sparse_mode=3), "uniform", 8),
    "bsnd_n64_window": (dict(layout="BSND", B=1, S1=48, S2=2048, N1=64, topk=64, sparse_mode=3), "window", 9),
    "bsnd_n48_hotcold_nomask": (dict(layout="BSND", B=2, S1=16, S2=400, N1=48, topk=96, sparse_mode=0),
                                "hot_cold", 10),
    # the rest of the head counts the constraints list (6, 24) and the largest batch count (256)
    "bsnd_n6_causal": (dict(layout="BSND", B=1, S1=30, S2=200, N1=6, topk=40, sparse_mode=3), "uniform", 11),
    "bsnd_n24_nomask": (dict(layout="BSND", B=1, S1=20, S2=150, N1=24, topk=50, sparse_mode=0), "uniform", 12),
    "bsnd_b256_n4": (dict(layout="BSND", B=256, S1=2, S2=24, N1=4, topk=8, sparse_mode=3), "uniform", 13),
    "tnd_b256_n2_varlen": (dict(layout="TND", B=256, seq_q=[(7 * b) % 5 for b in range(256)],
                                seq_kv=[1 + (11 * b) % 23 for b in range(256)], N1=2, topk=8, sparse_mode=3),
                           "uniform", 14),
    # the index sort's 16384-key windows (rows reaching past 8192 keys): one window, then two
    "bsnd_n8_sort_window_9k": (dict(layout="BSND", B=1, S1=12, S2=9000, N1=8, topk=200, sparse_mode=3), "uniform", 15),
    "bsnd_n8_sort_windows_20k": (dict(layout="BSND", B=1, S1=12, S2=20000, N1=8, topk=300, sparse_mode=3),
                                 "uniform", 16),
}


def make(name):
    kw, kind, seed = CASES[name]
    p = inputs.problem(**kw, name=name)
    inputs.generate(p, seed, index_kind=kind, window=256)
    return p


def check_all(case: Case, outs, label=""):
    dq, dk, dv, dqr, dkr = (from_dev(t) for t in outs)
    rdq, rdqr = case.ref_dq()
    rdk, rdkr, rdv = case.ref_dkv()
    res = {}
    res["dq"] = compare(label + "dq", dq, rdq)
    res["dq_rope"] = compare(label + "dq_rope", dqr, rdqr)
    res["dk"] = compare(label + "dk", dk, rdk)
    res["dk_rope"] = compare(label + "dk_rope", dkr, rdkr)
    res["dv"] = compare(label + "dv", dv, rdv)
    return res


@pytest.fixture(params=["dense", "scatter"])
def path(request, monkeypatch):
    """dK / dV path: key-major dense-masked kernels, or the per-pair partials path."""
    monkeypatch.setenv("SFAG_FORCE_PATH", request.param)
    return request.param


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("deterministic", [False, True])
def test_backward_matches_oracle(name, deterministic, path):
    case = Case(make(name))
    outs = case.run_gpu(deterministic=deterministic)
    res = check_all(case, outs, f"{name}/{path}/det={int(deterministic)}/")
    print(name, path, deterministic, {k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in res.items()})


def test_invalid_and_duplicate_indices(path):
    """Negative, out-of-range and causally masked indices are skipped; duplicates add."""
    p = inputs.problem("BSND", B=1, S1=33, S2=80, N1=16, topk=50, sparse_mode=3)
    inputs.generate(p, 21)
    r = np.random.default_rng(5)
    idx = r.integers(-3, 90, size=(33, 50)).astype(np.int32)
    idx[:, 1] = idx[:, 0]                              # duplicated slot in every row
    p.idx = idx.reshape(p.idx_shape())
    case = Case(p)
    check_all(case, case.run_gpu(), "messy/")
    check_all(case, case.run_gpu(deterministic=True), "messy-det/")


def test_all_slots_invalid_gives_zeros(path):
    p = inputs.problem("BSND", B=1, S1=8, S2=16, N1=8, topk=40, sparse_mode=3)
    inputs.generate(p, 22)
    p.idx = np.full(p.idx_shape(), -1, np.int32)
    case = Case(p)
    for det in (False, True):
        for t in case.run_gpu(deterministic=det):
            assert not from_dev(t).any()


def test_slot_permutation_invariance(path):
    p = make("bsnd_n64_short_prefix")
    case = Case(p)
    a = [from_dev(t) for t in case.run_gpu()]
    perm = np.stack([np.random.default_rng(i).permutation(p.topk) for i in range(p.rows)])
    p.idx = np.take_along_axis(p.idx.reshape(p.rows, p.topk), perm, axis=1).reshape(p.idx_shape())
    case2 = Case(p)
    b = [from_dev(t) for t in case2.run_gpu()]
    for x, y in zip(a, b):
        # only the order of fp32 accumulation changes: a few bf16 rounding flips, each at most
        # one ulp (2^-7 relative) of the element's own magnitude
        assert (np.abs(x - y) <= 2e-2 + 2.0 ** -7 * np.abs(x)).all()


@pytest.mark.parametrize("name", ["bsnd_n64_short_prefix", "tnd_n16_varlen_empty_seq", "bsnd_n128_nomask",
                                  "bsnd_n3"])
def test_forward_matches_oracle(name):
    import sparse_mla_flash_amd as sf
    p = make(name)
    case = Case(p)
    d = case.device_inputs()
    out, smax, ssum = sf.sparse_flash_attention_forward(
        d["query"], d["key"], d["value"], d["sparse_indices"], p.seq_q, p.seq_kv, d["query_rope"],
        d["key_rope"], scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)
    compare(name + "/out", from_dev(out), case.out64)
    m, l = from_dev(smax), from_dev(ssum)
    assert np.abs(m - case.m64).max() <= 1e-4 * max(1.0, np.abs(case.m64).max())
    assert np.abs(l - case.l64).max() <= 1e-4 * max(1.0, np.abs(case.l64).max())


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_forward_max_rising_far_after_the_first_chunk(dtype):
    """One key, selected by row r only after its first 32 slots, is a multiple of r's head-0 query:
    that head's logit for it lies about 100 nats above everything in the row's first chunk.  The
    forward's reference max comes from the first chunk, so its probabilities would overflow
    (exp of about 144 in log2 units) unless the row is recomputed against the true max."""
    import sparse_mla_flash_amd as sf
    p = inputs.problem(layout="BSND", B=1, S1=16, S2=256, N1=16, topk=128, sparse_mode=0,
                       name=f"rising_max_{dtype}", dtype=dtype)
    inputs.generate(p, 41)
    idx = p.idx.reshape(p.rows, p.topk)
    r = 5
    first = set(int(j) for j in idx[r, :32])
    j = next(int(x) for x in idx[r, 40:] if x >= 0 and int(x) not in first)
    qh = inputs.bits_to_f64(p.q, dtype).reshape(p.rows, p.N1, p.D)[r, 0]
    factor = 100.0 / (p.scale * float(qh @ qh))
    k = p.k.reshape(p.S2, p.D)
    k[j] = inputs.f32_to_bits((factor * qh).astype(np.float32), dtype)
    p.v = p.k.copy()
    case = Case(p)
    assert case.m64.max() > 90.0                  # the planted logit is the row's maximum
    d = case.device_inputs()
    out, smax, ssum = sf.sparse_flash_attention_forward(
        d["query"], d["key"], d["value"], d["sparse_indices"], p.seq_q, p.seq_kv, d["query_rope"],
        d["key_rope"], scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)
    u = 2.0 ** -11 if dtype == "fp16" else 2.0 ** -8
    got = from_dev(out)
    assert np.isfinite(got).all()
    compare(p.name + "/out", got, case.out64, u=u)
    m, l = from_dev(smax), from_dev(ssum)
    assert np.abs(m - case.m64).max() <= 1e-4 * max(1.0, np.abs(case.m64).max())
    assert np.abs(l - case.l64).max() <= 1e-4 * max(1.0, np.abs(case.l64).max())


BLOCK_CASES = {
    # name: (problem kwargs, seed); block selection, the last block cut by the key length
    "bsnd_n16_block4_causal": (dict(layout="BSND", B=1, S1=40, S2=301, N1=16, topk=20, sparse_mode=3,
                                    block=4), 31),
    "tnd_n64_block16_varlen": (dict(layout="TND", B=2, seq_q=[30, 17], seq_kv=[200, 95], N1=64, topk=6,
                                    sparse_mode=3, block=16), 32),
    "bsnd_n8_block64_nomask": (dict(layout="BSND", B=1, S1=12, S2=700, N1=8, topk=5, sparse_mode=0,
                                    block=64), 33),
}


def make_block(name):
    kw, seed = BLOCK_CASES[name]
    p = inputs.problem(**kw, name=name)
    inputs.generate(p, seed)
    return p


@pytest.mark.parametrize("name", sorted(BLOCK_CASES))
@pytest.mark.parametrize("deterministic", [False, True])
def test_block_selection_matches_oracle(name, deterministic, path):
    """sparseBlockSize > 1: every index names a block of consecutive keys."""
    case = Case(make_block(name))
    outs = case.run_gpu(deterministic=deterministic)
    res = check_all(case, outs, f"{name}/{path}/det={int(deterministic)}/")
    print(name, path, deterministic, {k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in res.items()})


@pytest.mark.parametrize("name", sorted(BLOCK_CASES))
def test_block_selection_forward_matches_oracle(name):
    import sparse_mla_flash_amd as sf
    p = make_block(name)
    case = Case(p)
    d = case.device_inputs()
    out, smax, ssum = sf.sparse_flash_attention_forward(
        d["query"], d["key"], d["value"], d["sparse_indices"], p.seq_q, p.seq_kv, d["query_rope"],
        d["key_rope"], scale_value=p.scale, sparse_block_size=p.block, layout=p.layout,
        sparse_mode=p.sparse_mode)
    compare(name + "/out", from_dev(out), case.out64)
    m, l = from_dev(smax), from_dev(ssum)
    assert np.abs(m - case.m64).max() <= 1e-4 * max(1.0, np.abs(case.m64).max())
    assert np.abs(l - case.l64).max() <= 1e-4 * max(1.0, np.abs(case.l64).max())


@pytest.mark.parametrize("name", ["bsnd_n64_short_prefix", "tnd_n16_varlen_empty_seq"])
def test_ropeless_matches_oracle(name, path):
    """No rope inputs (queryRopeOptional / keyRopeOptional absent): the oracle with zero rope
    tensors is the reference; no rope gradients are returned."""
    import sparse_mla_flash_amd as sf
    case = Case(make(name), rope=False)
    p = case.p
    d = case.device_inputs()
    for det in (False, True):
        dq, dk, dv, dqr, dkr = sf.sparse_flash_attention_grad(
            d["query"], d["key"], d["value"], d["sparse_indices"], d["d_out"], d["out"], d["softmax_max"],
            d["softmax_sum"], p.seq_q, p.seq_kv, None, None, scale_value=p.scale, layout=p.layout,
            sparse_mode=p.sparse_mode, deterministic=det)
        assert dqr is None and dkr is None
        rdq, _ = case.ref_dq()
        rdk, _, rdv = case.ref_dkv()
        compare(f"{name}/ropeless/{path}/dq", from_dev(dq), rdq)
        compare(f"{name}/ropeless/{path}/dk", from_dev(dk), rdk)
        compare(f"{name}/ropeless/{path}/dv", from_dev(dv), rdv)
    out, smax, ssum = sf.sparse_flash_attention_forward(
        d["query"], d["key"], d["value"], d["sparse_indices"], p.seq_q, p.seq_kv, None, None,
        scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)
    compare(name + "/ropeless/out", from_dev(out), case.out64)
    m = from_dev(smax)
    assert np.abs(m - case.m64).max() <= 1e-4 * max(1.0, np.abs(case.m64).max())


def test_heavy_duplicates(path):
    """Rows repeating a few keys many times: more than 256 positions fall in one 256-key block
    and keys repeat dozens of times; every repeat contributes separately."""
    p = inputs.problem("BSND", B=1, S1=24, S2=64, N1=16, topk=300, sparse_mode=0)
    inputs.generate(p, 23)
    r = np.random.default_rng(6)
    p.idx = r.integers(0, 10, size=p.idx_shape()).astype(np.int32)
    case = Case(p)
    check_all(case, case.run_gpu(), "dups/")


FP16_CASES = ["bsnd_n8_causal_tail", "bsnd_n64_short_prefix", "bsnd_n128_nomask", "bsnd_n48_padded_batches",
              "tnd_n16_varlen_empty_seq", "bsnd_n64_window", "bsnd_n6_causal"]


def make_fp16(name):
    kw, kind, seed = CASES[name]
    p = inputs.problem(**kw, name=name, dtype="fp16")
    inputs.generate(p, seed, index_kind=kind, window=256)
    return p


@pytest.mark.parametrize("name", FP16_CASES)
def test_fp16_backward_matches_oracle(name, path):
    """fp16 tensors (the page's second dtype) on both dK / dV paths.  fp16 carries 11 significant
    bits against bf16's 8, so the bound uses fp16's unit roundoff and rel-L2 <= 1e-3: a path that
    rounded its MFMA operands to bf16 would miss it (about 3e-3 here)."""
    import torch
    case = Case(make_fp16(name))
    outs = case.run_gpu()
    assert all(t.dtype == torch.float16 for t in outs if t is not None)
    dq, dk, dv, dqr, dkr = (from_dev(t) for t in outs)
    rdq, rdqr = case.ref_dq()
    rdk, rdkr, rdv = case.ref_dkv()
    u = 2.0 ** -11
    res = {}
    for nm, got, ref in (("dq", dq, rdq), ("dq_rope", dqr, rdqr), ("dk", dk, rdk), ("dk_rope", dkr, rdkr),
                         ("dv", dv, rdv)):
        res[nm] = compare(f"{name}/{path}/fp16/{nm}", got, ref, rel_l2=1e-3, u=u)
    print(name, path, "fp16", {k: f"{v[0]:.2e}/{v[1]:.2e}" for k, v in res.items()})


@pytest.mark.parametrize("name", ["bsnd_n64_short_prefix", "tnd_n16_varlen_empty_seq"])
def test_fp16_forward_matches_oracle(name):
    import sparse_mla_flash_amd as sf
    import torch
    p = make_fp16(name)
    case = Case(p)
    d = case.device_inputs()
    out, smax, ssum = sf.sparse_flash_attention_forward(
        d["query"], d["key"], d["value"], d["sparse_indices"], p.seq_q, p.seq_kv, d["query_rope"],
        d["key_rope"], scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)
    assert out.dtype == torch.float16
    compare(name + "/fp16/out", from_dev(out), case.out64, rel_l2=1e-3, u=2.0 ** -11)
    m, l = from_dev(smax), from_dev(ssum)
    assert np.abs(m - case.m64).max() <= 1e-4 * max(1.0, np.abs(case.m64).max())
    assert np.abs(l - case.l64).max() <= 1e-4 * max(1.0, np.abs(case.l64).max())


def test_fp16_and_bf16_calls_agree_on_the_same_values():
    """Inputs that both types hold exactly (bf16 values inside fp16's range) give the same
    gradients up to the output rounding of each type, so neither path reads the other's bits."""
    import torch
    name = "bsnd_n64_short_prefix"
    case = Case(make(name))
    d16 = {k: (v.to(torch.float16) if v is not None and v.dtype == torch.bfloat16 else v)
           for k, v in case.device_inputs().items()}
    a = case.run_gpu()
    b = case.run_gpu(dev=d16)
    assert b[0].dtype == torch.float16
    for nm, x, y in zip(("dq", "dk", "dv", "dq_rope", "dk_rope"), a, b):
        compare(f"{name}/bf16-vs-fp16/{nm}", from_dev(y), from_dev(x))      # the bf16 bar
