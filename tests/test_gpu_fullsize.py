"""Full-size workloads, run in the launch configuration the benchmark times.

* The small workload (BSND, S1 = 128 at the end of S2 = 4096, N1 = 8, topk = 1024, causal) is
  checked element by element against the fp64 oracle.
* The large workloads are checked on samples.  The oracle forward runs only on a set of
  "live" query rows; every other row keeps out = 0 and softmaxSum = 0, so by the operator's
  definition (p = 0 when softmaxSum <= 0) it contributes nothing.  The GPU still runs every
  row, key block and launch at full size.  Then:
  - dQ of sampled live rows must match the oracle;
  - dQ of every other row must be exactly 0;
  - dK / dV of sampled keys must match the oracle's sums over the live rows;
  - every output must be finite.
* On fully consistent inputs (every row's out and statistics from the library's forward), the
  column-sum identities hold at any size: Σ_j dK[j] ≈ 0, Σ_j dKRope[j] ≈ 0, and
  Σ_j dV[j] = Σ over rows with a valid slot of dO.  Both modes must also be bit-reproducible.

All large-size comparisons use the stated bar unscaled: max abs <= 2e-2, rel-L2 <= 5e-3.
"""

import numpy as np
import pytest

from sparse_mla_flash_amd import inputs
from tests.common import Case, compare, from_dev

pytestmark = pytest.mark.gpu


def _check_sampled(case: Case, outs, live_rows, dq_rows, key_sets, label):
    """dq_rows: live rows whose dQ is compared; key_sets: (keys, row_lo, row_hi) triples whose
    dK / dV the oracle sums over rows [row_lo, row_hi) (which must hold every live row that
    can reach those keys)."""
    p = case.p
    dq, dk, dv, dqr, dkr = (from_dev(t) for t in outs)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dq_rope", dqr), ("dk_rope", dkr)):
        assert np.isfinite(t).all(), f"{label}: non-finite {name}"
    dq2 = dq.reshape(p.rows, p.N1, p.D)
    dqr2 = dqr.reshape(p.rows, p.N1, p.Dr)
    dead = np.setdiff1d(np.arange(p.rows), live_rows)
    assert not dq2[dead].any() and not dqr2[dead].any(), f"{label}: dQ of rows without probability mass"
    rdq, rdqr = case.ref_dq(rows=dq_rows)
    compare(label + "dq", dq2[dq_rows], rdq, scaled=False)
    compare(label + "dq_rope", dqr2[dq_rows], rdqr, scaled=False)
    dk2 = dk.reshape(-1, p.D)
    dkr2 = dkr.reshape(-1, p.Dr)
    dv2 = dv.reshape(-1, p.D)
    for keys, lo, hi in key_sets:
        rdk, rdkr, rdv = case.ref_dkv(keys=keys, row_lo=lo, row_hi=hi)
        compare(label + "dk", dk2[keys], rdk, scaled=False)
        compare(label + "dk_rope", dkr2[keys], rdkr, scaled=False)
        compare(label + "dv", dv2[keys], rdv, scaled=False)


def test_small_workload_every_element():
    p = inputs.workload(1)
    case = Case(p)
    rdq, rdqr = case.ref_dq()
    rdk, rdkr, rdv = case.ref_dkv()
    for det in (False, True):
        dq, dk, dv, dqr, dkr = (from_dev(t) for t in case.run_gpu(deterministic=det))
        lab = f"{p.name}/det={int(det)}/"
        compare(lab + "dq", dq, rdq, scaled=False)
        compare(lab + "dq_rope", dqr, rdqr, scaled=False)
        compare(lab + "dk", dk, rdk, scaled=False)
        compare(lab + "dk_rope", dkr, rdkr, scaled=False)
        compare(lab + "dv", dv, rdv, scaled=False)


@pytest.fixture(scope="module")
def s8k():
    """The benchmarked workload: BSND, S1 = S2 = 8192, N1 = 64, topk = 2048, causal."""
    return inputs.workload(2)


def test_s8k_sampled_against_oracle(s8k):
    p = s8k
    live = np.arange(p.rows - 256, p.rows)                      # the last 256 query rows
    case = Case(p, fwd_rows=live)
    rng = np.random.default_rng(202)
    dq_rows = np.sort(rng.choice(live, 24, replace=False))
    keys = np.unique(np.concatenate([rng.choice(p.S2, 48, replace=False), np.arange(p.S2 - 40, p.S2)]))
    dev = case.device_inputs()
    outs = case.run_gpu(deterministic=False, dev=dev)
    _check_sampled(case, outs, live, dq_rows, [(keys, live[0], live[-1] + 1)], f"{p.name}/sampled/")


def test_s8k_column_sums_and_reproducibility(s8k):
    import torch
    import sparse_mla_flash_amd as sf
    p = s8k
    dev = {k: inputs_to_dev(v, raw) for k, (v, raw) in {
        "query": (p.q, False), "key": (p.k, False), "value": (p.v, False), "query_rope": (p.qr, False),
        "key_rope": (p.kr, False), "d_out": (p.dout, False), "sparse_indices": (p.idx, True)}.items()}
    out, smax, ssum = sf.sparse_flash_attention_forward(
        dev["query"], dev["key"], dev["value"], dev["sparse_indices"], p.seq_q, p.seq_kv, dev["query_rope"],
        dev["key_rope"], scale_value=p.scale, layout=p.layout, sparse_mode=p.sparse_mode)

    def run(det):
        return sf.sparse_flash_attention_grad(
            dev["query"], dev["key"], dev["value"], dev["sparse_indices"], dev["d_out"], out, smax, ssum,
            p.seq_q, p.seq_kv, dev["query_rope"], dev["key_rope"], scale_value=p.scale, layout=p.layout,
            sparse_mode=p.sparse_mode, deterministic=det)

    first = run(False)
    again = run(False)
    det = run(True)
    for a, b, c in zip(first, again, det):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    dq, dk, dv, dqr, dkr = (from_dev(t) for t in first)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.isfinite(t).all(), name
    # rows with at least one valid slot carry probability mass 1
    idx = p.idx.reshape(p.rows, p.topk)
    pos = np.arange(p.rows)[:, None]
    has_valid = ((idx >= 0) & (idx <= pos)).any(axis=1)
    dout = inputs.bf16_bits_to_f64(p.dout).reshape(p.rows, p.N1, p.D)
    want_dv = dout[has_valid].sum(axis=(0, 1))
    got_dv = dv.reshape(-1, p.D).sum(axis=0)
    assert np.linalg.norm(got_dv - want_dv) <= 1e-2 * np.linalg.norm(want_dv)
    for name, t, width in (("dk", dk, p.D), ("dk_rope", dkr, p.Dr)):
        rows = t.reshape(-1, width)
        no_cancel = np.sqrt((rows ** 2).sum())              # size of the sum if nothing cancelled
        assert np.linalg.norm(rows.sum(axis=0)) <= 2e-2 * no_cancel, name


def inputs_to_dev(bits, raw):
    from tests.common import to_dev
    return to_dev(bits, "raw" if raw else "bf16")


def test_block_selection_workload_sampled():
    """BSND S1 = S2 = 8192, N1 = 64, causal, 32 blocks of 64 keys per token (sparseBlockSize
    64): sampled rows and keys against the oracle, on both dK / dV modes."""
    p = inputs.workload(6)
    live = np.arange(p.rows - 128, p.rows)
    case = Case(p, fwd_rows=live)
    rng = np.random.default_rng(606)
    dq_rows = np.sort(rng.choice(live, 16, replace=False))
    idx0 = p.idx.reshape(p.rows, p.topk)
    sel = idx0[live[-1]]
    block_keys = (sel[sel >= 0][:3, None] * p.block + np.arange(p.block)[None, :]).reshape(-1)
    keys = np.unique(np.concatenate([rng.choice(p.S2, 32, replace=False), block_keys[block_keys < p.S2]]))
    dev = case.device_inputs()
    for det in (False, True):
        outs = case.run_gpu(deterministic=det, dev=dev)
        _check_sampled(case, outs, live, dq_rows, [(keys, live[0], live[-1] + 1)],
                       f"{p.name}/det={int(det)}/sampled/")


def test_hot_cold_deterministic_workload_sampled():
    """BSND B = 2, S1 = 4096, S2 = 32768, N1 = 48 (a partial head group), topk = 8192, no mask,
    deterministic; every token selects all hot keys plus distinct cold keys."""
    p = inputs.workload(5)
    lq = p.S1
    live = np.concatenate([np.arange(lq - 48, lq), np.arange(2 * lq - 48, 2 * lq)])
    case = Case(p, fwd_rows=live)
    rng = np.random.default_rng(505)
    dq_rows = np.sort(rng.choice(live, 12, replace=False))
    idx0 = p.idx.reshape(p.rows, p.topk)
    key_sets = []
    for b in range(2):
        local = rng.choice(p.S2, 40, replace=False)
        hot_local = idx0[b * lq + lq - 1][:4]                   # keys the last live row selected
        keys = np.unique(np.concatenate([local, hot_local])) + b * p.S2
        key_sets.append((keys, b * lq + lq - 48, b * lq + lq))
    dev = case.device_inputs()
    a = case.run_gpu(deterministic=True, dev=dev)
    b = case.run_gpu(deterministic=True, dev=dev)
    import torch
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    _check_sampled(case, a, live, dq_rows, key_sets, f"{p.name}/sampled/")


def _check_tail(t, outs, dq_pos, keys, label):
    """Sampled check of a TailCase run: dQ of live rows self.live[dq_pos], dQ = 0 on every other
    row, dK / dKRope / dV of `keys` against the oracle's sums over all live rows."""
    from tests.common import TailCase  # noqa: F401  (type of t)
    p = t.p
    dq, dk, dv, dqr, dkr = (from_dev(x) for x in outs)
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv), ("dq_rope", dqr), ("dk_rope", dkr)):
        assert np.isfinite(x).all(), f"{label}: non-finite {name}"
    dq2 = dq.reshape(p.rows, p.N1, p.D)
    dqr2 = dqr.reshape(p.rows, p.N1, p.Dr)
    dead = np.ones(p.rows, bool)
    dead[t.live] = False
    assert not dq2[dead].any() and not dqr2[dead].any(), f"{label}: dQ of rows without probability mass"
    rdq, rdqr = t.ref_dq(dq_pos)
    compare(label + "dq", dq2[t.live[dq_pos]], rdq, scaled=False)
    compare(label + "dq_rope", dqr2[t.live[dq_pos]], rdqr, scaled=False)
    rdk, rdkr, rdv = t.ref_dkv(keys)
    compare(label + "dk", dk.reshape(-1, p.D)[keys], rdk, scaled=False)
    compare(label + "dk_rope", dkr.reshape(-1, p.Dr)[keys], rdkr, scaled=False)
    compare(label + "dv", dv.reshape(-1, p.D)[keys], rdv, scaled=False)


@pytest.mark.timeout(900)
def test_tnd_varlen_n128_sampled_across_segments():
    """TND, 4 sequences of 2K / 4K / 8K / 16K tokens, N1 = 128 (two head groups), topk = 2048,
    causal.  Live rows: the last 1030 rows of the 4K sequence (three 512-row segments of the
    key-major kernel), the last 64 of the 2K and the last 128 of the 16K sequence.  The sampled
    keys are each selected by live rows of at least three segments, so the ordered sum over
    (head group, segment) partials is checked element by element; both deterministic settings."""
    from tests.common import TailCase
    p = inputs.workload(3)
    print(f"# {p.name}: generated", flush=True)
    t = TailCase(p, [64, 1030, 0, 128])
    print(f"# {p.name}: oracle forward on {len(t.live)} rows done", flush=True)
    rng = np.random.default_rng(303)
    dq_pos = np.sort(rng.choice(len(t.live), 16, replace=False))
    multi = t.keys_from_segments(rng, 40, seg_rows=512, min_segments=3)
    assert len(multi) >= 20
    other = np.concatenate([p.k_offset(0) + rng.choice(p.lkv(0), 8, replace=False),
                            p.k_offset(3) + rng.choice(p.lkv(3), 8, replace=False),
                            p.k_offset(2) + rng.choice(p.lkv(2), 4, replace=False)])   # seq 2: no live row
    keys = np.unique(np.concatenate([multi, other]))
    dev = t.device_inputs()
    for det in (False, True):
        outs = t.run_gpu(dev, deterministic=det)
        import sparse_mla_flash_amd as sf
        assert sf.sfag_last_path() == 0, "this workload takes the key-major path"
        _check_tail(t, outs, dq_pos, keys, f"{p.name}/det={int(det)}/")
        print(f"# {p.name}: det={int(det)} ok", flush=True)


@pytest.mark.timeout(900)
def test_long_context_window_sampled_both_modes():
    """BSND B = 1, 16384 queries at the end of 131072 keys, N1 = 128, topk = 2048, half the
    slots from the local window [pos - 4095, pos] and half uniform: the per-pair (scatter) path
    at its full 131072-key accumulator, in both deterministic settings.  Live rows: the last
    200; sampled keys from the window, from the uniform part and unselected ones."""
    from tests.common import TailCase
    import sparse_mla_flash_amd as sf
    p = inputs.workload(4)
    print(f"# {p.name}: generated", flush=True)
    t = TailCase(p, [200])
    print(f"# {p.name}: oracle forward on {len(t.live)} rows done", flush=True)
    rng = np.random.default_rng(404)
    dq_pos = np.sort(rng.choice(len(t.live), 16, replace=False))
    idx = p.idx.reshape(p.rows, p.topk)
    last = idx[t.live[-1]]
    win = last[last >= p.S2 - 4096]
    far = last[last < p.S2 - 4096]
    keys = np.unique(np.concatenate([rng.choice(win, 24, replace=False), rng.choice(far, 24, replace=False),
                                     rng.choice(p.S2, 8, replace=False)]))
    dev = t.device_inputs()
    for det in (False, True):
        outs = t.run_gpu(dev, deterministic=det)
        assert sf.sfag_last_path() == 1, "this workload takes the per-pair path"
        _check_tail(t, outs, dq_pos, keys, f"{p.name}/det={int(det)}/")
        print(f"# {p.name}: det={int(det)} ok", flush=True)
