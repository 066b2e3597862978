#!/usr/bin/env python3
"""Benchmark of the SparseFlashAttentionGrad backward on one MI355X.

One step = one full backward call (every launch of the library's backward: index sort,
query-major kernel, key-major kernel, ordered reduce and cast) over the BSND workload
S1 = S2 = 8192, N1 = 64, topk = 2048, causal (sparseMode 3), with every input already
resident in HBM.  Prints one JSON line:

  value      effective TFLOP/s = valid (row, slot) pairs x N1 x 5504 flop / step time
             (5504 = the five topk-wide contractions: 2*576 score recompute,
             2*512 dP, 2*512 dV, 2*576 dQ, 2*576 dK)
  roofline   the dominant kernel's algorithmic flops / its average duration, measured
             with HIP events that the library records on its own stream around that
             kernel, against the 2.5 PFLOP/s bf16 dense MFMA peak.  Key-major path: the
             query-major kernel does 3328 flop per (pair, head) (scores, dP, dQ) and the
             key-major kernel 2176 (dK, dV); scatter path: one kernel does all 5504.
             `traffic` comes from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
             of that kernel when it matches the current kernel sources, else null
  cpu_baseline  the fp64 CPU oracle on a bounded sample of rows of the same workload

Inputs are seeded synthetic tensors (sparse_mla_flash_amd.inputs); out / softmaxMax /
softmaxSum come from the library's sparse forward (timing inputs only).

  python bench.py [--steps K] [--warmup W] [--workload N] [--deterministic]
  python bench.py --copy-calibration     # plain 1 GiB device copies, for counter scaling
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLOP_PER_PAIR_HEAD = 2 * 576 + 2 * 512 + 2 * 512 + 2 * 576 + 2 * 576   # 5504
GATHER_BYTES_PER_PAIR = 576 * 2                                        # bf16 key row (nope | rope)
SCATTER_BYTES_PER_PAIR = 1088 * 4                                      # fp32 dK | dKRope | dV row
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
METRIC = "effective TFLOP/s + ms/call, sparse attn bwd (S=8K, topk=2048, N1=64) on 1 MI355X"
FLOP_Q_KERNEL = 2 * 576 + 2 * 512 + 2 * 576                                  # 3328: S, dP, dQ
FLOP_KV_KERNEL = 2 * 576 + 2 * 512                                           # 2176: dK, dV
CSRC = os.path.join("sparse_mla_flash_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                        if f.endswith((".hip", ".h", ".cpp")))


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def valid_per_row(p):
    """Number of valid (row, slot) pairs of every query row (host-side bookkeeping)."""
    import numpy as np
    idx = p.idx.reshape(p.rows, p.topk).astype(np.int64)
    bs = p.block
    counts = np.zeros(p.rows, dtype=np.int64)
    for b in range(p.B):
        r0 = p.q_offset(b)
        lq, lkv = p.lq(b), p.lkv(b)
        rows = idx[r0:r0 + lq]
        i = np.arange(lq)[:, None]
        hi = np.minimum(i + lkv - lq, lkv - 1) if p.sparse_mode == 3 else np.full((lq, 1), lkv - 1)
        # keys j*bs .. j*bs + bs - 1 of every block index j >= 0 that do not pass hi
        n = np.clip(hi - rows * bs + 1, 0, bs)
        counts[r0:r0 + lq] = np.where(rows >= 0, n, 0).sum(axis=1)
    return counts


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}))


def traffic_from_profile(kernel: str, workload_name: str):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(p, nrows: int, per_row):
    """Time the fp64 oracle backward on the last `nrows` query rows of the workload."""
    import numpy as np
    import oracle
    from sparse_mla_flash_amd import inputs
    g = oracle.Geometry.of(p)
    q, k, qr, kr = (inputs.bf16_bits_to_f64(x) for x in (p.q, p.k, p.qr, p.kr))
    dout = inputs.bf16_bits_to_f64(p.dout)
    lo, hi = p.rows - nrows, p.rows
    rows = np.arange(lo, hi)
    out, m, l = oracle.forward(g, q, k, k, qr, kr, p.idx, rows=rows)     # input preparation, untimed
    t0 = time.perf_counter()
    oracle.backward_dq(g, q, k, k, qr, kr, p.idx, dout, out, m, l, rows=rows)
    oracle.backward_dkv(g, q, k, k, qr, kr, p.idx, dout, out, m, l, row_lo=lo, row_hi=hi)
    dt = time.perf_counter() - t0
    pairs = int(per_row[lo:hi].sum())
    flops = pairs * p.N1 * FLOP_PER_PAIR_HEAD
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle backward (dQ pass + dK/dV pass) over query rows {lo}..{hi - 1} "
                      f"({pairs} valid pairs x {p.N1} heads) of the same workload; forward for those rows "
                      f"untimed; {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the kernel is measured on a single "
              "MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    import sparse_mla_flash_amd as sf
    from sparse_mla_flash_amd import inputs

    t_gen = time.perf_counter()
    p = inputs.workload(args.workload)
    t_gen = time.perf_counter() - t_gen
    print(f"# generated workload {p.name} in {t_gen:.1f} s", file=sys.stderr, flush=True)

    def dev(bits, raw=False):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a if raw else a.view(np.int16))
        return (t if raw else t.view(torch.bfloat16)).cuda()

    q, k, v, qr, kr, dout = (dev(x) for x in (p.q, p.k, p.v, p.qr, p.kr, p.dout))
    idx = dev(p.idx, raw=True)
    out, smax, ssum = sf.sparse_flash_attention_forward(q, k, v, idx, p.seq_q, p.seq_kv, qr, kr,
                                                        scale_value=p.scale, sparse_block_size=p.block,
                                                        layout=p.layout, sparse_mode=p.sparse_mode)
    det = bool(args.deterministic or p.deterministic)
    dims = sf._dims_from(q, k, idx, p.layout, p.seq_q, p.seq_kv)
    ws_bytes = sf.sfag_get_workspace_size(dims, p.seq_q, p.seq_kv, p.scale, p.block, p.layout, p.sparse_mode,
                                          2 ** 31 - 1, 2 ** 31 - 1, det)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    dqr, dkr = torch.empty_like(qr), torch.empty_like(kr)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        st = sf.sfag_sparse_flash_attention_grad(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(), dout.data_ptr(), out.data_ptr(),
            smax.data_ptr(), ssum.data_ptr(), p.seq_q, p.seq_kv, qr.data_ptr(), kr.data_ptr(), dims, p.scale, p.block,
            p.layout, p.sparse_mode, 2 ** 31 - 1, 2 ** 31 - 1, det, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            dqr.data_ptr(), dkr.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if st != 0:
            raise sf.SfagError(st, sf.sfag_last_error())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    ev = HipEvents()
    evs = [[ev.create() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sf.sfag_set_profile_events(*evs[i])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sf.sfag_set_profile_events()
    path = "key-major" if sf.sfag_last_path() == 0 else "scatter"
    s1 = sum(ev.elapsed_ms(e[0], e[1]) for e in evs) / args.steps
    s2 = sum(ev.elapsed_ms(e[2], e[3]) for e in evs) / args.steps if path == "key-major" else 0.0
    for e in evs:
        for x in e:
            ev.destroy(x)

    ms_per_step = (t1 - t0) / args.steps * 1e3
    per_row = valid_per_row(p)
    npairs = int(per_row.sum())
    nominal = p.rows * p.topk * p.block
    flops = npairs * p.N1 * FLOP_PER_PAIR_HEAD
    value = flops / (ms_per_step * 1e-3) / 1e12
    if path == "key-major":
        stages = {"bwd_q_kernel": (s1, FLOP_Q_KERNEL), "kv_dense_kernel": (s2, FLOP_KV_KERNEL)}
    else:
        stages = {("bwd_main_kernel<partial> + sort + reduce" if det else "bwd_main_kernel<atomic>"):
                  (s1, FLOP_PER_PAIR_HEAD)}
    kernel = max(stages, key=lambda n: stages[n][0])
    kern_avg, kflop = stages[kernel]
    achieved = npairs * p.N1 * kflop / (kern_avg * 1e-3) / 1e12
    # logical gather rate (one bf16 key row per valid pair, read by the kernel that forms the
    # scores) and scatter rate (one fp32 dK | dKRope | dV row per valid pair)
    gather_ms = s1
    scatter_ms = s2 if path == "key-major" else s1
    gather_gbs = npairs * GATHER_BYTES_PER_PAIR / (gather_ms * 1e-3) / 1e9
    scatter_gbs = npairs * SCATTER_BYTES_PER_PAIR / (scatter_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": p.name, "layout": p.layout, "B": p.B, "S1": p.S1, "S2": p.S2, "N1": p.N1,
            "topk": p.topk, "sparse_block_size": p.block, "sparse_mode": p.sparse_mode, "deterministic": det,
            "valid_pairs": npairs, "nominal_pairs": nominal,
            "effective_tflops_nominal": round(nominal * p.N1 * FLOP_PER_PAIR_HEAD / (ms_per_step * 1e-3) / 1e12, 3),
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 5),
            "traffic": traffic_from_profile(kernel.split("<")[0], p.name),
            "kernel": kernel,
            "kernel_ms": round(kern_avg, 4),
            "kernel_flop_per_pair_head": kflop,
            "path": path,
            "stages_ms": {n: round(v[0], 4) for n, v in stages.items()},
            "stages_tflops": {n: round(npairs * p.N1 * v[1] / (v[0] * 1e-3) / 1e12, 2) for n, v in stages.items()},
            "gather_logical_gbs": round(gather_gbs, 1),
            "gather_hbm_frac": round(gather_gbs / HBM_PEAK_GBS, 4),
            "scatter_logical_gbs": round(scatter_gbs, 1),
            "scatter_hbm_frac": round(scatter_gbs / HBM_PEAK_GBS, 4),
        },
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(p, min(args.cpu_rows, p.rows), per_row)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
