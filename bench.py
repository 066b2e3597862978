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
             key-major kernel 2176 (dK, dV); per-pair path: the chunk loop (query-major
             kernel, slots, partials, per-key sums) is timed as one stage with all 5504.
             `traffic` comes from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
             of that kernel when it matches the current kernel sources, else null
  cpu_baseline  the fp64 CPU oracle on a bounded sample of rows of the same workload

Inputs are seeded synthetic tensors (sparse_mla_flash_amd.inputs); out / softmaxMax /
softmaxSum come from the library's sparse forward (timing inputs only).

  python bench.py [--steps K] [--warmup W] [--workload N] [--deterministic]
  python bench.py --copy-calibration     # plain 1 GiB device copies, for counter scaling
  python bench.py --ceilings             # measured MFMA rate / shader clock, HBM copy, LDS and
                                         # atomic rates (sparse_mla_flash_amd/microbench)

Timing: `ms_per_step` is the wall-clock mean over the K timed steps (bracketed by device
synchronisation); `call_ms` gives the median, min and max of the same K calls measured one by
one with HIP events on the library's stream.  Per-kernel `hbm_gbs` divide the committed
rocprofv3 FETCH_SIZE + WRITE_SIZE bytes of that kernel (scaled by the same counters on a plain
copy) by its event-timed duration, and are null once the kernel sources change.
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
# the source file of each profiled kernel; with the two shared headers it fixes the kernel's code
KERNEL_FILES = {"bwd_q_kernel": "sfag_q.hip", "kv_dense_kernel": "sfag_dense.hip", "sort_rows_kernel": "sfag_dense.hip",
                "kv_reduce_kernel": "sfag_dense.hip", "pair_kv_kernel": "sfag_pair.hip",
                "pair_sum_kernel": "sfag_pair.hip", "pair_slots_kernel": "sfag_pair.hip", "fwd_kernel": "sfag_fwd.hip"}


def kernel_sha(kernel: str) -> str:
    """Hash of a kernel's source file and the shared device / launch headers."""
    h = hashlib.sha256()
    for f in (KERNEL_FILES[kernel], "sfag_device.h", "sfag_launch.h"):
        with open(os.path.join(ROOT, CSRC, f), "rb") as fh:
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

    def record(self, e, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert self.hip.hipEventRecord(e, stream) == 0


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
    if kernel not in KERNEL_FILES or t.get("kernel_sha") != kernel_sha(kernel):
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(p, nrows: int, per_row):
    """Time the fp64 oracle backward on the last `nrows` query rows of the workload."""
    import numpy as np
    import oracle
    from sparse_mla_flash_amd import inputs
    g = oracle.Geometry.of(p)
    q, k, qr, kr = (inputs.bits_to_f64(x, p.dtype) for x in (p.q, p.k, p.qr, p.kr))
    dout = inputs.bits_to_f64(p.dout, p.dtype)
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


INDEXER_WORKLOADS = {
    # name: (indexer_problem kwargs, seed); index heads 64 x 128 wide, causal
    "ix_bsnd_s4096_n64_g64_causal": (dict(layout="BSND", B=1, S1=4096, S2=4096, N1=64, G=64, sparse_mode=3), 101),
    "ix_bsnd_s8192_n128_g64_causal": (dict(layout="BSND", B=1, S1=8192, S2=8192, N1=128, G=64, sparse_mode=3), 102),
}


def indexer_bench(args):
    """Lightning-indexer backward (KL loss): one call per step on a seeded workload.  Inputs and
    both sets of forward statistics are prepared on the GPU with torch (fp32 products of the
    16-bit inputs); the timed region is the library call only."""
    import numpy as np
    import torch
    import sparse_mla_flash_amd as sf
    from sparse_mla_flash_amd import inputs
    name = args.indexer
    kw, seed = INDEXER_WORKLOADS[name]
    p = inputs.indexer_generate(inputs.indexer_problem(**kw, dtype=args.dtype, name=name), seed)
    elem = torch.float16 if args.dtype == "fp16" else torch.bfloat16

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(elem).cuda()

    q, qr, k, kr, qi, ki, w = (dev(x) for x in (p.q, p.qr, p.k, p.kr, p.qi, p.ki, p.w))
    S1, S2, N1 = p.S1, p.S2, p.N1
    smax = torch.zeros(1, N1, S1, device="cuda")
    ssum = torch.zeros_like(smax)
    mi = torch.zeros(1, S1, device="cuda")
    si = torch.zeros_like(mi)
    kf = torch.cat([k[0, :, 0].float(), kr[0, :, 0].float()], 1)            # [S2, 576]
    kif = ki[0, :, 0].float()                                                # [S2, 128]
    pos = torch.arange(S2, device="cuda")
    for r0 in range(0, S1, 256):
        r1 = min(S1, r0 + 256)
        qf = torch.cat([q[0, r0:r1].float(), qr[0, r0:r1].float()], 2)      # [R, N1, 576]
        hi = torch.arange(r0, r1, device="cuda")[:, None] + (S2 - S1)        # causal bound
        mask = pos[None, :] <= hi                                            # [R, S2]
        z = p.scale * torch.matmul(qf, kf.t().contiguous())                  # [R, N1, S2]
        z = z.masked_fill(~mask[:, None, :], float("-inf"))
        m = z.amax(2)
        smax[0, :, r0:r1] = m.t()
        ssum[0, :, r0:r1] = torch.exp(z - m[:, :, None]).sum(2).t()
        sc = torch.matmul(qi[0, r0:r1].float(), kif.t().contiguous())        # [R, G, S2]
        iv = (w[0, r0:r1].float()[:, :, None] * torch.relu(sc)).sum(1).masked_fill(~mask, float("-inf"))
        im = iv.amax(1)
        mi[0, r0:r1] = im
        si[0, r0:r1] = torch.exp(iv - im[:, None]).sum(1)
        del z, sc, iv
    torch.cuda.synchronize()
    dims = sf._indexer_dims(q, k, qi, w, "BSND", None)
    ws_bytes = sf.sfag_lightning_indexer_grad_get_workspace_size(dims, None, None, "BSND", p.sparse_mode)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    dqi, dki, dw = torch.empty_like(qi), torch.empty_like(ki), torch.empty_like(w)
    loss = torch.empty(1, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        st = sf.sfag_dense_lightning_indexer_grad_kl_loss(
            q.data_ptr(), k.data_ptr(), qi.data_ptr(), ki.data_ptr(), w.data_ptr(), smax.data_ptr(),
            ssum.data_ptr(), mi.data_ptr(), si.data_ptr(), qr.data_ptr(), kr.data_ptr(), None, None, dims, p.scale,
            "BSND", p.sparse_mode, 2 ** 31 - 1, 2 ** 31 - 1, dqi.data_ptr(), dki.data_ptr(), dw.data_ptr(),
            loss.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if st != 0:
            raise sf.SfagError(st, sf.sfag_last_error())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    evs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        ev.record(e0, stream)
        step()
        ev.record(e1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    calls = sorted(ev.elapsed_ms(a, b) for a, b in evs)
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    pairs = sum(min(S2, i + 1 + (S2 - S1)) for i in range(S1) if i + (S2 - S1) >= 0)
    flop_pair = 2 * 576 * N1 + 3 * 2 * p.Di * p.G       # main scores; index scores, dq~, dK~
    med = calls[len(calls) // 2]
    tf = pairs * flop_pair / (med * 1e-3) / 1e12
    rec = {"metric": "lightning-indexer backward (KL loss) TFLOP/s on 1 MI355X", "value": round(tf, 3),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round((t1 - t0) / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
           "config": {"workload": name, "layout": "BSND", "S1": S1, "S2": S2, "N1": N1, "G": p.G, "Di": p.Di,
                      "sparse_mode": p.sparse_mode, "admitted_pairs": pairs, "flop_per_pair": flop_pair},
           "call_ms": {"median": round(med, 4), "min": round(calls[0], 4), "max": round(calls[-1], 4),
                       "n": len(calls)},
           "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5), "traffic": None,
                        "kernel": "whole call (ix_query_kernel + ix_key_kernel + ix_finish_kernel)"},
           "loss": float(loss.item()), "device": device_info()}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = indexer_cpu_baseline(p, flop_pair, smax, ssum, mi, si)
    print(json.dumps(rec), flush=True)


def forward_bench(args, p, q, k, v, idx, qr, kr):
    """The sparse forward on the same workload: one call per step, HIP events per call."""
    import torch
    import sparse_mla_flash_amd as sf
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        return sf.sparse_flash_attention_forward(q, k, v, idx, p.seq_q, p.seq_kv, qr, kr, scale_value=p.scale,
                                                 sparse_block_size=p.block, layout=p.layout,
                                                 sparse_mode=p.sparse_mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    evs = [(ev.create(), ev.create()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        ev.record(e0, stream)
        step()
        ev.record(e1, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    calls = sorted(ev.elapsed_ms(a, b) for a, b in evs)
    for a, b in evs:
        ev.destroy(a)
        ev.destroy(b)
    npairs = int(valid_per_row(p).sum())
    flop = 2 * 576 + 2 * 512                              # S and P V per (pair, head)
    med = calls[len(calls) // 2]
    tf = npairs * p.N1 * flop / (med * 1e-3) / 1e12
    print(json.dumps({
        "metric": "sparse forward TFLOP/s on 1 MI355X", "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round((t1 - t0) / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": p.name, "valid_pairs": npairs, "N1": p.N1, "flop_per_pair_head": flop},
        "call_ms": {"median": round(med, 4), "min": round(calls[0], 4), "max": round(calls[-1], 4), "n": len(calls)},
        "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5), "traffic": None, "kernel": "fwd_kernel"},
        "device": device_info()}), flush=True)


def indexer_cpu_baseline(p, flop_pair, smax, ssum, mi, si, nrows: int = 512):
    """The fp64 indexer oracle on the last `nrows` query rows of the same workload."""
    import numpy as np
    from oracle import indexer as ix
    from sparse_mla_flash_amd import inputs
    geo = ix.IndexerGeometry(p.layout, p.B, p.S1, p.S2, p.N1, p.G, p.Di, p.D, p.Dr, p.seq_q, p.seq_kv,
                             p.sparse_mode, p.scale)
    f = lambda x: inputs.bits_to_f64(x, p.dtype)
    rows = list(range(p.rows - nrows, p.rows))
    cpu = lambda t: t.detach().double().cpu().numpy()
    t0 = time.perf_counter()
    ix.indexer_grad(geo, f(p.q), f(p.k), f(p.qr), f(p.kr), cpu(smax), cpu(ssum), f(p.qi), f(p.ki), f(p.w),
                    cpu(mi), cpu(si), rows=rows)
    dt = time.perf_counter() - t0
    pairs = sum(min(p.S2, i + 1 + (p.S2 - p.S1)) for i in range(p.S1 - nrows, p.S1))
    import os as _os
    return {"value": pairs * flop_pair / dt / 1e12, "unit": "TFLOP/s", "cores": _os.cpu_count(), "kind": "oracle",
            "sample": f"fp64 numpy indexer oracle over query rows {rows[0]}..{rows[-1]} ({pairs} admitted pairs); "
                      f"{dt:.2f} s wall"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _ceilings_lib():
    path = os.path.join(ROOT, "sparse_mla_flash_amd", "microbench", "libceilings.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.ceil_device_info.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.ceil_mfma.restype = ctypes.c_float
    L.ceil_mfma.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
    L.ceil_copy.restype = ctypes.c_float
    L.ceil_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    L.ceil_lds.restype = ctypes.c_float
    L.ceil_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    L.ceil_atomic.restype = ctypes.c_float
    L.ceil_atomic.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp]
    L.ceil_gather.restype = ctypes.c_float
    L.ceil_gather.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp]
    return L


def device_info():
    """Name, compute-unit count and peak shader / memory clocks from hipGetDeviceProperties."""
    L = _ceilings_lib()
    if L is None:
        return None
    name = ctypes.create_string_buffer(256)
    cus, clk, mclk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    if L.ceil_device_info(name, 256, ctypes.byref(cus), ctypes.byref(clk), ctypes.byref(mclk)) != 0:
        return None
    return {"name": name.value.decode(), "compute_units": cus.value, "peak_sclk_mhz": clk.value / 1000.0,
            "mem_clk_mhz": mclk.value / 1000.0}


def ceilings():
    """Measured ceilings: the bf16 MFMA rate with every CU busy and the shader clock it runs at,
    HBM copy bandwidth, LDS instruction rates (bytes per clock per CU at that clock) and the
    fp32 global atomic-add rate on random 4352-byte rows."""
    import torch
    L = _ceilings_lib()
    if L is None:
        raise SystemExit("libceilings.so is missing: run python -m sparse_mla_flash_amd.build")
    dev = device_info()
    cus = dev["compute_units"]
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    res = {"device": dev}
    # MFMA: 4 waves per SIMD, 8 independent 16x16x32 bf16 chains per wave
    blocks, iters = cus * 4, 20000
    best = None
    for _ in range(3):
        ms = L.ceil_mfma(out.data_ptr(), blocks, iters, clk.data_ptr(), stream)
        torch.cuda.synchronize()
        ticks, cyc = (int(x) for x in clk.tolist())
        if ms > 0 and (best is None or ms < best[0]):
            best = (ms, ticks, cyc)
    flop = blocks * 4 * iters * 8 * (16 * 16 * 32 * 2)
    ms, ticks, cyc = best
    sclk = cyc / ticks * 100.0 if ticks > 0 else None          # s_memrealtime runs at 100 MHz
    res["mfma_bf16"] = {"tflops": round(flop / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4),
                        "sclk_mhz_under_load": None if sclk is None else round(sclk, 1),
                        "flop_per_clk_per_cu": None if sclk is None else
                        round(flop / (ms * 1e-3) / (sclk * 1e6) / cus, 1)}
    # HBM copy, 2 GiB each way
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    times = [L.ceil_copy(a.data_ptr(), b.data_ptr(), n, cus * 16, stream) for _ in range(5)]
    torch.cuda.synchronize()
    t = min(x for x in times if x > 0)
    res["hbm_copy"] = {"gbs": round(2 * n / (t * 1e-3) / 1e9, 1), "bytes_each_way": n, "ms": round(t, 4)}
    del a, b
    # LDS rates at the shader clock measured above
    names = {0: "ds_add_f32", 1: "ds_write_b32", 2: "ds_read_b32", 3: "ds_write_b128", 4: "ds_read_b128",
             5: "ds_read_b64_tr_b16"}
    width = {0: 4, 1: 4, 2: 4, 3: 16, 4: 16, 5: 8}
    lds = {}
    lblocks, liters = cus * 2, 4000
    for mode in range(6):
        t = min(L.ceil_lds(mode, lblocks, liters, out.data_ptr(), stream) for _ in range(3))
        torch.cuda.synchronize()
        nbytes = lblocks * 256 * liters * 16 * width[mode]
        lds[names[mode]] = {"bytes_per_clk_per_cu": None if sclk is None else
                            round(nbytes / (t * 1e-3) / (sclk * 1e6) / cus, 1),
                            "tb_per_s": round(nbytes / (t * 1e-3) / 1e12, 2)}
    res["lds"] = lds
    # fp32 atomics: 65536 workgroups, each adding into one random row of 1088 floats, 4 times
    g = torch.Generator(device="cpu").manual_seed(7)
    for rows_total, label in ((131072, "rows_131072"), (8192, "rows_8192")):
        acc = torch.zeros(rows_total * 1088, dtype=torch.float32, device="cuda")
        rows = torch.randint(0, rows_total, (65536,), generator=g, dtype=torch.int32).cuda()
        t = min(L.ceil_atomic(acc.data_ptr(), rows.data_ptr(), 65536, 4, stream) for _ in range(3))
        torch.cuda.synchronize()
        ops = 65536 * 1088 * 4
        res["atomic_add_f32_" + label] = {"g_ops_per_s": round(ops / (t * 1e-3) / 1e9, 1), "ms": round(t, 3)}
        del acc, rows
    # direct-to-LDS gather of 32 random key rows (1152 B each) per chunk, 2048 workgroups x 128
    # chunks, two lane mappings: 32 B of 32 keys per 1 KB load, or whole 128-byte runs of 8 keys
    nkeys, gblocks, nch = 8192, 2048, 128
    kv = torch.ones(nkeys * 1024, dtype=torch.uint8, device="cuda")
    kr = torch.ones(nkeys * 128, dtype=torch.uint8, device="cuda")
    gi = torch.randint(0, nkeys, (gblocks * nch, 32), generator=g, dtype=torch.int32).sort(dim=1).values
    gi = gi.contiguous().cuda()
    gather = {}
    for mode, label in ((0, "32_keys_x_32B_per_load"), (1, "8_keys_x_128B_per_load")):
        t = min(L.ceil_gather(mode, kv.data_ptr(), kr.data_ptr(), gi.data_ptr(), gblocks, nch, out.data_ptr(), stream)
                for _ in range(5))
        torch.cuda.synchronize()
        nbytes = gblocks * nch * 36 * 1024
        gather[label] = {"gb_per_s": round(nbytes / (t * 1e-3) / 1e9, 1),
                         "bytes_per_clk_per_cu": None if sclk is None else
                         round(nbytes / (t * 1e-3) / (sclk * 1e6) / cus, 1), "ms": round(t, 4)}
    res["key_row_gather"] = gather
    del kv, kr, gi
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default="bf16",
                    help="element type of the 16-bit tensors (the workload's values rounded to it)")
    ap.add_argument("--cpu-rows", type=int, default=768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceilings", action="store_true")
    ap.add_argument("--forward", action="store_true",
                    help="time the sparse forward (out, softmaxMax, softmaxSum) on the workload instead")
    ap.add_argument("--indexer", choices=sorted(INDEXER_WORKLOADS), default=None,
                    help="time the lightning-indexer backward on this workload instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the kernel is measured on a single "
              "MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceilings:
        ceilings()
        return
    if args.indexer:
        indexer_bench(args)
        return

    import numpy as np
    import torch
    import sparse_mla_flash_amd as sf
    from sparse_mla_flash_amd import inputs

    t_gen = time.perf_counter()
    p = inputs.workload(args.workload, dtype=args.dtype)
    t_gen = time.perf_counter() - t_gen
    print(f"# generated workload {p.name} in {t_gen:.1f} s", file=sys.stderr, flush=True)

    elem = torch.float16 if args.dtype == "fp16" else torch.bfloat16

    def dev(bits, raw=False):
        a = np.ascontiguousarray(bits)
        t = torch.from_numpy(a if raw else a.view(np.int16))
        return (t if raw else t.view(elem)).cuda()

    q, k, v, qr, kr, dout = (dev(x) for x in (p.q, p.k, p.v, p.qr, p.kr, p.dout))
    idx = dev(p.idx, raw=True)
    out, smax, ssum = sf.sparse_flash_attention_forward(q, k, v, idx, p.seq_q, p.seq_kv, qr, kr,
                                                        scale_value=p.scale, sparse_block_size=p.block,
                                                        layout=p.layout, sparse_mode=p.sparse_mode)
    if args.forward:
        forward_bench(args, p, q, k, v, idx, qr, kr)
        return
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
    evs = [[ev.create() for _ in range(6)] for _ in range(args.steps)]   # call begin / end + 4 stage events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sf.sfag_set_profile_events(*evs[i][2:6])
        ev.record(evs[i][0], stream)
        step()
        ev.record(evs[i][1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sf.sfag_set_profile_events()
    path = "key-major" if sf.sfag_last_path() == 0 else "per-pair"
    calls = sorted(ev.elapsed_ms(e[0], e[1]) for e in evs)
    s1 = sum(ev.elapsed_ms(e[2], e[3]) for e in evs) / args.steps
    s2 = sum(ev.elapsed_ms(e[4], e[5]) for e in evs) / args.steps if path == "key-major" else 0.0
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
        # one event pair around the whole chunk loop (query-major kernel, slots, partials, sums)
        stages = {"per-pair chunk loop": (s1, FLOP_PER_PAIR_HEAD)}
    kernel = max(stages, key=lambda n: stages[n][0])
    kern_avg, kflop = stages[kernel]
    achieved = npairs * p.N1 * kflop / (kern_avg * 1e-3) / 1e12
    stage_rec = {}
    for n, (ms, fl) in stages.items():
        tr = traffic_from_profile(n.split("<")[0].split(" ")[0], p.name)
        stage_rec[n] = {
            "ms": round(ms, 4),
            "tflops": round(npairs * p.N1 * fl / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(npairs * p.N1 * fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            # HBM bytes moved by this kernel (rocprofv3 counters, copy-calibrated) over its time
            "hbm_gbs": None if tr is None else round(tr / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": None if tr is None else round(tr / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    # logical gather rate: one bf16 key row per valid pair, mostly served by L2 / MALL, so this
    # is an on-chip rate, not an HBM one
    gather_gbs = npairs * GATHER_BYTES_PER_PAIR / (s1 * 1e-3) / 1e9
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
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": p.name, "layout": p.layout, "B": p.B, "S1": p.S1, "S2": p.S2, "N1": p.N1,
            "topk": p.topk, "sparse_block_size": p.block, "sparse_mode": p.sparse_mode, "deterministic": det,
            "valid_pairs": npairs, "nominal_pairs": nominal,
            "effective_tflops_nominal": round(nominal * p.N1 * FLOP_PER_PAIR_HEAD / (ms_per_step * 1e-3) / 1e12, 3),
        },
        "call_ms": {"median": round(calls[len(calls) // 2], 4), "min": round(calls[0], 4),
                    "max": round(calls[-1], 4), "n": len(calls),
                    "effective_tflops_median": round(flops / (calls[len(calls) // 2] * 1e-3) / 1e12, 3)},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 5),
            "traffic": traffic_from_profile(kernel.split("<")[0].split(" ")[0], p.name),
            "kernel": kernel,
            "kernel_ms": round(kern_avg, 4),
            "kernel_flop_per_pair_head": kflop,
            "path": path,
            "stages": stage_rec,
            "gather_logical_gbs": round(gather_gbs, 1),
        },
        "device": device_info(),
        "host_cpu": cpu_model(),
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(p, min(args.cpu_rows, p.rows), per_row)
        rec["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
