// sfag_bwd.hip -- SparseFlashAttentionGrad backward kernels for gfx950.
//
// Operation (SparseFlashAttentionGrad README, "function description"): per query row and
// head, over the key rows named by sparseIndices (gather), recompute the logits
// z = scale (q.k + qRope.kRope) and P = exp(z - softmaxMax) / softmaxSum, then
//   stage 1  dP = dO V^T          dV[u] += P^T dO
//   stage 2  dS = P * (dP - D)    D = rowsum(dO * out)   (FlashSoftmaxGrad)
//   stage 3  dQ = scale dS K      dK[u] += scale dS^T Q
// with V = K (the page's constraint that value equals key) and the rope columns
// handled as 64 extra columns of Q and K.
//
// Work decomposition: one workgroup (4 waves) per (query row, group of <= 64 heads).  All
// heads of a row share the gathered key rows, so the five contractions are small dense
// GEMMs on the 16x16x32 bf16 MFMA:
//   S  [heads x keys]  = Q  [heads x 576] . K^T      wave w owns head tile w
//   dP [heads x keys]  = dO [heads x 512] . K^T
//   dQ [heads x 576]  += dS [heads x keys] . K       (fp32 accumulators in registers)
//   dK [keys x 576]    = dS^T . Q                     wave w owns dK column tiles 9w..9w+8
//   dV [keys x 512]    = P^T  . dO                    wave w owns dV column tiles 8w..8w+7
// Q lives in LDS for the whole row; each chunk of 32 selected keys is gathered into LDS with
// 16-byte loads; dS and P pass through LDS as [key][head] bf16 tiles.  Row-major LDS tiles
// are read in both orientations (direct 16-byte reads, and ds_read_b64_tr_b16 transpose
// reads), so no transposed copies are stored.
//
// The dK/dV contributions of each chunk leave the workgroup either as fp32 atomic adds into
// an fp32 accumulator (default) or as plain stores into a per-pair partial buffer that a
// later ordered reduction sums (deterministic mode).
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

constexpr int kKC = 32;               // selected keys per chunk
constexpr int kThreads = 256;         // 4 waves
constexpr int kQChunks = kDk / 8;     // 72 16-byte chunks per 576-wide row
constexpr int kHtChunks = 64 / 8;     // 8 chunks per 64-wide [key][head] row
constexpr float kLog2e = 1.4426950408889634f;

// LDS carve-up (bytes)
constexpr int kLdsQ = 64 * kDk * 2;            // Qs [64 heads][576]
constexpr int kLdsK = kKC * kDk * 2;           // Ks [32 keys][576]
constexpr int kLdsHT = kKC * 64 * 2;           // DSt / PSt [32 keys][64 heads]
constexpr int kLdsBwd = kLdsQ + kLdsK + 2 * kLdsHT + kKC * 8 + 3 * 64 * 4 + 2 * 257 * 4;

// Stage this row's Q (nope | rope) for heads [h0, h0 + nh) into Qs; rows nh..63 are zero.
__device__ __forceinline__ void load_q_tile(uint16_t* Qs, const uint16_t* q, const uint16_t* qr,
                                            int64_t row, int N1, int h0, int nh) {
  for (int c = threadIdx.x; c < 64 * kQChunks; c += kThreads) {
    const int h = c / kQChunks, part = c % kQChunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < nh) {
      const int64_t hh = row * N1 + h0 + h;
      if (part < 64) v = *reinterpret_cast<const uint4*>(q + hh * kDn + part * 8);
      else if (qr) v = *reinterpret_cast<const uint4*>(qr + hh * kDr + (part - 64) * 8);
    }
    *reinterpret_cast<uint4*>(Qs + swz(h, part * 8, kQChunks)) = v;
  }
}

// Gather the selected key rows (nope | rope) of one chunk into Ks; invalid slots are zero rows.
__device__ __forceinline__ void gather_k_tile(uint16_t* Ks, const uint16_t* k, const uint16_t* kr,
                                              const int64_t* keyrow) {
  for (int c = threadIdx.x; c < kKC * kQChunks; c += kThreads) {
    const int key = c / kQChunks, part = c % kQChunks;
    const int64_t kr_ = keyrow[key];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kr_ >= 0) {
      if (part < 64) v = *reinterpret_cast<const uint4*>(k + kr_ * kDn + part * 8);
      else if (kr) v = *reinterpret_cast<const uint4*>(kr + kr_ * kDr + (part - 64) * 8);
    }
    *reinterpret_cast<uint4*>(Ks + swz(key, part * 8, kQChunks)) = v;
  }
}

template <int kMode>
__global__ void __launch_bounds__(kThreads, 1) bwd_main_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + kLdsQ);
  uint16_t* DSt = reinterpret_cast<uint16_t*>(smem + kLdsQ + kLdsK);
  uint16_t* PSt = reinterpret_cast<uint16_t*>(smem + kLdsQ + kLdsK + kLdsHT);
  int64_t* keyrow = reinterpret_cast<int64_t*>(smem + kLdsQ + kLdsK + 2 * kLdsHT);
  float* sD = reinterpret_cast<float*>(smem + kLdsQ + kLdsK + 2 * kLdsHT + kKC * 8);
  float* sM = sD + 64;
  float* sIL = sM + 64;
  int32_t* cum = reinterpret_cast<int32_t*>(sIL + 64);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = a.row_begin + blockIdx.x;
  const int hg = blockIdx.y;
  const int h0 = hg * 64;
  const int nh = min(64, a.N1 - h0);
  const int ntile = (nh + 15) >> 4;       // head tiles of 16 with at least one real head
  const int kst = (nh + 31) >> 5;         // 32-head K steps of the dK / dV contractions
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);

  if (!geo.active || geo.hi < 0) {
    // padded or empty row: zero dQ / dQRope
    for (int e = threadIdx.x; e < nh * kDn; e += kThreads)
      a.dq[(row * a.N1 + h0) * kDn + e] = 0;
    for (int e = threadIdx.x; e < nh * kDr; e += kThreads)
      if (a.dqr) a.dqr[(row * a.N1 + h0) * kDr + e] = 0;
    return;
  }

  // ---- per-row setup -------------------------------------------------------------------
  load_q_tile(Qs, a.q, a.qr, row, a.N1, h0, nh);
  // statistics and FlashSoftmaxGrad D = rowsum(dO * out), one head per 4 threads
  {
    const int h = threadIdx.x >> 2, part = threadIdx.x & 3;
    float d = 0.f;
    if (h < nh) {
      const uint16_t* dor = a.dout + (row * a.N1 + h0 + h) * kDn + part * 128;
      const uint16_t* otr = a.out + (row * a.N1 + h0 + h) * kDn + part * 128;
      for (int e = 0; e < 128; e += 8) {
        const uint4 x = *reinterpret_cast<const uint4*>(dor + e);
        const uint4 y = *reinterpret_cast<const uint4*>(otr + e);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          d += __uint_as_float(xs[w] << 16) * __uint_as_float(ys[w] << 16);
          d += __uint_as_float(xs[w] & 0xffff0000u) * __uint_as_float(ys[w] & 0xffff0000u);
        }
      }
    }
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    if (part == 0) {
      float m = 0.f, il = 0.f;
      if (h < nh) {
        const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
        const float l = a.ssum[st];
        m = a.smax[st];
        il = l > 0.f ? 1.f / l : 0.f;
      }
      sD[h] = d;
      sM[h] = m * kLog2e;
      sIL[h] = il;
    }
  }
  // dO fragments: A operand of dP for this wave's head tile, B operand of dV for its column tiles.
  // Staged through Ks in two 32-head halves so every global read is a coalesced 16-byte load.
  bf16x8 doA[16];
  bf16x8 doB[8][2];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) doA[ks] = bf16x8{};
#pragma unroll
  for (int ft = 0; ft < 8; ++ft) doB[ft][0] = doB[ft][1] = bf16x8{};
  for (int half = 0; half < kst; ++half) {
    __syncthreads();
    for (int cidx = threadIdx.x; cidx < 32 * 64; cidx += kThreads) {
      const int h = cidx >> 6, part = cidx & 63;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (32 * half + h < nh)
        v = *reinterpret_cast<const uint4*>(a.dout + (row * a.N1 + h0 + 32 * half + h) * kDn + part * 8);
      *reinterpret_cast<uint4*>(Ks + swz(h, part * 8, kQChunks)) = v;
    }
    __syncthreads();
    if ((wave >> 1) == half && wave < ntile) {
      const int hr = 16 * (wave & 1) + c;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) doA[ks] = lds_read8(Ks, hr, 32 * ks + 8 * g, kQChunks);
    }
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) {
      const bf16x8 f = lds_frag_tr(Ks, 0, 16 * (8 * wave + ft), kQChunks, lane);
      if (half == 0) doB[ft][0] = f; else doB[ft][1] = f;
    }
  }
  __syncthreads();
  float mrow[4], ilrow[4], drow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 16 * wave + 4 * g + v;
    mrow[v] = sM[h & 63];
    ilrow[v] = sIL[h & 63];
    drow[v] = sD[h & 63];
  }
  const float zscale = a.scale * kLog2e;

  f32x4 dqacc[36];
#pragma unroll
  for (int ft = 0; ft < 36; ++ft) dqacc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* idxrow = a.idx + row * (a.topk / a.bs);
  const int64_t pair_base = (row - a.row_begin) * a.topk;
  const int nslots = a.topk;

  for (int c0 = 0; c0 < nslots; c0 += kKC) {
    // ---- indices and validity --------------------------------------------------------
    int any = 0;
    if (threadIdx.x < kKC) {
      const int s = c0 + threadIdx.x;
      int64_t kr_ = -1;
      if (s < nslots) {
        const int j = slot_key(idxrow, s, a.bs);
        if (j >= 0 && j <= geo.hi) kr_ = geo.kstart + j;
      }
      keyrow[threadIdx.x] = kr_;
      any = kr_ >= 0;
    }
    if (!__syncthreads_or(any)) continue;

    // ---- gather ------------------------------------------------------------------------
    gather_k_tile(Ks, a.k, a.kr, keyrow);
    __syncthreads();

    // ---- S, dP, P, dS for this wave's head tile ------------------------------------------
    if (wave < ntile) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 pacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kDk / 32; ++ks) {
        const bf16x8 qa = lds_read8(Qs, 16 * wave + c, 32 * ks + 8 * g, kQChunks);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kb = lds_read8(Ks, 16 * kt + c, 32 * ks + 8 * g, kQChunks);
          sacc[kt] = mfma(qa, kb, sacc[kt]);
          if (ks < 16) pacc[kt] = mfma(doA[ks], kb, pacc[kt]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bool valid = keyrow[16 * kt + c] >= 0;
        uint16_t pb[4], db[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = valid ? exp2f(sacc[kt][v] * zscale - mrow[v]) * ilrow[v] : 0.f;
          const float ds = p * (pacc[kt][v] - drow[v]);
          pb[v] = f2bf(p);
          db[v] = f2bf(ds);
        }
        const int key = 16 * kt + c, hcol = 16 * wave + 4 * g;
        const uint2 pw = make_uint2(pb[0] | ((uint32_t)pb[1] << 16), pb[2] | ((uint32_t)pb[3] << 16));
        const uint2 dw = make_uint2(db[0] | ((uint32_t)db[1] << 16), db[2] | ((uint32_t)db[3] << 16));
        *reinterpret_cast<uint2*>(PSt + swz(key, hcol, kHtChunks)) = pw;
        *reinterpret_cast<uint2*>(DSt + swz(key, hcol, kHtChunks)) = dw;
      }
    } else if (16 * wave < 32 * kst) {
      // zero-pad head columns that the 32-deep dK / dV contractions read
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 16 * kt + c, hcol = 16 * wave + 4 * g;
        *reinterpret_cast<uint2*>(PSt + swz(key, hcol, kHtChunks)) = make_uint2(0, 0);
        *reinterpret_cast<uint2*>(DSt + swz(key, hcol, kHtChunks)) = make_uint2(0, 0);
      }
    }
    __syncthreads();

    // ---- dQ += dS K  (this wave's head tile, all 36 column tiles) -------------------------
    if (wave < ntile) {
      const bf16x8 dsa = lds_frag_tr(DSt, 0, 16 * wave, kHtChunks, lane);
#pragma unroll
      for (int ft = 0; ft < 36; ++ft) {
        const bf16x8 kb = lds_frag_tr(Ks, 0, 16 * ft, kQChunks, lane);
        dqacc[ft] = mfma(dsa, kb, dqacc[ft]);
      }
    }

    // ---- dK = scale dS^T Q, dV = P^T dO for this chunk ----------------------------------------
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      bf16x8 sa[2], pa[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        sa[ks] = ks < kst ? lds_read8(DSt, 16 * kt + c, 32 * ks + 8 * g, kHtChunks) : bf16x8{};
        pa[ks] = ks < kst ? lds_read8(PSt, 16 * kt + c, 32 * ks + 8 * g, kHtChunks) : bf16x8{};
      }
      int64_t outrow[4];
      int64_t pairrow[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = 16 * kt + 4 * g + v;
        outrow[v] = keyrow[key];
        pairrow[v] = ((int64_t)hg * a.pairs_per_launch + pair_base + c0 + key) * kDacc;
      }
      // dK | dKRope columns
      for (int t = 0; t < 9; ++t) {
        const int ft = 9 * wave + t;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < kst; ++ks)
          acc = mfma(sa[ks], lds_frag_tr(Qs, 32 * ks, 16 * ft, kQChunks, lane), acc);
        const int col = 16 * ft + c;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (outrow[v] < 0) continue;
          const float val = acc[v] * a.scale;
          if (kMode == 0)
            __hip_atomic_fetch_add(a.acc + outrow[v] * kDacc + col, val, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          else
            a.partial[pairrow[v] + col] = val;
        }
      }
      // dV columns
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        acc = mfma(pa[0], doB[t][0], acc);
        if (kst > 1) acc = mfma(pa[1], doB[t][1], acc);
        const int col = kDk + 16 * (8 * wave + t) + c;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (outrow[v] < 0) continue;
          if (kMode == 0)
            __hip_atomic_fetch_add(a.acc + outrow[v] * kDacc + col, acc[v], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          else
            a.partial[pairrow[v] + col] = acc[v];
        }
      }
    }
    __syncthreads();
  }

  // ---- dQ / dQRope out ------------------------------------------------------------------
  if (wave < ntile) {
#pragma unroll
    for (int ft = 0; ft < 36; ++ft) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * wave + 4 * g + v;
        if (h >= nh) continue;
        const int col = 16 * ft + c;
        const uint16_t bv = f2bf(dqacc[ft][v] * a.scale);
        const int64_t hh = row * a.N1 + h0 + h;
        if (col < kDn) a.dq[hh * kDn + col] = bv;
        else if (a.dqr) a.dqr[hh * kDr + col - kDn] = bv;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Small kernels: accumulator fill, fp32 -> bf16 cast, deterministic sort keys and reduction.
// ------------------------------------------------------------------------------------------

__global__ void fill_zero_kernel(float4* p, int64_t n4) {
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// acc [keys][dK 512 | dKRope 64 | dV 512] fp32 -> dk [keys][512], dkr [keys][64], dv [keys][512]
__global__ void cast_kernel(const float* acc, uint16_t* dk, uint16_t* dkr, uint16_t* dv, int64_t keys) {
  const int64_t n = keys * (kDacc / 4);
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / (kDacc / 4);
    const int col = (int)(e % (kDacc / 4)) * 4;
    const float4 x = *reinterpret_cast<const float4*>(acc + r * kDacc + col);
    const uint2 w = make_uint2(f2bf(x.x) | ((uint32_t)f2bf(x.y) << 16), f2bf(x.z) | ((uint32_t)f2bf(x.w) << 16));
    if (col < kDn) *reinterpret_cast<uint2*>(dk + r * kDn + col) = w;
    else if (col < kDk) {
      if (dkr) *reinterpret_cast<uint2*>(dkr + r * kDr + col - kDn) = w;
    }
    else *reinterpret_cast<uint2*>(dv + r * kDn + col - kDk) = w;
  }
}

// sort key of every (row, slot) of the launch: (key row << 32) | pair, or ~0 for skipped slots
__global__ void pair_keys_kernel(BwdArgs a, uint64_t* keys, int64_t nrows) {
  __shared__ int32_t cum[2 * 257];
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const int64_t n = nrows * a.topk;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = a.row_begin + e / a.topk;
    const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, r, a.mode3);
    const int j = slot_key(a.idx + r * (a.topk / a.bs), (int)(e % a.topk), a.bs);
    uint64_t kv = ~0ull;
    if (geo.active && j >= 0 && j <= geo.hi) kv = ((uint64_t)(geo.kstart + j) << 32) | (uint64_t)e;
    keys[e] = kv;
  }
}

__device__ __forceinline__ int64_t lower_bound64(const uint64_t* a, int64_t n, uint64_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// acc[key] += sum over the launch's pairs of that key, in ascending pair order, head groups
// in ascending order within a pair.  One workgroup per key row.
__global__ void __launch_bounds__(256) det_reduce_kernel(const uint64_t* sorted, int64_t n,
                                                         const float* partial, int64_t pairs_per_launch,
                                                         int hg_count, float* acc, int64_t key_begin) {
  const int64_t key = key_begin + blockIdx.x;
  __shared__ int64_t range[2];
  if (threadIdx.x == 0) {
    range[0] = lower_bound64(sorted, n, (uint64_t)key << 32);
    range[1] = lower_bound64(sorted, n, (uint64_t)(key + 1) << 32);
  }
  __syncthreads();
  const int64_t lo = range[0], hi = range[1];
  if (lo >= hi) return;
  for (int col = threadIdx.x; col < kDacc; col += blockDim.x) {
    float s = 0.f;
    for (int64_t e = lo; e < hi; ++e) {
      const int64_t pair = (int64_t)(sorted[e] & 0xffffffffull);
      for (int h = 0; h < hg_count; ++h) s += partial[((int64_t)h * pairs_per_launch + pair) * kDacc + col];
    }
    acc[key * kDacc + col] += s;
  }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------

hipError_t launch_bwd_main(const BwdArgs& a, int64_t nrows, int hg_count, int mode, hipStream_t st) {
  dim3 grid((unsigned)nrows, (unsigned)hg_count);
  if (mode == 1)
    hipLaunchKernelGGL(bwd_main_kernel<1>, grid, dim3(kThreads), kLdsBwd, st, a);
  else
    hipLaunchKernelGGL(bwd_main_kernel<0>, grid, dim3(kThreads), kLdsBwd, st, a);
  return hipGetLastError();
}

hipError_t set_bwd_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_main_kernel<0>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBwd);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_main_kernel<1>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBwd);
}

hipError_t launch_fill_zero(float* p, int64_t nfloats, hipStream_t st) {
  const int64_t n4 = nfloats / 4;
  if (n4 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_cast(const float* acc, uint16_t* dk, uint16_t* dkr, uint16_t* dv, int64_t keys,
                       hipStream_t st) {
  const int64_t n = keys * (kDacc / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(cast_kernel, dim3(blocks), dim3(256), 0, st, acc, dk, dkr, dv, keys);
  return hipGetLastError();
}

hipError_t launch_pair_keys(const BwdArgs& a, uint64_t* keys, int64_t nrows, hipStream_t st) {
  const int64_t n = nrows * a.topk;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(pair_keys_kernel, dim3(blocks), dim3(256), 0, st, a, keys, nrows);
  return hipGetLastError();
}

hipError_t launch_det_reduce(const uint64_t* sorted, int64_t n, const float* partial,
                             int64_t pairs_per_launch, int hg_count, float* acc, int64_t keys,
                             hipStream_t st) {
  // grid.x is limited to 2^31 - 1; key rows are at most 256 * 131072
  hipLaunchKernelGGL(det_reduce_kernel, dim3((unsigned)keys), dim3(256), 0, st, sorted, n, partial,
                     pairs_per_launch, hg_count, acc, (int64_t)0);
  return hipGetLastError();
}

}  // namespace sfag
