// sfag_q.hip -- query-major half of the SparseFlashAttentionGrad backward for the key-major
// dK / dV path (gfx950).
//
// Per query row and group of <= 64 heads, over the row's valid key positions in ascending
// order (sorted beforehand), in chunks of 32 keys:
//   S  = Q K^T, dP = dO V^T (V = K, the page's value-equals-key constraint)      [MFMA]
//   P  = exp(S scale - softmaxMax) / softmaxSum,  dS = P (dP - rowsum(dO * out))   [registers]
//   dQ += dS K                                                                     [MFMA]
// and the bf16 dS and P of every (row, key) pair are written as a 256-byte record for the
// key-major kernel that forms dK = scale dS^T Q and dV = P^T dO (SparseFlashAttentionGrad
// README, "function description", stages 1-3).
//
// Pipeline: the gathered key chunk is double-buffered in LDS.  While chunk c is multiplied,
// the K rows of chunk c+1 stream from global memory directly into the other buffer
// (global_load_lds; their key rows were staged in LDS one chunk earlier); two barriers per
// chunk.
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kKC = 32;
constexpr int kThreads = 256;
constexpr int kPitch = kDk + 8;                  // 584: padded row of Q / key tiles
constexpr int kRowChunks = kPitch / 8;           // 73 16-byte chunks per padded row
constexpr int kHtPitch = 64 + 8;                 // DSt row pitch
constexpr int kBlocks = (kKC * kRowChunks + 63) / 64;   // 37 blocks of 64 chunks per key tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsQ = 64 * kPitch * 2;           // Qs [64 heads][584]
constexpr int kLdsK = kBlocks * 64 * 16;         // one key chunk [32][584], rounded to whole blocks
constexpr int kLdsHT = kKC * kHtPitch * 2;       // DSt [32 keys][72]
constexpr int kLdsTotal = kLdsQ + 2 * kLdsK + kLdsHT + 3 * kKC * 8 + 3 * 64 * 4 + 2 * 257 * 4;
static_assert(kLdsTotal <= 160 * 1024, "LDS budget");
}  // namespace

__global__ void __launch_bounds__(kThreads, 1) bwd_q_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Ks0 = reinterpret_cast<uint16_t*>(smem + kLdsQ);
  uint16_t* Ks1 = reinterpret_cast<uint16_t*>(smem + kLdsQ + kLdsK);
  uint16_t* DSt = reinterpret_cast<uint16_t*>(smem + kLdsQ + 2 * kLdsK);
  int64_t* krow3 = reinterpret_cast<int64_t*>(smem + kLdsQ + 2 * kLdsK + kLdsHT);   // [3][32]
  float* sD = reinterpret_cast<float*>(krow3 + 3 * kKC);
  float* sM = sD + 64;
  float* sIL = sM + 64;
  int32_t* cum = reinterpret_cast<int32_t*>(sIL + 64);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = blockIdx.x;
  const int hg = blockIdx.y;
  const int h0 = hg * 64;
  const int nh = min(64, a.N1 - h0);
  const int ntile = (nh + 15) >> 4;
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  const int count = a.count[row];
  if (!geo.active || geo.hi < 0 || count == 0) {
    for (int e = threadIdx.x; e < nh * kDn; e += kThreads) a.dq[(row * a.N1 + h0) * kDn + e] = 0;
    for (int e = threadIdx.x; e < nh * kDr; e += kThreads) a.dqr[(row * a.N1 + h0) * kDr + e] = 0;
    return;
  }
  const int32_t* srow = a.sorted + row * a.topk;
  const int nchunk = (count + kKC - 1) / kKC;

  // ---- per-row setup: Q tile, statistics, D = rowsum(dO * out) ---------------------------
  for (int cc = threadIdx.x; cc < 64 * (kDk / 8); cc += kThreads) {
    const int h = cc / (kDk / 8), part = cc % (kDk / 8);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < nh) {
      const int64_t hh = row * a.N1 + h0 + h;
      v = part < 64 ? *reinterpret_cast<const u32x4*>(a.q + hh * kDn + part * 8)
                    : *reinterpret_cast<const u32x4*>(a.qr + hh * kDr + (part - 64) * 8);
    }
    *reinterpret_cast<u32x4*>(Qs + h * kPitch + part * 8) = v;
  }
  {
    const int h = threadIdx.x >> 2, part = threadIdx.x & 3;
    float d = 0.f;
    if (h < nh) {
      const uint16_t* dor = a.dout + (row * a.N1 + h0 + h) * kDn + part * 128;
      const uint16_t* otr = a.out + (row * a.N1 + h0 + h) * kDn + part * 128;
      for (int e = 0; e < 128; e += 8) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(dor + e);
        const u32x4 y = *reinterpret_cast<const u32x4*>(otr + e);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          d += __uint_as_float(x[w] << 16) * __uint_as_float(y[w] << 16);
          d += __uint_as_float(x[w] & 0xffff0000u) * __uint_as_float(y[w] & 0xffff0000u);
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
  // dO A fragments for this wave's head tile, staged through the key buffers
  bf16x8 doA[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) doA[ks] = bf16x8{};
  {
    uint16_t* stage = Ks0;   // 64 x 584 elements span both key buffers
    for (int cc = threadIdx.x; cc < 64 * 64; cc += kThreads) {
      const int h = cc >> 6, part = cc & 63;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (h < nh) v = *reinterpret_cast<const u32x4*>(a.dout + (row * a.N1 + h0 + h) * kDn + part * 8);
      *reinterpret_cast<u32x4*>(stage + h * kPitch + part * 8) = v;
    }
    __syncthreads();
    if (wave < ntile) {
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) doA[ks] = lds_read8p(stage, 16 * wave + c, 32 * ks + 8 * g, kPitch);
    }
  }
  // key rows of chunks 0 and 1
  if (threadIdx.x < 2 * kKC) {
    const int e = threadIdx.x;
    krow3[e] = e < count ? geo.kstart + srow[e] : -1;
  }
  __syncthreads();
  float mrow[4], ilrow[4], drow[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = (16 * wave + 4 * g + v) & 63;
    mrow[v] = sM[h];
    ilrow[v] = sIL[h];
    drow[v] = sD[h];
  }
  const float zscale = a.scale * kLog2e;

  // Gather of one 32-key chunk straight from global memory into a key buffer: the buffer is
  // 37 blocks of 64 consecutive 16-byte chunks, and lane i of a block lands at chunk
  // block * 64 + i (global_load_lds), so each lane loads the source chunk of that position.
  // Padding positions and slots past the row's valid count read the zero row.
#define SFAG_GATHER_ASYNC(KS, KR)                                                              \
  {                                                                                            \
    for (int blk = wave; blk < kBlocks; blk += 4) {                                            \
      const int P = blk * 64 + lane;                                                           \
      const int rk = P / kRowChunks, lc = P % kRowChunks;                                      \
      const int64_t r = rk < kKC ? (KR)[rk] : -1;                                              \
      const uint16_t* src = (r < 0 || lc >= kDk / 8) ? a.zero_row                              \
                          : (lc < 64 ? a.k + r * kDn + lc * 8 : a.kr + r * kDr + (lc - 64) * 8); \
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KS) + blk * 512), 16, 0, 0); \
    }                                                                                          \
  }

  f32x4 dqacc[36];
#pragma unroll
  for (int ft = 0; ft < 36; ++ft) dqacc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};

  SFAG_GATHER_ASYNC(Ks0, krow3)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int ci = 0; ci < nchunk; ++ci) {
    const int c0 = ci * kKC;
    uint16_t* Ks = (ci & 1) ? Ks1 : Ks0;
    uint16_t* Kn = (ci & 1) ? Ks0 : Ks1;
    const int64_t* kr_cur = krow3 + (ci % 3) * kKC;
    const int64_t* kr_nxt = krow3 + ((ci + 1) % 3) * kKC;
    // loads of chunk ci+1 and the key rows of chunk ci+2 go out first
    const bool more = ci + 1 < nchunk;
    if (more) SFAG_GATHER_ASYNC(Kn, kr_nxt)
    int64_t kr2 = -1;
    if (threadIdx.x < kKC) {
      const int e = c0 + 2 * kKC + threadIdx.x;
      if (e < count) kr2 = geo.kstart + srow[e];
    }

    // ---- S, dP, P, dS for this wave's head tile --------------------------------------------
    if (wave < ntile) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 pacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kDk / 32; ++ks) {
        const bf16x8 qa = lds_read8p(Qs, 16 * wave + c, 32 * ks + 8 * g, kPitch);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kb = lds_read8p(Ks, 16 * kt + c, 32 * ks + 8 * g, kPitch);
          sacc[kt] = mfma(qa, kb, sacc[kt]);
          if (ks < 16) pacc[kt] = mfma(doA[ks], kb, pacc[kt]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 16 * kt + c;
        const bool valid = kr_cur[key] >= 0;
        uint32_t pw[2], dw[2];
#pragma unroll
        for (int v2 = 0; v2 < 2; ++v2) {
          uint32_t pbits = 0, dbits = 0;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int v = 2 * v2 + h2;
            const float p = valid ? exp2f(sacc[kt][v] * zscale - mrow[v]) * ilrow[v] : 0.f;
            const float ds = p * (pacc[kt][v] - drow[v]);
            pbits |= (uint32_t)f2bf(p) << (16 * h2);
            dbits |= (uint32_t)f2bf(ds) << (16 * h2);
          }
          pw[v2] = pbits;
          dw[v2] = dbits;
        }
        const int hcol = 16 * wave + 4 * g;
        *reinterpret_cast<uint2*>(DSt + key * kHtPitch + hcol) = make_uint2(dw[0], dw[1]);
        if (valid) {
          uint16_t* rec = a.dsp + (((int64_t)row * a.topk + c0 + key) * a.hgc + hg) * 128;
          *reinterpret_cast<uint2*>(rec + hcol) = make_uint2(dw[0], dw[1]);
          *reinterpret_cast<uint2*>(rec + 64 + hcol) = make_uint2(pw[0], pw[1]);
        }
      }
    } else {
      // head columns without real heads: zero records (the key-major kernel reads 64 heads)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 16 * kt + c;
        if (kr_cur[key] >= 0) {
          const int hcol = 16 * wave + 4 * g;
          uint16_t* rec = a.dsp + (((int64_t)row * a.topk + c0 + key) * a.hgc + hg) * 128;
          *reinterpret_cast<uint2*>(rec + hcol) = make_uint2(0, 0);
          *reinterpret_cast<uint2*>(rec + 64 + hcol) = make_uint2(0, 0);
        }
      }
    }
    __syncthreads();

    // ---- dQ += dS K --------------------------------------------------------------------------
    if (wave < ntile) {
      const bf16x8 dsa = lds_frag_trp(DSt, 0, 16 * wave, kHtPitch, lane);
#pragma unroll
      for (int ft = 0; ft < 36; ++ft) dqacc[ft] = mfma(dsa, lds_frag_trp(Ks, 0, 16 * ft, kPitch, lane), dqacc[ft]);
    }
    if (threadIdx.x < kKC) krow3[((ci + 2) % 3) * kKC + threadIdx.x] = kr2;
    __builtin_amdgcn_s_waitcnt(0);      // the next chunk's direct-to-LDS loads have landed
    __syncthreads();
  }

  // ---- dQ / dQRope out ------------------------------------------------------------------------
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
        else a.dqr[hh * kDr + col - kDn] = bv;
      }
    }
  }
}

#undef SFAG_GATHER_ASYNC

hipError_t launch_bwd_q(const BwdArgs& a, int64_t nrows, int hg_count, hipStream_t st) {
  hipLaunchKernelGGL(bwd_q_kernel, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), kLdsTotal, st, a);
  return hipGetLastError();
}

hipError_t set_q_attributes() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_q_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsTotal);
}

}  // namespace sfag
