// sfag_fwd.hip -- sparse attention forward over the selected keys (gfx950).
//
// Produces the backward's inputs out, softmaxMax and softmaxSum: per query row and head,
// over the valid selected slots, z = scale (q.k + qRope.kRope), softmaxMax = max z,
// softmaxSum = sum exp(z - max), out = sum softmax(z) v with v = k[:512] (SparseAttnSharedkv
// README, "function description": O = softmax(Q K~^T scale) V~ with K~ = V~; the statistics
// are the forward intermediates the SparseFlashAttentionGrad page names).
//
// Same decomposition as the backward: one workgroup per (row, <= 64 heads), Q in LDS, 32-key
// chunks gathered into LDS, S = Q K^T on 16x16x32 bf16 MFMA, an online softmax with running
// max / sum per head, and O += P V with P passed through LDS and V read with transpose loads.
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kKC = 32;
constexpr int kThreads = 256;
constexpr int kQChunks = kDk / 8;
constexpr int kHtChunks = 64 / 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsQ = 64 * kDk * 2;
constexpr int kLdsK = kKC * kDk * 2;
constexpr int kLdsHT = kKC * 64 * 2;
constexpr int kLdsFwd = kLdsQ + kLdsK + kLdsHT + kKC * 8 + 2 * 257 * 4;
}  // namespace

template <bool F16>
__global__ void __launch_bounds__(kThreads, 1) fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + kLdsQ);
  uint16_t* PSt = reinterpret_cast<uint16_t*>(smem + kLdsQ + kLdsK);
  int64_t* keyrow = reinterpret_cast<int64_t*>(smem + kLdsQ + kLdsK + kLdsHT);
  int32_t* cum = reinterpret_cast<int32_t*>(smem + kLdsQ + kLdsK + kLdsHT + kKC * 8);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = blockIdx.x;
  const int h0 = blockIdx.y * 64;
  const int nh = min(64, a.N1 - h0);
  const int ntile = (nh + 15) >> 4;
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);

  if (!geo.active || geo.hi < 0) {
    for (int e = threadIdx.x; e < nh * kDn; e += kThreads) a.out[(row * a.N1 + h0) * kDn + e] = 0;
    for (int h = threadIdx.x; h < nh; h += kThreads) {
        const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
        a.smax[st] = 0.f;
        a.ssum[st] = 0.f;
    }
    return;
  }

  for (int cc = threadIdx.x; cc < 64 * kQChunks; cc += kThreads) {
    const int h = cc / kQChunks, part = cc % kQChunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < nh) {
      const int64_t hh = row * a.N1 + h0 + h;
      v = part < 64 ? *reinterpret_cast<const uint4*>(a.q + hh * kDn + part * 8)
                    : (a.qr ? *reinterpret_cast<const uint4*>(a.qr + hh * kDr + (part - 64) * 8) : uint4{0, 0, 0, 0});
    }
    *reinterpret_cast<uint4*>(Qs + swz(h, part * 8, kQChunks)) = v;
  }

  const float zscale = a.scale * kLog2e;
  float mrun[4], lrun[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { mrun[v] = -INFINITY; lrun[v] = 0.f; }
  f32x4 oacc[32];
#pragma unroll
  for (int ft = 0; ft < 32; ++ft) oacc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* idxrow = a.idx + row * (a.topk / a.bs);
  for (int c0 = 0; c0 < a.topk; c0 += kKC) {
    int any = 0;
    if (threadIdx.x < kKC) {
      const int s = c0 + threadIdx.x;
      int64_t kr_ = -1;
      if (s < a.topk) {
        const int j = slot_key(idxrow, s, a.bs);
        if (j >= 0 && j <= geo.hi) kr_ = geo.kstart + j;
      }
      keyrow[threadIdx.x] = kr_;
      any = kr_ >= 0;
    }
    if (!__syncthreads_or(any)) continue;
    for (int cc = threadIdx.x; cc < kKC * kQChunks; cc += kThreads) {
      const int key = cc / kQChunks, part = cc % kQChunks;
      const int64_t kr_ = keyrow[key];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kr_ >= 0)
        v = part < 64 ? *reinterpret_cast<const uint4*>(a.k + kr_ * kDn + part * 8)
                      : (a.kr ? *reinterpret_cast<const uint4*>(a.kr + kr_ * kDr + (part - 64) * 8) : uint4{0, 0, 0, 0});
      *reinterpret_cast<uint4*>(Ks + swz(key, part * 8, kQChunks)) = v;
    }
    __syncthreads();

    if (wave < ntile) {
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kDk / 32; ++ks) {
        const bf16x8 qa = lds_read8(Qs, 16 * wave + c, 32 * ks + 8 * g, kQChunks);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          sacc[kt] = mfma_t<F16>(qa, lds_read8(Ks, 16 * kt + c, 32 * ks + 8 * g, kQChunks), sacc[kt]);
      }
      float z[2][4];
      float cmax[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) cmax[v] = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bool valid = keyrow[16 * kt + c] >= 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          z[kt][v] = valid ? sacc[kt][v] * zscale : -INFINITY;
          cmax[v] = fmaxf(cmax[v], z[kt][v]);
        }
      }
      // max over the 16 lanes that hold the other keys of the same heads
#pragma unroll
      for (int v = 0; v < 4; ++v)
        for (int o = 1; o < 16; o <<= 1) cmax[v] = fmaxf(cmax[v], __shfl_xor(cmax[v], o));
      float alpha[4], mnew[4], psum[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        mnew[v] = fmaxf(mrun[v], cmax[v]);
        alpha[v] = mrun[v] == -INFINITY ? 0.f : exp2f(mrun[v] - mnew[v]);
        psum[v] = 0.f;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        uint16_t pb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = z[kt][v] == -INFINITY ? 0.f : exp2f(z[kt][v] - mnew[v]);
          psum[v] += p;
          pb[v] = f2x<F16>(p);
        }
        const int key = 16 * kt + c, hcol = 16 * wave + 4 * g;
        *reinterpret_cast<uint2*>(PSt + swz(key, hcol, kHtChunks)) =
            make_uint2(pb[0] | ((uint32_t)pb[1] << 16), pb[2] | ((uint32_t)pb[3] << 16));
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        for (int o = 1; o < 16; o <<= 1) psum[v] += __shfl_xor(psum[v], o);
        lrun[v] = lrun[v] * alpha[v] + psum[v];
        mrun[v] = mnew[v];
      }
#pragma unroll
      for (int ft = 0; ft < 32; ++ft)
#pragma unroll
        for (int v = 0; v < 4; ++v) oacc[ft][v] *= alpha[v];
    }
    __syncthreads();
    if (wave < ntile) {
      const bf16x8 pa = lds_frag_tr(PSt, 0, 16 * wave, kHtChunks, lane);
#pragma unroll
      for (int ft = 0; ft < 32; ++ft) oacc[ft] = mfma_t<F16>(pa, lds_frag_tr(Ks, 0, 16 * ft, kQChunks, lane), oacc[ft]);
    }
    __syncthreads();
  }

  if (wave < ntile) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * wave + 4 * g + v;
      if (h >= nh) continue;
      const float inv = lrun[v] > 0.f ? 1.f / lrun[v] : 0.f;
      const int64_t hh = row * a.N1 + h0 + h;
#pragma unroll
      for (int ft = 0; ft < 32; ++ft) a.out[hh * kDn + 16 * ft + c] = f2x<F16>(oacc[ft][v] * inv);
      if (c == 0) {
        const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
        a.smax[st] = lrun[v] > 0.f ? mrun[v] / kLog2e : 0.f;
        a.ssum[st] = lrun[v];
      }
    }
  }
}

hipError_t launch_fwd(const FwdArgs& a, int64_t nrows, int hg_count, hipStream_t st) {
  if (a.f16)
    hipLaunchKernelGGL(fwd_kernel<true>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), kLdsFwd, st, a);
  else
    hipLaunchKernelGGL(fwd_kernel<false>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), kLdsFwd, st, a);
  return hipGetLastError();
}

hipError_t set_fwd_attributes() {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<false>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsFwd);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_kernel<true>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsFwd);
}

}  // namespace sfag
