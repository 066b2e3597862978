// sfag_fwd.hip -- sparse attention forward over the selected keys (gfx950).
//
// Produces the backward's inputs out, softmaxMax and softmaxSum: per query row and head, over
// the valid selected slots, z = scale (q.k + qRope.kRope), softmaxMax = max z, softmaxSum =
// sum exp(z - max), out = sum softmax(z) v with v = k[:512] (SparseAttnSharedkv README,
// "function description": O = softmax(Q K~^T scale) V~ with K~ = V~; the statistics are the
// forward intermediates the SparseFlashAttentionGrad page names).
//
// One workgroup of 8 waves per (row, group of <= 64 heads), over the row's slots in chunks of
// 32 (slots past the row's last valid one are not visited; invalid slots inside are masked):
//   score waves (0-3): wave w keeps Q | QRope of heads 16 w .. + 15 in registers, forms S for
//     both 16-key tiles of the chunk on the 16x16x32 MFMA, and accumulates P = exp(S - mu)
//     (zero for invalid slots) against a fixed reference mu per head: the max of the first chunk
//     with a valid slot.  The running max m is kept alongside; P goes to LDS as a [key][head]
//     tile.  No accumulator is ever rescaled.  If some head's m rises more than kLazy (log2
//     units) above its mu -- P would no longer be bounded by 2^kLazy -- the row is computed a
//     second time with mu = the final m of every head (P <= 1 then).  At the end softmaxMax = m
//     and softmaxSum = sum P exp(mu - m), the statistics of the true max.
//   output waves (4-7): wave 4 + w owns output dims 128 w .. + 127 of all 64 heads (fp32
//     accumulators across all chunks); in step c it adds P V of chunk c - 1 (transposing LDS
//     reads of P and of the key tile's value dims); it also gathers the key rows of chunk c + 2
//     straight from global memory into LDS (global_load_lds, 16 bytes per lane) and marks which
//     of that chunk's slots are valid.
// One barrier per step; key tiles quadruple-buffered (a gather has two steps to land), P tiles
// double-buffered.  Key tiles use the swizzled [chunk group][key][slot] layout of
// sfag_ktile.h: output wave w gathers keys 8 w .. 8 w + 7 of every chunk, eight whole 128-byte
// runs of key rows per load.
#include "sfag_device.h"
#include "sfag_dpp.h"
#include "sfag_ktile.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kKC = 32;
constexpr int kThreads = 512;                    // 4 score waves + 4 output waves
constexpr int kChunks = kDk / 8;                 // 72 16-byte chunks per key row (64 value + 8 rope)
constexpr int kHtPitch = 64 + 8;                 // P tile row pitch
constexpr int kBlocks = kChunks / 2;             // 36 direct-to-LDS blocks of 1 KB per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 15.f;                    // bound on m - mu (log2 units): P <= 2^15 fits fp16
constexpr int kLdsK = kBlocks * 64 * 16;         // one key tile
static_assert(kLdsK == kTileBytes, "key tile size");
// s_waitcnt operands with expcnt and lgkmcnt at zero: vmcnt(9) (all but the 9 loads of the
// newest gather) and vmcnt(10) (all but a gather and one position load)
constexpr int kWaitVm9 = 0x0009;
constexpr int kWaitVm10 = 0x000a;
}  // namespace

template <bool F16>
__global__ void __launch_bounds__(kThreads, 1) fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Kb0[kLdsK / 2], Kb1[kLdsK / 2], Kb2[kLdsK / 2], Kb3[kLdsK / 2];
  __shared__ __attribute__((aligned(16))) uint16_t Pb0[kKC * kHtPitch], Pb1[kKC * kHtPitch];
  __shared__ __attribute__((aligned(16))) float sIL[64];
  __shared__ int32_t sVal[4][kKC];
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t s_last, s_over[2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool swave = wave < 4;
  const int rw = wave & 3;
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = (int64_t)gridDim.x - 1 - blockIdx.x;     // long rows first
  const int hg = blockIdx.y;
  const int h0 = hg * 64;
  const int nh = min(64, a.N1 - h0);
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  const int32_t* irow = a.idx + row * (a.topk / a.bs);
  // slots past the last valid one are never visited
  if (threadIdx.x == 0) {
    s_last = -1;
    s_over[0] = s_over[1] = 0;
  }
  __syncthreads();
  if (geo.active && geo.hi >= 0) {
    int last = -1;
    for (int s = threadIdx.x; s < a.topk; s += kThreads) {
      const int j = slot_key(irow, s, a.bs);
      if (j >= 0 && j <= geo.hi) last = s;
    }
    if (last >= 0) atomicMax(&s_last, last);
  }
  __syncthreads();
  const int nslots = s_last + 1;
  if (nslots == 0) {
    for (int e = threadIdx.x; e < nh * kDn; e += kThreads) a.out[(row * a.N1 + h0) * kDn + e] = 0;
    for (int h = threadIdx.x; h < nh; h += kThreads) {
      const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
      a.smax[st] = 0.f;
      a.ssum[st] = 0.f;
    }
    return;
  }
  const int nchunk = (nslots + kKC - 1) / kKC;
  const float zscale = a.scale * kLog2e;

  auto uniform = [](const void* p) {               // a workgroup-uniform pointer, made scalar
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<uint16_t*>(((uint64_t)hi << 32) | lo);
  };
  const uint16_t* kbase = uniform(a.k + geo.kstart * kDn);
  const bool rope = a.kr != nullptr;
  // without rope inputs the rope chunks are read from the key's value row (their Q is zero)
  const uint16_t* krbase = uniform(rope ? a.kr + geo.kstart * kDr : a.k + geo.kstart * kDn);
  asm volatile("" : "+s"(kbase), "+s"(krbase));

  if (swave) {
    // Q | QRope fragments (A operands of S: lane (g, c) holds head 16 rw + c, dims 32 ks + 8 g)
    bf16x8 qA[18];
    {
      const int h = 16 * rw + c;
      const bool hv = h < nh;
      const int64_t hrow = row * a.N1 + h0 + (hv ? h : 0);
      const uint16_t* qrow = a.q + hrow * kDn + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
        qA[ks] = hv ? qv : bf16x8{};
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        qA[16 + ks] = bf16x8{};
        if (hv && a.qr) qA[16 + ks] = *reinterpret_cast<const bf16x8*>(a.qr + hrow * kDr + 32 * ks + 8 * g);
      }
    }
    const int kse = ktile_off(g, c);                // chunk g of key c
    f32x4 sacc[2];
    // state of heads 16 rw + 4 g + v (log2 domain of the scaled logits): running max m and
    // reference mu (the same in the 16 lanes of a head), this lane's part of the sum of P
    float m[4], mu[4], l[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) mu[v] = -INFINITY;
    for (int pass = 0;; ++pass) {
      bool over = false;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        m[v] = -INFINITY;
        l[v] = 0.f;
      }
      lds_barrier();                                // chunks 0, 1 gathered, their slots marked
// Scores and P of chunk CI on key buffer KS into P buffer PD.
#define SFAG_FSTEP(CI, KS, PD)                                                                 \
  {                                                                                            \
    if ((CI) < nchunk) {                                                                       \
      sacc[0] = sacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};                                           \
      /* step ks reads chunk 4 ks + g of keys c and 16 + c: group ks / 2, slot bit 2 = ks % 2 */ \
      const uint16_t* kre = (KS) + kse;                                                        \
      const uint16_t* kro = (KS) + (kse ^ 32);                                                 \
      bf16x8 kf0[18], kf1[18];                                                                 \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                       \
        const uint16_t* kr_ = (ks & 1) ? kro : kre;                                            \
        kf0[ks] = *reinterpret_cast<const bf16x8*>(kr_ + (ks >> 1) * 2048);                    \
        kf1[ks] = *reinterpret_cast<const bf16x8*>(kr_ + (ks >> 1) * 2048 + 1024);             \
      }                                                                                        \
      _Pragma("unroll") for (int ks = 0; ks < 18; ++ks) {                                      \
        if (ks + 2 < 18) {                                                                     \
          const uint16_t* kr_ = ((ks + 2) & 1) ? kro : kre;                                    \
          kf0[ks + 2] = *reinterpret_cast<const bf16x8*>(kr_ + ((ks + 2) >> 1) * 2048);        \
          kf1[ks + 2] = *reinterpret_cast<const bf16x8*>(kr_ + ((ks + 2) >> 1) * 2048 + 1024); \
        }                                                                                      \
        sacc[0] = mfma_t<F16>(qA[ks], kf0[ks], sacc[0]);                                       \
        sacc[1] = mfma_t<F16>(qA[ks], kf1[ks], sacc[1]);                                       \
      }                                                                                        \
      const bool ok0 = sVal[(CI) & 3][c] != 0, ok1 = sVal[(CI) & 3][16 + c] != 0;              \
      const int hcol = 16 * rw + 4 * g;                                                        \
      float p[2][4];                                                                           \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) {                                          \
        const float s0 = ok0 ? sacc[0][v] * zscale : -INFINITY;                                \
        const float s1 = ok1 ? sacc[1][v] * zscale : -INFINITY;                                \
        const float mc = fmaxf(m[v], row16_max(fmaxf(s0, s1)));                                \
        /* mu is taken from the first chunk with a valid slot (mc finite) */                   \
        mu[v] = mu[v] == -INFINITY ? mc : mu[v];                                               \
        over = over || mc > mu[v] + kLazy;                                                     \
        const bool fin = mu[v] != -INFINITY;                                                   \
        p[0][v] = fin ? __builtin_amdgcn_exp2f(s0 - mu[v]) : 0.f;                              \
        p[1][v] = fin ? __builtin_amdgcn_exp2f(s1 - mu[v]) : 0.f;                              \
        l[v] += p[0][v] + p[1][v];                                                             \
        m[v] = mc;                                                                             \
      }                                                                                        \
      _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                       \
        const uint32_t pw0 = pack_x2<F16>(p[kt][0], p[kt][1]), pw1 = pack_x2<F16>(p[kt][2], p[kt][3]); \
        *reinterpret_cast<uint2*>((PD) + (16 * kt + c) * kHtPitch + hcol) = make_uint2(pw0, pw1); \
      }                                                                                        \
    }                                                                                          \
    lds_barrier();                                                                             \
  }
      int ci = 0;
      for (; ci + 3 <= nchunk; ci += 4) {
        SFAG_FSTEP(ci, Kb0, Pb0)
        SFAG_FSTEP(ci + 1, Kb1, Pb1)
        SFAG_FSTEP(ci + 2, Kb2, Pb0)
        SFAG_FSTEP(ci + 3, Kb3, Pb1)
      }
      if (ci <= nchunk) {
        SFAG_FSTEP(ci, Kb0, Pb0)
        ++ci;
      }
      if (ci <= nchunk) {
        SFAG_FSTEP(ci, Kb1, Pb1)
        ++ci;
      }
      if (ci <= nchunk) SFAG_FSTEP(ci, Kb2, Pb0)
#undef SFAG_FSTEP
      if (over) s_over[pass] = 1;
      lds_barrier();                                // every wave's verdict in s_over
      if (pass == 0 && s_over[0] != 0) {
        // second pass against the true maxima (unchanged where a head had no valid slot)
#pragma unroll
        for (int v = 0; v < 4; ++v) mu[v] = m[v];
        continue;
      }
      break;
    }
    // statistics out (natural-log domain) and 1 / sum for the output waves
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * rw + 4 * g + v;
      const float ls = row16_sum(l[v]);
      if (c == 0) {
        sIL[h] = ls > 0.f ? 1.f / ls : 0.f;
        if (h < nh) {
          const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
          a.smax[st] = ls > 0.f ? m[v] / kLog2e : 0.f;
          a.ssum[st] = ls > 0.f ? ls * __builtin_amdgcn_exp2f(mu[v] - m[v]) : 0.f;
        }
      }
    }
    lds_barrier();
  } else {
    // gathering lane: key gkey of every chunk, 16 bytes at gcol of each 128-byte run of its row
    const int gkey = ktile_gather_key(rw, lane);
    const uint32_t gcol = ktile_gather_col(rw, lane);
    const char* kgat[kBlocks / 4 - 1];
#pragma unroll
    for (int j = 0; j < kBlocks / 4 - 1; ++j) {
      kgat[j] = reinterpret_cast<const char*>(uniform(kbase + 64 * j));
      asm volatile("" : "+s"(kgat[j]));
    }
    const char* rgat = reinterpret_cast<const char*>(uniform(krbase));
    asm volatile("" : "+s"(rgat));
    // key position of slot s (clamped to the last visited slot); invalid slots read key 0
    auto slot_pos = [&](int s) { return slot_key(irow, min(s, nslots - 1), a.bs); };
    auto gather_pos = [&](int j) { return (j >= 0 && j <= geo.hi) ? j : 0; };
#define SFAG_GATHER_ASYNC(KS, SV)                                                              \
  {                                                                                            \
    const uint32_t ko_ = (uint32_t)(SV) * (uint32_t)(kDn * 2) + gcol;                          \
    const uint32_t ro_ = (uint32_t)(SV) * (uint32_t)((rope ? kDr : kDn) * 2) + gcol;           \
    _Pragma("unroll") for (int j = 0; j < kBlocks / 4; ++j) {                                  \
      const char* src = j < kBlocks / 4 - 1 ? kgat[j] + ko_ : rgat + ro_;                      \
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KS) + (4 * j + rw) * 512), 16, 0, 0); \
    }                                                                                          \
  }
    // slot validity of chunk CH from the raw position J (one lane per key)
#define SFAG_MARK(CH, J)                                                                       \
  {                                                                                            \
    if ((lane & 7) == 0)                                                                       \
      sVal[(CH) & 3][gkey] = ((CH) * kKC + gkey < nslots && (J) >= 0 && (J) <= geo.hi) ? 1 : 0; \
  }
    // Transposing reads of the chunk's keys in the order 4 g + j, 4 g + 16 + j (j = 0..3) for
    // lane group g, the same for P and V.  Key tile: lane (g, c) points at key tk = 4 g + c / 4
    // and dims 128 rw + 16 nt + 4 (c % 4), i.e. chunk 16 rw + 2 nt + (c % 4) / 2 (group
    // 2 rw + nt / 4, slot (2 (nt % 4) + (c % 4) / 2) ^ swz(tk)): element (kq0 ^ 16 (nt % 4)) +
    // 2048 (nt / 4); keys + 16 are 1024 elements on.  P tile ([key][head]): key tk, head
    // 4 (c % 4), keys + 16 at 16 rows on.
    const int tk = 4 * g + (c >> 2);
    const int kq0 = 2 * rw * 2048 + tk * 64 + 4 * (c & 1) + ((((c & 3) >> 1) ^ ktile_swz(tk)) << 3);
    const int psoff = tk * kHtPitch + 4 * (c & 3);
    f32x4 oacc[4][8];
    for (int pass = 0;; ++pass) {
      int gkey_ = gkey, psoff_ = psoff;
      uint32_t gcol_ = gcol;
      asm volatile("" : "+v"(gkey_), "+v"(psoff_), "+v"(gcol_));
#define gkey gkey_
#define psoff psoff_
#define gcol gcol_
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) oacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      int32_t raw = slot_pos(gkey);
      SFAG_MARK(0, raw)
      SFAG_GATHER_ASYNC(Kb0, gather_pos(raw))
      raw = slot_pos(kKC + gkey);
      SFAG_MARK(1, raw)
      SFAG_GATHER_ASYNC(Kb1, gather_pos(raw))
      int32_t gsv = slot_pos(2 * kKC + gkey);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(kWaitVm10);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
// Output step CI (>= 1): the position of chunk CI + 3's slot, the slot marks of chunk CI + 2,
// then O += P V of chunk CI - 1 from KP / PP with the gather of chunk CI + 2 into KN issued one
// 1 KB load per column tile between the MFMAs (the loads queue on the vector memory path behind
// the other waves'; ahead of the MFMAs they would hold them up).  Ends by waiting for chunk
// CI + 1's gather and the position load, leaving this step's gather in flight.
#define SFAG_OSTEP(CI, KP, KN, PP)                                                             \
  {                                                                                            \
    const int32_t sv = slot_pos(((CI) + 3) * kKC + gkey);                                      \
    asm volatile("" ::: "memory");                                                             \
    SFAG_MARK((CI) + 2, gsv)                                                                   \
    const int32_t gp_ = gather_pos(gsv);                                                       \
    const uint32_t ko_ = (uint32_t)gp_ * (uint32_t)(kDn * 2) + gcol;                           \
    const uint32_t ro_ = (uint32_t)gp_ * (uint32_t)((rope ? kDr : kDn) * 2) + gcol;            \
    const uint16_t* pq_ = (PP) + psoff;                                                        \
    bf16x8 pa[4];                                                                              \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) pa[t] = tr_frag(pq_ + 16 * t, 16 * kHtPitch); \
    /* the lane offset is made opaque per step so that its per-buffer sums are not hoisted */   \
    int kq_ = kq0;                                                                             \
    asm volatile("" : "+v"(kq_));                                                              \
    bf16x8 kb = tr_frag((KP) + kq_, 1024);                                                     \
    _Pragma("unroll") for (int nt = 0; nt < 8; ++nt) {                                         \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      _Pragma("unroll") for (int j = nt; j < (nt == 7 ? 9 : nt + 1); ++j) {                   \
        const char* src = j < kBlocks / 4 - 1 ? kgat[j] + ko_ : rgat + ro_;                    \
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KN) + (4 * j + rw) * 512), 16, 0, 0); \
      }                                                                                        \
      bf16x8 nb = kb;                                                                          \
      if (nt < 7) nb = tr_frag((KP) + (kq_ ^ (16 * ((nt + 1) & 3))) + 2048 * ((nt + 1) >> 2), 1024); \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) oacc[t][nt] = mfma_t<F16>(pa[t], kb, oacc[t][nt]); \
      kb = nb;                                                                                 \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    asm volatile("" ::: "memory");                                                             \
    __builtin_amdgcn_s_waitcnt(kWaitVm9);                                                      \
    gsv = sv;                                                                                  \
    __builtin_amdgcn_s_barrier();                                                              \
    asm volatile("" ::: "memory");                                                             \
  }
      // step 0: no P V yet (chunk 0 is being scored), only the position of chunk 3's slot and
      // the gather of chunk 2
      {
        const int32_t sv = slot_pos(3 * kKC + gkey);
        asm volatile("" ::: "memory");
        SFAG_MARK(2, gsv)
        SFAG_GATHER_ASYNC(Kb2, gather_pos(gsv))
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm9);
        gsv = sv;
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      int ci = 1;
      for (; ci + 3 <= nchunk; ci += 4) {
        SFAG_OSTEP(ci, Kb0, Kb3, Pb0)
        SFAG_OSTEP(ci + 1, Kb1, Kb0, Pb1)
        SFAG_OSTEP(ci + 2, Kb2, Kb1, Pb0)
        SFAG_OSTEP(ci + 3, Kb3, Kb2, Pb1)
      }
      if (ci <= nchunk) {
        SFAG_OSTEP(ci, Kb0, Kb3, Pb0)
        ++ci;
      }
      if (ci <= nchunk) {
        SFAG_OSTEP(ci, Kb1, Kb0, Pb1)
        ++ci;
      }
      if (ci <= nchunk) SFAG_OSTEP(ci, Kb2, Kb1, Pb0)
#undef SFAG_OSTEP
      __builtin_amdgcn_s_waitcnt(0);                    // no gather may still write LDS
      lds_barrier();                                    // the score waves' verdict in s_over
      if (pass == 0 && s_over[0] != 0) continue;        // second pass (see the score waves)
      break;
#undef gkey
#undef psoff
#undef gcol
    }
#undef SFAG_MARK
#undef SFAG_GATHER_ASYNC
    lds_barrier();                                        // sIL from the score waves
    // out: lane holds heads 16 t + 4 g + v, dims 128 rw + 16 nt + c
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4 il = *reinterpret_cast<const f32x4*>(sIL + 16 * t + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * t + 4 * g + v;
        if (h >= nh) continue;
        uint16_t* orow = a.out + (row * a.N1 + h0 + h) * kDn + 128 * rw + c;
        // lanes c and c ^ 1 hold neighbouring dims: the even lane stores both as one word
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const float x = oacc[t][nt][v] * il[v];
          const float y = dpp_f<kDppXor1>(x);
          if ((c & 1) == 0) *reinterpret_cast<uint32_t*>(orow + 16 * nt) = pack_x2<F16>(x, y);
        }
      }
    }
  }
}

hipError_t launch_fwd(const FwdArgs& a, int64_t nrows, int hg_count, hipStream_t st) {
  if (a.f16)
    hipLaunchKernelGGL(fwd_kernel<true>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(fwd_kernel<false>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}


}  // namespace sfag
