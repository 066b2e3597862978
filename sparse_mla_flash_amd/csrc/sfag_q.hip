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
// Work split of the 4 waves (an LDS read of up to 16 bytes per lane costs the same LDS time,
// and a transposing read delivers only 8):
//   scores: wave w owns head tile w (heads 16 w .. 16 w + 15) over the whole contraction
//     (512 value + 64 rope dims) for both 16-key tiles of the chunk.  Its Q and dO fragments
//     stay in registers for the whole row; every 16-byte key fragment read from LDS feeds the
//     S and dP MFMAs of its key tile, and no partial sums change hands.
//   dQ: wave w owns output dims 144 w .. 144 w + 143 for all 64 heads, so each gathered key
//     element is read (transposed) once per workgroup.
// Key tiles are stored chunk-major in LDS ([72 chunks of 16 B][32 keys]): one direct-to-LDS
// block (64 lanes x 16 B) is then two chunk columns of all 32 keys, so a gathering lane always
// handles the same key (lane % 32) and each of its loads is one add to that key's row address.
// Pipeline: key tiles are triple-buffered in LDS and gathered straight from global memory
// one chunk ahead (global_load_lds).  The score MFMAs of chunk c and the dQ MFMAs of chunk
// c - 1 sit in one block so that the scheduler can interleave them; one barrier per chunk.
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kKC = 32;
constexpr int kThreads = 256;
constexpr int kChunks = kDk / 8;                 // 72 16-byte chunks per key row (64 value + 8 rope)
constexpr int kHtPitch = 64 + 8;                 // DSt row pitch
constexpr int kBlocks = kChunks / 2;             // 36 direct-to-LDS blocks (2 chunk columns) per tile
static_assert(kBlocks % 4 == 0, "gather blocks per wave");
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsK = kBlocks * 64 * 16;         // one key tile, chunk-major: [72 chunks][32 keys][16 B]
constexpr int kLdsDS = kKC * kHtPitch * 2;       // DSt [32 keys][72]
constexpr int kLdsTotal = 3 * kLdsK + 3 * kLdsDS + 3 * 64 * 4 + 2 * 257 * 4;
static_assert(kLdsTotal <= 160 * 1024, "LDS budget");
// s_waitcnt operands.  kWaitVmem: vmcnt(0), expcnt and lgkmcnt at their maximum (issued just
// before a chunk's record stores).  kWaitAllButRecords: vmcnt(4), lgkmcnt(0): at the end of a
// chunk the only vector memory operations that can be in flight are the chunk's 4 record
// stores, so this leaves them in flight and waits for this wave's LDS writes.
constexpr int kWaitVmem = 0x0f70;
constexpr int kWaitAllButRecords = 0x0074;
}  // namespace

__global__ void __launch_bounds__(kThreads, 1) bwd_q_kernel(BwdArgs a) {
  // Separate LDS arrays (not one carved buffer): the compiler can then prove that the
  // direct-to-LDS gather into one key buffer does not alias reads of the others, and does not
  // wait for the gather before every LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t Kb0[kLdsK / 2], Kb1[kLdsK / 2], Kb2[kLdsK / 2];
  __shared__ __attribute__((aligned(16))) uint16_t Db0[kKC * kHtPitch], Db1[kKC * kHtPitch], Db2[kKC * kHtPitch];
  __shared__ __attribute__((aligned(16))) float sD[64], sM[64], sIL[64];
  __shared__ int32_t cum[2 * 257];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
  const int g = lane >> 4, c = lane & 15;
  // longest rows (highest positions under the causal mask) first
  const int64_t row = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int hg = blockIdx.y;
  const int h0 = hg * 64;
  const int nh = min(64, a.N1 - h0);
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  const int count = a.count[row];
  if (!geo.active || geo.hi < 0 || count == 0) {
    for (int e = threadIdx.x; e < nh * kDn; e += kThreads) a.dq[(row * a.N1 + h0) * kDn + e] = 0;
    if (a.dqr)
      for (int e = threadIdx.x; e < nh * kDr; e += kThreads) a.dqr[(row * a.N1 + h0) * kDr + e] = 0;
    return;
  }
  const int32_t* srow = a.sorted + row * a.topk;
  const int nchunk = (count + kKC - 1) / kKC;

  // ---- per-row setup --------------------------------------------------------------------------
  // gathering lanes: key slot gkey of every chunk, chunk column gcol of every block
  const int gkey = lane & 31, gcol = lane >> 5;
  int32_t gsv = srow[min(gkey, count - 1)];               // sorted position of chunk 0's key
  // D = rowsum(dO * out) and the statistics of every head
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
  // Q and dO fragments of this wave, straight from global memory (A operands of S and dP:
  // lane (g, c) holds head 16 wave + c, dims 32 ks + 8 g .. + 7; steps 16 and 17 are the rope
  // dims); zero for padded heads
  bf16x8 qA[18], doA[16];
  {
    const int h = 16 * wave + c;
    const bool hv = h < nh;
    const int64_t hrow = row * a.N1 + h0 + (hv ? h : 0);
    const uint16_t* qrow = a.q + hrow * kDn + 8 * g;
    const uint16_t* drow = a.dout + hrow * kDn + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
      const bf16x8 dv = *reinterpret_cast<const bf16x8*>(drow + 32 * ks);
      qA[ks] = hv ? qv : bf16x8{};
      doA[ks] = hv ? dv : bf16x8{};
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qA[16 + ks] = bf16x8{};
      if (hv && a.qr) qA[16 + ks] = *reinterpret_cast<const bf16x8*>(a.qr + hrow * kDr + 32 * ks + 8 * g);
    }
  }
  __syncthreads();
  const float zscale = a.scale * kLog2e;
  // Loop-invariant bases, held in SGPRs: the empty asm makes them opaque, so the compiler
  // cannot re-load them from the kernel arguments inside the loop (a scalar load in flight
  // forces LDS waits to drain completely).
  auto uniform = [](const void* p) {               // a workgroup-uniform pointer, made scalar
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<uint16_t*>(((uint64_t)hi << 32) | lo);
  };
  const uint16_t* kbase = uniform(a.k + geo.kstart * kDn);
  const bool rope = a.kr != nullptr;                // without rope inputs the rope terms are absent
  const uint16_t* krbase = uniform(rope ? a.kr + geo.kstart * kDr : a.zero_row);
  const uint16_t* zrow = uniform(a.zero_row);
  // The record pointers lose their address space through the scalar round trip; stores through
  // them are made global explicitly, because a generic (flat) store might hit LDS and would then
  // wait for every direct-to-LDS gather load in flight.
  typedef __attribute__((address_space(1))) uint64_t GlobalU64;
  uint16_t* recrow = uniform(a.dsp + ((int64_t)row * a.topk * a.hgc + hg) * 128);   // slot 0 of this row
  uint16_t* trash = uniform(a.trash);
  const int recstride = a.hgc * 128;                                          // elements per slot
  asm volatile("" : "+s"(kbase), "+s"(krbase), "+s"(zrow), "+s"(recrow), "+s"(trash));

  // Gather of chunk CH (this lane's key: sorted position SV) into key buffer KS: block b of the
  // tile holds chunk columns 2 b and 2 b + 1; wave w loads blocks w, w + 4, ..., w + 32 (the
  // last one: rope chunks).  Slots past the row's valid count read the zero row.
#define SFAG_GATHER_ASYNC(KS, CH, SV)                                                          \
  {                                                                                            \
    const bool ok_ = (CH) * kKC + gkey < count;                                                \
    const uint16_t* pk_ = ok_ ? kbase + (int64_t)(SV) * kDn : zrow;                            \
    const uint16_t* pr_ = ok_ && rope ? krbase + (int64_t)(SV) * kDr : zrow;                   \
    _Pragma("unroll") for (int j = 0; j < kBlocks / 4; ++j) {                                  \
      const int blk = wave + 4 * j;                                                            \
      const uint16_t* src = j < kBlocks / 4 - 1 ? pk_ + (2 * blk + gcol) * 8                   \
                                                : pr_ + (2 * blk + gcol - 64) * 8;             \
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KS) + blk * 512), 16, 0, 0); \
    }                                                                                          \
  }

// S and dP of this wave's head tile for both key tiles of chunk buffer KS.
#define SFAG_SCORES(KS)                                                                        \
  {                                                                                            \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                         \
      sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                    \
      pacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                    \
    }                                                                                          \
    /* chunk-major tile: element (chunk, key) at (chunk * 32 + key) * 8; lane (g, c) of step  \
       ks reads chunk 4 ks + g of key 16 kt + c */                                             \
    const uint16_t* kr0 = (KS) + (g * kKC + c) * 8;                                            \
    const uint16_t* kr1 = (KS) + (g * kKC + 16 + c) * 8;                                       \
    bf16x8 kf0[18], kf1[18];                /* key fragments, read two steps ahead */         \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                         \
      kf0[ks] = *reinterpret_cast<const bf16x8*>(kr0 + 4 * ks * kKC * 8);                      \
      kf1[ks] = *reinterpret_cast<const bf16x8*>(kr1 + 4 * ks * kKC * 8);                      \
    }                                                                                          \
    _Pragma("unroll") for (int ks = 0; ks < 18; ++ks) {                                        \
      if (ks + 2 < 18) {                                                                       \
        kf0[ks + 2] = *reinterpret_cast<const bf16x8*>(kr0 + 4 * (ks + 2) * kKC * 8);          \
        kf1[ks + 2] = *reinterpret_cast<const bf16x8*>(kr1 + 4 * (ks + 2) * kKC * 8);          \
      }                                                                                        \
      sacc[0] = mfma(qA[ks], kf0[ks], sacc[0]);                                                \
      sacc[1] = mfma(qA[ks], kf1[ks], sacc[1]);                                                \
      if (ks < 16) {                                                                           \
        pacc[0] = mfma(doA[ks], kf0[ks], pacc[0]);                                             \
        pacc[1] = mfma(doA[ks], kf1[ks], pacc[1]);                                             \
      }                                                                                        \
    }                                                                                          \
    /* issue order: the first four fragments, then per step the fragments two steps ahead and \
       the step's MFMAs.  The vector-memory slots of steps 0-8 take the sorted-position load;   \
       the gather itself sits in its own (conditional) block before the scores: all 9 loads   \
       issued together measured faster than spread among the MFMAs */                        \
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                         \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                        \
      if (ks < 9) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                           \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                       \
    }                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                         \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                         \
  }

// dQ[64 heads][144 w .. 144 w + 143] += dS[64][32 keys] K[32 keys][dims] of the previous chunk
#define SFAG_DQ(KS, DST)                                                                       \
  {                                                                                            \
    bf16x8 dsa[4];                                                                             \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) dsa[t] = lds_frag_trp((DST), 0, 16 * t, kHtPitch, lane); \
    bf16x8 kb = lds_frag_tr_cm((KS), 144 * wave, lane);                                        \
    _Pragma("unroll") for (int nt = 0; nt < 9; ++nt) {                                         \
      bf16x8 nb = kb;                                                                          \
      if (nt < 8) nb = lds_frag_tr_cm((KS), 144 * wave + 16 * (nt + 1), lane);                 \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) dqacc[t][nt] = mfma(dsa[t], kb, dqacc[t][nt]); \
      kb = nb;                                                                                 \
    }                                                                                          \
  }

// P and dS of this wave's head tile for both key tiles: records and the DSt tile of this
// chunk.  Every lane issues exactly 4 record stores (invalid slots write to the sink), so that
// the end-of-chunk wait can leave them in flight.
#define SFAG_FINISH(CI, DST)                                                                   \
  {                                                                                            \
    const int c0 = (CI) * kKC;                                                                 \
    const int hcol = 16 * wave + 4 * g;          /* heads hcol .. hcol + 3 */                   \
    const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + hcol);                               \
    const f32x4 iv = *reinterpret_cast<const f32x4*>(sIL + hcol);                              \
    const f32x4 dv = *reinterpret_cast<const f32x4*>(sD + hcol);                               \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                         \
      const int key = 16 * kt + c;                                                             \
      const bool valid = c0 + key < count;                                                     \
      uint16_t* rec = valid ? recrow + (int64_t)(c0 + key) * recstride : trash;                \
      float p[4], ds[4];                                                                       \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) {                                          \
        /* v_exp_f32: results below 2^-126 flush to 0, far under bf16 resolution here */       \
        const float e_ = __builtin_amdgcn_exp2f(sacc[kt][v] * zscale - mv[v]) * iv[v];         \
        p[v] = valid ? e_ : 0.f;                                                               \
        ds[v] = p[v] * (pacc[kt][v] - dv[v]);                                                  \
      }                                                                                        \
      const uint32_t pw[2] = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};               \
      const uint32_t dw[2] = {pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])};           \
      *reinterpret_cast<uint2*>((DST) + key * kHtPitch + hcol) = make_uint2(dw[0], dw[1]);     \
      /* the next chunk's gather is in before any record store is issued */                    \
      if (kt == 0) __builtin_amdgcn_s_waitcnt(kWaitVmem);                                      \
      *(GlobalU64*)(rec + hcol) = ((uint64_t)dw[1] << 32) | dw[0];                             \
      *(GlobalU64*)(rec + 64 + hcol) = ((uint64_t)pw[1] << 32) | pw[0];                        \
    }                                                                                          \
  }

  f32x4 sacc[2], pacc[2];
  f32x4 dqacc[4][9];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int nt = 0; nt < 9; ++nt) dqacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  SFAG_GATHER_ASYNC(Kb0, 0, gsv)
  gsv = srow[min(kKC + gkey, count - 1)];                 // chunk 1

  // The row's Q | QRope | dO with the 64 heads innermost (bt[row][hg][col][h]), the key-major
  // kernel's B operand, written from the fragments already in registers.  Per 64-column block
  // (two steps of every wave) the [64 heads][64 cols] tile goes through LDS (pitch 72, the
  // key buffers 1 and 2 in turn, unused until the loop) and comes back by transposing reads:
  // lane (g, c) of wave w stores heads 32 s + 8 g .. + 7 of column 64 k + 16 w + c.
  {
    uint16_t* bto = a.bt + ((int64_t)row * a.hgc + hg) * (int64_t)kDacc * 64;
    const int hrow = 16 * wave + c;
#pragma unroll
    for (int k = 0; k < kDacc / 64; ++k) {
      uint16_t* t = (k & 1) ? Kb2 : Kb1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = 2 * k + j;                         // 32-column step over Q | QRope | dO
        const bf16x8 v = ks < 18 ? qA[ks] : doA[ks - 18];
        *reinterpret_cast<bf16x8*>(t + hrow * 72 + 32 * j + 8 * g) = v;
      }
      lds_barrier();
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const bf16x8 v = lds_frag_trp(t, 32 * sh, 16 * wave, 72, lane);
        *reinterpret_cast<bf16x8*>(bto + (64 * k + 16 * wave + c) * 64 + 32 * sh + 8 * g) = v;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

// One chunk CI: gather of chunk CI + 1 into KN, scores of chunk CI (buffer KC), dQ of chunk
// CI - 1 (buffers KP, DP; skipped for chunk 0), finish into DC.  The sorted position
// of this lane's key of chunk CI + 2 is loaded branch-free and only used after the
// end-of-chunk wait.
#define SFAG_CHUNK(CI, KC, KP, KN, DC, DP, WITH_DQ)                                            \
  {                                                                                            \
    const int ci_ = (CI);                                                                      \
    if (ci_ + 1 < nchunk) SFAG_GATHER_ASYNC(KN, ci_ + 1, gsv)                                  \
    const int32_t sv = srow[min((ci_ + 2) * kKC + gkey, count - 1)];                           \
    SFAG_SCORES(KC)                                                                            \
    if (WITH_DQ) SFAG_DQ(KP, DP)                                                               \
    SFAG_FINISH(ci_, DC)                                                                       \
    /* everything but the 4 record stores just issued */                                      \
    __builtin_amdgcn_s_waitcnt(kWaitAllButRecords);                                            \
    gsv = sv;                                                                                  \
    /* a plain barrier: the data exchanged is in LDS, and a release fence would also wait for  \
       the record stores */                                                                    \
    asm volatile("" ::: "memory");                                                             \
    __builtin_amdgcn_s_barrier();                                                              \
    asm volatile("" ::: "memory");                                                             \
  }

  SFAG_CHUNK(0, Kb0, Kb2, Kb1, Db0, Db2, false)
  // chunk ci lives in key / dS buffers ci % 3; unrolled by 3 so every access names its buffer
  int ci = 1;
  for (; ci + 2 < nchunk; ci += 3) {
    SFAG_CHUNK(ci, Kb1, Kb0, Kb2, Db1, Db0, true)
    SFAG_CHUNK(ci + 1, Kb2, Kb1, Kb0, Db2, Db1, true)
    SFAG_CHUNK(ci + 2, Kb0, Kb2, Kb1, Db0, Db2, true)
  }
  if (ci < nchunk) {
    SFAG_CHUNK(ci, Kb1, Kb0, Kb2, Db1, Db0, true)
    ++ci;
  }
  if (ci < nchunk) {
    SFAG_CHUNK(ci, Kb2, Kb1, Kb0, Db2, Db1, true)
    ++ci;
  }
  // dQ of the last chunk
  switch ((nchunk - 1) % 3) {
    case 0: SFAG_DQ(Kb0, Db0) break;
    case 1: SFAG_DQ(Kb1, Db1) break;
    default: SFAG_DQ(Kb2, Db2) break;
  }

#undef SFAG_GATHER_ASYNC
#undef SFAG_SCORES
#undef SFAG_DQ
#undef SFAG_FINISH
#undef SFAG_CHUNK

  // ---- dQ / dQRope out: lane holds heads 16 t + 4 g + v, dims 144 w + 16 nt + c ------------------
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 16 * t + 4 * g + v;
      if (h >= nh) continue;
      const int64_t hh2 = row * a.N1 + h0 + h;
#pragma unroll
      for (int nt = 0; nt < 9; ++nt) {
        const int col = 144 * wave + 16 * nt + c;
        const uint16_t bv = f2bf(dqacc[t][nt][v] * a.scale);
        if (col < kDn) a.dq[hh2 * kDn + col] = bv;
        else if (a.dqr) a.dqr[hh2 * kDr + col - kDn] = bv;
      }
    }
  }
}

hipError_t launch_bwd_q(const BwdArgs& a, int64_t nrows, int hg_count, hipStream_t st) {
  hipLaunchKernelGGL(bwd_q_kernel, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t set_q_attributes() { return hipSuccess; }

}  // namespace sfag
