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
// Work split: 8 waves, two per SIMD, in two roles, so that one wave of every SIMD can issue
// MFMAs while the other waits for LDS, the exponentials or its stores:
//   score waves (0-3): wave w keeps the Q and dO fragments of heads 16 w .. 16 w + 15 for the
//     whole contraction (512 value + 64 rope dims) in registers and, for chunk c, computes S
//     and dP of its head tile for both 16-key tiles (every 16-byte key fragment read from LDS
//     feeds the S and dP MFMAs of its key tile), then P and dS in registers, the chunk's dS
//     tile in LDS ([key][head]) and the 256-byte dS | P record of every (row, key) pair.
//   dQ waves (4-7): wave 4 + w owns the output dims of 16-dim column tiles w, w + 4, .., w + 32
//     (144 dims) for all 64 heads (fp32 accumulators across all chunks) and in step c adds dS K
//     of chunk c - 1 (each gathered key element is read, transposed, once per workgroup); it also
//     gathers keys 8 w .. 8 w + 7 of chunk c + 2 straight from global memory into LDS
//     (global_load_lds, 16 bytes per lane).
// Records are stored chunk-major: per (row, head group) and chunk of 32 sorted positions, 8 KB
// = [dS | P][head tile of 16][32 positions][16 heads] bf16, so that each record store
// instruction of a score wave writes 512 contiguous bytes.
// One barrier per step.  Key tiles are quadruple-buffered and gathered two chunks ahead, so a
// gather has two steps to land; dS tiles are double-buffered.  Key tiles use the swizzled
// [chunk group][key][slot] layout of sfag_ktile.h: each direct-to-LDS load reads eight whole
// 128-byte runs of key rows, and a gathering lane always handles the same key.
#include "sfag_device.h"
#include "sfag_dpp.h"
#include "sfag_ktile.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kKC = 32;
constexpr int kThreads = 512;                    // 4 score waves + 4 dQ waves
constexpr int kChunks = kDk / 8;                 // 72 16-byte chunks per key row (64 value + 8 rope)
constexpr int kHtPitch = 64 + 8;                 // DSt row pitch
constexpr int kBlocks = kChunks / 2;             // 36 direct-to-LDS blocks of 1 KB per tile
static_assert(kBlocks % 4 == 0, "gather blocks per dQ wave");
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsK = kBlocks * 64 * 16;         // one key tile
static_assert(kLdsK == kTileBytes, "key tile size");
constexpr int kLdsDS = kKC * kHtPitch * 2;       // DSt [32 keys][72]
constexpr int kLdsTotal = 4 * kLdsK + 2 * kLdsDS + 3 * 64 * 4 + 2 * 257 * 4;
static_assert(kLdsTotal <= 160 * 1024, "LDS budget");
// s_waitcnt operands with expcnt and lgkmcnt at zero: vmcnt(9) (all but the 9 loads of the
// newest gather) and vmcnt(10) (all but a gather and one position load)
constexpr int kWaitVm9 = 0x0009;
constexpr int kWaitVm10 = 0x000a;
// rounds of the heads-innermost copy (17 blocks of 64 columns, up to 8 per round), two
// barriers each
constexpr int kCopyRounds = (kDacc / 64 + 7) / 8;
static_assert(8 * 64 * 72 * 2 <= 2 * kLdsK, "a copy round's tiles fit key buffers 2 and 3");
}  // namespace

template <bool F16>
__global__ void __launch_bounds__(kThreads, 1) bwd_q_kernel(BwdArgs a) {
  // Separate LDS arrays (not one carved buffer): the compiler can then prove that the
  // direct-to-LDS gather into one key buffer does not alias reads of the others, and does not
  // wait for the gather before every LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t Kb0[kLdsK / 2], Kb1[kLdsK / 2], Kb2[kLdsK / 2], Kb3[kLdsK / 2];
  __shared__ __attribute__((aligned(16))) uint16_t Db0[kKC * kHtPitch], Db1[kKC * kHtPitch];
  __shared__ __attribute__((aligned(16))) float sD[64], sM[64], sIL[64];
  __shared__ int32_t cum[2 * 257];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
  const bool swave = wave < 4;                      // score wave; otherwise dQ wave
  const int rw = wave & 3;                          // index within the role
  const int g = lane >> 4, c = lane & 15;
  // longest rows (highest positions under the causal mask) first
  const int64_t lrow = (int64_t)gridDim.x - 1 - blockIdx.x;     // row within this launch
  const int64_t row = a.row_begin + lrow;
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

  // ---- per-row setup: D and the statistics are formed by the score waves (below) --------------
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
  // The record pointers lose their address space through the scalar round trip; stores through
  // them are made global explicitly (a generic store might address LDS).
  typedef __attribute__((address_space(1))) uint64_t GlobalU64;
  uint16_t* recrow = uniform(a.dsp + (lrow * a.hgc + hg) * (int64_t)a.rec_chunks * kRecChunk);
  asm volatile("" : "+s"(kbase), "+s"(krbase), "+s"(recrow));

  // gathering lanes of the dQ waves: key gkey of every chunk, the 16 bytes at gcol of each
  // 128-byte run of its row
  const int gkey = ktile_gather_key(rw, lane);
  const uint32_t gcol = ktile_gather_col(rw, lane);
  // byte bases of the gather: value chunk group j of key 0, and the rope row (the zero row
  // without rope inputs); held as opaque scalars so that every load is one scalar base plus the
  // lane's 32-bit offset
  const char* kgat[kBlocks / 4 - 1];
#pragma unroll
  for (int j = 0; j < kBlocks / 4 - 1; ++j) {
    kgat[j] = reinterpret_cast<const char*>(uniform(kbase + 64 * j));
    asm volatile("" : "+s"(kgat[j]));
  }
  const char* rgat = reinterpret_cast<const char*>(uniform(krbase));
  asm volatile("" : "+s"(rgat));

  // Gather of chunk CH (this lane's key: sorted position SV) into key buffer KS (dQ waves): dQ
  // wave rw loads keys 8 rw .. 8 rw + 7 of chunk groups 0 .. 8 (the last one: the rope row) into
  // blocks 4 j + rw.
#define SFAG_GATHER_ASYNC(KS, CH, SV)                                                          \
  {                                                                                            \
    /* slots past the row's valid count repeat its last valid key (their p is 0) */           \
    const uint32_t ko_ = (uint32_t)(SV) * (uint32_t)(kDn * 2) + gcol;                          \
    const uint32_t ro_ = rope ? (uint32_t)(SV) * (uint32_t)(kDr * 2) + gcol : gcol;            \
    _Pragma("unroll") for (int j = 0; j < kBlocks / 4; ++j) {                                  \
      const char* src = j < kBlocks / 4 - 1 ? kgat[j] + ko_ : rgat + ro_;                      \
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KS) + (4 * j + rw) * 512), 16, 0, 0); \
    }                                                                                          \
  }

// S and dP of this score wave's head tile for both key tiles of chunk buffer KS.
#define SFAG_SCORES(KS)                                                                        \
  {                                                                                            \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                         \
      sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                    \
      pacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                    \
    }                                                                                          \
    /* lane (g, c) of step ks reads chunk 4 ks + g of keys c and 16 + c: chunk group ks / 2,   \
       slot bit 2 = ks % 2 (key 16 + c is 1024 elements after key c) */                        \
    const uint16_t* kre = (KS) + kse;                                                          \
    const uint16_t* kro = (KS) + (kse ^ 32);                                                   \
    bf16x8 kf0[18], kf1[18];                /* key fragments, read two steps ahead */         \
    _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                         \
      const uint16_t* kr_ = (ks & 1) ? kro : kre;                                              \
      kf0[ks] = *reinterpret_cast<const bf16x8*>(kr_ + (ks >> 1) * 2048);                      \
      kf1[ks] = *reinterpret_cast<const bf16x8*>(kr_ + (ks >> 1) * 2048 + 1024);               \
    }                                                                                          \
    _Pragma("unroll") for (int ks = 0; ks < 18; ++ks) {                                        \
      if (ks + 2 < 18) {                                                                       \
        const uint16_t* kr_ = ((ks + 2) & 1) ? kro : kre;                                      \
        kf0[ks + 2] = *reinterpret_cast<const bf16x8*>(kr_ + ((ks + 2) >> 1) * 2048);          \
        kf1[ks + 2] = *reinterpret_cast<const bf16x8*>(kr_ + ((ks + 2) >> 1) * 2048 + 1024);   \
      }                                                                                        \
      sacc[0] = mfma_t<F16>(qA[ks], kf0[ks], sacc[0]);                                                \
      sacc[1] = mfma_t<F16>(qA[ks], kf1[ks], sacc[1]);                                                \
      if (ks < 16) {                                                                           \
        pacc[0] = mfma_t<F16>(doA[ks], kf0[ks], pacc[0]);                                             \
        pacc[1] = mfma_t<F16>(doA[ks], kf1[ks], pacc[1]);                                             \
      }                                                                                        \
    }                                                                                          \
    /* issue order: the first four fragments, then per step the fragments two steps ahead and \
       the step's MFMAs */                                                                     \
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                         \
    _Pragma("unroll") for (int ks = 0; ks < 16; ++ks) {                                        \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                                       \
    }                                                                                          \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                         \
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                         \
  }

// dQ[64 heads][column tiles rw + 4 nt] += dS[64][32 keys] K[32 keys][dims] of one chunk.  A
// operands (dS^T, heads 16 t + c) from the [key][head] tile, B operands (K, dims 16 (rw + 4 nt)
// + c: chunk group nt, slot pair rw) from the key tile, both by transposing reads at one
// per-lane offset plus constants (2048 elements per column tile).  The contraction takes the
// chunk's keys in the order 4 g + j, 4 g + 16 + j (j = 0..3) for lane group g in both operands.
#define SFAG_DQ(KS, DST)                                                                       \
  {                                                                                            \
    const uint16_t* kq_ = (KS) + kqoff;                                                        \
    const uint16_t* dq_ = (DST) + dsoff;                                                       \
    bf16x8 dsa[4];                                                                             \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) dsa[t] = tr_frag(dq_ + 16 * t, 16 * kHtPitch); \
    bf16x8 kb = tr_frag(kq_, 1024);                                                            \
    _Pragma("unroll") for (int nt = 0; nt < 9; ++nt) {                                         \
      bf16x8 nb = kb;                                                                          \
      if (nt < 8) nb = tr_frag(kq_ + 2048 * (nt + 1), 1024);                                   \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) dqacc[t][nt] = mfma_t<F16>(dsa[t], kb, dqacc[t][nt]); \
      kb = nb;                                                                                 \
    }                                                                                          \
  }

// The same with the gather of chunk CH (sorted position SV) into key buffer KN issued one block
// per column tile, so that the gather queues behind the MFMAs instead of ahead of them.
#define SFAG_DQ_GATHER(KS, DST, KN, SV)                                                        \
  {                                                                                            \
    const uint32_t ko_ = (uint32_t)(SV) * (uint32_t)(kDn * 2) + gcol;                          \
    const uint32_t ro_ = rope ? (uint32_t)(SV) * (uint32_t)(kDr * 2) + gcol : gcol;            \
    const uint16_t* kq_ = (KS) + kqoff;                                                        \
    const uint16_t* dq_ = (DST) + dsoff;                                                       \
    bf16x8 dsa[4];                                                                             \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) dsa[t] = tr_frag(dq_ + 16 * t, 16 * kHtPitch); \
    bf16x8 kb = tr_frag(kq_, 1024);                                                            \
    _Pragma("unroll") for (int nt = 0; nt < 9; ++nt) {                                         \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      {                                                                                        \
        const char* src = nt < kBlocks / 4 - 1 ? kgat[nt] + ko_ : rgat + ro_;                  \
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)((KN) + (4 * nt + rw) * 512), 16, 0, 0); \
      }                                                                                        \
      bf16x8 nb = kb;                                                                          \
      if (nt < 8) nb = tr_frag(kq_ + 2048 * (nt + 1), 1024);                                   \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) dqacc[t][nt] = mfma_t<F16>(dsa[t], kb, dqacc[t][nt]); \
      kb = nb;                                                                                 \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }

// P and dS of this score wave's head tile for both key tiles: the DSt tile of this chunk and the
// chunk's records (positions past the valid count get p = dS = 0).  Lane (g, c) stores heads
// 16 rw + 4 g .. + 3 of position 16 kt + c at ((rw * 32 + 16 kt + c) * 16 + 4 g) of each half.
#define SFAG_FINISH(CI, DST)                                                                   \
  {                                                                                            \
    const int c0 = (CI) * kKC;                                                                 \
    const int hcol = 16 * rw + 4 * g;            /* heads hcol .. hcol + 3 */                   \
    const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + hcol);                               \
    const f32x4 iv = *reinterpret_cast<const f32x4*>(sIL + hcol);                              \
    const f32x4 dv = *reinterpret_cast<const f32x4*>(sD + hcol);                               \
    uint16_t* rec = recrow + (int64_t)(CI) * kRecChunk + (rw * kKC + c) * 16 + 4 * g;          \
    _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                         \
      const int key = 16 * kt + c;                                                             \
      const bool valid = c0 + key < count;                                                     \
      float p[4], ds[4];                                                                       \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) {                                          \
        /* v_exp_f32: results below 2^-126 flush to 0, far under bf16 resolution here */       \
        const float e_ = __builtin_amdgcn_exp2f(sacc[kt][v] * zscale - mv[v]) * iv[v];         \
        p[v] = valid ? e_ : 0.f;                                                               \
        ds[v] = p[v] * (pacc[kt][v] - dv[v]);                                                  \
      }                                                                                        \
      const uint32_t pw[2] = {pack_x2<F16>(p[0], p[1]), pack_x2<F16>(p[2], p[3])};               \
      const uint32_t dw[2] = {pack_x2<F16>(ds[0], ds[1]), pack_x2<F16>(ds[2], ds[3])};           \
      *reinterpret_cast<uint2*>((DST) + key * kHtPitch + hcol) = make_uint2(dw[0], dw[1]);     \
      *(GlobalU64*)(rec + 16 * 16 * kt) = ((uint64_t)dw[1] << 32) | dw[0];                     \
      *(GlobalU64*)(rec + kRecHalf + 16 * 16 * kt) = ((uint64_t)pw[1] << 32) | pw[0];          \
    }                                                                                          \
  }

  // Steps 0 .. nchunk.  In step ci the score waves take chunk ci and the dQ waves gather chunk
  // ci + 2 and add dQ of chunk ci - 1.  Chunk ci lives in key buffer ci % 4 and dS buffer ci % 2,
  // so the loops are unrolled by 4 and every access names its buffer.  The two roles run
  // separate loops (their register sets are never live together) with one barrier per step.
  if (swave) {
    // Q and dO fragments straight from global memory (A operands of S and dP: lane (g, c) holds
    // head 16 rw + c, dims 32 ks + 8 g .. + 7; steps 16 and 17 are the rope dims); zero for
    // padded heads
    // requested in the order they are used: Q | QRope and dO (the copy below), then out and the
    // statistics (D, formed after the copy)
    bf16x8 qA[18], doA[16];
    u32x4 oy[16];
    float smv = 0.f, ssv = 0.f;
    const int h = 16 * rw + c;
    const bool hv = h < nh;
    {
      const int64_t hrow = row * a.N1 + h0 + (hv ? h : 0);
      const uint16_t* qrow = a.q + hrow * kDn + 8 * g;
      const uint16_t* drow = a.dout + hrow * kDn + 8 * g;
      const uint16_t* orow = a.out + hrow * kDn + 8 * g;
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
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 dv = *reinterpret_cast<const bf16x8*>(drow + 32 * ks);
        doA[ks] = hv ? dv : bf16x8{};
      }
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) oy[ks] = *reinterpret_cast<const u32x4*>(orow + 32 * ks);
      if (hv && g == 0) {
        const int64_t st = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h0 + h);
        smv = a.smax[st];
        ssv = a.ssum[st];
      }
    }
    // The row's Q | QRope | dO with the 64 heads innermost (bt[row][hg][col][h]), the key-major
    // kernel's B operand, written from the fragments already in registers.  The 17 blocks of 64
    // columns go in rounds of up to 8: each block's [64 heads][64 cols] tile goes through LDS
    // (pitch 72; key buffers 2 and 3, unused until the loop, hold four tiles each) and comes back
    // by transposing reads: lane (g, c) of score wave w stores heads 32 s + 8 g .. + 7 of column
    // 64 k + 16 w + c.  Two barriers per round; the dQ waves pass as many meanwhile.  These
    // stores drain during the loop.
    {
      uint16_t* bto = a.bt + (lrow * a.hgc + hg) * (int64_t)kDacc * 64;
      const int hrow = 16 * rw + c;
#pragma unroll
      for (int r = 0; r < kCopyRounds; ++r) {
        const int kb = 8 * r, kn = min(8, kDacc / 64 - kb);
#pragma unroll
        for (int i = 0; i < kn; ++i) {
          uint16_t* t = (i < 4 ? Kb2 : Kb3) + (i & 3) * (64 * 72);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int ks = 2 * (kb + i) + j;                // 32-column step over Q | QRope | dO
            const bf16x8 v = ks < 18 ? qA[ks] : doA[ks - 18];
            *reinterpret_cast<bf16x8*>(t + hrow * 72 + 32 * j + 8 * g) = v;
          }
        }
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kn; ++i) {
          const uint16_t* t = (i < 4 ? Kb2 : Kb3) + (i & 3) * (64 * 72);
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            const bf16x8 v = lds_frag_trp(t, 32 * sh, 16 * rw, 72, lane);
            *reinterpret_cast<bf16x8*>(bto + (64 * (kb + i) + 16 * rw + c) * 64 + 32 * sh + 8 * g) = v;
          }
        }
        lds_barrier();
      }
    }
    {
      // D = rowsum(dO * out) of this lane's head: its dO fragments times the same elements of
      // out, summed over the 4 lanes (g) that hold the head; then the head's statistics
      float d = 0.f;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const u32x4 y = oy[ks];
        const u32x4 x = __builtin_bit_cast(u32x4, doA[ks]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          d += x2f<F16>((uint16_t)(x[w] & 0xffffu)) * x2f<F16>((uint16_t)(y[w] & 0xffffu));
          d += x2f<F16>((uint16_t)(x[w] >> 16)) * x2f<F16>((uint16_t)(y[w] >> 16));
        }
      }
      d += __shfl_xor(d, 16);
      d += __shfl_xor(d, 32);
      if (g == 0) {
        sD[h] = d;                                    // padded heads: 0 (their dO is zero)
        sM[h] = smv * kLog2e;
        sIL[h] = ssv > 0.f ? 1.f / ssv : 0.f;
      }
    }
    f32x4 sacc[2], pacc[2];
    const int kse = ktile_off(g, c);                // chunk g of key c
// Score step CI on key buffer KC and dS buffer DC; ends by waiting for this wave's LDS accesses
// (the record stores stay in flight).
#define SFAG_SSTEP(CI, KC, DC)                                                                 \
  {                                                                                            \
    if ((CI) < nchunk) {                                                                       \
      SFAG_SCORES(KC)                                                                          \
      SFAG_FINISH(CI, DC)                                                                      \
    }                                                                                          \
    lds_barrier();                                                                             \
  }
    int ci = 0;
    for (; ci + 3 <= nchunk; ci += 4) {
      SFAG_SSTEP(ci, Kb0, Db0)
      SFAG_SSTEP(ci + 1, Kb1, Db1)
      SFAG_SSTEP(ci + 2, Kb2, Db0)
      SFAG_SSTEP(ci + 3, Kb3, Db1)
    }
    if (ci <= nchunk) {
      SFAG_SSTEP(ci, Kb0, Db0)
      ++ci;
    }
    if (ci <= nchunk) {
      SFAG_SSTEP(ci, Kb1, Db1)
      ++ci;
    }
    if (ci <= nchunk) SFAG_SSTEP(ci, Kb2, Db0)
#undef SFAG_SSTEP
  } else {
    // chunks 0 and 1 in flight before the score waves' copy of Q | QRope | dO (chunk 1 repeats
    // chunk 0's last position when the row has one chunk); the position of chunk 2's key is
    // loaded too.  Loads complete in order, so vmcnt(10) leaves chunk 1's gather and that position
    // load outstanding.
    int32_t gsv = srow[min(gkey, count - 1)];
    SFAG_GATHER_ASYNC(Kb0, 0, gsv)
    gsv = srow[min(kKC + gkey, count - 1)];
    SFAG_GATHER_ASYNC(Kb1, 1, gsv)
    gsv = srow[min(2 * kKC + gkey, count - 1)];
    for (int k = 0; k < 2 * kCopyRounds - 1; ++k) lds_barrier();   // the score waves' copy of Q | QRope | dO
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitVm10);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // transposing-read lane offsets (keys 4 g + c / 4 and, at the second read, + 16): K tile
    // (dims 16 rw + 4 (c % 4) of chunk group 0, i.e. chunk 2 rw + (c % 4) / 2) and dS tile
    // ([key][head], pitch 72; head 4 (c % 4))
    const int tk = 4 * g + (c >> 2);
    const int kqoff = tk * 64 + (((2 * rw + ((c & 3) >> 1)) ^ ktile_swz(tk)) << 3) + 4 * (c & 1);
    const int dsoff = tk * kHtPitch + 4 * (c & 3);
    f32x4 dqacc[4][9];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int nt = 0; nt < 9; ++nt) dqacc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
// dQ step CI: the position of chunk CI + 3's key, the gather of chunk CI + 2 into KN, dQ of chunk
// CI - 1 from KP / DP.  Ends by waiting for chunk CI + 1's gather (issued a step earlier) and the
// position load, leaving this step's gather in flight, and for the LDS reads.  Every step issues
// the same vector memory operations (past the last chunk the gather repeats the row's last
// position into the free buffer KN), so that one wait count fits all and the compiler's own
// wait analysis sees the same pattern on every path.
#define SFAG_QSTEP(CI, KP, KN, DP)                                                             \
  {                                                                                            \
    const int32_t sv = srow[min(((CI) + 3) * kKC + gkey, count - 1)];                          \
    /* the position load must be issued before the gather for the wait count below */          \
    asm volatile("" ::: "memory");                                                             \
    SFAG_DQ_GATHER(KP, DP, KN, gsv)                                                            \
    asm volatile("" ::: "memory");                                                             \
    __builtin_amdgcn_s_waitcnt(kWaitVm9);                                                      \
    gsv = sv;                                                                                  \
    __builtin_amdgcn_s_barrier();                                                              \
    asm volatile("" ::: "memory");                                                             \
  }
    // step 0: no dQ yet (chunk 0 is being scored), only the position of chunk 3 and the gather
    // of chunk 2
    {
      const int32_t sv = srow[min(3 * kKC + gkey, count - 1)];
      asm volatile("" ::: "memory");
      SFAG_GATHER_ASYNC(Kb2, 2, gsv)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(kWaitVm9);
      gsv = sv;
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    int ci = 1;
    for (; ci + 3 <= nchunk; ci += 4) {
      SFAG_QSTEP(ci, Kb0, Kb3, Db0)
      SFAG_QSTEP(ci + 1, Kb1, Kb0, Db1)
      SFAG_QSTEP(ci + 2, Kb2, Kb1, Db0)
      SFAG_QSTEP(ci + 3, Kb3, Kb2, Db1)
    }
    if (ci <= nchunk) {
      SFAG_QSTEP(ci, Kb0, Kb3, Db0)
      ++ci;
    }
    if (ci <= nchunk) {
      SFAG_QSTEP(ci, Kb1, Kb0, Db1)
      ++ci;
    }
    if (ci <= nchunk) SFAG_QSTEP(ci, Kb2, Kb1, Db0)
#undef SFAG_QSTEP
    __builtin_amdgcn_s_waitcnt(0);                        // no gather may still write LDS at exit

    // ---- dQ / dQRope out: lane holds heads 16 t + 4 g + v, dims 16 (rw + 4 nt) + c -------------
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int h = 16 * t + 4 * g + v;
        if (h >= nh) continue;
        const int64_t hh2 = row * a.N1 + h0 + h;
#pragma unroll
        for (int nt = 0; nt < 9; ++nt) {
          // lanes c and c ^ 1 hold neighbouring dims: the even lane stores both as one word
          const float x = dqacc[t][nt][v] * a.scale;
          const float y = dpp_f<kDppXor1>(x);
          const int col = 16 * (rw + 4 * nt) + c;
          if ((c & 1) == 0) {
            const uint32_t pv = pack_x2<F16>(x, y);
            if (col < kDn) *reinterpret_cast<uint32_t*>(a.dq + hh2 * kDn + col) = pv;
            else if (a.dqr) *reinterpret_cast<uint32_t*>(a.dqr + hh2 * kDr + col - kDn) = pv;
          }
        }
      }
    }
  }

#undef SFAG_GATHER_ASYNC
#undef SFAG_SCORES
#undef SFAG_DQ
#undef SFAG_DQ_GATHER
#undef SFAG_FINISH
}

hipError_t launch_bwd_q(const BwdArgs& a, int64_t nrows, int hg_count, hipStream_t st) {
  if (a.f16)
    hipLaunchKernelGGL(bwd_q_kernel<true>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_q_kernel<false>, dim3((unsigned)nrows, (unsigned)hg_count), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}


}  // namespace sfag
