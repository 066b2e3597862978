// sfag_indexer.hip -- backward of the lightning indexer with its KL loss (gfx950).
//
// DenseLightningIndexerGradKLLoss README, "function description": per query token t and the keys
// s its mask admits,
//   index scores  S[g, s] = q~[t, g] . K~[s],   I[s] = sum_g W[t, g] ReLU(S[g, s])
//   target        p[s] = head-summed main-attention softmax, L1-normalised over s
//   loss          sum_t KL(p || Softmax(I))
//   gradients     dI = Softmax(I) - p,  dW[t, g] = sum_s dI[s] ReLU(S[g, s]),
//                 dS = dI W [S > 0],  dq~[t, g] = sum_s dS[g, s] K~[s],  dK~[s] += dS^T q~[t].
// The main softmax is rebuilt from the forward's statistics on the MLA logits q . k + qRope .
// kRope (times scaleValue), and Softmax(I) from the indexer forward's statistics.
//
// Kernels:
//   ix_query_kernel  one workgroup of 8 waves per query row, keys in chunks of 32 (key rows
//                    staged in LDS, next chunk loaded while this one is computed).  Main waves
//                    0-3 (head tiles w, w + 4) form the main scores on the MFMA and the chunk's
//                    head-summed softmax; index waves 4-7 (index-head tile w - 4) form S and
//                    their part of I.  After a barrier the index waves form Softmax(I) and the
//                    gradient terms, and add dq~ on the MFMA.  The head sum's L1 norm is known
//                    only after the last chunk, so the chunk terms use 1 / (heads) and a second
//                    accumulator carries the correction (1 / heads - 1 / norm), applied at the
//                    end: exact for any statistics, and without cancellation in 16-bit operands
//                    (the main term is the small difference itself).  Writes dq~, dW, the row's
//                    loss and norm, and the head sum of every (row, key) for the key kernel.
//   ix_key_kernel    workgroup = (64 keys, part of the query rows): per query row, S for its
//                    keys (recomputed on the MFMA), Softmax(I), dI = Softmax(I) - sum / norm,
//                    dS, and dK~ += dS^T q~ on the MFMA into registers; fp32 partials per part.
//   ix_finish_kernel dK~ = sum of the parts in part order, and the loss = sum of the rows' losses
//                    in row order (one workgroup); deterministic.
#include "sfag_device.h"
#include "sfag_dpp.h"
#include "sfag_ktile.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kIxThreads = 512;                   // query kernel: 8 waves
constexpr int kIxKC = 32;                         // keys per chunk
constexpr int kKPitch = kDk + 8;                  // 584: main key rows (512 + 64 rope) in LDS
constexpr int kIPitch = kIxDi + 8;                // 136: index rows in LDS
constexpr int kDsPitch = kIxKC + 8;               // 40: [16 heads][32 keys] gradient tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeyThreads = 256;                  // key kernel: 4 waves of 16 keys
constexpr int kKeyTile = 64;
constexpr int kDkPitch = 64 + 8;                  // [16 keys][64 index heads] dS tile per wave

__device__ __forceinline__ float wsum16(float v) {  // sum over the 16 lanes c of a 16-lane group
  return row16_sum(v);
}
}  // namespace

// ------------------------------------------------------------------------------------------
template <bool F16>
__global__ void __launch_bounds__(kIxThreads, 1) ix_query_kernel(IxArgs a) {
  // chunk buffers: three for the main key rows (9 chunk groups; separate arrays, so that the
  // compiler can tell a direct-to-LDS load into one from reads of the others) and four for the
  // index key rows (2 chunk groups; read one step longer), both in the swizzled [chunk
  // group][key][slot] layout of sfag_ktile.h
  __shared__ __attribute__((aligned(16))) uint16_t Kt0[kIxKC * kDk], Kt1[kIxKC * kDk], Kt2[kIxKC * kDk];
  __shared__ __attribute__((aligned(16))) uint16_t Kib[4][kIxKC * kIxDi];   // index rows, chunk c in Kib[c % 4]
  __shared__ __attribute__((aligned(16))) uint16_t Dt[4][2][16 * kDsPitch];   // per index wave: dS', T
  __shared__ float sP[2][4][kIxKC];              // chunk c % 2, per main wave: softmax summed over its heads
  __shared__ float sI[2][4][kIxKC];              // chunk c % 2, per index wave: its part of I
  __shared__ float sM[128], sIL[128];            // main statistics (log2 domain), 1 / sum
  __shared__ float sRed[4];
  __shared__ int32_t cum[2 * 257];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = (int64_t)gridDim.x - 1 - blockIdx.x;     // long rows first
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  const int G = a.G;
  const int nit = (G + 15) >> 4;                  // index-head tiles (<= 4)
  const int nmt = (a.N1 + 15) >> 4;               // main-head tiles (<= 8)
  const bool live = geo.active && geo.hi >= 0 && a.ssum_i[row] > 0.f;
  if (!live) {
    for (int e = threadIdx.x; e < G * kIxDi; e += kIxThreads) a.dqi[row * G * kIxDi + e] = 0;
    for (int e = threadIdx.x; e < G; e += kIxThreads) a.dw[row * G + e] = 0;
    if (threadIdx.x == 0) {
      a.lrow[row] = 0.f;
      a.norm[row] = 0.f;
    }
    return;
  }
  const int nkeys = geo.hi + 1;
  const int nchunk = (nkeys + kIxKC - 1) / kIxKC;
  const float zscale = a.scale * kLog2e;
  // main statistics; heads with an empty sum take no part (their softmax is zero)
  for (int h = threadIdx.x; h < 128; h += kIxThreads) {
    float m = 0.f, il = 0.f;
    if (h < a.N1) {
      const int64_t j = stat_index(a.layout_tnd, geo, row, a.N1, a.S1, h);
      const float l = a.ssum[j];
      if (l > 0.f) {
        m = a.smax[j] * kLog2e;
        il = 1.f / l;
      }
    }
    sM[h] = m;
    sIL[h] = il;
  }
  __syncthreads();
  int heads = 0;
  for (int h = 0; h < a.N1; ++h) heads += sIL[h] > 0.f ? 1 : 0;
  const float inv_heads = heads > 0 ? 1.f / (float)heads : 0.f;
  const float max_i = a.smax_i[row], lsum_i = __logf(a.ssum_i[row]);

  // Gathers: the keys of a chunk are consecutive rows, clamped to the last admitted key (the
  // clamped copies are masked).  A direct-to-LDS block (64 lanes x 16 bytes) is one 128-byte run
  // (chunk group) of 8 keys: main wave w loads keys 8 w .. 8 w + 7 of the 9 groups of the main
  // rows (value groups 0..7, rope group 8; a rope-less call reads value columns instead, whose Q
  // is zero) and of the 2 groups of the index rows.  The index waves issue no direct-to-LDS
  // loads: while one is in flight the compiler makes a wave's ordinary LDS accesses wait for all
  // its loads, and the index waves read and write LDS through ordinary accesses every step.
  const int gkey = ktile_gather_key(wave & 3, lane);
  const uint32_t gcol = ktile_gather_col(wave & 3, lane);
  const int kse = ktile_off(g, c);               // fragment reads: chunk g of key c
  const bool has_rope = a.kr != nullptr;
  const char* kb8 = reinterpret_cast<const char*>(a.k + geo.kstart * kDn);
  const char* kr8 = has_rope ? reinterpret_cast<const char*>(a.kr + geo.kstart * kDr) : kb8;
  const char* ki8 = reinterpret_cast<const char*>(a.ki + geo.kstart * kIxDi);
  typedef __attribute__((address_space(3))) void LdsVoid;
#define IX_GATHER_MAIN(KT, CH)                                                                  \
  {                                                                                            \
    const uint32_t key_ = (uint32_t)min((CH) * kIxKC + gkey, nkeys - 1);                       \
    _Pragma("unroll") for (int j = 0; j < 9; ++j) {                                            \
      const char* src_ = j < 8 ? kb8 + key_ * (uint32_t)(kDn * 2) + j * 128 + gcol             \
                               : (has_rope ? kr8 + key_ * (uint32_t)(kDr * 2) + gcol           \
                                           : kb8 + key_ * (uint32_t)(kDn * 2) + gcol);          \
      __builtin_amdgcn_global_load_lds(src_, (LdsVoid*)((KT) + (4 * j + wave) * 512), 16, 0, 0); \
    }                                                                                          \
  }
#define IX_GATHER_INDEX(KI, CH)                                                                 \
  {                                                                                            \
    const uint32_t key_ = (uint32_t)min((CH) * kIxKC + gkey, nkeys - 1);                       \
    _Pragma("unroll") for (int j = 0; j < 2; ++j)                                              \
      __builtin_amdgcn_global_load_lds(ki8 + key_ * (uint32_t)(kIxDi * 2) + j * 128 + gcol,    \
                                       (LdsVoid*)((KI) + (4 * j + wave) * 512), 16, 0, 0);     \
  }
  // fragment read of step ks (chunk 4 ks + g) of key tile kt (keys 16 kt + c): chunk group ks / 2,
  // slot bit 2 = ks % 2, key 16 + c 1024 elements after key c
#define IX_KFRAG(KC, KS, KT) \
  (*reinterpret_cast<const bf16x8*>((KC) + (((KS) & 1) ? (kse ^ 32) : kse) + ((KS) >> 1) * 2048 + (KT) * 1024))
  // s_waitcnt operand with expcnt and lgkmcnt at zero: vmcnt(11): all but a main wave's newest
  // gather (9 main-row and 2 index-row loads)
  constexpr int kWaitMain = 0x000b;

  // Two roles with separate loops (their registers are never live together) and the same
  // barriers: one before step 0, one per step.  Step c: the main waves gather chunk c + 2 into
  // the buffers chunk c - 1 (main rows) and c - 2 (index rows) used, form the scores of chunk c
  // and its head-summed softmax, and wait for chunk c + 1; meanwhile the index waves form the
  // gradient terms of chunk c - 1 (from the head sums and partial I of the previous step), add
  // dq~ of chunk c - 1, and form the index scores of chunk c.
  if (wave < 4) {
    // A operands: Q of head 16 t + c (dims 32 ks + 8 g; steps 16, 17: rope), for t = w, w + 4
    bf16x8 qA[2][18];
    bool has[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = wave + 4 * u;
      has[u] = t < nmt;
      const int h = 16 * t + c;
      const bool okh = has[u] && h < a.N1;
      const uint16_t* qrow = a.q + (row * a.N1 + min(h, a.N1 - 1)) * kDn;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qA[u][ks] = okh ? *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g) : bf16x8{};
#pragma unroll
      for (int ks = 16; ks < 18; ++ks)
        qA[u][ks] = (okh && a.qr)
                        ? *reinterpret_cast<const bf16x8*>(a.qr + (row * a.N1 + h) * kDr + 32 * (ks - 16) + 8 * g)
                        : bf16x8{};
    }
    IX_GATHER_MAIN(Kt0, 0)
    IX_GATHER_INDEX(Kib[0], 0)
    IX_GATHER_MAIN(Kt1, 1)
    IX_GATHER_INDEX(Kib[1], 1)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitMain);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#define IX_MSTEP(CI, KC, KN)                                                                   \
  {                                                                                            \
    IX_GATHER_MAIN(KN, min((CI) + 2, nchunk - 1))                                              \
    IX_GATHER_INDEX(Kib[((CI) + 2) & 3], min((CI) + 2, nchunk - 1))                            \
    if ((CI) < nchunk) {                                                                       \
      float ps[2] = {0.f, 0.f};                                                                \
      _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                          \
        if (!has[u]) continue;                                                                 \
        const int t = wave + 4 * u;                                                            \
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};                \
        _Pragma("unroll") for (int ks = 0; ks < 18; ++ks)                                      \
          _Pragma("unroll") for (int kt = 0; kt < 2; ++kt)                                     \
            sacc[kt] = mfma_t<F16>(qA[u][ks], IX_KFRAG(KC, ks, kt), sacc[kt]);                 \
        const f32x4 mv = *reinterpret_cast<const f32x4*>(sM + 16 * t + 4 * g);                 \
        const f32x4 iv = *reinterpret_cast<const f32x4*>(sIL + 16 * t + 4 * g);                \
        _Pragma("unroll") for (int kt = 0; kt < 2; ++kt)                                       \
          _Pragma("unroll") for (int v = 0; v < 4; ++v)                                        \
            ps[kt] += __builtin_amdgcn_exp2f(sacc[kt][v] * zscale - mv[v]) * iv[v];            \
      }                                                                                        \
      _Pragma("unroll") for (int kt = 0; kt < 2; ++kt) {                                       \
        const float p_ = col4_sum(ps[kt]);                                                     \
        if (g == 0) sP[(CI) & 1][wave][16 * kt + c] = (CI) * kIxKC + 16 * kt + c < nkeys ? p_ : 0.f; \
      }                                                                                        \
    }                                                                                          \
    asm volatile("" ::: "memory");                                                             \
    __builtin_amdgcn_s_waitcnt(kWaitMain);                                                     \
    __builtin_amdgcn_s_barrier();                                                              \
    asm volatile("" ::: "memory");                                                             \
  }
    int ci = 0;
    for (; ci + 3 <= nchunk + 1; ci += 3) {
      IX_MSTEP(ci, Kt0, Kt2)
      IX_MSTEP(ci + 1, Kt1, Kt0)
      IX_MSTEP(ci + 2, Kt2, Kt1)
    }
    if (ci <= nchunk) {
      IX_MSTEP(ci, Kt0, Kt2)
      ++ci;
    }
    if (ci <= nchunk) IX_MSTEP(ci, Kt1, Kt0)
#undef IX_MSTEP
    __builtin_amdgcn_s_waitcnt(0);                // no gather may still write LDS at exit
    __syncthreads();                              // the index waves' row results
    return;
  }

  const int it = wave - 4;
  const bool hasi = it < nit;
  bf16x8 qiA[4];
  float wv[4];                                    // W of this lane's C rows (index heads 16 it + 4 g + v)
  {
    const int h = 16 * it + c;
    const bool okh = hasi && h < G;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qiA[ks] = okh ? *reinterpret_cast<const bf16x8*>(a.qi + (row * G + h) * kIxDi + 32 * ks + 8 * g) : bf16x8{};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hh = 16 * it + 4 * g + v;
      wv[v] = (hasi && hh < G) ? x2f<F16>(a.w[row * G + hh]) : 0.f;
    }
  }
  // dq~ contraction over the chunk's keys in the order 4 g + j, 4 g + 16 + j (j = 0..3) for lane
  // group g, in both operands: the dS' / T tiles hold key 16 kt + c at 8 (c / 4) + c % 4 + 4 kt;
  // the transposing reads of the index key tile point lane (g, c) at key 4 g + c / 4 and dims
  // 16 nt + 4 (c % 4) (chunk group nt / 4, slot (2 (nt % 4) + (c % 4) / 2) ^ swz), keys + 16 at
  // 1024 elements on
  const int tk = 4 * g + (c >> 2);
  const int kq0 = tk * 64 + 4 * (c & 1) + ((((c & 3) >> 1) ^ ktile_swz(tk)) << 3);
  // accumulators: dq~ (main term and correction term), dW terms, loss terms
  f32x4 qacc[8], tacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) qacc[nt] = tacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float aw[4] = {0.f, 0.f, 0.f, 0.f}, bw[4] = {0.f, 0.f, 0.f, 0.f};
  float l1 = 0.f, nrm = 0.f;
  f32x4 iprev[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};   // S of the previous chunk

  // chunks 0 and 1 are gathered by the main waves
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  for (int ci = 0; ci <= nchunk; ++ci) {
    if (hasi && ci >= 1) {
      // gradient terms of chunk ci - 1: head sums (main waves) and partial I (index waves) of
      // the previous step
      const int s0 = (ci - 1) * kIxKC, pb = (ci - 1) & 1;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = 16 * kt + c;
        const int kpos = 8 * (c >> 2) + (c & 3) + 4 * kt;     // key's place in the dq~ key order
        const bool valid = s0 + key < nkeys;
        const float tot = valid ? sP[pb][0][key] + sP[pb][1][key] + sP[pb][2][key] + sP[pb][3][key] : 0.f;
        float ival = 0.f;
        for (int u = 0; u < nit; ++u) ival += sI[pb][u][key];
        const float lsm = ival - max_i - lsum_i;             // log Softmax(I)
        const float sm = valid ? __expf(lsm) : 0.f;
        const float dip = sm - tot * inv_heads;              // dI with the provisional norm
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float sv_ = iprev[kt][v];
          const float relu = fmaxf(sv_, 0.f);
          aw[v] += dip * relu;
          bw[v] += tot * relu;
          Dt[it][0][(4 * g + v) * kDsPitch + kpos] = f2x<F16>(sv_ > 0.f ? dip : 0.f);
          Dt[it][1][(4 * g + v) * kDsPitch + kpos] = f2x<F16>(sv_ > 0.f ? tot : 0.f);
        }
        if (it == 0 && g == 0 && valid) {
          if (tot > 0.f) l1 += tot * (__logf(tot) - lsm);
          nrm += tot;
          a.tot[row * a.kstride + s0 + key] = tot;           // the head sum, for the key kernel
        }
      }
      // dq~ += dS' K~ and the correction term T K~ of chunk ci - 1 (this wave's own tiles)
      const uint16_t* KP = Kib[(ci + 3) & 3];
      const bf16x8 da = *reinterpret_cast<const bf16x8*>(&Dt[it][0][c * kDsPitch + 8 * g]);
      const bf16x8 ta = *reinterpret_cast<const bf16x8*>(&Dt[it][1][c * kDsPitch + 8 * g]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 kb_ = tr_frag(KP + ((kq0 ^ (16 * (nt & 3))) + 2048 * (nt >> 2)), 1024);
        qacc[nt] = mfma_t<F16>(da, kb_, qacc[nt]);
        tacc[nt] = mfma_t<F16>(ta, kb_, tacc[nt]);
      }
    }
    if (hasi && ci < nchunk) {
      // index scores of chunk ci and this wave's part of I
      const uint16_t* KC = Kib[ci & 3];
      f32x4 iacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) iacc[kt] = mfma_t<F16>(qiA[ks], IX_KFRAG(KC, ks, kt), iacc[kt]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float is = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) is += wv[v] * fmaxf(iacc[kt][v], 0.f);
        is = col4_sum(is);
        if (g == 0) sI[ci & 1][it][16 * kt + c] = is;
        iprev[kt] = iacc[kt];
      }
    }
    lds_barrier();
  }
#undef IX_GATHER_MAIN
#undef IX_GATHER_INDEX
#undef IX_KFRAG
  __builtin_amdgcn_s_waitcnt(0);                  // no gather may still write LDS at exit

  // ---- row results ----
  if (it == 0) {
    l1 = wsum16(l1);
    nrm = wsum16(nrm);
    if (lane == 0) {
      sRed[0] = l1;
      sRed[1] = nrm;
    }
  }
  __syncthreads();
  const float norm = sRed[1];
  const float corr = norm > 0.f ? inv_heads - 1.f / norm : 0.f;
  if (wave == 4 && lane == 0) {
    a.norm[row] = norm;
    a.lrow[row] = norm > 0.f ? sRed[0] / norm - __logf(norm) : 0.f;
  }
  if (hasi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float d = wsum16(aw[v]) + corr * wsum16(bw[v]);
      const int hh = 16 * it + 4 * g + v;
      if (c == 0 && hh < G) a.dw[row * G + hh] = f2x<F16>(d);
    }
    // lanes c and c ^ 1 hold neighbouring dims: the even lane stores both as one word
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int hh = 16 * it + 4 * g + v;
        const float x = wv[v] * (qacc[nt][v] + corr * tacc[nt][v]);
        const float y = dpp_f<kDppXor1>(x);
        if (hh < G && (c & 1) == 0)
          *reinterpret_cast<uint32_t*>(a.dqi + (row * G + hh) * kIxDi + 16 * nt + c) = pack_x2<F16>(x, y);
      }
  }
}

// ------------------------------------------------------------------------------------------
// dK~ partials: workgroup = (64 keys of one batch, part of that batch's query rows); wave w owns
// keys 16 w .. 16 w + 15 of the tile.  Per query row: S'[key][head] = K~[key] . q~[head] (A =
// this wave's K~ rows, held in registers; B = the row's q~ tile in LDS), I, Softmax(I),
// dI = Softmax(I) - sum / norm, dS'[key][head] = dI W [S' > 0] (through a per-wave LDS tile),
// and dK~[key][dims] += dS' q~ on the MFMA.
template <bool F16>
__global__ void __launch_bounds__(kKeyThreads, 2) ix_key_kernel(IxArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][64 * kIPitch];     // [index head][dims]
  __shared__ __attribute__((aligned(16))) uint16_t Dk[4][16 * kDkPitch];    // per wave [key][head]
  __shared__ float sW[2][64];
  __shared__ int32_t cum[2 * 257], kbase_tile[257];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int G = a.G;
  // tile -> batch: tiles of 64 keys per batch, numbered batch by batch
  for (int t = threadIdx.x; t <= a.B; t += blockDim.x) {
    int32_t sq = 0, skv = 0, nt = 0;
    for (int b = 0; b < t; ++b) {
      const int lq = a.layout_tnd ? a.lens.lq[b] : (int)a.S1;
      const int lk = a.layout_tnd ? a.lens.lkv[b] : (int)a.S2;
      sq += lq;
      skv += lk;
      nt += (lk + kKeyTile - 1) / kKeyTile;
    }
    cum[t] = sq;
    cum[257 + t] = skv;
    kbase_tile[t] = nt;
  }
  __syncthreads();
  const int tile = blockIdx.x, part = blockIdx.y;
  int b = 0;
  {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (kbase_tile[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
  const int nk = a.layout_tnd ? lkv : (int)a.S2;     // key rows of the batch (BSND: padded too)
  const int kt0 = (tile - kbase_tile[b]) * kKeyTile;
  const int64_t q0 = cum[b], k0 = cum[257 + b];
  // query rows that admit a key of the tile: i >= kt0 - (lkv - lq) under the causal mode
  int ilo = 0;
  if (a.mode3) ilo = max(0, kt0 - (lkv - lq));
  if (kt0 >= lkv) ilo = lq;                           // padded keys: no row admits them
  const int span = max(0, lq - ilo);
  const int per = (span + a.parts - 1) / a.parts;
  const int i0 = min(lq, ilo + part * per), i1 = min(lq, i0 + per);

  // this wave's keys: rows of the A operand (K~, dims 32 ks + 8 g), zero past the batch's keys
  const int mykey = kt0 + 16 * wave + c;
  bf16x8 kA[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    kA[ks] = mykey < lkv ? *reinterpret_cast<const bf16x8*>(a.ki + (k0 + mykey) * kIxDi + 32 * ks + 8 * g)
                         : bf16x8{};
  f32x4 dacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) dacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nit = (G + 15) >> 4;

  // q~ tile staging: 64 heads x 16 pieces of 16 bytes, 4 per thread (heads past G read zeros)
  u32x4 st[4];
  float stw = 0.f;
  auto load_row = [&](int i) {
    const int64_t r = q0 + i;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = (int)threadIdx.x + kKeyThreads * u;
      const int h = e >> 4, j = e & 15;
      st[u] = h < G ? *reinterpret_cast<const u32x4*>(a.qi + (r * G + h) * kIxDi + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
    stw = threadIdx.x < 64 && (int)threadIdx.x < G ? x2f<F16>(a.w[r * G + threadIdx.x]) : 0.f;
  };
  auto store_row = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = (int)threadIdx.x + kKeyThreads * u;
      const int h = e >> 4, j = e & 15;
      *reinterpret_cast<u32x4*>(&Qt[buf][h * kIPitch + 8 * j]) = st[u];
    }
    if (threadIdx.x < 64) sW[buf][threadIdx.x] = stw;
  };

  if (i0 < i1) {
    load_row(i0);
    store_row(0);
  }
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    const int buf = (i - i0) & 1;
    if (i + 1 < i1) load_row(i + 1);
    const int64_t r = q0 + i;
    // keys this row admits: positions <= hi
    const int hi = a.mode3 ? min(lkv - 1, i + lkv - lq) : lkv - 1;
    const float norm = a.norm[r];
    const float inv_norm = norm > 0.f ? 1.f / norm : 0.f;
    const float max_i = a.smax_i[r];
    const float sum_i = a.ssum_i[r];
    const float lsum_i = sum_i > 0.f ? __logf(sum_i) : 0.f;
    // S'[key 4 g + v][head 16 nt + c]
    f32x4 sacc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt < nit)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sacc[nt] = mfma_t<F16>(kA[ks], lds_read8p(Qt[buf], 16 * nt + c, 32 * ks + 8 * g, kIPitch), sacc[nt]);
    }
    float wl[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) wl[nt] = sW[buf][16 * nt + c];
    const int kb = kt0 + 16 * wave + 4 * g;       // first key of this lane's C rows
    float tot4[4];
    {
      const float* tp = a.tot + r * a.kstride;
#pragma unroll
      for (int v = 0; v < 4; ++v) tot4[v] = (kb + v <= hi && sum_i > 0.f) ? tp[kb + v] : 0.f;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float is = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) is += wl[nt] * fmaxf(sacc[nt][v], 0.f);
      is = wsum16(is);
      const bool valid = kb + v <= hi && sum_i > 0.f;
      const float sm = valid ? __expf(is - max_i - lsum_i) : 0.f;
      const float di = sm - tot4[v] * inv_norm;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        Dk[wave][(4 * g + v) * kDkPitch + 16 * nt + c] = f2x<F16>(sacc[nt][v] > 0.f ? di * wl[nt] : 0.f);
    }
    // the tile is read by other lanes of this wave only
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bf16x8 dA[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) dA[ks] = *reinterpret_cast<const bf16x8*>(&Dk[wave][c * kDkPitch + 32 * ks + 8 * g]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        dacc[nt] = mfma_t<F16>(dA[ks], lds_frag_trp(Qt[buf], 32 * ks, 16 * nt, kIPitch, lane), dacc[nt]);
    if (i + 1 < i1) store_row(buf ^ 1);
    lds_barrier();
  }
  // partial rows (all 64 keys of the tile that exist in the batch's key rows)
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int key = kt0 + 16 * wave + 4 * g + v;
    if (key < nk)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        a.dkp[((int64_t)part * a.keys + k0 + key) * kIxDi + 16 * nt + c] = dacc[nt][v];
  }
}

// ------------------------------------------------------------------------------------------
// blockIdx.x < keys: one key row, dK~ = sum of the parts in part order.  The last workgroup
// (blockIdx.x == keys) sums the rows' losses in row order.
template <bool F16>
__global__ void __launch_bounds__(kIxDi) ix_finish_kernel(IxArgs a) {
  const int64_t key = blockIdx.x;
  if (key < a.keys) {
    float s = 0.f;
    for (int p = 0; p < a.parts; ++p) s += a.dkp[((int64_t)p * a.keys + key) * kIxDi + threadIdx.x];
    a.dki[key * kIxDi + threadIdx.x] = f2x<F16>(s);
    return;
  }
  __shared__ float part[kIxDi];
  float s = 0.f;
  for (int64_t r = threadIdx.x; r < a.rows; r += kIxDi) s += a.lrow[r];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int j = 0; j < kIxDi; ++j) t += part[j];
    a.loss[0] = t;
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_indexer(const IxArgs& a, int64_t key_tiles, hipStream_t st) {
  if (a.rows > 0) {
    if (a.f16) hipLaunchKernelGGL(ix_query_kernel<true>, dim3((unsigned)a.rows), dim3(kIxThreads), 0, st, a);
    else hipLaunchKernelGGL(ix_query_kernel<false>, dim3((unsigned)a.rows), dim3(kIxThreads), 0, st, a);
  }
  if (key_tiles > 0) {
    const dim3 grid((unsigned)key_tiles, (unsigned)a.parts);
    if (a.f16) hipLaunchKernelGGL(ix_key_kernel<true>, grid, dim3(kKeyThreads), 0, st, a);
    else hipLaunchKernelGGL(ix_key_kernel<false>, grid, dim3(kKeyThreads), 0, st, a);
  }
  if (a.f16) hipLaunchKernelGGL(ix_finish_kernel<true>, dim3((unsigned)(a.keys + 1)), dim3(kIxDi), 0, st, a);
  else hipLaunchKernelGGL(ix_finish_kernel<false>, dim3((unsigned)(a.keys + 1)), dim3(kIxDi), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfag
