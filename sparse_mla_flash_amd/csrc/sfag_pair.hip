// sfag_pair.hip -- per-pair dK / dV for SparseFlashAttentionGrad selections too sparse for the
// key-major kernel (gfx950).
//
// The page's stage 1 and stage 3 scatter each query row's contributions into the selected key
// rows: dV[u] += P^T dO and dK[u] += scale dS^T Q (SparseFlashAttentionGrad README, "function
// description").  When every row selects a small fraction of the keys it can reach, the
// key-major kernel would multiply mostly zeros, so here the work follows the pairs:
//   pair_slots_kernel  per 256-key block, a stable counting sort of the chunk's pairs of the block
//                      by key: every pair gets its slot, every key its run of slots;
//   pair_kv_kernel     per query row, the [positions x heads] dS (or P) records times the row's
//                      [heads x 1088] Q | QRope (or dO) on the MFMA: one fp32 partial row of
//                      1088 values per valid (row, position) pair, written to its slot;
//   pair_sum_kernel    per key, its run of partial rows added in slot order (one wave per key).
// Slots are numbered key-major: the pairs of key block 0 first, inside a block key by key, and
// the pairs of one key in ascending (row, position) order.  A key's sum therefore runs over its
// pairs in a fixed order, and query rows are taken in fixed chunks in order: the result is
// bit-reproducible, with or without the deterministic flag.
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kThreads = 256;

// Per-batch tables in LDS: first query row / key row of every batch (cum[0..B], cum[257..257+B])
// and the first key block of every batch (bstart[0..B]).  The reduce covers ceil(S2 / 256) blocks
// per batch for BSND (padded key rows included, so they get zeros) and ceil(Lkv / 256) for TND.
__device__ __forceinline__ void pair_tables(const PairArgs& a, int32_t* cum, int32_t* bstart) {
  for (int t = threadIdx.x; t <= a.B; t += blockDim.x) {
    int32_t sq = 0, skv = 0, nb = 0;
    for (int b = 0; b < t; ++b) {
      sq += a.layout_tnd ? a.lens.lq[b] : (int32_t)a.S1;
      skv += a.layout_tnd ? a.lens.lkv[b] : (int32_t)a.S2;
      nb += ((a.layout_tnd ? a.lens.lkv[b] : (int32_t)a.S2) + kBk - 1) / kBk;
    }
    cum[t] = sq;
    cum[257 + t] = skv;
    bstart[t] = nb;
  }
}

// batch of global key block gb (last batch whose first block is <= gb)
__device__ __forceinline__ int batch_of_block(const int32_t* bstart, int B, int gb) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bstart[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}
}  // namespace

// ------------------------------------------------------------------------------------------
// Slots of one chunk of query rows, per key block gb (batch b, block lb): the block's pairs, in
// (row, position) order, counting-sorted by key.  16 waves; wave w takes a contiguous range of
// the chunk's rows of batch b.  Pass 1 counts every key's pairs per wave; the counts are turned
// into starting offsets (keys ascending, waves ascending inside a key); pass 2 walks the same
// pairs again and gives each its offset: a pair's slot is bbase[gb] + loc.  Within a wave, 64
// consecutive pairs are ranked at once: lanes holding the same key find each other with eight
// ballots over the key's bits.
constexpr int kSlotWaves = 16;

// lanes of this wave holding the same key byte (valid lanes only)
__device__ __forceinline__ uint64_t same_key_lanes(int key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool bit = (key >> i) & 1;
    const uint64_t on = __ballot(bit);
    m &= bit ? on : ~on;
  }
  return m;
}

template <bool kRank>
__device__ __forceinline__ void slot_pass(const PairArgs& a, int32_t* wcnt, int32_t* wpre, int32_t* wo,
                                          int64_t rbeg, int64_t rend, int lb, int lane) {
  const uint64_t lt = (1ull << lane) - 1;
  for (int64_t rt = rbeg; rt < rend; rt += 64) {
    const int64_t r = rt + lane;
    int n = 0, o = 0;
    if (r < rend) {
      const int32_t* orow = a.offs + r * (a.maxblk + 1) + lb;
      o = orow[0];
      n = orow[1] - o;
    }
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, 63);
    // wave-private LDS: run starts of the 64 rows (flattened) and their first positions
    wpre[lane] = incl - n;
    wo[lane] = o;
    asm volatile("" ::: "memory");
    for (int f0 = 0; f0 < total; f0 += 256) {
      int key[4];
      int64_t pidx[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = f0 + 64 * u + lane;
        ok[u] = f < total;
        int j = 0;                                  // last row whose run starts at or before f
#pragma unroll
        for (int st = 32; st; st >>= 1)
          if (wpre[j + st] <= f) j += st;
        const int p = wo[j] + (f - wpre[j]);
        const int64_t row = rt + j;
        key[u] = ok[u] ? (a.sorted[row * a.topk + p] & (kBk - 1)) : 0;
        pidx[u] = (row - a.row_begin) * a.topk + p;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t peers = same_key_lanes(key[u], ok[u]);
        const int before = __popcll(peers & lt);
        const int c = __popcll(peers);
        if (kRank) {
          if (ok[u]) {
            const int base = wcnt[key[u]];          // read by every lane of the key before the
            a.loc[pidx[u]] = base + before;         // first of them moves it on
            if (before == 0) wcnt[key[u]] = base + c;
          }
        } else if (ok[u] && before == 0) {
          wcnt[key[u]] += c;
        }
      }
    }
    asm volatile("" ::: "memory");
  }
}

__global__ void __launch_bounds__(kSlotWaves * 64) pair_slots_kernel(PairArgs a) {
  __shared__ int32_t cum[2 * 257], bstart[257];
  __shared__ int32_t cnt[kSlotWaves][kBk];
  __shared__ int32_t s_pre[kSlotWaves][65], s_o[kSlotWaves][64];
  __shared__ int32_t s_wsum[4];
  pair_tables(a, cum, bstart);
  for (int e = threadIdx.x; e < kSlotWaves * kBk; e += blockDim.x) (&cnt[0][0])[e] = 0;
  __syncthreads();
  const int gb = blockIdx.x;
  const int b = batch_of_block(bstart, a.B, gb);
  const int lb = gb - bstart[b];
  const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
  const int nkeys = a.layout_tnd ? lkv : (int)a.S2;
  const int nvalid = min(kBk, nkeys - lb * kBk);
  const int64_t kg0 = (int64_t)cum[257 + b] + lb * kBk;
  const int64_t q0 = cum[b];                      // first query row of batch b
  const int64_t r0 = max((int64_t)a.row_begin, q0), r1 = min(a.row_begin + a.nrows, q0 + lq);
  const bool live = lb * kBk < lkv && r1 > r0;    // keys of later blocks cannot be selected
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t per = live ? (r1 - r0 + kSlotWaves - 1) / kSlotWaves : 0;
  const int64_t rbeg = min(r1, r0 + wave * per), rend = min(r1, rbeg + per);
  if (live) slot_pass<false>(a, cnt[wave], s_pre[wave], s_o[wave], rbeg, rend, lb, lane);
  __syncthreads();
  int tot = 0, incl = 0;
  if (threadIdx.x < kBk) {
    const int k = threadIdx.x;
#pragma unroll
    for (int w = 0; w < kSlotWaves; ++w) tot += cnt[w][k];
    incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
  }
  __syncthreads();
  if (threadIdx.x < kBk) {
    const int k = threadIdx.x;
    int base = incl - tot;
    for (int v = 0; v < wave; ++v) base += s_wsum[v];
    if (k < nvalid) {
      a.kcnt[kg0 + k] = tot;
      a.koff[kg0 + k] = base;
    }
#pragma unroll
    for (int w = 0; w < kSlotWaves; ++w) {
      const int t = cnt[w][k];
      cnt[w][k] = base;
      base += t;
    }
    if (k == kBk - 1) a.btotal[gb] = base;
  }
  __syncthreads();
  if (live) slot_pass<true>(a, cnt[wave], s_pre[wave], s_o[wave], rbeg, rend, lb, lane);
}

// Exclusive scan of the block totals: bbase[gb] = first slot of block gb; bbase[nblocks] = all.
__global__ void __launch_bounds__(1024) block_base_kernel(PairArgs a) {
  __shared__ int32_t s_wsum[16];
  __shared__ int32_t s_base;
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int p0 = 0; p0 < a.nblocks; p0 += 1024) {
    const int i = p0 + threadIdx.x;
    const int n = i < a.nblocks ? a.btotal[i] : 0;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int base = s_base;
    for (int v = 0; v < wave; ++v) base += s_wsum[v];
    if (i < a.nblocks) a.bbase[i] = base + incl - n;
    __syncthreads();
    if (threadIdx.x == 1023) s_base = base + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.bbase[a.nblocks] = s_base;
}

// ------------------------------------------------------------------------------------------
// Partials of one chunk row.  Workgroup = (chunk row, column slice); slices 0, 1: dK | dKRope
// columns 288 s .. + 287 (18 column tiles, from dS), slices 2, 3: dV columns 256 (s - 2) .. + 255
// (16 tiles, from P).  The row's [heads x slice columns] Q | QRope (or dO), from the heads-
// innermost copy of every head group, sits in LDS for the whole row; wave w takes the row's
// chunks of 32 sorted positions w, w + 4, ...:
//   C[column][position] += A[column][heads] B[heads][position]  (16x16x32 bf16 MFMA)
// with A from LDS and B straight from the chunk-major records (lane (g, c): position c, and for
// head step ks the heads 16 g + 8 ks .. + 7 of head tile g, so both steps are one 32-byte run;
// A reads the same heads).  Lane (g, c) ends with columns 16 ft + 4 g .. + 3 of position c: one
// 16-byte store per column tile into the pair's slot.
constexpr int kPairCols = 288;                      // widest slice (18 column tiles)
constexpr int kPairLds = 2 * kPairCols * 64;        // two head groups, elements

template <int NFT, bool F16>
__device__ __forceinline__ void pair_kv_row(const PairArgs& a, uint16_t* Bs, int64_t row, int lr, int b,
                                            int colbase, int half, float mul, int lane, int wave,
                                            const int32_t* bstart) {
  const int g = lane >> 4, c = lane & 15;
  const int count = a.count[row];
  const int nck = (count + 31) >> 5;
  const int32_t* srow = a.sorted + row * a.topk;
  const int32_t* lrow = a.loc + (int64_t)lr * a.topk;
  const int64_t hgstride = (int64_t)a.rec_chunks * kRecChunk;
  const uint16_t* rec = a.dsp + (int64_t)lr * a.hgc * hgstride + half + g * 512 + c * 16;
  for (int pc = wave; pc < nck; pc += 4) {
    f32x4 acc[NFT][2];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) acc[ft][0] = acc[ft][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int hg = 0; hg < a.hgc; ++hg) {
      bf16x8 f[2][2];
      const uint16_t* rp = rec + hg * hgstride + (int64_t)pc * kRecChunk;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) f[pt][ks] = *reinterpret_cast<const bf16x8*>(rp + pt * 256 + 8 * ks);
      const uint16_t* bs = Bs + hg * kPairCols * 64;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const int col = 16 * ft + c;
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(bs + col * 64 + (((2 * g + ks) ^ (col & 7)) << 3));
          acc[ft][0] = mfma_t<F16>(af, f[0][ks], acc[ft][0]);
          acc[ft][1] = mfma_t<F16>(af, f[1][ks], acc[ft][1]);
        }
    }
    // slots of this lane's two positions (pt = 0, 1)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int p = 32 * pc + 16 * pt + c;
      if (p >= count) continue;
      const int64_t slot = (int64_t)a.bbase[bstart[b] + (srow[p] >> 8)] + lrow[p];
      float* dst = a.part + slot * kDacc + colbase + 4 * g;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        const f32x4 v = acc[ft][pt];
        *reinterpret_cast<float4*>(dst + 16 * ft) = make_float4(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
      }
    }
  }
}

template <bool F16>
__global__ void __launch_bounds__(kThreads, 2) pair_kv_kernel(PairArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kPairLds];
  __shared__ int32_t cum[2 * 257], bstart[257];
  const int lr = blockIdx.x;                      // row within the chunk
  const int64_t row = a.row_begin + lr;
  const int s = blockIdx.y;
  if (a.count[row] == 0) return;
  pair_tables(a, cum, bstart);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nft = s < 2 ? 18 : 16;
  const int colbase = s < 2 ? 288 * s : kDk + 256 * (s - 2);
  // stage the slice of every head group: LDS row = column (64 heads, 8 chunks of 16 bytes,
  // chunk j stored at j ^ (column % 8))
  for (int hg = 0; hg < a.hgc; ++hg) {
    const uint16_t* src = a.bt + (((int64_t)lr * a.hgc + hg) * kDacc + colbase) * 64;
    for (int e = threadIdx.x; e < nft * 16 * 8; e += kThreads) {
      const int col = e >> 3, j = e & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + col * 64 + j * 8);
      *reinterpret_cast<u32x4*>(Bs + hg * kPairCols * 64 + col * 64 + ((j ^ (col & 7)) << 3)) = v;
    }
  }
  __syncthreads();
  int b = 0;
  if (a.layout_tnd) {
    while (b + 1 < a.B && cum[b + 1] <= row) ++b;
  } else {
    b = (int)(row / a.S1);
  }
  if (s < 2) pair_kv_row<18, F16>(a, Bs, row, lr, b, colbase, 0, a.scale, lane, wave, bstart);
  else pair_kv_row<16, F16>(a, Bs, row, lr, b, colbase, kRecHalf, 1.f, lane, wave, bstart);
}

// ------------------------------------------------------------------------------------------
// Sum of one chunk, one wave per key: the key's run of partial rows, in slot order, added to the
// fp32 accumulator row (zero in the first chunk).  Lane l holds columns 4 l + 256 j .. + 3 for
// j < 4 and column 1024 + l.  Middle chunks skip keys without pairs; the last chunk writes bf16
// dK / dKRope / dV for every key (zeros for keys no row selected).
template <bool F16>
__device__ __forceinline__ void store_x4(uint16_t* p, f32x4 v) {
  const uint32_t lo = (uint32_t)f2x<F16>(v[0]) | ((uint32_t)f2x<F16>(v[1]) << 16);
  const uint32_t hi = (uint32_t)f2x<F16>(v[2]) | ((uint32_t)f2x<F16>(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

template <bool F16>
__global__ void __launch_bounds__(kThreads) pair_sum_kernel(PairArgs a) {
  __shared__ int32_t cum[2 * 257], bstart[257];
  pair_tables(a, cum, bstart);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t kg = (int64_t)blockIdx.x * 4 + wave;
  if (kg >= a.keys) return;
  const int n = a.kcnt[kg];
  if (n == 0 && !a.first && !a.last) return;
  int b = 0;
  if (a.layout_tnd) {
    int lo = 0, hi = a.B - 1;                     // last batch whose first key is <= kg
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[257 + mid] <= kg) lo = mid; else hi = mid - 1;
    }
    b = lo;
  } else {
    b = (int)(kg / a.S2);
  }
  const int lk = (int)(kg - cum[257 + b]);
  const int64_t s0 = (int64_t)a.bbase[bstart[b] + (lk >> 8)] + a.koff[kg];
  f32x4 v[4];
  float t = 0.f;
  float* accrow = a.acc + kg * kDacc;
  if (a.first) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const f32x4*>(accrow + 256 * j + 4 * lane);
    t = accrow[1024 + lane];
  }
  const float* src = a.part + s0 * kDacc;
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    f32x4 x[4][4];
    float y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* sp = src + (int64_t)(i + u) * kDacc;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[u][j] = *reinterpret_cast<const f32x4*>(sp + 256 * j + 4 * lane);
      y[u] = sp[1024 + lane];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += x[u][j];
      t += y[u];
    }
  }
  for (; i < n; ++i) {
    const float* sp = src + (int64_t)i * kDacc;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += *reinterpret_cast<const f32x4*>(sp + 256 * j + 4 * lane);
    t += sp[1024 + lane];
  }
  if (!a.last) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(accrow + 256 * j + 4 * lane) = v[j];
    accrow[1024 + lane] = t;
    return;
  }
  // columns 0..511 dK, 512..575 dKRope, 576..1087 dV
  store_x4<F16>(a.dk + kg * kDn + 4 * lane, v[0]);
  store_x4<F16>(a.dk + kg * kDn + 256 + 4 * lane, v[1]);
  if (lane < 16) {
    if (a.dkr) store_x4<F16>(a.dkr + kg * kDr + 4 * lane, v[2]);
  } else {
    store_x4<F16>(a.dv + kg * kDn + 4 * lane - 64, v[2]);
  }
  store_x4<F16>(a.dv + kg * kDn + 192 + 4 * lane, v[3]);
  a.dv[kg * kDn + 448 + lane] = f2x<F16>(t);
}

// ------------------------------------------------------------------------------------------
hipError_t launch_pair_chunk(const PairArgs& a, hipStream_t st) {
  if (a.nblocks > 0) {
    hipLaunchKernelGGL(pair_slots_kernel, dim3((unsigned)a.nblocks), dim3(kSlotWaves * 64), 0, st, a);
    hipLaunchKernelGGL(block_base_kernel, dim3(1), dim3(1024), 0, st, a);
  }
  if (a.nrows > 0) {
    if (a.f16) hipLaunchKernelGGL(pair_kv_kernel<true>, dim3((unsigned)a.nrows, 4), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(pair_kv_kernel<false>, dim3((unsigned)a.nrows, 4), dim3(kThreads), 0, st, a);
  }
  if (a.keys > 0) {
    const dim3 grid((unsigned)((a.keys + 3) / 4));
    if (a.f16) hipLaunchKernelGGL(pair_sum_kernel<true>, grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL(pair_sum_kernel<false>, grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sfag
