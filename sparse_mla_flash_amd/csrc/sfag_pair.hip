// sfag_pair.hip -- per-pair dK / dV for SparseFlashAttentionGrad selections too sparse for the
// key-major kernel (gfx950).
//
// The page's stage 1 and stage 3 scatter each query row's contributions into the selected key
// rows: dV[u] += P^T dO and dK[u] += scale dS^T Q (SparseFlashAttentionGrad README, "function
// description").  When every row selects a small fraction of the keys it can reach, the
// key-major kernel would multiply mostly zeros, so here the work follows the pairs:
//   pair_kv_kernel      per query row, the [positions x heads] dS (or P) records times the row's
//                       [heads x 1088] Q | QRope (or dO) on the MFMA: one fp32 partial row of
//                       1088 values per valid (row, position) pair, written to its slot;
//   pair_reduce_kernel  per 256-key block and 64-column slice, the block's partials added into
//                       the block's accumulator rows in slot order.
// Slots are numbered key-block-major: the pairs of key block lb come together, rows ascending,
// positions (ascending keys) within a row.  A row's pairs of one block are a contiguous run of
// its sorted positions, so a slot is the block's base + the row's offset within the block (an
// exclusive scan over rows, block_slots_kernel) + the pair's rank in its run.  The sum of a key
// therefore runs over its pairs in ascending (row, position) order, and query rows are taken in
// fixed chunks in order: the result is bit-reproducible, with or without the deterministic flag.
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
// Slot offsets of one chunk of query rows: for key block gb (batch b, block lb) and every chunk
// row r of batch b, rowoff[r][lb] = number of the block's pairs in earlier chunk rows; btotal[gb]
// = the block's pairs in the chunk.  One workgroup per block, 256 rows per scan step.
__global__ void __launch_bounds__(kThreads) block_slots_kernel(PairArgs a) {
  __shared__ int32_t cum[2 * 257], bstart[257];
  __shared__ int32_t s_wsum[kThreads / 64];
  pair_tables(a, cum, bstart);
  __syncthreads();
  const int gb = blockIdx.x;
  const int b = batch_of_block(bstart, a.B, gb);
  const int lb = gb - bstart[b];
  const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
  const int64_t q0 = cum[b];                      // first query row of batch b
  const int64_t r0 = max((int64_t)a.row_begin, q0), r1 = min(a.row_begin + a.nrows, q0 + lq);
  const bool live = lb * kBk < lkv;               // keys of later blocks cannot be selected
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int running = 0;
  if (live) {
    for (int64_t p0 = r0; p0 < r1; p0 += kThreads) {
      const int64_t r = p0 + threadIdx.x;
      int n = 0;
      if (r < r1) {
        const int32_t* o = a.offs + r * (a.maxblk + 1) + lb;
        n = o[1] - o[0];
      }
      int incl = n;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      if (lane == 63) s_wsum[wave] = incl;
      __syncthreads();
      int base = running;
      for (int v = 0; v < wave; ++v) base += s_wsum[v];
      if (r < r1) a.rowoff[(r - a.row_begin) * a.maxblk + lb] = base + incl - n;
      running += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) a.btotal[gb] = running;
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

template <int NFT>
__device__ __forceinline__ void pair_kv_row(const PairArgs& a, uint16_t* Bs, int64_t row, int lr, int b,
                                            int colbase, int half, float mul, int lane, int wave,
                                            const int32_t* bstart) {
  const int g = lane >> 4, c = lane & 15;
  const int count = a.count[row];
  const int nck = (count + 31) >> 5;
  const int32_t* srow = a.sorted + row * a.topk;
  const int32_t* orow = a.offs + row * (a.maxblk + 1);
  const int32_t* rrow = a.rowoff + (int64_t)lr * a.maxblk;
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
          acc[ft][0] = mfma(af, f[0][ks], acc[ft][0]);
          acc[ft][1] = mfma(af, f[1][ks], acc[ft][1]);
        }
    }
    // slots of this lane's two positions (pt = 0, 1)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int p = 32 * pc + 16 * pt + c;
      if (p >= count) continue;
      const int key = srow[p];
      const int lb = key >> 8;
      const int64_t slot = (int64_t)a.bbase[bstart[b] + lb] + rrow[lb] + (p - orow[lb]);
      float* dst = a.part + slot * kDacc + colbase + 4 * g;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        const f32x4 v = acc[ft][pt];
        *reinterpret_cast<float4*>(dst + 16 * ft) = make_float4(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
      }
      if (colbase == 0 && g == 0) a.keyb[slot] = (uint8_t)(key & (kBk - 1));
    }
  }
}

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
  if (s < 2) pair_kv_row<18>(a, Bs, row, lr, b, colbase, 0, a.scale, lane, wave, bstart);
  else pair_kv_row<16>(a, Bs, row, lr, b, colbase, kRecHalf, 1.f, lane, wave, bstart);
}

// ------------------------------------------------------------------------------------------
// Ordered reduce of one chunk.  Workgroup = (key block gb, 64-column slice cs); the block's 256
// accumulator rows of the slice sit in LDS (starting from zero in the first chunk, from the fp32
// accumulator otherwise).  The block's slots are streamed in order; wave w adds the pairs of
// keys 64 w .. 64 w + 63 (lane = column), so the pairs of one key are added by one wave in slot
// order.  The last chunk writes bf16 dK / dKRope / dV (zeros for keys no row selected).
__global__ void __launch_bounds__(kThreads, 2) pair_reduce_kernel(PairArgs a) {
  __shared__ __attribute__((aligned(16))) float accs[kBk * 64];
  __shared__ int32_t cum[2 * 257], bstart[257];
  pair_tables(a, cum, bstart);
  __syncthreads();
  const int gb = blockIdx.x, cs = blockIdx.y;
  const int b = batch_of_block(bstart, a.B, gb);
  const int lb = gb - bstart[b];
  const int nkeys = a.layout_tnd ? a.lens.lkv[b] : (int)a.S2;
  const int nvalid = min(kBk, nkeys - lb * kBk);
  const int64_t krow0 = (int64_t)cum[257 + b] + lb * kBk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = cs * 64 + lane;
  for (int k = wave; k < kBk; k += 4)
    accs[k * 64 + lane] = (a.first || k >= nvalid) ? 0.f : a.acc[(krow0 + k) * kDacc + col];
  __syncthreads();
  const int64_t lo = a.bbase[gb], hi = a.bbase[gb + 1];
  const int k0 = 64 * wave;
  for (int64_t s0 = lo; s0 < hi; s0 += 64) {
    const int64_t sl = s0 + lane;
    const int kb = sl < hi ? (int)a.keyb[sl] : -1;
    uint64_t mine = __ballot(kb >= k0 && kb < k0 + 64);
    while (mine) {
      // up to 8 of this wave's pairs at a time: loads first, then the adds in slot order
      int bit[8], key[8];
      float val[8];
      int n = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bit[i] = -1;
        if (mine) {
          bit[i] = __builtin_ctzll(mine);
          mine &= mine - 1;
          ++n;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        key[i] = bit[i] >= 0 ? __shfl(kb, bit[i]) : 0;
        val[i] = bit[i] >= 0 ? a.part[(s0 + bit[i]) * kDacc + col] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) accs[key[i] * 64 + lane] += val[i];
    }
  }
  __syncthreads();
  for (int k = wave; k < nvalid; k += 4) {
    const float v = accs[k * 64 + lane];
    const int64_t kr = krow0 + k;
    if (!a.last) {
      a.acc[kr * kDacc + col] = v;
    } else {
      const uint16_t bv = f2bf(v);
      if (col < kDn) a.dk[kr * kDn + col] = bv;
      else if (col < kDk) {
        if (a.dkr) a.dkr[kr * kDr + col - kDn] = bv;
      } else {
        a.dv[kr * kDn + col - kDk] = bv;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_pair_chunk(const PairArgs& a, hipStream_t st) {
  if (a.nblocks > 0) {
    hipLaunchKernelGGL(block_slots_kernel, dim3((unsigned)a.nblocks), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(block_base_kernel, dim3(1), dim3(1024), 0, st, a);
  }
  if (a.nrows > 0) hipLaunchKernelGGL(pair_kv_kernel, dim3((unsigned)a.nrows, 4), dim3(kThreads), 0, st, a);
  if (a.nblocks > 0)
    hipLaunchKernelGGL(pair_reduce_kernel, dim3((unsigned)a.nblocks, kDacc / 64), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfag
