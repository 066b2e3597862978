// sfag_dense.hip -- key-major dK / dV for SparseFlashAttentionGrad (gfx950).
//
// The page's stage 1 and stage 3 scatter each query row's contributions into the selected
// key rows (dV[u] += P^T dO, dK[u] += scale dS^T Q).  Accumulating those per (row, slot)
// contributions with fp32 atomics costs one L2 atomic lane-op per value (1088 per pair), far
// slower than the MFMA work.  Here the accumulation is turned around: a workgroup owns a
// block of 256 consecutive keys and a slice of the 1088 output columns and walks the query
// rows of one row segment in order.  For every row that selects keys in the block it multiplies
// the row's dense [256 keys x 64 heads] dS (or P) -- zero where the row did not select the key,
// loaded as MFMA fragments straight from the pair records -- by the row's [64 heads x cols]
// Q (or dO) slice, staged in LDS, on the 16x16x32 bf16 MFMA into fp32 registers.  Rows with no
// key in the block cost nothing; rows that select a fraction f of the block cost 1/f of the
// useful flops.  The per-segment partial sums are then added in segment order, so the result
// does not depend on scheduling (deterministic by construction).
//
// Kernels:
//   sort_rows_kernel   per row: valid key positions sorted ascending, their count, the largest
//                      multiplicity of a repeated key, the start of every 256-key block and
//                      the key -> position map
//   kv_dense_kernel    (item = key block x row segment, column slice, head group) partial sums
//   kv_reduce_kernel   per key row: sum of the partials in (head group, segment) order -> bf16
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kThreads = 256;
constexpr int32_t kNoKey = 0x7fffffff;

// Per-batch tables in LDS: query / key row starts (cum, as in cum_lengths) and the first item
// (key block x row segment) of every batch.
__device__ __forceinline__ void item_tables(const Lens& L, int B, int tnd, int64_t S1, int64_t S2,
                                            int32_t* cum, int32_t* ibase) {
  for (int t = threadIdx.x; t <= B; t += blockDim.x) {
    int32_t sq = 0, skv = 0, it = 0;
    for (int b = 0; b < t; ++b) {
      sq += tnd ? L.lq[b] : (int32_t)S1;
      skv += tnd ? L.lkv[b] : (int32_t)S2;
      it += ((L.lkv[b] + kBk - 1) / kBk) * ((L.lq[b] + kSegRows - 1) / kSegRows);
    }
    cum[t] = sq;
    cum[257 + t] = skv;
    ibase[t] = it;
  }
}
}  // namespace

// ------------------------------------------------------------------------------------------
// Counting sort of one row's valid key positions.  The valid keys lie in [0, hi], which the
// map covers in full blocks; the range is walked in windows of kSortWin keys.  Per window:
// 16-bit occurrence counts in LDS (two per word, LDS atomics), then each thread takes 64
// consecutive keys, and a block-wide exclusive scan of the threads' totals gives every key's
// first sorted position.  From that one pass come the sorted list (each key written as often as
// it occurs), the key -> first-position map (-1: not selected), the block starts (the position
// of the first key >= 256 lb) and the largest multiplicity.  Slots past the count hold kNoKey.
constexpr int kSortWin = 64 * kThreads;           // 16384 keys per window
constexpr int kSortWords = kSortWin / 2;

__global__ void __launch_bounds__(kThreads) sort_rows_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t cw[kSortWords];   // 16-bit counts, 32 KB
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t s_wsum[kThreads / 64], s_base, s_dup;
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (row == 0)
    for (int i = t; i < kDk; i += kThreads) a.zero_row[i] = 0;
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  const int map_end = (geo.active && geo.hi >= 0) ? min(a.kstride, ((geo.hi + kBk) / kBk) * kBk) : 0;
  const int32_t* irow = a.idx + row * (a.topk / a.bs);
  int32_t* srow = a.sorted + row * a.topk;
  int16_t* kp = a.kpos + row * a.kstride;
  int32_t* orow = a.offs + row * (a.maxblk + 1);
  if (t == 0) {
    s_base = 0;
    s_dup = 1;
  }
  int dup = 1;
  for (int w0 = 0; w0 < map_end; w0 += kSortWin) {
    const int w1 = min(map_end, w0 + kSortWin);
    for (int k = t; k < kSortWords; k += kThreads) cw[k] = 0u;
    __syncthreads();
    for (int i = t; i < a.topk; i += kThreads) {
      const int j = slot_key(irow, i, a.bs);
      if (j >= 0 && j <= geo.hi && j >= w0 && j < w1) {
        const int k = j - w0;
        atomicAdd(&cw[k >> 1], 1u << (16 * (k & 1)));
      }
    }
    __syncthreads();
    // this thread's 64 keys: w0 + 64 t .. + 63 (32 count words)
    const uint32_t* mine = &cw[32 * t];
    int tsum = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(mine + 4 * q);
      tsum += (int)((v.x & 0xffffu) + (v.x >> 16) + (v.y & 0xffffu) + (v.y >> 16) + (v.z & 0xffffu) + (v.z >> 16) +
                    (v.w & 0xffffu) + (v.w >> 16));
    }
    // block-wide exclusive scan of tsum
    int incl = tsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int pos = s_base + incl - tsum;
    for (int v = 0; v < wave; ++v) pos += s_wsum[v];
    const int k0 = w0 + 64 * t;
    // w1 - w0 is a multiple of 256, so a thread's 64 keys are all inside or all outside
    if (k0 < w1) {
      if ((k0 & (kBk - 1)) == 0) orow[k0 / kBk] = pos;                   // block start
#pragma unroll
      for (int q = 0; q < 8; ++q) {                                       // 8 keys per step
        const u32x4 v = *reinterpret_cast<const u32x4*>(mine + 4 * q);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        i16x8 m;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = (int)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
          m[e] = n > 0 ? (short)pos : (short)-1;
          for (int r = 0; r < n; ++r) srow[pos + r] = k0 + 8 * q + e;
          pos += n;
          dup = max(dup, n);
        }
        *reinterpret_cast<i16x8*>(kp + k0 + 8 * q) = m;
      }
    }
    __syncthreads();
    if (t == kThreads - 1) s_base = pos;                                // total so far
    __syncthreads();
  }
  if (dup > 1) atomicMax(&s_dup, dup);
  __syncthreads();
  const int cnt = s_base;
  for (int i = cnt + t; i < a.topk; i += kThreads) srow[i] = kNoKey;
  const int nblk = (geo.lkv + kBk - 1) / kBk;
  for (int lb = map_end / kBk + t; lb <= nblk; lb += kThreads) orow[lb] = cnt;
  if (t == 0) {
    a.count[row] = cnt;
    a.maxdup[row] = s_dup;
  }
}

// ------------------------------------------------------------------------------------------
// Live items: items (key block x row segment, numbered per batch segment-major: item =
// segment * blocks + block) that the causal mask does not rule out, listed in item order.
// imap[item] = position in the list or -1.  One workgroup; the host computes the same count.
__global__ void __launch_bounds__(1024) item_list_kernel(DenseArgs a) {
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t wcount[16];
  __shared__ int32_t s_base;
  item_tables(a.lens, a.B, a.layout_tnd, a.S1, a.S2, cum, ibase);
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t0 = 0; t0 < a.items; t0 += 1024) {
    const int t = t0 + threadIdx.x;
    bool live = false;
    if (t < a.items) {
      int lo = 0, hi = a.B - 1;           // last batch whose first item is <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ibase[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
      const int nblk = (lkv + kBk - 1) / kBk;
      const int local = t - ibase[b];
      const int seg = local / nblk, lb = local % nblk;
      const int i1 = min(lq, (seg + 1) * kSegRows);
      live = !(a.mode3 && (i1 - 1) + lkv - lq < lb * kBk);
    }
    const uint64_t m = __ballot(live);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int base = s_base;
    for (int w = 0; w < wave; ++w) base += wcount[w];
    if (t < a.items) {
      const int k = live ? base + below : -1;
      a.imap[t] = k < a.citems ? k : -1;
      if (live && k < a.citems) a.ilist[k] = t;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wcount[w];
      s_base += tot;
    }
    __syncthreads();
  }
}

// Workgroup = (live item, column slice, head group).  Workgroups are dealt to the 8 XCDs
// round-robin (x = w % 8), so XCD x is given the contiguous run of live items
// [x n, x n + n) and walks it as  half (dK slices, then dV slices) > item > slice: the
// workgroups resident on one XCD are then neighbouring key blocks of one row segment x the 4
// column slices of one half, which share the segment's Q / dO rows and dS / P records in
// that XCD's L2.
// Column slices 0..3: dK columns 144 s .. 144 s + 143 (the last one holds the rope columns);
// 4..7: dV columns 128 (s - 4) .. + 127.  Wave w owns keys kb0 + 64 w .. + 63.
//
// For every row of the segment that selects keys of the block (a "unit"; a row that repeats
// keys gives one unit per repeat layer L, the L-th occurrence of each key):
//   A = [256 keys x 64 heads] of dS (dK slices) or P (dV slices), zero where the row did not
//       select the key.  MFMA A fragments come straight from the pair records in global
//       memory: lane (g, c) handles keys kb0 + 64 w + 4 c + kt (kt = 0..3) as row c of key
//       tile kt and needs heads 8 g .. 8 g + 7 (+ 32) of each, found through the row's
//       key -> position map (one 8-byte load for the 4 keys); unselected keys load nothing.
//   B = the row's [64 heads x cols] Q (or dO) slice, read from the column-major copy written by
//       the query-major kernel (one contiguous run of 2 KB per column tile), staged in LDS as
//       [column][8 chunks of 8 heads + 1 pad chunk] and read as whole 16-byte fragments.
//   acc[keys][cols] += A B  on the 16x16x32 bf16 MFMA, fp32 in registers; accumulator row
//       4 g + v of key tile kt is key kb0 + 64 w + 4 (4 g + v) + kt.
// Two workgroups share a CU (at most 256 registers per lane), so each unit is simple: its
// records are requested and used at once, the map and the B tile of the next unit are
// requested before its MFMAs, and the other workgroup runs while this one waits.
constexpr int kBtColChunks = 9;                       // B tile column: 8 chunks of 8 heads + 1 pad
constexpr int kBtElems = 144 * kBtColChunks * 8;      // up to 144 columns

// Shared state of one key-major workgroup, set up by kv_dense_kernel.
struct KvCtx {
  const int16_t* s_row;
  const uint16_t* s_lay;
  int64_t qstart;
  int i0, nrows, kb0, colbase, hg, which, citem;
  bool isdk;
};

// Main loop of one workgroup with NFT column tiles (9: dK slice, 8: dV slice).  DUPS: some
// row of the item repeats keys, so units are (row, layer) pairs; otherwise units are rows.
template <int NFT, bool DUPS>
__device__ __forceinline__ void kv_dense_units(const DenseArgs& a, const KvCtx& x, uint16_t* Bt0, uint16_t* Bt1) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int nrows = x.nrows;
  const int16_t* s_row = x.s_row;
  const uint16_t* s_lay = x.s_lay;
  constexpr int kBLoads = (NFT * 128 + kThreads - 1) / kThreads;
  constexpr int kQ = 2 * NFT;                        // (column tile, head step) steps

  // B tile: chunk P = t + 256 i of the row's contiguous run goes to LDS chunk 9 (P / 8) + P % 8;
  // threads past the run copy chunk P - 128 into the pad chunk of column P - 1152
  uint32_t bsrc[kBLoads];
  int bdst[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int P = (int)threadIdx.x + kThreads * i;
    const bool pad = P >= NFT * 128;
    bsrc[i] = (uint32_t)(pad ? P - 128 : P) * 16u;
    bdst[i] = pad ? ((P - NFT * 128) * kBtColChunks + 8) * 8 : ((P >> 3) * kBtColChunks + (P & 7)) * 8;
  }
  const int64_t bt_row = (int64_t)a.hgc * kDacc * 64;
  const uint16_t* bt_base = a.bt + ((int64_t)x.hg * kDacc + x.colbase) * 64;
  const uint32_t rstride = (uint32_t)a.hgc * 128u;
  const int kmap = x.kb0 + 64 * wave + 4 * c;        // first of this lane's 4 keys
  const int64_t row0 = x.qstart + x.i0;
  const int64_t rec_row = (int64_t)a.topk * a.hgc * 128;
  const uint16_t* rec_base = a.dsp + (int64_t)x.hg * 128 + x.which + 8 * g;

  f32x4 acc[4][NFT];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) acc[kt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};

#define KV_MAP_LOAD(MP, ROW)                                                                   \
  MP = *reinterpret_cast<const i16x4*>(a.kpos + (row0 + (ROW)) * a.kstride + kmap);
#define KV_B_LOAD(SP, ROW)                                                                     \
  {                                                                                            \
    const char* run_ = reinterpret_cast<const char*>(bt_base + (row0 + (ROW)) * bt_row);       \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i)                                        \
      SP[i] = *reinterpret_cast<const u32x4*>(run_ + bsrc[i]);                                 \
  }
#define KV_B_STORE(BT, SP)                                                                     \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i)                                        \
      *reinterpret_cast<u32x4*>((BT) + bdst[i]) = SP[i];                                       \
  }
#define KV_BFRAG(BT, Q)                                                                        \
  (*reinterpret_cast<const bf16x8*>((BT) + ((16 * ((Q) >> 1) + c) * kBtColChunks + 4 * ((Q) & 1) + g) * 8))

  // unit cursor: row index ri (into s_row) and repeat layer L; the next unit's row is rn
  auto advance = [&](int& ri, int& L) {
    if (DUPS && L + 1 < (int)s_lay[ri]) {
      ++L;
    } else {
      L = 0;
      ++ri;
    }
  };
  int ri = 0, L = 0;
  i16x4 mc;                                          // map of the current unit's row
  u32x4 bs[kBLoads];
  {
    const int r0 = __builtin_amdgcn_readfirstlane((int)s_row[0]);
    KV_MAP_LOAD(mc, r0)
    KV_B_LOAD(bs, r0)
    KV_B_STORE(Bt0, bs)
  }
  lds_barrier();

  for (int u = 0; ri < nrows; ++u) {
    uint16_t* BC = (u & 1) ? Bt1 : Bt0;
    uint16_t* BN = (u & 1) ? Bt0 : Bt1;
    const int r = __builtin_amdgcn_readfirstlane((int)s_row[ri]);
    int ri2 = ri, L2 = L;
    advance(ri2, L2);
    const int rn = __builtin_amdgcn_readfirstlane((int)s_row[min(ri2, nrows - 1)]);
    // records of this unit (layer L: the L-th occurrence of each key)
    const uint16_t* rb = rec_base + (row0 + r) * rec_row;
    bf16x8 f[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      int e = mc[kt];
      bool ok = e >= 0;
      if (DUPS && L > 0) {
        e += L;
        ok = ok && e < a.topk && a.sorted[(row0 + r) * a.topk + min(e, a.topk - 1)] == kmap + kt;
      }
      f[kt][0] = bf16x8{};
      f[kt][1] = bf16x8{};
      if (ok) {
        const uint16_t* src = rb + (uint32_t)e * rstride;
        f[kt][0] = *reinterpret_cast<const bf16x8*>(src);
        f[kt][1] = *reinterpret_cast<const bf16x8*>(src + 32);
      }
    }
    i16x4 mn;
    KV_MAP_LOAD(mn, rn)
    KV_B_LOAD(bs, rn)
    {
      bf16x8 bq[kQ];
      bq[0] = KV_BFRAG(BC, 0);
      bq[1] = KV_BFRAG(BC, 1);
      bq[2] = KV_BFRAG(BC, 2);
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q + 3 < kQ) bq[q + 3] = KV_BFRAG(BC, q + 3);
        const int ft = q >> 1, ks = q & 1;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt][ft] = mfma(f[kt][ks], bq[q], acc[kt][ft]);
      }
      // issue order: the next unit's map and B tile loads, three fragments, then (fragment
      // three steps ahead, 4 MFMAs) pairs
      __builtin_amdgcn_sched_group_barrier(0x020, kBLoads + 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q + 3 < kQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
    KV_B_STORE(BN, bs)
    lds_barrier();
    mc = mn;
    ri = ri2;
    L = L2;
  }
#undef KV_BFRAG
#undef KV_B_STORE
#undef KV_B_LOAD
#undef KV_MAP_LOAD

  const float mul = x.isdk ? a.scale : 1.f;
  float* part = a.part + ((int64_t)x.hg * a.citems + x.citem) * (int64_t)kBk * kDacc;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = 64 * wave + 4 * (4 * g + v) + kt;
        part[(int64_t)kk * kDacc + x.colbase + 16 * ft + c] = acc[kt][ft][v] * mul;
      }
}

__global__ void __launch_bounds__(kThreads, 2) kv_dense_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Bt0[kBtElems], Bt1[kBtElems];
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t s_b, s_nrows, s_dups;
  __shared__ int16_t s_row[kSegRows];      // segment rows that select keys in the block, in order
  __shared__ uint16_t s_lay[kSegRows];     // their repeat layers (1 without repeated keys)
  __shared__ int32_t s_wcnt[4];

  const int w = blockIdx.x;
  const int xcd = w & 7, j = w >> 3;
  const int per_xcd = (a.citems + 7) >> 3;
  const int half = j / (4 * per_xcd), r = j - half * 4 * per_xcd;
  const int citem = xcd * per_xcd + (r >> 2);
  const int sl = 4 * half + (r & 3);
  const int hg = blockIdx.y;
  if (half >= 2 || citem >= a.citems) return;
  const int item = a.ilist[citem];
  if (item < 0 || item >= a.items) return;     // host and device agree on the live count
  item_tables(a.lens, a.B, a.layout_tnd, a.S1, a.S2, cum, ibase);
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = 0;
    while (b + 1 < a.B && ibase[b + 1] <= item) ++b;
    s_b = b;
  }
  __syncthreads();
  const int b = s_b;
  const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
  const int nblk = (lkv + kBk - 1) / kBk;
  const int local = item - ibase[b];
  const int seg = local / nblk, lb = local % nblk;
  const int kb0 = lb * kBk;
  const int64_t qstart = cum[b];
  const int i0 = seg * kSegRows, i1 = min(lq, i0 + kSegRows);
  int32_t* flag = a.flag + (int64_t)hg * a.citems + citem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ordered list of the segment's rows with keys in the block; s_dups: some listed row repeats
  // keys (its units are (row, layer) pairs)
  if (threadIdx.x == 0) {
    s_nrows = 0;
    s_dups = 0;
  }
  for (int p0 = i0; p0 < i1; p0 += kThreads) {
    const int i = p0 + threadIdx.x;
    int n = 0, lay = 1;
    if (i < i1 && !(a.mode3 && i + lkv - lq < kb0)) {
      const int64_t row = qstart + i;
      const int32_t* offr = a.offs + row * (a.maxblk + 1);
      n = offr[lb + 1] - offr[lb];
      if (n > 0) lay = a.maxdup[row];
    }
    const uint64_t m = __ballot(n > 0);
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int base = s_nrows;
    for (int v = 0; v < wave; ++v) base += s_wcnt[v];
    if (n > 0) {
      const int at = base + __popcll(m & ((1ull << lane) - 1ull));
      s_row[at] = (int16_t)(i - i0);
      s_lay[at] = (uint16_t)min(lay, 65535);
      if (lay > 1) s_dups = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_nrows += s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
    __syncthreads();
  }
  const int nrows = s_nrows;
  const bool dups = s_dups != 0;
  if (nrows == 0) {
    if (threadIdx.x == 0) *flag = 0;
    return;
  }
  KvCtx x;
  x.s_row = s_row;
  x.s_lay = s_lay;
  x.qstart = qstart;
  x.i0 = i0;
  x.nrows = nrows;
  x.kb0 = kb0;
  x.isdk = sl < 4;
  x.colbase = x.isdk ? 144 * sl : kDk + 128 * (sl - 4);
  x.hg = hg;
  x.which = x.isdk ? 0 : 64;
  x.citem = citem;
  if (x.isdk) {
    if (dups) kv_dense_units<9, true>(a, x, Bt0, Bt1);
    else kv_dense_units<9, false>(a, x, Bt0, Bt1);
  } else {
    if (dups) kv_dense_units<8, true>(a, x, Bt0, Bt1);
    else kv_dense_units<8, false>(a, x, Bt0, Bt1);
  }
  if (threadIdx.x == 0) *flag = 1;
}

// ------------------------------------------------------------------------------------------
// One workgroup per key row: sum of the partials of its block over (head group, segment) in
// that fixed order, written as bf16 dK | dKRope | dV.  Padded key rows get zeros.
__global__ void __launch_bounds__(kThreads) kv_reduce_kernel(DenseArgs a) {
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t s_b;
  __shared__ int32_t fl[kMaxSegs];
  item_tables(a.lens, a.B, a.layout_tnd, a.S1, a.S2, cum, ibase);
  __syncthreads();
  const int64_t krow = blockIdx.x;
  if (threadIdx.x == 0) {
    int b = 0;
    while (b + 1 < a.B && cum[257 + b + 1] <= krow) ++b;
    s_b = b;
  }
  __syncthreads();
  const int b = s_b;
  const int j = (int)(krow - cum[257 + b]);
  const int lq = a.lens.lq[b], lkv = a.lens.lkv[b];
  const int nseg = (lq + kSegRows - 1) / kSegRows;
  const int nblk = (lkv + kBk - 1) / kBk;
  const int lb = j / kBk, kr = j % kBk;
  const bool live = j < lkv && lq > 0;
  if (live)
    for (int t = threadIdx.x; t < a.hgc * nseg; t += kThreads) {
      const int hg = t / nseg, seg = t % nseg;
      const int ci = a.imap[ibase[b] + seg * nblk + lb];
      fl[t] = (ci >= 0 && a.flag[(int64_t)hg * a.citems + ci]) ? ci : -1;
    }
  __syncthreads();
  for (int col = threadIdx.x; col < kDacc; col += kThreads) {
    float s = 0.f;
    if (live)
      for (int hg = 0; hg < a.hgc; ++hg)
        for (int seg = 0; seg < nseg; ++seg) {
          const int ci = fl[hg * nseg + seg];
          if (ci < 0) continue;
          s += a.part[(((int64_t)hg * a.citems + ci) * kBk + kr) * kDacc + col];
        }
    const uint16_t v = f2bf(s);
    if (col < kDn) a.dk[krow * kDn + col] = v;
    else if (col < kDk) {
      if (a.dkr) a.dkr[krow * kDr + col - kDn] = v;
    }
    else a.dv[krow * kDn + col - kDk] = v;
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_sort_rows(const DenseArgs& a, int64_t rows, hipStream_t st) {
  hipLaunchKernelGGL(sort_rows_kernel, dim3((unsigned)rows), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_item_list(const DenseArgs& a, hipStream_t st) {
  if (a.items == 0) return hipSuccess;
  hipLaunchKernelGGL(item_list_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_dense(const DenseArgs& a, hipStream_t st) {
  if (a.citems == 0) return hipSuccess;
  const unsigned per_xcd = (unsigned)((a.citems + 7) / 8);   // 8 XCDs x per_xcd items x 8 slices
  hipLaunchKernelGGL(kv_dense_kernel, dim3(per_xcd * 64, (unsigned)a.hgc), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_reduce(const DenseArgs& a, int64_t keys, hipStream_t st) {
  hipLaunchKernelGGL(kv_reduce_kernel, dim3((unsigned)keys), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t set_dense_attributes() { return hipSuccess; }

}  // namespace sfag
