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
// map covers in full blocks; the range is walked in windows of KPT * 256 keys.  Per window:
// 16-bit occurrence counts in LDS (two per word, LDS atomics), then each thread takes KPT
// consecutive keys, and a block-wide exclusive scan of the threads' totals gives every key's
// first sorted position.  From that one pass come the sorted list (each key written as often as
// it occurs), the key -> first-position map (-1: not selected), the block starts (the position
// of the first key >= 256 lb) and the largest multiplicity.  Slots past the count hold kNoKey.
// Each thread replaces its counts in LDS by its keys' map entries, 8 keys per step, and the
// whole window's map then leaves LDS in the permuted layout as 16-byte stores.  KPT = 32 (a
// 16 KB count window, twice the workgroups per CU) serves calls whose rows all fit one window.
template <int KPT>
__global__ void __launch_bounds__(kThreads) sort_rows_kernel(DenseArgs a) {
  constexpr int kWin = KPT * kThreads;                // keys per window
  constexpr int kWords = kWin / 2;
  constexpr int kTw = KPT / 2;                        // count words per thread
  __shared__ __attribute__((aligned(16))) uint32_t cw[kWords];   // 16-bit counts, then map entries
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
  // keys [0, map_end) are sorted (whole 256-key blocks covering [0, hi]); the key -> position map
  // is written only when the caller keeps one (kstride > 0, which then covers map_end)
  const int map_end = (geo.active && geo.hi >= 0) ? ((geo.hi + kBk) / kBk) * kBk : 0;
  const bool keep_map = a.kstride > 0;
  const int32_t* irow = a.idx + row * (a.topk / a.bs);
  int32_t* srow = a.sorted + row * a.topk;
  int16_t* kp = a.kpos + row * a.kstride;
  int32_t* orow = a.offs + row * (a.maxblk + 1);
  if (t == 0) {
    s_base = 0;
    s_dup = 1;
  }
  int dup = 1;
  for (int w0 = 0; w0 < map_end; w0 += kWin) {
    const int w1 = min(map_end, w0 + kWin);
    const int nw = (w1 - w0) / 2;                     // count words in use (a multiple of 128)
    for (int k = t; k < nw; k += kThreads) cw[k] = 0u;
    __syncthreads();
    for (int i = t; i < a.topk; i += kThreads) {
      const int j = slot_key(irow, i, a.bs);
      if (j >= 0 && j <= geo.hi && j >= w0 && j < w1) {
        const int k = j - w0;
        atomicAdd(&cw[k >> 1], 1u << (16 * (k & 1)));
      }
    }
    __syncthreads();
    // this thread's KPT keys: w0 + KPT t .. + KPT - 1; w1 - w0 is a multiple of 256, so they are
    // all inside or all outside the window
    const int k0 = w0 + KPT * t;
    const bool mine_in = k0 < w1;
    uint32_t* mine = &cw[kTw * t];
    int tsum = 0;
    if (mine_in) {
#pragma unroll
      for (int q = 0; q < kTw / 4; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(mine + 4 * q);
        tsum += (int)((v.x & 0xffffu) + (v.x >> 16) + (v.y & 0xffffu) + (v.y >> 16) + (v.z & 0xffffu) +
                      (v.z >> 16) + (v.w & 0xffffu) + (v.w >> 16));
      }
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
    if (mine_in) {
      if ((k0 & (kBk - 1)) == 0) orow[k0 / kBk] = pos;                   // block start
#pragma unroll 1
      for (int q = 0; q < kTw / 4; ++q) {                                 // 8 keys per step
        const u32x4 v = *reinterpret_cast<const u32x4*>(mine + 4 * q);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t m[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t packed = 0u;
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int n = (int)((w[h] >> (16 * e2)) & 0xffffu);
            const int key = k0 + 8 * q + 2 * h + e2;
            // map entry: the first position as 16 bits, 0xffff (-1) when not selected
            packed |= (n > 0 ? ((uint32_t)pos & 0xffffu) : 0xffffu) << (16 * e2);
            if (n > 0) srow[pos] = key;
            if (n > 1)
              for (int r = 1; r < n; ++r) srow[pos + r] = key;          // a repeated key
            pos += n;
            dup = max(dup, n);
          }
          m[h] = packed;
        }
        *reinterpret_cast<u32x4*>(mine + 4 * q) = u32x4{m[0], m[1], m[2], m[3]};
      }
    }
    __syncthreads();
    // the window's map, stored permuted inside each 64-key group: key 16 kt + c at 4 c + kt, so
    // that 8-entry chunk q of a group holds keys 16 (e % 4) + 2 q + e / 4, e = 0..7
    if (keep_map) {
      const uint16_t* m16 = reinterpret_cast<const uint16_t*>(cw);
      for (int ch = t; ch < (w1 - w0) / 8; ch += kThreads) {
        const int grp = ch >> 3, q = ch & 7;
        const uint16_t* g16 = m16 + 64 * grp;
        i16x8 m;
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = (short)g16[16 * (e & 3) + 2 * q + (e >> 2)];
        *reinterpret_cast<i16x8*>(kp + w0 + 8 * ch) = m;
      }
    }
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

// Workgroup = (head group, live item, column slice), or a part of one (KvShape: the positions
// of an XCD's last partial round are split over consecutive ranges of the item's rows).
// Workgroups are dealt to the 8 XCDs round-robin (x = w % 8), so XCD x is given the contiguous
// run of live items [x n, x n + n) and walks it as  head group > half (dK slices, then dV
// slices) > item > slice: the workgroups resident on one XCD are then neighbouring key blocks of
// one row segment x the 4 column slices of one half, which share the segment's Q / dO rows and
// dS / P records in that XCD's L2.
// Column slices 0..3: dK columns 144 s .. 144 s + 143 (the last one holds the rope columns);
// 4..7: dV columns 128 (s - 4) .. + 127.  Wave w owns keys kb0 + 64 w .. + 63.
//
// For every row of the segment that selects keys of the block (a "unit"; a row that repeats
// keys gives one unit per repeat layer L, the L-th occurrence of each key):
//   A = [256 keys x 64 heads] of dS (dK slices) or P (dV slices), zero where the row did not
//       select the key.  MFMA A fragments come straight from the pair records in global
//       memory: lane (g, c) handles key kb0 + 64 w + 16 kt + c (kt = 0..3) as row c of key
//       tile kt, found through the row's key -> position map; unselected keys load nothing.
//       The heads are contracted in the order that matches the record layout: head step ks of
//       lane (g, c) covers heads 32 ks + 8 g .. + 7, so the lanes of one head step read both
//       16-byte halves of head tiles 2 ks and 2 ks + 1 of every position (whole 32-byte runs).
//   B = the row's [64 heads x cols] Q (or dO) slice, read from the column-major copy written by
//       the query-major kernel (one contiguous run of 2 KB per column tile), staged in LDS as
//       [column][8 chunks of 8 heads + 1 pad chunk] and read as whole 16-byte fragments (head
//       chunk 4 ks + g for head step ks).
//   acc[keys][cols] += A B  on the 16x16x32 bf16 MFMA, fp32 in registers; accumulator row
//       4 g + v of key tile kt is key kb0 + 64 w + 16 kt + 4 g + v.
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

// Main loop of one workgroup with NFT column tiles (9: dK slice, 8: dV slice) over the listed
// rows ri_begin .. ri_end - 1 of the item.  DUPS: some row of the item repeats keys, so units are
// (row, layer) pairs; otherwise units are rows.  The sums go to out[key][ocol + column] (row pitch
// `pitch` floats), zeros for an empty range.
template <int NFT, bool DUPS, bool F16>
__device__ __forceinline__ void kv_dense_units(const DenseArgs& a, const KvCtx& x, uint16_t* Bt0, uint16_t* Bt1,
                                               int ri_begin, int ri_end, float* out, int pitch, int ocol) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
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

  const int kmap = x.kb0 + 64 * wave + c;            // this lane's key of key tile kt: kmap + 16 kt
  const int kb0w = x.kb0 + 64 * wave;                 // first key of this wave's 64-key group
  const int64_t row0 = x.qstart + x.i0;
  // records of (row, hg): chunk-major [chunk][dS | P][head tile of 16][32 positions][16 heads].
  // The contraction over heads is taken in the order that makes each record load read whole
  // 32-byte runs: head step ks of lane (g, c) covers heads 32 ks + 8 g .. + 7 (half g % 2 of head
  // tile 2 ks + g / 2), so one load instruction reads both halves of every position of two head
  // tiles; the B fragments read the same heads of Q / dO.
  const int64_t rec_row = (int64_t)a.hgc * a.rec_chunks * kRecChunk;
  const uint16_t* rec_base = a.dsp + (int64_t)x.hg * a.rec_chunks * kRecChunk + x.which;
  const uint32_t rec_lane = (uint32_t)((g >> 1) * 512 + 8 * (g & 1));
  const uint16_t* zrow = a.zero_row;                 // 576 zero elements

  f32x4 acc[4][NFT];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) acc[kt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};

#define KV_MAP_LOAD(MP, ROW)                                                                   \
  {                                                                                            \
    /* the map stores key 16 kt + c of each 64-key group at 4 c + kt: one 8-byte load */       \
    MP = *reinterpret_cast<const i16x4*>(a.kpos + (row0 + (ROW)) * a.kstride + kb0w + 4 * c); \
  }
#define KV_B_LOAD(SP, ROW, I0, I1)                                                             \
  {                                                                                            \
    const char* run_ = reinterpret_cast<const char*>(bt_base + (row0 + (ROW)) * bt_row);       \
    _Pragma("unroll") for (int i = (I0); i < (I1); ++i)                                        \
      SP[i - (I0)] = *reinterpret_cast<const u32x4*>(run_ + bsrc[i]);                          \
  }
#define KV_B_STORE(BT, SP, I0, I1)                                                             \
  {                                                                                            \
    _Pragma("unroll") for (int i = (I0); i < (I1); ++i)                                        \
      *reinterpret_cast<u32x4*>((BT) + bdst[i]) = SP[i - (I0)];                                \
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
  int ri = ri_begin, L = 0;
  i16x4 mc;                                          // map of the current unit's row
  constexpr int kBHalf = (kBLoads + 1) / 2;          // B loads staged in the first half-unit
  u32x4 bs[kBHalf];
  bf16x8 f[4][2];                                    // A fragments: [key tile][head step]
  // records of unit (row R, layer LL, map MP), head step KS, into f[*][KS] (zero where the row
  // did not select the key)
#define KV_REC_LOAD(R, LL, MP, KS)                                                             \
  {                                                                                            \
    const uint16_t* rb_ = rec_base + (row0 + (R)) * rec_row;                                   \
    /* opaque here, so that nothing derived from the map is computed (and waited for) earlier */ \
    i16x4 mp_ = (MP);                                                                          \
    asm volatile("" : "+v"(mp_));                                                              \
    _Pragma("unroll") for (int kt = 0; kt < 4; ++kt) {                                         \
      int e = mp_[kt];                                                                         \
      bool ok = e >= 0;                                                                        \
      if (DUPS && (LL) > 0) {                                                                  \
        e += (LL);                                                                             \
        ok = ok && e < a.topk && a.sorted[(row0 + (R)) * a.topk + min(e, a.topk - 1)] == kmap + 16 * kt; \
      }                                                                                        \
      /* unselected keys read 16 zero bytes: every unit issues the same loads */               \
      const uint16_t* src_ = ok ? rb_ + (rec_lane + 1024u * (KS) + (uint32_t)(e >> 5) * (uint32_t)kRecChunk + (uint32_t)(e & 31) * 16u) : zrow; \
      f[kt][KS] = *reinterpret_cast<const bf16x8*>(src_);                                      \
    }                                                                                          \
  }
  if (ri_begin < ri_end) {
    const int r0 = __builtin_amdgcn_readfirstlane((int)s_row[ri_begin]);
    KV_MAP_LOAD(mc, r0)
    KV_B_LOAD(bs, r0, 0, kBHalf)
    KV_B_STORE(Bt0, bs, 0, kBHalf)
    KV_B_LOAD(bs, r0, kBHalf, kBLoads)
    KV_B_STORE(Bt0, bs, kBHalf, kBLoads)
    KV_REC_LOAD(r0, 0, mc, 0)
    KV_REC_LOAD(r0, 0, mc, 1)
    lds_barrier();
  }

  // Unit loop.  The MFMAs of a unit run head step by head step (all column tiles with the first
  // head step's A fragments, then all with the second), so that the registers of the first head
  // step are free halfway: the next unit's first-half records are requested there, its second
  // half at the end of the unit, each with the other half-unit (and the other workgroup) to land.
  for (int u = 0; ri < ri_end; ++u) {
    uint16_t* BC = (u & 1) ? Bt1 : Bt0;
    uint16_t* BN = (u & 1) ? Bt0 : Bt1;
    int ri2 = ri, L2 = L;
    advance(ri2, L2);
    const int rn = __builtin_amdgcn_readfirstlane((int)s_row[min(ri2, ri_end - 1)]);
    i16x4 mn;
    KV_MAP_LOAD(mn, rn)
    KV_B_LOAD(bs, rn, 0, kBHalf)
    // fixed phase order (nothing is moved across these): the loads above, per head step its
    // MFMAs, then its record loads for the next unit (and the B tile halves)
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 bq[NFT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // a wave in its MFMA phase outranks the other workgroup's wave on the SIMD, so that a
      // head step's MFMAs issue back to back and the other wave's record loads and B-tile
      // stores (at priority 0) fill the gaps
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      bq[0] = KV_BFRAG(BC, ks);
      bq[1] = KV_BFRAG(BC, 2 + ks);
      bq[2] = KV_BFRAG(BC, 4 + ks);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        if (ft + 3 < NFT) bq[ft + 3] = KV_BFRAG(BC, 2 * (ft + 3) + ks);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[kt][ft] = mfma_t<F16>(f[kt][ks], bq[ft], acc[kt][ft]);
      }
      // issue order: three fragments, then (fragment three tiles ahead, 4 MFMAs) per column tile
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        if (ft + 3 < NFT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
      // this head step's fragments are consumed: request the next unit's; the next unit's B tile
      // goes to LDS in two halves, the second loaded while the second head step runs
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      KV_REC_LOAD(rn, L2, mn, ks)      /* past the last unit: the last row again, unused */
      if (ks == 0) {
        KV_B_STORE(BN, bs, 0, kBHalf)
        KV_B_LOAD(bs, rn, kBHalf, kBLoads)
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    KV_B_STORE(BN, bs, kBHalf, kBLoads)
    // the next unit's map and B-tile loads, issued right after the barrier, go first as well
    __builtin_amdgcn_s_setprio(1);
    lds_barrier();
    mc = mn;
    ri = ri2;
    L = L2;
  }
#undef KV_REC_LOAD
#undef KV_BFRAG
#undef KV_B_STORE
#undef KV_B_LOAD
#undef KV_MAP_LOAD

  const float mul = x.isdk ? a.scale : 1.f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = 64 * wave + 16 * kt + 4 * g + v;
        out[(int64_t)kk * pitch + ocol + 16 * ft + c] = acc[kt][ft][v] * mul;
      }
}

template <bool F16>
__global__ void __launch_bounds__(kThreads, 2) kv_dense_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Bt0[kBtElems], Bt1[kBtElems];
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t s_b, s_nrows, s_dups;
  __shared__ int16_t s_row[kSegRows];      // segment rows that select keys in the block, in order
  __shared__ uint16_t s_lay[kSegRows];     // their repeat layers (1 without repeated keys)
  __shared__ int32_t s_wcnt[4];

  const KvShape shp = kv_shape(a.citems, a.hgc);
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  if (j >= shp.wgs_per_xcd()) return;
  const KvWork wk = kv_work(shp, xcd, j);
  const int citem = wk.citem, sl = wk.sl, hg = wk.hg;
  if (citem >= a.citems) return;
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
  x.which = x.isdk ? 0 : kRecHalf;
  x.citem = citem;
  // rows of this part: consecutive ranges of the listed rows, all of a row's repeat layers in one
  const int ri0 = (int)((int64_t)nrows * wk.part / wk.nparts);
  const int ri1 = (int)((int64_t)nrows * (wk.part + 1) / wk.nparts);
  float* out;
  int pitch, ocol;
  if (wk.part == 0) {
    out = a.part + ((int64_t)hg * a.citems + citem) * (int64_t)kBk * kDacc;
    pitch = kDacc;
    ocol = x.colbase;
  } else {
    out = a.xpart + (int64_t)(wk.xslot + wk.part - 1) * kBk * kKvXCols;
    pitch = kKvXCols;
    ocol = 0;
  }
  if (x.isdk) {
    if (dups) kv_dense_units<9, true, F16>(a, x, Bt0, Bt1, ri0, ri1, out, pitch, ocol);
    else kv_dense_units<9, false, F16>(a, x, Bt0, Bt1, ri0, ri1, out, pitch, ocol);
  } else {
    if (dups) kv_dense_units<8, true, F16>(a, x, Bt0, Bt1, ri0, ri1, out, pitch, ocol);
    else kv_dense_units<8, false, F16>(a, x, Bt0, Bt1, ri0, ri1, out, pitch, ocol);
  }
  if (threadIdx.x == 0) *flag = 1;
}

// ------------------------------------------------------------------------------------------
// One workgroup per key row: sum of the partials of its block over (head group, segment) in
// that fixed order, written as bf16 dK | dKRope | dV.  Padded key rows get zeros.
template <bool F16>
__global__ void __launch_bounds__(kThreads) kv_reduce_kernel(DenseArgs a) {
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t s_b;
  __shared__ int32_t fl[kMaxSegs];
  __shared__ int32_t xs[kMaxSegs * 8];    // first extra slot of (head group, segment, slice), -1: none
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
  const KvShape shp = kv_shape(a.citems, a.hgc);
  if (live)
    for (int t = threadIdx.x; t < a.hgc * nseg; t += kThreads) {
      const int hg = t / nseg, seg = t % nseg;
      const int ci = a.imap[ibase[b] + seg * nblk + lb];
      fl[t] = (ci >= 0 && a.flag[(int64_t)hg * a.citems + ci]) ? ci : -1;
    }
  __syncthreads();
  if (live && shp.parts > 1)
    for (int i = threadIdx.x; i < a.hgc * nseg * 8; i += kThreads) {
      const int t = i >> 3, ci = fl[t];
      xs[i] = ci >= 0 ? kv_xslot(shp, t / nseg, ci, i & 7) : -1;
    }
  __syncthreads();
  // bit 30 of fl: some slice of this (head group, segment) is split (few are: only an XCD's tail)
  if (live && shp.parts > 1)
    for (int t = threadIdx.x; t < a.hgc * nseg; t += kThreads) {
      bool any = false;
      for (int sl = 0; sl < 8; ++sl) any = any || xs[8 * t + sl] >= 0;
      if (any) fl[t] |= 1 << 30;
    }
  __syncthreads();
  // each thread sums the columns threadIdx.x + 256 i (i < 5; the last only for the first 64
  // threads) over the (head group, segment) entries t = hg * nseg + seg in order, a split
  // position's parts after its first; the partials of 4 entries x all of the thread's columns are
  // requested together, then added in entry order
  constexpr int kCols = (kDacc + kThreads - 1) / kThreads;
  int sl[kCols], xcol[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    const int col = threadIdx.x + kThreads * i;
    sl[i] = col < kDk ? col / 144 : 4 + (col - kDk) / 128;       // slice holding the column
    xcol[i] = col < kDk ? col - 144 * sl[i] : col - kDk - 128 * (sl[i] - 4);
  }
  float s[kCols];
#pragma unroll
  for (int i = 0; i < kCols; ++i) s[i] = 0.f;
  if (live) {
    const int nt = a.hgc * nseg;
    for (int t0 = 0; t0 < nt; t0 += 4) {
      int e[4];
      float v[kCols][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = t0 + u < nt ? fl[t0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* pr = a.part + (((int64_t)((t0 + u) / nseg) * a.citems + (e[u] & 0x3fffffff)) * kBk + kr) * kDacc;
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
          const int col = threadIdx.x + kThreads * i;
          v[i][u] = (e[u] >= 0 && col < kDacc) ? pr[col] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (e[u] < 0) continue;
#pragma unroll
        for (int i = 0; i < kCols; ++i) {
          s[i] += v[i][u];
          if (e[u] & (1 << 30)) {
            const int x0 = xs[8 * (t0 + u) + sl[i]];
            if (x0 >= 0 && threadIdx.x + kThreads * i < kDacc)   // parts 1.., in part order
              for (int q = 0; q < shp.parts - 1; ++q)
                s[i] += a.xpart[((int64_t)(x0 + q) * kBk + kr) * kKvXCols + xcol[i]];
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kCols; ++i) {
    const int col = threadIdx.x + kThreads * i;
    if (col >= kDacc) continue;
    const uint16_t v = f2x<F16>(s[i]);
    if (col < kDn) a.dk[krow * kDn + col] = v;
    else if (col < kDk) {
      if (a.dkr) a.dkr[krow * kDr + col - kDn] = v;
    }
    else a.dv[krow * kDn + col - kDk] = v;
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_sort_rows(const DenseArgs& a, int64_t rows, hipStream_t st) {
  // every row's keys fit one 8192-key window: the half-size window (twice the workgroups per CU)
  if ((int64_t)a.maxblk * kBk <= 32 * kThreads)
    hipLaunchKernelGGL(sort_rows_kernel<32>, dim3((unsigned)rows), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(sort_rows_kernel<64>, dim3((unsigned)rows), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_item_list(const DenseArgs& a, hipStream_t st) {
  if (a.items == 0) return hipSuccess;
  hipLaunchKernelGGL(item_list_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_dense(const DenseArgs& a, hipStream_t st) {
  if (a.citems == 0) return hipSuccess;
  const KvShape shp = kv_shape(a.citems, a.hgc);
  const unsigned grid = 8u * (unsigned)shp.wgs_per_xcd();
  if (a.f16)
    hipLaunchKernelGGL(kv_dense_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(kv_dense_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_reduce(const DenseArgs& a, int64_t keys, hipStream_t st) {
  if (a.f16)
    hipLaunchKernelGGL(kv_reduce_kernel<true>, dim3((unsigned)keys), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(kv_reduce_kernel<false>, dim3((unsigned)keys), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}


}  // namespace sfag
