// sfag_dense.hip -- key-major dK / dV for SparseFlashAttentionGrad (gfx950).
//
// The page's stage 1 and stage 3 scatter each query row's contributions into the selected
// key rows (dV[u] += P^T dO, dK[u] += scale dS^T Q).  Accumulating those per (row, slot)
// contributions with fp32 atomics costs one L2 atomic lane-op per value (1088 per pair), far
// slower than the MFMA work.  Here the accumulation is turned around: a workgroup owns a
// block of 256 consecutive keys and a slice of the 1088 output columns and walks the query
// rows of one row segment in order.  For every row that selects keys in the block it builds a
// dense [256 keys x 64 heads] tile of dS (or P) -- zero where the row did not select the key
// -- in LDS, and accumulates  tile . Q_row  (or  tile . dO_row) on the 16x16x32 bf16 MFMA into
// fp32 registers.  Rows with no key in the block cost nothing; rows that select a fraction f
// of the block cost 1/f of the useful flops.  The per-segment partial sums are then added in
// segment order, so the result does not depend on scheduling (deterministic by construction).
//
// Kernels:
//   sort_rows_kernel   per row: valid key positions sorted ascending, their count, the largest
//                      multiplicity of a repeated key, and the start of every 256-key block
//   kv_dense_kernel    (item = key block x row segment, column slice, head group) partial sums
//   kv_reduce_kernel   per key row: sum of the partials in (head group, segment) order -> bf16
#include "sfag_device.h"
#include "sfag_launch.h"

namespace sfag {

namespace {
constexpr int kThreads = 256;
constexpr int kHtChunks = 64 / 8;          // [key][64 heads] tile rows: 8 chunks
constexpr int kBtChunks = 24;              // [64 heads][<=144 cols] tile rows padded to 192 cols
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
__global__ void __launch_bounds__(kThreads) sort_rows_kernel(DenseArgs a, int np) {
  extern __shared__ __attribute__((aligned(16))) int32_t keys[];
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t s_cnt, s_dup;
  if (a.layout_tnd) {
    cum_lengths(a.lens, a.B, cum);
    __syncthreads();
  }
  const int64_t row = blockIdx.x;
  if (row == 0)
    for (int i = threadIdx.x; i < kDk; i += kThreads) a.zero_row[i] = 0;
  const RowGeo geo = row_geo(a.lens, cum, a.B, a.layout_tnd, a.S1, a.S2, row, a.mode3);
  for (int i = threadIdx.x; i < np; i += kThreads) {
    int32_t v = kNoKey;
    if (i < a.topk && geo.active) {
      const int j = a.idx[row * a.topk + i];
      if (j >= 0 && j <= geo.hi) v = j;
    }
    keys[i] = v;
  }
  if (threadIdx.x == 0) s_dup = 1;
  __syncthreads();
  // bitonic sort, ascending
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < np; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int32_t x = keys[i], y = keys[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    int lo = 0, hi = np;  // first kNoKey
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < kNoKey) lo = mid + 1; else hi = mid;
    }
    s_cnt = lo;
  }
  __syncthreads();
  const int cnt = s_cnt;
  // longest run of one repeated key
  for (int i = threadIdx.x; i < cnt; i += kThreads) {
    if (i == 0 || keys[i - 1] != keys[i]) {
      int e = i + 1;
      while (e < cnt && keys[e] == keys[i]) ++e;
      if (e - i > 1) atomicMax(&s_dup, e - i);
    }
  }
  for (int i = threadIdx.x; i < a.topk; i += kThreads) a.sorted[row * a.topk + i] = keys[i];
  const int nblk = (geo.lkv + kBk - 1) / kBk;
  for (int lb = threadIdx.x; lb <= nblk; lb += kThreads) {
    const int32_t start = lb * kBk;
    int lo = 0, hi = cnt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < start) lo = mid + 1; else hi = mid;
    }
    a.offs[row * (a.maxblk + 1) + lb] = lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
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
// [x n, x n + n) and walks it as  half (dK slices, then dV slices) > item > slice: the ~32
// workgroups resident on one XCD are then 8 neighbouring key blocks of one row segment x the
// 4 column slices of one half, which share the segment's Q / dO rows and dS / P records in
// that XCD's L2.
// Column slices 0..3: dK columns 144 s .. 144 s + 143 (the last one holds the rope columns);
// 4..7: dV columns 128 (s - 4) .. + 127.  Wave w owns key tiles 4w .. 4w + 3 (64 keys).
//
// The A (dS or P) and B (Q or dO) tiles are double-buffered.  Per selecting row u (and per
// repeat layer of a duplicated key) every thread
//   issues the global loads of unit u+1 into registers, clears in the other buffer the tile
//   rows it wrote for unit u-1, runs the MFMAs of unit u | barrier | stores unit u+1's
//   records and B tile into the other buffer | barrier
// so the loads of the next unit are in flight while the MFMAs of this one run, and a tile
// row is never cleared and written in the same barrier interval.
constexpr int kSegCap = kSegRows;   // rows of one segment staged in LDS

__global__ void __launch_bounds__(kThreads, 1) kv_dense_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t At2[2][kBk * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bt2[2][64 * kBtChunks * 8];
  __shared__ int32_t cum[2 * 257];
  __shared__ int32_t ibase[257];
  __shared__ int32_t s_b;
  __shared__ int32_t s_lo[kSegCap], s_n[kSegCap];
  __shared__ uint8_t s_dup[kSegCap];

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
  if (a.mode3 && (i1 - 1) + lkv - lq < kb0) {
    if (threadIdx.x == 0) *flag = 0;
    return;
  }
  // per-row pair ranges of this block and repeat counts, staged once
  for (int i = i0 + threadIdx.x; i < i1; i += kThreads) {
    int lo = 0, n = 0, dup = 1;
    if (!(a.mode3 && i + lkv - lq < kb0)) {
      const int64_t row = qstart + i;
      const int32_t* offr = a.offs + row * (a.maxblk + 1);
      lo = offr[lb];
      n = offr[lb + 1] - lo;
      dup = n > 0 ? a.maxdup[row] : 1;
    }
    s_lo[i - i0] = lo;
    s_n[i - i0] = n;
    s_dup[i - i0] = (uint8_t)min(dup, 255);
  }
  for (int p = threadIdx.x; p < 2 * kBk * 8; p += kThreads)
    *reinterpret_cast<uint4*>(&At2[0][0] + p * 8) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const bool isdk = sl < 4;
  const int nft = isdk ? 9 : 8;
  const int nbt = 64 * 2 * nft;                         // 16-byte pieces of the B tile
  const int colbase = isdk ? 144 * sl : kDk + 128 * (sl - 4);
  const int h0 = hg * 64;
  const int nh = min(64, a.N1 - h0);
  const int which = isdk ? 0 : 64;
  const int piece = threadIdx.x & 7;

  // ---- fast path: rows without repeated keys, one unit per (row, chunk of 256 positions) ----
  int cur = -1, chunk = 0;
  auto advance = [&](int& i, int& ch) {
    if (i >= 0 && (ch + 1) * kBk < s_n[i - i0]) { ++ch; return; }
    ch = 0;
    for (i = (i < 0 ? i0 : i + 1); i < i1; ++i)
      if (s_n[i - i0] > 0 && s_dup[i - i0] == 1) return;
    i = -1;
  };
  u32x4 rec[8];
  int key[8];                    // sorted key position of each prefetched record
  u32x4 btp[5];
  // B-tile pieces of this thread: element offset inside the row's Q / dO block (bit 31 set:
  // inside the row's rope block); padded heads and pieces past the tile read a valid address
  const uint16_t* bmain = (isdk ? a.q : a.dout) + (int64_t)h0 * kDn;
  int boff[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int p = min((int)threadIdx.x + kThreads * k, nbt - 1);
    const int h = min(p / (2 * nft), nh - 1), ch8 = (p % (2 * nft)) * 8;
    const int col = colbase + ch8;
    if (isdk && col >= kDn) boff[k] = (int)(0x80000000u | (unsigned)(h * kDr + col - kDn));
    else boff[k] = h * kDn + (isdk ? col : col - kDk);
  }
  int u_lo = 0, u_n = 0, u_ch = 0;

#define SFAG_PF_REC(k)                                                                         \
  {                                                                                            \
    const int pr = (threadIdx.x >> 3) + 32 * (k) + kBk * u_ch;                                 \
    const int e = u_lo + min(pr, u_n - 1);                                                     \
    key[k] = srow_[e];                                                                         \
    rec[k] = *reinterpret_cast<const u32x4*>(drow_ + (int64_t)e * a.hgc * 128);                \
  }
#define SFAG_PF_BT(k)                                                                          \
  btp[k] = *reinterpret_cast<const u32x4*>((boff[k] < 0 ? rope_row : main_row) + (boff[k] & 0x7fffffff));
#define SFAG_ST_REC(k)                                                                         \
  {                                                                                            \
    const int pr = (threadIdx.x >> 3) + 32 * (k) + kBk * u_ch;                                 \
    key[k] = pr < u_n ? key[k] - kb0 : -1;                                                     \
    if (key[k] >= 0) *reinterpret_cast<u32x4*>(At_ + swz(key[k], piece * 8, kHtChunks)) = rec[k]; \
  }
#define SFAG_ST_BT(k)                                                                          \
  {                                                                                            \
    const int p = threadIdx.x + kThreads * (k);                                                \
    if (p < nbt) {                                                                             \
      const int h = p / (2 * nft), ch8 = (p % (2 * nft)) * 8;                                  \
      *reinterpret_cast<u32x4*>(Bt_ + swz(h, ch8, kBtChunks)) = h < nh ? btp[k] : u32x4{0u, 0u, 0u, 0u}; \
    }                                                                                          \
  }

// Issue every global load of unit (I, CH) up front, with addresses clamped into range and no
// branches; nothing consumes them before the MFMAs of the current unit.
#define SFAG_PREFETCH(I, CH)                                                                   \
  {                                                                                            \
    const int64_t row_ = qstart + (I);                                                         \
    u_lo = s_lo[(I) - i0];                                                                     \
    u_n = s_n[(I) - i0];                                                                       \
    u_ch = (CH);                                                                               \
    const int32_t* srow_ = a.sorted + row_ * a.topk;                                           \
    const uint16_t* drow_ = a.dsp + (row_ * a.topk * a.hgc + hg) * 128 + which + piece * 8;    \
    SFAG_PF_REC(0) SFAG_PF_REC(1) SFAG_PF_REC(2) SFAG_PF_REC(3)                                \
    SFAG_PF_REC(4) SFAG_PF_REC(5) SFAG_PF_REC(6) SFAG_PF_REC(7)                                \
    if (u_ch == 0) {                                                                           \
      const uint16_t* main_row = bmain + row_ * a.N1 * kDn;                                    \
      const uint16_t* rope_row = a.qr + (row_ * a.N1 + h0) * kDr;                              \
      SFAG_PF_BT(0) SFAG_PF_BT(1) SFAG_PF_BT(2) SFAG_PF_BT(3) SFAG_PF_BT(4)                    \
    }                                                                                          \
  }

// Store the prefetched records into their key rows of buffer BUF and the B tile; key[k]
// becomes the tile row written (-1: none) so that it can be cleared later.
#define SFAG_STORE(BUF)                                                                        \
  {                                                                                            \
    uint16_t* At_ = At2[BUF];                                                                  \
    uint16_t* Bt_ = Bt2[BUF];                                                                  \
    SFAG_ST_REC(0) SFAG_ST_REC(1) SFAG_ST_REC(2) SFAG_ST_REC(3)                                \
    SFAG_ST_REC(4) SFAG_ST_REC(5) SFAG_ST_REC(6) SFAG_ST_REC(7)                                \
    if (u_ch == 0) {                                                                           \
      SFAG_ST_BT(0) SFAG_ST_BT(1) SFAG_ST_BT(2) SFAG_ST_BT(3) SFAG_ST_BT(4)                    \
    }                                                                                          \
  }

// MFMAs of one unit from buffer BUF: 4 key tiles x (8 or 9) column tiles x 2 head steps, the
// B fragments read three column tiles at a time.
#define SFAG_MMA(BUF)                                                                          \
  {                                                                                            \
    const uint16_t* At_ = At2[BUF];                                                            \
    const uint16_t* Bt_ = Bt2[BUF];                                                            \
    static_for<0, 2>([&](auto KS) {                                                            \
      constexpr int ks = decltype(KS)::value;                                                  \
      bf16x8 af[4];                                                                            \
      static_for<0, 4>([&](auto KT) {                                                          \
        constexpr int kt = decltype(KT)::value;                                                \
        af[kt] = lds_read8(At_, 16 * (4 * wave + kt) + c, 32 * ks + 8 * g, kHtChunks);         \
      });                                                                                      \
      static_for<0, 3>([&](auto FG) {                                                          \
        constexpr int fg = decltype(FG)::value;                                                \
        bf16x8 bfr[3];                                                                         \
        static_for<0, 3>([&](auto F) {                                                         \
          constexpr int f = decltype(F)::value;                                                \
          bfr[f] = lds_frag_tr(Bt_, 32 * ks, 16 * (3 * fg + f), kBtChunks, lane);              \
        });                                                                                    \
        static_for<0, 3>([&](auto F) {                                                         \
          constexpr int ft = 3 * fg + decltype(F)::value;                                      \
          if (ft < 8 || isdk)                                                                  \
            static_for<0, 4>([&](auto KT) {                                                    \
              constexpr int kt = decltype(KT)::value;                                          \
              acc[kt][ft] = mfma(af[kt], bfr[decltype(F)::value], acc[kt][ft]);                \
            });                                                                                \
        });                                                                                    \
      });                                                                                      \
    });                                                                                        \
  }

  f32x4 acc[4][9];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < 9; ++ft) acc[kt][ft] = f32x4{0.f, 0.f, 0.f, 0.f};

  advance(cur, chunk);
  bool any = cur >= 0;
  if (any) {
    SFAG_PREFETCH(cur, chunk);
    SFAG_STORE(0);
  }
  __syncthreads();
  int buf = 0;
  while (cur >= 0) {
    int nxt = cur, nchunk = chunk;
    advance(nxt, nchunk);
    if (nxt >= 0) SFAG_PREFETCH(nxt, nchunk);   // later chunks of a row keep btp from its first load
    // clear the other buffer's A tile (its last unit's MFMAs finished before the last barrier)
    {
      u32x4* Ac = reinterpret_cast<u32x4*>(At2[buf ^ 1]);
#pragma unroll
      for (int k = 0; k < kBk * 8 / kThreads; ++k) Ac[threadIdx.x + kThreads * k] = u32x4{0u, 0u, 0u, 0u};
    }
    if (buf == 0) SFAG_MMA(0) else SFAG_MMA(1)
    __syncthreads();
    if (nxt >= 0) {
      if (buf == 0) SFAG_STORE(1) else SFAG_STORE(0)
    }
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    chunk = nchunk;
  }

  // ---- slow path: rows that repeat a key.  Every repeat contributes separately, so such a
  // row is applied in layers (the L-th occurrence of each key) and 256-position chunks, with
  // the whole tile cleared each time.  Never taken when indices are distinct.
  for (int i = i0; i < i1; ++i) {
    if (s_n[i - i0] == 0 || s_dup[i - i0] == 1) continue;
    any = true;
    const int64_t row = qstart + i;
    const int lo = s_lo[i - i0], n = s_n[i - i0];
    const int32_t* srow = a.sorted + row * a.topk;
    for (int L = 0; L < (int)s_dup[i - i0]; ++L) {
      for (int ch = 0; ch * kBk < n; ++ch) {
        __syncthreads();
        for (int p = threadIdx.x; p < kBk * 8; p += kThreads)
          *reinterpret_cast<uint4*>(&At2[0][0] + p * 8) = make_uint4(0, 0, 0, 0);
        for (int p = threadIdx.x; p < nbt; p += kThreads) {
          const int h = p / (2 * nft), ch8 = (p % (2 * nft)) * 8;
          const int col = colbase + ch8;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (h < nh) {
            const int64_t hh = row * a.N1 + h0 + h;
            v = isdk ? *reinterpret_cast<const uint4*>(col < kDn ? a.q + hh * kDn + col : a.qr + hh * kDr + (col - kDn))
                     : *reinterpret_cast<const uint4*>(a.dout + hh * kDn + (col - kDk));
          }
          *reinterpret_cast<uint4*>(Bt2[0] + swz(h, ch8, kBtChunks)) = v;
        }
        __syncthreads();
        for (int p = threadIdx.x; p < kBk * 8; p += kThreads) {
          const int pr = ch * kBk + (p >> 3);
          if (pr >= n) continue;
          const int e = lo + pr;
          const int32_t kk = srow[e];
          const bool occ = e - L >= lo && srow[e - L] == kk && (e - L == lo || srow[e - L - 1] != kk);
          if (!occ) continue;
          const uint4 v = *reinterpret_cast<const uint4*>(
              a.dsp + ((row * a.topk + e) * a.hgc + hg) * 128 + which + (p & 7) * 8);
          *reinterpret_cast<uint4*>(At2[0] + swz(kk - kb0, (p & 7) * 8, kHtChunks)) = v;
        }
        __syncthreads();
        SFAG_MMA(0)
      }
    }
  }
#undef SFAG_PREFETCH
#undef SFAG_STORE
#undef SFAG_MMA
#undef SFAG_PF_REC
#undef SFAG_PF_BT
#undef SFAG_ST_REC
#undef SFAG_ST_BT
  if (!any) {
    if (threadIdx.x == 0) *flag = 0;
    return;
  }
  const float mul = isdk ? a.scale : 1.f;
  float* part = a.part + ((int64_t)hg * a.citems + citem) * (int64_t)kBk * kDacc;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int ft = 0; ft < 9; ++ft) {
      if (ft >= nft) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = 16 * (4 * wave + kt) + 4 * g + v;
        part[(int64_t)kk * kDacc + colbase + 16 * ft + c] = acc[kt][ft][v] * mul;
      }
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
  __shared__ int32_t fl[2 * 256];
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
    else if (col < kDk) a.dkr[krow * kDr + col - kDn] = v;
    else a.dv[krow * kDn + col - kDk] = v;
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_sort_rows(const DenseArgs& a, int64_t rows, int np, hipStream_t st) {
  hipLaunchKernelGGL(sort_rows_kernel, dim3((unsigned)rows), dim3(kThreads), (size_t)np * 4, st, a, np);
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

hipError_t set_dense_attributes() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&sort_rows_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
}

}  // namespace sfag
