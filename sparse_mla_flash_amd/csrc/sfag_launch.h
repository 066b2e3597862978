// sfag_launch.h -- kernel argument blocks and launchers shared by the host library and the
// HIP kernels of the SparseFlashAttentionGrad library (internal; not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfag {

// Per-batch valid query / key lengths, passed by value in the kernel arguments (B <= 256).
struct Lens {
  int32_t lq[256];
  int32_t lkv[256];
};

constexpr int kBk = 256;        // keys per block of the key-major dK / dV kernel
constexpr int kSegRows = 512;   // query rows per segment of the key-major dK / dV kernel
constexpr int kMaxSegs = 512;   // (head group, segment) pairs per batch the ordered reduce can hold
// Launch shape of the key-major dK / dV kernel.  A position is (head group, live item, column
// slice); workgroups are dealt round-robin to the 8 XCDs, and XCD x walks its run of per_xcd live
// items as  head group > half (dK slices 0..3, then dV slices 4..7) > item > slice of the half,
// n = hgc * per_xcd * 8 positions.  Two workgroups fit a CU, so an XCD runs 64 at a time; the
// last rem = n % 64 positions would run as one partial round with most of the XCD idle, so each
// of them is split into `parts` workgroups over consecutive ranges of the item's rows, with
// `parts` chosen to minimise the time of that tail (ceil(rem parts / 64) rounds of 1 / parts of
// a workgroup).  Part 0 of a split position writes the item's partial slot; parts 1.. write
// extra slots [kBk keys][kKvXCols] that the reduce adds after it, in part order.  Host and device
// derive the shape from (citems, hgc) alone, so the summation order depends on the shape only.
constexpr int kKvSlotsPerXcd = 64;
constexpr int kKvMaxParts = 4;
constexpr int kKvXCols = 144;   // column pitch of an extra slot (the widest slice)

struct KvShape {
  int per_xcd;   // live items per XCD run
  int n;         // positions per XCD
  int j0;        // positions before the tail
  int rem;       // tail positions
  int parts;     // workgroups per tail position (1: no split)
  __host__ __device__ int wgs_per_xcd() const { return j0 + rem * parts; }
  __host__ __device__ int extra_slots() const { return 8 * rem * (parts - 1); }
};

__host__ __device__ inline KvShape kv_shape(int citems, int hgc) {
  KvShape s;
  s.per_xcd = (citems + 7) / 8;
  s.n = hgc * s.per_xcd * 8;
  s.rem = s.n % kKvSlotsPerXcd;
  s.j0 = s.n - s.rem;
  s.parts = 1;
  int best_r = 1, best_p = 1;                      // unsplit: one round of whole workgroups
  for (int P = 2; P <= kKvMaxParts && s.rem > 0; ++P) {
    const int r = (s.rem * P + kKvSlotsPerXcd - 1) / kKvSlotsPerXcd;
    if (r * best_p < best_r * P) {                 // r / P < best_r / best_p
      best_r = r;
      best_p = P;
    }
  }
  s.parts = best_p;
  return s;
}

// Work of the j-th workgroup of XCD xcd.  xslot: first extra slot of a split position (its part
// p >= 1 writes slot xslot + p - 1), -1 when the position is not split.
struct KvWork {
  int hg, citem, sl, part, nparts, xslot;
};

__host__ __device__ inline KvWork kv_work(const KvShape& s, int xcd, int j) {
  KvWork w;
  int pos;
  if (j < s.j0 || s.parts == 1) {
    pos = j;
    w.part = 0;
    w.nparts = 1;
    w.xslot = -1;
  } else {
    const int t = j - s.j0, q = t / s.parts;
    pos = s.j0 + q;
    w.part = t - q * s.parts;
    w.nparts = s.parts;
    w.xslot = (xcd * s.rem + q) * (s.parts - 1);
  }
  const int per_hg = s.per_xcd * 8;
  w.hg = pos / per_hg;
  const int r1 = pos - w.hg * per_hg;
  const int half = r1 / (4 * s.per_xcd), r2 = r1 - half * 4 * s.per_xcd;
  w.citem = xcd * s.per_xcd + (r2 >> 2);
  w.sl = 4 * half + (r2 & 3);
  return w;
}

// The reduce's side: first extra slot of (head group, live item, slice), -1 when not split.
__host__ __device__ inline int kv_xslot(const KvShape& s, int hg, int citem, int sl) {
  if (s.parts == 1) return -1;
  const int xcd = citem / s.per_xcd, local = citem - xcd * s.per_xcd;
  const int pos = hg * s.per_xcd * 8 + (sl >> 2) * 4 * s.per_xcd + 4 * local + (sl & 3);
  if (pos < s.j0) return -1;
  return (xcd * s.rem + (pos - s.j0)) * (s.parts - 1);
}

// dS | P records, per (row, head group) and chunk of 32 sorted positions:
// [dS | P][head tile of 16][32 positions][16 heads] bf16
constexpr int kRecChunk = 2 * 4 * 32 * 16;   // elements per chunk (8 KB)
constexpr int kRecHalf = kRecChunk / 2;      // offset of the P half

struct BwdArgs {
  const uint16_t* q;      // [rows, N1, 512] bf16
  const uint16_t* qr;     // [rows, N1, 64]
  const uint16_t* k;      // [keys, 512]  (also plays V)
  const uint16_t* kr;     // [keys, 64]
  const uint16_t* dout;   // [rows, N1, 512]
  const uint16_t* out;    // [rows, N1, 512]
  const int32_t* idx;     // [rows, topk / bs] block indices (bs = 1: key positions)
  const float* smax;      // statistics (BSND [B, N1, S1], TND [N1, T1])
  const float* ssum;
  uint16_t* dq;           // [rows, N1, 512]
  uint16_t* dqr;          // [rows, N1, 64]
  const int32_t* sorted;  // [rows, topk] valid key positions, ascending
  const int32_t* count;   // [rows] number of valid positions
  // records and heads-innermost copy of the launch's rows (row - row_begin)
  uint16_t* dsp;          // [launch rows, head groups, rec_chunks, kRecChunk] bf16 dS | P records
  const uint16_t* zero_row;  // 576 zero bf16 (rope operand of rope-less calls)
  uint16_t* bt;           // [launch rows, hgc, 1088, 64] heads-innermost Q | QRope | dO
  Lens lens;
  int64_t S1;             // BSND S1 / TND T1 (statistics head stride)
  int64_t S2;             // BSND S2 / TND T2
  int64_t row_begin;      // first query row of this launch
  int B, N1, topk, mode3, layout_tnd, hgc;
  int bs;                 // sparseBlockSize: topk slots = index count x bs
  int rec_chunks;         // record chunks per (row, head group): ceil(topk / 32)
  float scale;
  int f16;                // 16-bit tensors are fp16 (else bf16)
};

struct DenseArgs {
  const uint16_t* q;      // [rows, N1, 512]
  const uint16_t* qr;     // [rows, N1, 64]
  const uint16_t* dout;   // [rows, N1, 512]
  const int32_t* idx;     // [rows, topk / bs]
  int32_t* sorted;        // [rows, topk]
  int32_t* count;         // [rows]
  int32_t* maxdup;        // [rows]
  int32_t* offs;          // [rows, maxblk + 1]
  int16_t* kpos;          // [rows, kstride] first sorted position of each key, -1: not selected;
                          // inside each 64-key group key 16 t + c is stored at 4 c + t
                          // (key-major path only; kstride = 0: not written)
  const uint16_t* dsp;    // [rows, hgc, rec_chunks, kRecChunk]
  const uint16_t* bt;     // [rows, hgc, 1088, 64] Q | QRope | dO with the 64 heads of a group innermost
  float* part;            // [hgc, citems, kBk, 1088]
  float* xpart;           // [kv_shape().extra_slots(), kBk, kKvXCols] parts 1.. of split positions
  int32_t* flag;          // [hgc, citems]
  int32_t* ilist;         // [citems] live item -> item (key block x row segment)
  int32_t* imap;          // [items]  item -> live item, -1 when the causal mask rules it out
  uint16_t* zero_row;     // 576 bf16, zeroed by the sort kernel
  uint16_t* dk;           // [keys, 512]
  uint16_t* dkr;          // [keys, 64]
  uint16_t* dv;           // [keys, 512]
  Lens lens;
  int64_t S1, S2;
  int B, N1, topk, mode3, layout_tnd, hgc, maxblk, items, citems, kstride;
  int bs;                 // sparseBlockSize: topk slots = index count x bs
  int rec_chunks;         // record chunks per (row, head group)
  float scale;
  int f16;                // 16-bit tensors are fp16 (else bf16)
};

// Per-pair dK / dV of one chunk of query rows [row_begin, row_begin + nrows).
struct PairArgs {
  const int32_t* sorted;  // [rows, topk] valid key positions, ascending
  const int32_t* count;   // [rows]
  const int32_t* offs;    // [rows, maxblk + 1] first sorted position of every 256-key block
  const uint16_t* dsp;    // [nrows, hgc, rec_chunks, kRecChunk] records of the chunk's rows
  const uint16_t* bt;     // [nrows, hgc, 1088, 64] heads-innermost Q | QRope | dO of the chunk's rows
  float* part;            // [slots, 1088] fp32 partials, key-major slot order
  int32_t* loc;           // [nrows, topk] slot of each (row, position) pair within its key block
  int32_t* kcnt;          // [keys] pairs of each key in the chunk
  int32_t* koff;          // [keys] first slot of each key within its key block
  int32_t* btotal;        // [nblocks] pairs of each key block in the chunk
  int32_t* bbase;         // [nblocks + 1] first slot of each key block
  float* acc;             // [keys, 1088] fp32 accumulator carried between chunks
  uint16_t* dk;           // [keys, 512]
  uint16_t* dkr;          // [keys, 64] (NULL: rope-less call)
  uint16_t* dv;           // [keys, 512]
  Lens lens;
  int64_t S1, S2;
  int64_t row_begin;
  int64_t keys;           // key rows (B x S2, or the sum of the key lengths)
  int nrows, B, topk, layout_tnd, hgc, maxblk, rec_chunks, nblocks;
  int first, last;        // the chunk is the first / the last one
  float scale;
  int f16;                // 16-bit tensors are fp16 (else bf16)
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* qr;
  const uint16_t* k;
  const uint16_t* kr;
  const int32_t* idx;
  uint16_t* out;
  float* smax;
  float* ssum;
  Lens lens;
  int64_t S1;
  int64_t S2;
  int B, N1, topk, mode3, layout_tnd;
  int bs;                 // sparseBlockSize: topk slots = index count x bs
  float scale;
  int f16;                // 16-bit tensors are fp16 (else bf16)
};

// Lightning-indexer backward with KL loss (index head width fixed at 128).
constexpr int kIxDi = 128;
struct IxArgs {
  const uint16_t* q;      // [rows, N1, 512] main query
  const uint16_t* qr;     // [rows, N1, 64] (NULL: no rope terms)
  const uint16_t* k;      // [keys, 512] main key
  const uint16_t* kr;     // [keys, 64] (NULL with qr)
  const uint16_t* qi;     // [rows, G, 128] queryIndex
  const uint16_t* ki;     // [keys, 128] keyIndex
  const uint16_t* w;      // [rows, G] weights
  const float* smax;      // main statistics ([B, N1, S1] / [N1, T1])
  const float* ssum;
  const float* smax_i;    // index statistics [rows]
  const float* ssum_i;
  uint16_t* dqi;          // [rows, G, 128]
  uint16_t* dki;          // [keys, 128]
  uint16_t* dw;           // [rows, G]
  float* loss;            // [1]
  float* tot;             // [rows, kstride] head-summed main softmax of every admitted (row, key)
  float* norm;            // [rows] its sum over the row's keys
  float* lrow;            // [rows] loss of every row
  float* dkp;             // [parts, keys, 128] fp32 dK~ partials
  Lens lens;
  int64_t S1, S2, kstride, rows, keys;
  int B, N1, G, mode3, layout_tnd, parts;
  float scale;
  int f16;
};

// statistics element of head h of a query row (BSND [B, N1, S1], TND [N1, T1])
template <typename Geo>
__host__ __device__ inline int64_t stat_index(int tnd, const Geo& g, int64_t row, int N1, int64_t S1, int h) {
  return tnd ? (int64_t)h * S1 + row : ((int64_t)g.b * N1 + h) * S1 + g.i;
}

hipError_t launch_fwd(const FwdArgs& a, int64_t nrows, int hg_count, hipStream_t st);
hipError_t launch_bwd_q(const BwdArgs& a, int64_t nrows, int hg_count, hipStream_t st);
hipError_t launch_pair_chunk(const PairArgs& a, hipStream_t st);
hipError_t launch_sort_rows(const DenseArgs& a, int64_t rows, hipStream_t st);
hipError_t launch_item_list(const DenseArgs& a, hipStream_t st);
hipError_t launch_kv_dense(const DenseArgs& a, hipStream_t st);
hipError_t launch_kv_reduce(const DenseArgs& a, int64_t keys, hipStream_t st);
hipError_t launch_indexer(const IxArgs& a, int64_t key_tiles, hipStream_t st);

}  // namespace sfag
