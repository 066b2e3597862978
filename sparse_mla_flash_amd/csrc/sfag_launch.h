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
  float* acc;             // [keys, 1088] fp32 accumulator (atomic mode)
  float* partial;         // [head groups, pairs_per_launch, 1088] (deterministic mode)
  const int32_t* sorted;  // [rows, topk] valid key positions, ascending (key-major mode)
  const int32_t* count;   // [rows] number of valid positions (key-major mode)
  uint16_t* dsp;          // [rows, head groups, rec_chunks, kRecChunk] bf16 dS | P records (key-major mode)
  const uint16_t* zero_row;  // 576 zero bf16 (key-major mode: rope operand of rope-less calls)
  uint16_t* bt;           // [rows, hgc, 1088, 64] heads-innermost Q | QRope | dO (key-major mode)
  Lens lens;
  int64_t S1;             // BSND S1 / TND T1 (statistics head stride)
  int64_t S2;             // BSND S2 / TND T2
  int64_t row_begin;      // first query row of this launch
  int64_t pairs_per_launch;
  int B, N1, topk, mode3, layout_tnd, hgc;
  int bs;                 // sparseBlockSize: topk slots = index count x bs
  int rec_chunks;         // record chunks per (row, head group): ceil(topk / 32)
  float scale;
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
  int16_t* kpos;          // [rows, kstride] first sorted position of each key, -1: not selected
  const uint16_t* dsp;    // [rows, hgc, rec_chunks, kRecChunk]
  const uint16_t* bt;     // [rows, hgc, 1088, 64] Q | QRope | dO with the 64 heads of a group innermost
  float* part;            // [hgc, citems, kBk, 1088]
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
};

// statistics element of head h of a query row (BSND [B, N1, S1], TND [N1, T1])
template <typename Geo>
__host__ __device__ inline int64_t stat_index(int tnd, const Geo& g, int64_t row, int N1, int64_t S1, int h) {
  return tnd ? (int64_t)h * S1 + row : ((int64_t)g.b * N1 + h) * S1 + g.i;
}

// mode 0: fp32 atomic dK/dV, 1: per-pair partials (deterministic mode)
hipError_t launch_bwd_main(const BwdArgs& a, int64_t nrows, int hg_count, int mode, hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, int64_t nrows, int hg_count, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t nfloats, hipStream_t st);
hipError_t launch_cast(const float* acc, uint16_t* dk, uint16_t* dkr, uint16_t* dv, int64_t keys,
                       hipStream_t st);
hipError_t launch_pair_keys(const BwdArgs& a, uint64_t* keys, int64_t nrows, hipStream_t st);
hipError_t launch_det_reduce(const uint64_t* sorted, int64_t n, const float* partial,
                             int64_t pairs_per_launch, int hg_count, float* acc, int64_t keys,
                             hipStream_t st);
hipError_t sort_pair_keys(void* temp, size_t temp_bytes, const uint64_t* in, uint64_t* out, int64_t n,
                          int end_bit, hipStream_t st);
size_t sort_temp_bytes(int64_t n, int end_bit);
hipError_t launch_bwd_q(const BwdArgs& a, int64_t nrows, int hg_count, hipStream_t st);
hipError_t set_q_attributes();
hipError_t launch_sort_rows(const DenseArgs& a, int64_t rows, hipStream_t st);
hipError_t launch_item_list(const DenseArgs& a, hipStream_t st);
hipError_t launch_kv_dense(const DenseArgs& a, hipStream_t st);
hipError_t launch_kv_reduce(const DenseArgs& a, int64_t keys, hipStream_t st);
hipError_t set_dense_attributes();
hipError_t set_bwd_attributes();
hipError_t set_fwd_attributes();

}  // namespace sfag
