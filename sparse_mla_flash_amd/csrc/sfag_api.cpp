// sfag_api.cpp -- host side of the SparseFlashAttentionGrad C ABI: argument validation
// (SparseFlashAttentionGrad README, "constraints"), workspace planning and the launch sequence.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sfag.h"
#include "sfag_launch.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev[4] = {nullptr, nullptr, nullptr, nullptr};
thread_local int32_t g_last_path = -1;

sfag_status fail(sfag_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sfag_status ok() {
  g_last_error.clear();
  return SFAG_OK;
}

constexpr int64_t kMaxSeq = 131072;           // S1, S2 up to 128K
constexpr int64_t kMaxTopk = 131072;
constexpr int kDacc = 1088;                   // fp32 accumulator row: dK 512 | dKRope 64 | dV 512
constexpr uint64_t kAlign = 256;
// per-chunk budget of the per-pair path's fp32 partials (a sixth of an MI355X's 288 GB: every
// chunk re-reads and re-writes the fp32 accumulator rows of the keys it reaches, so fewer, larger
// chunks move less).  Each key's sum runs over its pairs in row order whatever the chunking, so
// the result does not depend on the budget.
constexpr uint64_t kPartialBudget = 48ull << 30;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int tnd = 0;
  int64_t B = 0, S1 = 0, S2 = 0, N1 = 0, topk = 0;   // topk: slots per row (indices x block size)
  int bs = 1;
  int64_t rows = 0, keys = 0;
  int mode3 = 0, det = 0, hg_count = 0;
  float scale = 0.f;
  sfag::Lens lens;                 // per-batch valid lengths
  // path: key-major dense-masked dK / dV (dense = 1) or per-pair partials (dense = 0)
  int dense = 0;
  int f16 = 0;                     // 16-bit tensors are fp16 (else bf16)
  double waste = 0.0;              // dense-masked (row, key) entries per valid pair (upper bound)
  int64_t items = 0, citems = 0, maxblk = 0;
  int64_t rec_chunks = 0;          // record chunks of 32 positions per (row, head group)
  // workspace layout
  uint64_t off_acc = 0, off_loc = 0, off_kcnt = 0, off_koff = 0, off_btotal = 0, off_bbase = 0;
  uint64_t off_sorted = 0, off_count = 0, off_maxdup = 0, off_offs = 0, off_dsp = 0, off_part = 0, off_flag = 0;
  uint64_t off_xpart = 0;          // key-major: partial sums of the split tail positions
  uint64_t off_zero = 0, off_ilist = 0, off_imap = 0, off_kpos = 0, off_bt = 0;
  uint64_t bytes = 0;
  int64_t chunk_rows = 0;          // per-pair path: query rows per chunk
  int64_t pair_blocks = 0;         // per-pair path: key blocks of 256 the reduce covers
};

// Rows x candidate keys the key-major kernels visit vs. the most pairs the rows can hold:
// per batch, query i may select keys 0..i + Lkv - Lq (sparseMode 3) or 0..Lkv-1 (mode 0).
void path_stats(const Plan& p, double* range_sum, double* valid_max) {
  double rs = 0, vm = 0;
  for (int64_t b = 0; b < p.B; ++b) {
    const double lq = p.lens.lq[b], lkv = p.lens.lkv[b], k = (double)p.topk;
    if (lq <= 0 || lkv <= 0) continue;
    if (!p.mode3) {
      rs += lq * lkv;
      vm += lq * std::min(k, lkv);
      continue;
    }
    // range of row i is i + d for i >= i_lo, with d = Lkv - Lq + 1 (never above Lkv)
    const double d = lkv - lq + 1;
    const double ilo = std::max(0.0, 1.0 - d), ihi = lq - 1;
    if (ihi < ilo) continue;
    const auto series = [](double a, double z, double off) {  // sum_{i=a..z} (i + off)
      return z < a ? 0.0 : (z - a + 1) * ((a + z) / 2.0 + off);
    };
    rs += series(ilo, ihi, d);
    // rows whose range is at most topk contribute their range, the others topk
    const double isplit = std::min(ihi, std::floor(k - d));  // last i with i + d <= topk
    vm += series(ilo, isplit, d) + std::max(0.0, ihi - std::max(isplit, ilo - 1)) * k;
  }
  *range_sum = rs;
  *valid_max = vm;
}

bool n1_allowed(int64_t n) {
  static const int64_t ok_[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 128};
  for (int64_t v : ok_)
    if (v == n) return true;
  return false;
}

// Validate everything that needs no device pointer and build the plan.
sfag_status make_plan(const sfag_dims* dims, const int32_t* sq, const int32_t* skv, float scale,
                      int64_t block, const char* layout, int64_t mode, int32_t det, bool need_ws,
                      Plan* p) {
  if (!dims) return fail(SFAG_ERR_PARAM_NULLPTR, "dims is NULL");
  if (!layout) return fail(SFAG_ERR_PARAM_NULLPTR, "layout is NULL");
  if (std::strcmp(layout, "BSND") == 0) p->tnd = 0;
  else if (std::strcmp(layout, "TND") == 0) p->tnd = 1;
  else return fail(SFAG_ERR_PARAM_INVALID, "layout must be \"BSND\" or \"TND\", got \"%s\"", layout);
  if (dims->N2 != 1) return fail(SFAG_ERR_PARAM_INVALID, "N2 must be 1 (got %lld)", (long long)dims->N2);
  if (dims->D != 512) return fail(SFAG_ERR_PARAM_INVALID, "D must be 512 (got %lld)", (long long)dims->D);
  if (dims->Drope != 64)
    return fail(SFAG_ERR_PARAM_INVALID, "Drope must be 64 (got %lld)", (long long)dims->Drope);
  if (!n1_allowed(dims->N1))
    return fail(SFAG_ERR_PARAM_INVALID, "N1 must be one of 1,2,3,4,6,8,12,16,24,32,48,64,128 (got %lld)",
                (long long)dims->N1);
  if (dims->B < 1 || dims->B > 256) return fail(SFAG_ERR_PARAM_INVALID, "B must be in 1..256 (got %lld)", (long long)dims->B);
  if (dims->topk < 1 || dims->topk > kMaxTopk)
    return fail(SFAG_ERR_PARAM_INVALID, "topk must be in 1..%lld (got %lld)", (long long)kMaxTopk, (long long)dims->topk);
  if (block >= 1 && block > kMaxTopk / dims->topk)     // topk * block > kMaxTopk, without overflow
    return fail(SFAG_ERR_PARAM_INVALID, "topk * sparseBlockSize must be at most %lld (got %lld * %lld)",
                (long long)kMaxTopk, (long long)dims->topk, (long long)block);
  if (mode != 0 && mode != 3)
    return fail(SFAG_ERR_PARAM_INVALID, "sparseMode must be 0 or 3 (got %lld)", (long long)mode);
  if (block < 1) return fail(SFAG_ERR_PARAM_INVALID, "sparseBlockSize must be >= 1 (got %lld)", (long long)block);
  if (!std::isfinite(scale)) return fail(SFAG_ERR_PARAM_INVALID, "scaleValue must be finite");
  if (det != 0 && det != 1) return fail(SFAG_ERR_PARAM_INVALID, "deterministic must be 0 or 1");
  if (dims->dtype != SFAG_DTYPE_BF16 && dims->dtype != SFAG_DTYPE_FP16)
    return fail(SFAG_ERR_PARAM_INVALID, "dtype must be SFAG_DTYPE_BF16 (0) or SFAG_DTYPE_FP16 (1) (got %lld)",
                (long long)dims->dtype);
  p->f16 = dims->dtype == SFAG_DTYPE_FP16;

  p->B = dims->B;
  p->S1 = dims->S1;
  p->S2 = dims->S2;
  p->N1 = dims->N1;
  p->topk = dims->topk * block;     // slots per row: every index names a block of `block` keys
  p->bs = (int)block;
  p->mode3 = mode == 3;
  p->det = det;
  p->scale = scale;
  p->hg_count = (int)((dims->N1 + 63) / 64);
  std::memset(&p->lens, 0, sizeof(p->lens));
  if (!p->tnd) {
    if (p->S1 < 1 || p->S1 > kMaxSeq || p->S2 < 1 || p->S2 > kMaxSeq)
      return fail(SFAG_ERR_PARAM_INVALID, "S1 and S2 must be in 1..131072 (got %lld, %lld)",
                  (long long)p->S1, (long long)p->S2);
    for (int64_t b = 0; b < p->B; ++b) {
      const int64_t lq = sq ? sq[b] : p->S1, lkv = skv ? skv[b] : p->S2;
      if (lq < 0 || lq > p->S1 || lkv < 0 || lkv > p->S2)
        return fail(SFAG_ERR_PARAM_INVALID, "actual sequence lengths of batch %lld out of range (%lld, %lld)",
                    (long long)b, (long long)lq, (long long)lkv);
      p->lens.lq[b] = (int32_t)lq;
      p->lens.lkv[b] = (int32_t)lkv;
    }
    p->rows = p->B * p->S1;
    p->keys = p->B * p->S2;
  } else {
    if (!sq || !skv) return fail(SFAG_ERR_PARAM_NULLPTR, "TND layout needs both actual sequence length arrays");
    int64_t cq = 0, ckv = 0;
    for (int64_t b = 0; b < p->B; ++b) {
      if (sq[b] < 0 || sq[b] > kMaxSeq || skv[b] < 0 || skv[b] > kMaxSeq)
        return fail(SFAG_ERR_PARAM_INVALID, "sequence %lld lengths out of range (%d, %d)", (long long)b, sq[b], skv[b]);
      p->lens.lq[b] = sq[b];
      p->lens.lkv[b] = skv[b];
      cq += sq[b];
      ckv += skv[b];
    }
    if (cq != p->S1 || ckv != p->S2)
      return fail(SFAG_ERR_PARAM_INVALID, "TND: query / key lengths sum to %lld / %lld but dims give T1=%lld T2=%lld",
                  (long long)cq, (long long)ckv, (long long)p->S1, (long long)p->S2);
    if (cq < 1 || ckv < 1) return fail(SFAG_ERR_PARAM_INVALID, "TND: no query or key tokens");
    p->rows = cq;
    p->keys = ckv;
  }
  if (p->rows > INT32_MAX || p->keys * (int64_t)kDacc > (int64_t)1 << 40)
    return fail(SFAG_ERR_PARAM_INVALID, "problem too large");

  if (!need_ws) return SFAG_OK;

  // choose the dK / dV path: the key-major kernels pay for every candidate key of a block a
  // selecting row could have chosen; the scatter path pays 1088 fp32 adds per valid pair
  double range_sum = 0, valid_max = 0;
  path_stats(*p, &range_sum, &valid_max);
  p->waste = valid_max > 0 ? range_sum / valid_max : 0.0;
  int64_t max_lq = 0;
  for (int64_t b = 0; b < p->B; ++b) max_lq = std::max<int64_t>(max_lq, p->lens.lq[b]);
  const bool dense_fits = p->topk <= 16384 &&
      p->hg_count * ((max_lq + sfag::kSegRows - 1) / sfag::kSegRows) <= sfag::kMaxSegs;
  p->dense = dense_fits && p->waste <= 8.0;
  if (const char* f = std::getenv("SFAG_FORCE_PATH")) {
    if (std::strcmp(f, "dense") == 0 && dense_fits) p->dense = 1;
    if (std::strcmp(f, "scatter") == 0) p->dense = 0;
  }
  uint64_t off = 0;
  int64_t maxblk = 0;
  for (int64_t b = 0; b < p->B; ++b) maxblk = std::max<int64_t>(maxblk, (p->lens.lkv[b] + sfag::kBk - 1) / sfag::kBk);
  p->maxblk = maxblk;
  p->rec_chunks = (p->topk + 31) / 32;
  // shared by both paths: sorted positions, counts, repeat counts, block starts, zero row
  const uint64_t pairs = (uint64_t)p->rows * p->topk;
  p->off_sorted = off;
  off = align_up(off + pairs * 4);
  p->off_count = off;
  off = align_up(off + (uint64_t)p->rows * 4);
  p->off_maxdup = off;
  off = align_up(off + (uint64_t)p->rows * 4);
  p->off_offs = off;
  off = align_up(off + (uint64_t)p->rows * (maxblk + 1) * 4);
  p->off_zero = off;
  off = align_up(off + 576 * 2);
  const uint64_t rec_row = (uint64_t)p->hg_count * p->rec_chunks * sfag::kRecChunk * 2;   // records per row
  const uint64_t bt_row = (uint64_t)p->hg_count * kDacc * 64 * 2;                         // Q | QRope | dO copy
  if (p->dense) {
    int64_t items = 0;
    for (int64_t b = 0; b < p->B; ++b) {
      const int64_t nblk = (p->lens.lkv[b] + sfag::kBk - 1) / sfag::kBk;
      items += nblk * ((p->lens.lq[b] + sfag::kSegRows - 1) / sfag::kSegRows);
    }
    p->items = items;
    // live items: the key blocks of a row segment that the causal mask leaves reachable form a
    // prefix of the segment's blocks (same rule as the device-side list)
    int64_t citems = 0;
    for (int64_t b = 0; b < p->B; ++b) {
      const int64_t lq = p->lens.lq[b], lkv = p->lens.lkv[b];
      const int64_t nblk = (lkv + sfag::kBk - 1) / sfag::kBk, nseg = (lq + sfag::kSegRows - 1) / sfag::kSegRows;
      for (int64_t seg = 0; seg < nseg; ++seg) {
        if (!p->mode3) {
          citems += nblk;
          continue;
        }
        const int64_t i1 = std::min(lq, (seg + 1) * sfag::kSegRows);
        const int64_t hi = i1 - 1 + lkv - lq;     // last key reachable from the segment
        if (hi >= 0) citems += std::min(nblk, hi / sfag::kBk + 1);
      }
    }
    p->citems = citems;
    p->off_kpos = off;
    off = align_up(off + (uint64_t)p->rows * maxblk * sfag::kBk * 2);
    p->off_dsp = off;
    off = align_up(off + (uint64_t)p->rows * rec_row);
    p->off_part = off;
    off = align_up(off + (uint64_t)p->hg_count * citems * sfag::kBk * kDacc * 4);
    p->off_xpart = off;
    off = align_up(off + (uint64_t)sfag::kv_shape((int)citems, p->hg_count).extra_slots() * sfag::kBk *
                             sfag::kKvXCols * 4);
    p->off_flag = off;
    off = align_up(off + (uint64_t)p->hg_count * std::max<int64_t>(citems, 1) * 4);
    p->off_ilist = off;
    off = align_up(off + (uint64_t)std::max<int64_t>(citems, 1) * 4);
    p->off_imap = off;
    off = align_up(off + (uint64_t)std::max<int64_t>(items, 1) * 4);
    p->off_bt = off;                    // Q | QRope | dO, heads innermost (key-major B operand)
    off = align_up(off + (uint64_t)p->rows * bt_row);
    p->bytes = off;
    return SFAG_OK;
  }
  // per-pair path: rows in chunks whose fp32 partials fit the budget
  const uint64_t part_row = (uint64_t)p->topk * kDacc * 4;
  int64_t r = (int64_t)(kPartialBudget / part_row);
  r = std::max<int64_t>(1, std::min<int64_t>(r, p->rows));
  const int64_t nchunks = (p->rows + r - 1) / r;
  r = (p->rows + nchunks - 1) / nchunks;          // chunks of (nearly) equal size
  p->chunk_rows = r;
  int64_t nblocks = 0;
  for (int64_t b = 0; b < p->B; ++b)
    nblocks += ((p->tnd ? p->lens.lkv[b] : p->S2) + sfag::kBk - 1) / sfag::kBk;
  p->pair_blocks = nblocks;
  p->off_acc = off;
  off = align_up(off + (uint64_t)p->keys * kDacc * 4);
  p->off_dsp = off;
  off = align_up(off + (uint64_t)r * rec_row);
  p->off_bt = off;
  off = align_up(off + (uint64_t)r * bt_row);
  p->off_part = off;
  off = align_up(off + (uint64_t)r * part_row);
  p->off_loc = off;
  off = align_up(off + (uint64_t)r * p->topk * 4);
  p->off_kcnt = off;
  off = align_up(off + (uint64_t)std::max<int64_t>(p->keys, 1) * 4);
  p->off_koff = off;
  off = align_up(off + (uint64_t)std::max<int64_t>(p->keys, 1) * 4);
  p->off_btotal = off;
  off = align_up(off + (uint64_t)std::max<int64_t>(nblocks, 1) * 4);
  p->off_bbase = off;
  off = align_up(off + (uint64_t)(nblocks + 1) * 4);
  p->bytes = off;
  return SFAG_OK;
}

sfag_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(SFAG_ERR_PARAM_NULLPTR, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(SFAG_ERR_PARAM_INVALID, "%s must be 16-byte aligned", name);
  return SFAG_OK;
}

#define SFAG_HIP(call)                                                                    \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(SFAG_ERR_DEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

// Scratch of the no-allocation entry point: one array per GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: the device address of each
// GPU's copy is taken once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr uint64_t kScratchBytes = SFAG_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sfag_status scratch_of_current_device(void** out) {
  int dev = -1;
  SFAG_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(SFAG_ERR_DEVICE, "device %d out of range for the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    SFAG_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(SFAG_ERR_DEVICE, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SFAG_OK;
}

sfag_status backward(const void* query, const void* key, const void* value, const int32_t* sparse_indices,
                     const void* d_out, const void* out, const float* softmax_max, const float* softmax_sum,
                     const int32_t* seq_len_q_host, const int32_t* seq_len_kv_host, const void* query_rope,
                     const void* key_rope, const sfag_dims* dims, float scale_value, int64_t sparse_block_size,
                     const char* layout, int64_t sparse_mode, int32_t deterministic, void* d_query, void* d_key,
                     void* d_value, void* d_query_rope, void* d_key_rope, void* workspace, uint64_t workspace_size,
                     bool noalloc, void* stream);

}  // namespace

extern "C" {

const char* sfag_last_error(void) { return g_last_error.c_str(); }

const char* sfag_version(void) { return "sfag-mi355x 0.1 (gfx950)"; }

sfag_status sfag_set_profile_events(void* s1_begin, void* s1_end, void* s2_begin, void* s2_end) {
  g_ev[0] = reinterpret_cast<hipEvent_t>(s1_begin);
  g_ev[1] = reinterpret_cast<hipEvent_t>(s1_end);
  g_ev[2] = reinterpret_cast<hipEvent_t>(s2_begin);
  g_ev[3] = reinterpret_cast<hipEvent_t>(s2_end);
  return ok();
}

int32_t sfag_last_path(void) { return g_last_path; }

sfag_status sfag_get_workspace_size(const sfag_dims* dims, const int32_t* seq_len_q_host,
                                    const int32_t* seq_len_kv_host, float scale_value,
                                    int64_t sparse_block_size, const char* layout, int64_t sparse_mode,
                                    int64_t pre_tokens, int64_t next_tokens, int32_t deterministic,
                                    uint64_t* workspace_size) {
  (void)pre_tokens;
  (void)next_tokens;
  if (!workspace_size) return fail(SFAG_ERR_PARAM_NULLPTR, "workspace_size is NULL");
  Plan p;
  sfag_status st = make_plan(dims, seq_len_q_host, seq_len_kv_host, scale_value, sparse_block_size, layout,
                             sparse_mode, deterministic, true, &p);
  if (st != SFAG_OK) return st;
  *workspace_size = p.bytes;
  return ok();
}

sfag_status sfag_sparse_flash_attention_grad(
    const void* query, const void* key, const void* value, const int32_t* sparse_indices, const void* d_out,
    const void* out, const float* softmax_max, const float* softmax_sum, const int32_t* seq_len_q_host,
    const int32_t* seq_len_kv_host, const void* query_rope, const void* key_rope, const sfag_dims* dims,
    float scale_value, int64_t sparse_block_size, const char* layout, int64_t sparse_mode, int64_t pre_tokens,
    int64_t next_tokens, int32_t deterministic, void* d_query, void* d_key, void* d_value, void* d_query_rope,
    void* d_key_rope, void* workspace, uint64_t workspace_size, void* stream) {
  (void)pre_tokens;
  (void)next_tokens;
  return backward(query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum, seq_len_q_host,
                  seq_len_kv_host, query_rope, key_rope, dims, scale_value, sparse_block_size, layout, sparse_mode,
                  deterministic, d_query, d_key, d_value, d_query_rope, d_key_rope, workspace, workspace_size,
                  false, stream);
}

sfag_status sfag_sparse_flash_attention_grad_noalloc(
    const void* query, const void* key, const void* value, const int32_t* sparse_indices, const void* d_out,
    const void* out, const float* softmax_max, const float* softmax_sum, const int32_t* seq_len_q_host,
    const int32_t* seq_len_kv_host, const void* query_rope, const void* key_rope, const sfag_dims* dims,
    float scale_value, int64_t sparse_block_size, const char* layout, int64_t sparse_mode, int64_t pre_tokens,
    int64_t next_tokens, int32_t deterministic, void* d_query, void* d_key, void* d_value, void* d_query_rope,
    void* d_key_rope, void* stream) {
  (void)pre_tokens;
  (void)next_tokens;
  return backward(query, key, value, sparse_indices, d_out, out, softmax_max, softmax_sum, seq_len_q_host,
                  seq_len_kv_host, query_rope, key_rope, dims, scale_value, sparse_block_size, layout, sparse_mode,
                  deterministic, d_query, d_key, d_value, d_query_rope, d_key_rope, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

sfag_status backward(const void* query, const void* key, const void* value, const int32_t* sparse_indices,
                     const void* d_out, const void* out, const float* softmax_max, const float* softmax_sum,
                     const int32_t* seq_len_q_host, const int32_t* seq_len_kv_host, const void* query_rope,
                     const void* key_rope, const sfag_dims* dims, float scale_value, int64_t sparse_block_size,
                     const char* layout, int64_t sparse_mode, int32_t deterministic, void* d_query, void* d_key,
                     void* d_value, void* d_query_rope, void* d_key_rope, void* workspace, uint64_t workspace_size,
                     bool noalloc, void* stream) {
  sfag_status st;
  const struct { const void* p; const char* n; } req[] = {
      {query, "query"}, {key, "key"}, {value, "value"}, {sparse_indices, "sparse_indices"},
      {d_out, "d_out"}, {out, "out"}, {softmax_max, "softmax_max"}, {softmax_sum, "softmax_sum"},
      {d_query, "d_query"}, {d_key, "d_key"}, {d_value, "d_value"}};
  for (const auto& r : req)
    if ((st = check_ptr(r.p, r.n)) != SFAG_OK) return st;
  // rope inputs: both given (then both rope gradients are required) or both absent (no rope
  // terms; the rope gradient pointers are ignored)
  const bool has_rope = query_rope || key_rope;
  if (has_rope) {
    const struct { const void* p; const char* n; } rope[] = {
        {query_rope, "query_rope"}, {key_rope, "key_rope"}, {d_query_rope, "d_query_rope"}, {d_key_rope, "d_key_rope"}};
    for (const auto& r : rope)
      if ((st = check_ptr(r.p, r.n)) != SFAG_OK) return st;
  } else {
    d_query_rope = nullptr;
    d_key_rope = nullptr;
  }
  Plan p;
  st = make_plan(dims, seq_len_q_host, seq_len_kv_host, scale_value, sparse_block_size, layout, sparse_mode,
                 deterministic, true, &p);
  if (st != SFAG_OK) return st;
  if (noalloc) {
    if (p.bytes > kScratchBytes)
      return fail(SFAG_ERR_WORKSPACE,
                  "this problem needs %llu bytes of scratch; the no-allocation entry point holds %llu",
                  (unsigned long long)p.bytes, (unsigned long long)kScratchBytes);
    if ((st = scratch_of_current_device(&workspace)) != SFAG_OK) return st;
    workspace_size = kScratchBytes;
  }
  if (workspace_size < p.bytes || (p.bytes > 0 && !workspace))
    return fail(SFAG_ERR_WORKSPACE, "workspace of %llu bytes needed, got %llu%s", (unsigned long long)p.bytes,
                (unsigned long long)workspace_size, workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(SFAG_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);

  sfag::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(query);
  a.qr = static_cast<const uint16_t*>(query_rope);
  a.k = static_cast<const uint16_t*>(key);
  a.kr = static_cast<const uint16_t*>(key_rope);
  a.dout = static_cast<const uint16_t*>(d_out);
  a.out = static_cast<const uint16_t*>(out);
  a.idx = sparse_indices;
  a.smax = softmax_max;
  a.ssum = softmax_sum;
  a.dq = static_cast<uint16_t*>(d_query);
  a.dqr = static_cast<uint16_t*>(d_query_rope);
  a.lens = p.lens;
  a.S1 = p.S1;
  a.S2 = p.S2;
  a.B = (int)p.B;
  a.N1 = (int)p.N1;
  a.topk = (int)p.topk;
  a.bs = p.bs;
  a.mode3 = p.mode3;
  a.layout_tnd = p.tnd;
  a.hgc = p.hg_count;
  a.rec_chunks = (int)p.rec_chunks;
  a.scale = scale_value;
  a.f16 = p.f16;

  // index sort (both paths): sorted positions, counts, block starts (and the key -> position map
  // of the key-major path)
  sfag::DenseArgs da{};
  da.q = a.q;
  da.qr = a.qr;
  da.dout = a.dout;
  da.idx = sparse_indices;
  da.sorted = reinterpret_cast<int32_t*>(ws + p.off_sorted);
  da.count = reinterpret_cast<int32_t*>(ws + p.off_count);
  da.maxdup = reinterpret_cast<int32_t*>(ws + p.off_maxdup);
  da.offs = reinterpret_cast<int32_t*>(ws + p.off_offs);
  da.kpos = p.dense ? reinterpret_cast<int16_t*>(ws + p.off_kpos) : nullptr;
  da.kstride = p.dense ? (int)(p.maxblk * sfag::kBk) : 0;
  da.zero_row = reinterpret_cast<uint16_t*>(ws + p.off_zero);
  da.dk = static_cast<uint16_t*>(d_key);
  da.dkr = static_cast<uint16_t*>(d_key_rope);
  da.dv = static_cast<uint16_t*>(d_value);
  da.lens = p.lens;
  da.S1 = p.S1;
  da.S2 = p.S2;
  da.B = (int)p.B;
  da.N1 = (int)p.N1;
  da.topk = (int)p.topk;
  da.bs = p.bs;
  da.mode3 = p.mode3;
  da.layout_tnd = p.tnd;
  da.hgc = p.hg_count;
  da.maxblk = (int)p.maxblk;
  da.rec_chunks = (int)p.rec_chunks;
  da.scale = scale_value;
  da.f16 = p.f16;
  a.sorted = da.sorted;
  a.count = da.count;
  a.zero_row = da.zero_row;

  if (p.dense) {
    da.dsp = reinterpret_cast<uint16_t*>(ws + p.off_dsp);
    da.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
    da.part = reinterpret_cast<float*>(ws + p.off_part);
    da.xpart = reinterpret_cast<float*>(ws + p.off_xpart);
    da.flag = reinterpret_cast<int32_t*>(ws + p.off_flag);
    da.items = (int)p.items;
    da.citems = (int)p.citems;
    da.ilist = reinterpret_cast<int32_t*>(ws + p.off_ilist);
    da.imap = reinterpret_cast<int32_t*>(ws + p.off_imap);
    a.dsp = reinterpret_cast<uint16_t*>(ws + p.off_dsp);
    a.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
    a.row_begin = 0;
    SFAG_HIP(sfag::launch_item_list(da, s));
    SFAG_HIP(sfag::launch_sort_rows(da, p.rows, s));
    if (g_ev[0]) SFAG_HIP(hipEventRecord(g_ev[0], s));
    SFAG_HIP(sfag::launch_bwd_q(a, p.rows, p.hg_count, s));
    if (g_ev[1]) SFAG_HIP(hipEventRecord(g_ev[1], s));
    if (g_ev[2]) SFAG_HIP(hipEventRecord(g_ev[2], s));
    SFAG_HIP(sfag::launch_kv_dense(da, s));
    if (g_ev[3]) SFAG_HIP(hipEventRecord(g_ev[3], s));
    SFAG_HIP(sfag::launch_kv_reduce(da, p.keys, s));
    g_last_path = 0;
    return ok();
  }

  // per-pair path, in chunks of query rows: query-major kernel, slots (counting sort by key),
  // partials, per-key sums (the last chunk writes the bf16 key gradients)
  SFAG_HIP(sfag::launch_sort_rows(da, p.rows, s));
  sfag::PairArgs pa{};
  pa.sorted = da.sorted;
  pa.count = da.count;
  pa.offs = da.offs;
  pa.dsp = reinterpret_cast<uint16_t*>(ws + p.off_dsp);
  pa.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
  pa.part = reinterpret_cast<float*>(ws + p.off_part);
  pa.loc = reinterpret_cast<int32_t*>(ws + p.off_loc);
  pa.kcnt = reinterpret_cast<int32_t*>(ws + p.off_kcnt);
  pa.koff = reinterpret_cast<int32_t*>(ws + p.off_koff);
  pa.keys = p.keys;
  pa.btotal = reinterpret_cast<int32_t*>(ws + p.off_btotal);
  pa.bbase = reinterpret_cast<int32_t*>(ws + p.off_bbase);
  pa.acc = reinterpret_cast<float*>(ws + p.off_acc);
  pa.dk = static_cast<uint16_t*>(d_key);
  pa.dkr = static_cast<uint16_t*>(d_key_rope);
  pa.dv = static_cast<uint16_t*>(d_value);
  pa.lens = p.lens;
  pa.S1 = p.S1;
  pa.S2 = p.S2;
  pa.B = (int)p.B;
  pa.topk = (int)p.topk;
  pa.layout_tnd = p.tnd;
  pa.hgc = p.hg_count;
  pa.maxblk = (int)p.maxblk;
  pa.rec_chunks = (int)p.rec_chunks;
  pa.nblocks = (int)p.pair_blocks;
  pa.scale = scale_value;
  pa.f16 = p.f16;
  a.dsp = const_cast<uint16_t*>(pa.dsp);
  a.bt = const_cast<uint16_t*>(pa.bt);
  if (g_ev[0]) SFAG_HIP(hipEventRecord(g_ev[0], s));
  for (int64_t r0 = 0; r0 < p.rows; r0 += p.chunk_rows) {
    const int64_t nr = std::min<int64_t>(p.chunk_rows, p.rows - r0);
    a.row_begin = r0;
    SFAG_HIP(sfag::launch_bwd_q(a, nr, p.hg_count, s));
    pa.row_begin = r0;
    pa.nrows = (int)nr;
    pa.first = r0 == 0;
    pa.last = r0 + nr >= p.rows;
    SFAG_HIP(sfag::launch_pair_chunk(pa, s));
  }
  if (g_ev[1]) SFAG_HIP(hipEventRecord(g_ev[1], s));
  g_last_path = 1;
  return ok();
}

// ---- lightning-indexer backward --------------------------------------------------------------
struct IxPlan {
  int tnd = 0, mode3 = 0;
  int64_t B = 0, S1 = 0, S2 = 0, N1 = 0, G = 0, rows = 0, keys = 0, kstride = 0, key_tiles = 0;
  int parts = 1;
  sfag::Lens lens;
  uint64_t off_tot = 0, off_norm = 0, off_lrow = 0, off_dkp = 0, bytes = 0;
};

constexpr int kIxKeyTile = 64;

sfag_status make_ix_plan(const sfag_indexer_dims* d, const int64_t* sq, const int64_t* skv, const char* layout,
                         int64_t mode, IxPlan* p) {
  if (!d) return fail(SFAG_ERR_PARAM_NULLPTR, "dims is NULL");
  if (!layout) return fail(SFAG_ERR_PARAM_NULLPTR, "layout is NULL");
  if (std::strcmp(layout, "BSND") == 0) p->tnd = 0;
  else if (std::strcmp(layout, "TND") == 0) p->tnd = 1;
  else return fail(SFAG_ERR_PARAM_INVALID, "layout must be \"BSND\" or \"TND\", got \"%s\"", layout);
  if (d->D != 512) return fail(SFAG_ERR_PARAM_INVALID, "D must be 512 (got %lld)", (long long)d->D);
  if (d->Drope != 64) return fail(SFAG_ERR_PARAM_INVALID, "Drope must be 64 (got %lld)", (long long)d->Drope);
  if (d->Di != sfag::kIxDi) return fail(SFAG_ERR_PARAM_INVALID, "Di must be 128 (got %lld)", (long long)d->Di);
  if (d->N1 < 1 || d->N1 > 128) return fail(SFAG_ERR_PARAM_INVALID, "N1 must be in 1..128 (got %lld)", (long long)d->N1);
  if (d->G < 1 || d->G > 64) return fail(SFAG_ERR_PARAM_INVALID, "G must be in 1..64 (got %lld)", (long long)d->G);
  if (d->B < 1 || d->B > 256) return fail(SFAG_ERR_PARAM_INVALID, "B must be in 1..256 (got %lld)", (long long)d->B);
  if (d->dtype != SFAG_DTYPE_BF16 && d->dtype != SFAG_DTYPE_FP16)
    return fail(SFAG_ERR_PARAM_INVALID, "dtype must be SFAG_DTYPE_BF16 (0) or SFAG_DTYPE_FP16 (1) (got %lld)",
                (long long)d->dtype);
  if (mode != 0 && mode != 3) return fail(SFAG_ERR_PARAM_INVALID, "sparseMode must be 0 or 3 (got %lld)", (long long)mode);
  p->mode3 = mode == 3;
  p->B = d->B;
  p->S1 = d->S1;
  p->S2 = d->S2;
  p->N1 = d->N1;
  p->G = d->G;
  std::memset(&p->lens, 0, sizeof(p->lens));
  int64_t maxkv = 0;
  if (!p->tnd) {
    if (p->S1 < 1 || p->S1 > kMaxSeq || p->S2 < 1 || p->S2 > kMaxSeq)
      return fail(SFAG_ERR_PARAM_INVALID, "S1 and S2 must be in 1..131072 (got %lld, %lld)", (long long)p->S1,
                  (long long)p->S2);
    for (int64_t b = 0; b < p->B; ++b) {
      const int64_t lq = sq ? sq[b] : p->S1, lkv = skv ? skv[b] : p->S2;
      if (lq < 0 || lq > p->S1 || lkv < 0 || lkv > p->S2)
        return fail(SFAG_ERR_PARAM_INVALID, "actual sequence lengths of batch %lld out of range (%lld, %lld)",
                    (long long)b, (long long)lq, (long long)lkv);
      p->lens.lq[b] = (int32_t)lq;
      p->lens.lkv[b] = (int32_t)lkv;
    }
    p->rows = p->B * p->S1;
    p->keys = p->B * p->S2;
    maxkv = p->S2;
  } else {
    if (!sq || !skv) return fail(SFAG_ERR_PARAM_NULLPTR, "TND layout needs both actual sequence length arrays");
    int64_t cq = 0, ckv = 0;
    for (int64_t b = 0; b < p->B; ++b) {
      if (sq[b] < 0 || sq[b] > kMaxSeq || skv[b] < 0 || skv[b] > kMaxSeq)
        return fail(SFAG_ERR_PARAM_INVALID, "sequence %lld lengths out of range (%lld, %lld)", (long long)b,
                    (long long)sq[b], (long long)skv[b]);
      p->lens.lq[b] = (int32_t)sq[b];
      p->lens.lkv[b] = (int32_t)skv[b];
      cq += sq[b];
      ckv += skv[b];
      maxkv = std::max<int64_t>(maxkv, skv[b]);
    }
    if (cq != p->S1 || ckv != p->S2)
      return fail(SFAG_ERR_PARAM_INVALID, "TND: query / key lengths sum to %lld / %lld but dims give T1=%lld T2=%lld",
                  (long long)cq, (long long)ckv, (long long)p->S1, (long long)p->S2);
    if (cq < 1 || ckv < 1) return fail(SFAG_ERR_PARAM_INVALID, "TND: no query or key tokens");
    p->rows = cq;
    p->keys = ckv;
  }
  p->kstride = std::max<int64_t>(maxkv, 1);
  int64_t tiles = 0;
  for (int64_t b = 0; b < p->B; ++b)
    tiles += ((p->tnd ? p->lens.lkv[b] : p->S2) + kIxKeyTile - 1) / kIxKeyTile;
  p->key_tiles = tiles;
  // split every key tile's query rows so that the key kernel has about 1024 workgroups
  const int64_t t1 = std::max<int64_t>(tiles, 1);
  p->parts = (int)std::max<int64_t>(1, std::min<int64_t>(32, (1024 + t1 - 1) / t1));
  uint64_t off = 0;
  p->off_tot = off;
  off = align_up(off + (uint64_t)p->rows * p->kstride * 4);
  p->off_norm = off;
  off = align_up(off + (uint64_t)p->rows * 4);
  p->off_lrow = off;
  off = align_up(off + (uint64_t)p->rows * 4);
  p->off_dkp = off;
  off = align_up(off + (uint64_t)p->parts * p->keys * sfag::kIxDi * 4);
  p->bytes = off;
  return SFAG_OK;
}

}  // namespace

extern "C" {

sfag_status sfag_sparse_flash_attention_forward(const void* query, const void* key, const void* value,
                                                const int32_t* sparse_indices, const int32_t* seq_len_q_host,
                                                const int32_t* seq_len_kv_host, const void* query_rope,
                                                const void* key_rope, const sfag_dims* dims, float scale_value,
                                                int64_t sparse_block_size, const char* layout, int64_t sparse_mode,
                                                int64_t pre_tokens, int64_t next_tokens, void* out,
                                                float* softmax_max, float* softmax_sum, void* stream) {
  (void)pre_tokens;
  (void)next_tokens;
  sfag_status st;
  const struct { const void* p; const char* n; } req[] = {
      {query, "query"}, {key, "key"}, {value, "value"}, {sparse_indices, "sparse_indices"},
      {out, "out"}, {softmax_max, "softmax_max"}, {softmax_sum, "softmax_sum"}};
  for (const auto& r : req)
    if ((st = check_ptr(r.p, r.n)) != SFAG_OK) return st;
  if (query_rope || key_rope) {             // both or neither (no rope terms)
    if ((st = check_ptr(query_rope, "query_rope")) != SFAG_OK) return st;
    if ((st = check_ptr(key_rope, "key_rope")) != SFAG_OK) return st;
  }
  Plan p;
  st = make_plan(dims, seq_len_q_host, seq_len_kv_host, scale_value, sparse_block_size, layout, sparse_mode, 0,
                 false, &p);
  if (st != SFAG_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  sfag::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(query);
  a.qr = static_cast<const uint16_t*>(query_rope);
  a.k = static_cast<const uint16_t*>(key);
  a.kr = static_cast<const uint16_t*>(key_rope);
  a.idx = sparse_indices;
  a.out = static_cast<uint16_t*>(out);
  a.smax = softmax_max;
  a.ssum = softmax_sum;
  a.lens = p.lens;
  a.S1 = p.S1;
  a.S2 = p.S2;
  a.B = (int)p.B;
  a.N1 = (int)p.N1;
  a.topk = (int)p.topk;
  a.bs = p.bs;
  a.mode3 = p.mode3;
  a.layout_tnd = p.tnd;
  a.scale = scale_value;
  a.f16 = p.f16;
  SFAG_HIP(sfag::launch_fwd(a, p.rows, p.hg_count, s));
  return ok();
}

sfag_status sfag_lightning_indexer_grad_get_workspace_size(const sfag_indexer_dims* dims,
                                                         const int64_t* seq_len_q_host,
                                                         const int64_t* seq_len_kv_host, const char* layout,
                                                         int64_t sparse_mode, uint64_t* workspace_size) {
  if (!workspace_size) return fail(SFAG_ERR_PARAM_NULLPTR, "workspace_size is NULL");
  IxPlan p;
  const sfag_status st = make_ix_plan(dims, seq_len_q_host, seq_len_kv_host, layout, sparse_mode, &p);
  if (st != SFAG_OK) return st;
  *workspace_size = p.bytes;
  return ok();
}

sfag_status sfag_dense_lightning_indexer_grad_kl_loss(
    const void* query, const void* key, const void* query_index, const void* key_index, const void* weights,
    const float* softmax_max, const float* softmax_sum, const float* softmax_max_index,
    const float* softmax_sum_index, const void* query_rope, const void* key_rope, const int64_t* seq_len_q_host,
    const int64_t* seq_len_kv_host, const sfag_indexer_dims* dims, double scale_value, const char* layout,
    int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens, void* d_query_index, void* d_key_index,
    void* d_weights, float* loss, void* workspace, uint64_t workspace_size, void* stream) {
  (void)pre_tokens;
  (void)next_tokens;
  sfag_status st;
  // 16-byte rows are read as whole pieces and dq~ is written in 4-byte pairs: these need 16-byte
  // alignment; the others are accessed element by element
  const struct { const void* p; const char* n; bool al; } req[] = {
      {query, "query", true}, {key, "key", true}, {query_index, "query_index", true},
      {key_index, "key_index", true}, {weights, "weights", false}, {softmax_max, "softmax_max", false},
      {softmax_sum, "softmax_sum", false}, {softmax_max_index, "softmax_max_index", false},
      {softmax_sum_index, "softmax_sum_index", false}, {d_query_index, "d_query_index", true},
      {d_key_index, "d_key_index", false}, {d_weights, "d_weights", false}, {loss, "loss", false}};
  for (const auto& r : req) {
    if (!r.p) return fail(SFAG_ERR_PARAM_NULLPTR, "%s is NULL", r.n);
    if (r.al && (st = check_ptr(r.p, r.n)) != SFAG_OK) return st;
  }
  if ((query_rope == nullptr) != (key_rope == nullptr))
    return fail(SFAG_ERR_PARAM_INVALID, "query_rope and key_rope must both be given or both be NULL");
  if (query_rope) {
    if ((st = check_ptr(query_rope, "query_rope")) != SFAG_OK) return st;
    if ((st = check_ptr(key_rope, "key_rope")) != SFAG_OK) return st;
  }
  if (!std::isfinite(scale_value)) return fail(SFAG_ERR_PARAM_INVALID, "scaleValue must be finite");
  IxPlan p;
  if ((st = make_ix_plan(dims, seq_len_q_host, seq_len_kv_host, layout, sparse_mode, &p)) != SFAG_OK) return st;
  if (workspace_size < p.bytes || (p.bytes > 0 && !workspace))
    return fail(SFAG_ERR_WORKSPACE, "workspace of %llu bytes needed, got %llu%s", (unsigned long long)p.bytes,
                (unsigned long long)workspace_size, workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(SFAG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  sfag::IxArgs a{};
  a.q = static_cast<const uint16_t*>(query);
  a.qr = static_cast<const uint16_t*>(query_rope);
  a.k = static_cast<const uint16_t*>(key);
  a.kr = static_cast<const uint16_t*>(key_rope);
  a.qi = static_cast<const uint16_t*>(query_index);
  a.ki = static_cast<const uint16_t*>(key_index);
  a.w = static_cast<const uint16_t*>(weights);
  a.smax = softmax_max;
  a.ssum = softmax_sum;
  a.smax_i = softmax_max_index;
  a.ssum_i = softmax_sum_index;
  a.dqi = static_cast<uint16_t*>(d_query_index);
  a.dki = static_cast<uint16_t*>(d_key_index);
  a.dw = static_cast<uint16_t*>(d_weights);
  a.loss = loss;
  a.tot = reinterpret_cast<float*>(ws + p.off_tot);
  a.norm = reinterpret_cast<float*>(ws + p.off_norm);
  a.lrow = reinterpret_cast<float*>(ws + p.off_lrow);
  a.dkp = reinterpret_cast<float*>(ws + p.off_dkp);
  a.lens = p.lens;
  a.S1 = p.S1;
  a.S2 = p.S2;
  a.kstride = p.kstride;
  a.rows = p.rows;
  a.keys = p.keys;
  a.B = (int)p.B;
  a.N1 = (int)p.N1;
  a.G = (int)p.G;
  a.mode3 = p.mode3;
  a.layout_tnd = p.tnd;
  a.parts = p.parts;
  a.scale = (float)scale_value;
  a.f16 = dims->dtype == SFAG_DTYPE_FP16;
  SFAG_HIP(sfag::launch_indexer(a, p.key_tiles, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"
