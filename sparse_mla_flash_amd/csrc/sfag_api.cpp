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
// per-launch budget of the deterministic partial buffer; the row chunk it implies depends
// only on the shape, so the summation order (and the result) is fixed for a given shape
constexpr uint64_t kPartialBudget = 4ull << 30;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int tnd = 0;
  int64_t B = 0, S1 = 0, S2 = 0, N1 = 0, topk = 0;   // topk: slots per row (indices x block size)
  int bs = 1;
  int64_t rows = 0, keys = 0;
  int mode3 = 0, det = 0, hg_count = 0;
  float scale = 0.f;
  sfag::Lens lens;                 // per-batch valid lengths
  // path: key-major dense-masked dK / dV (dense = 1) or per-pair scatter (dense = 0)
  int dense = 0;
  double waste = 0.0;              // dense-masked (row, key) entries per valid pair (upper bound)
  int64_t items = 0, citems = 0, maxblk = 0;
  // workspace layout
  uint64_t off_acc = 0, off_partial = 0, off_keys0 = 0, off_keys1 = 0, off_sorttmp = 0;
  uint64_t off_sorted = 0, off_count = 0, off_maxdup = 0, off_offs = 0, off_dsp = 0, off_part = 0, off_flag = 0;
  uint64_t off_zero = 0, off_ilist = 0, off_imap = 0, off_trash = 0, off_kpos = 0, off_bt = 0;
  uint64_t sort_tmp_bytes = 0, bytes = 0;
  int64_t det_rows = 0;            // query rows per deterministic launch
  int end_bit = 64;
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
  if (block >= 1 && dims->topk * block > kMaxTopk)
    return fail(SFAG_ERR_PARAM_INVALID, "topk * sparseBlockSize must be at most %lld (got %lld * %lld)",
                (long long)kMaxTopk, (long long)dims->topk, (long long)block);
  if (mode != 0 && mode != 3)
    return fail(SFAG_ERR_PARAM_INVALID, "sparseMode must be 0 or 3 (got %lld)", (long long)mode);
  if (block < 1) return fail(SFAG_ERR_PARAM_INVALID, "sparseBlockSize must be >= 1 (got %lld)", (long long)block);
  if (!std::isfinite(scale)) return fail(SFAG_ERR_PARAM_INVALID, "scaleValue must be finite");
  if (det != 0 && det != 1) return fail(SFAG_ERR_PARAM_INVALID, "deterministic must be 0 or 1");

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
  if (p->dense) {
    int64_t items = 0, maxblk = 0;
    for (int64_t b = 0; b < p->B; ++b) {
      const int64_t nblk = (p->lens.lkv[b] + sfag::kBk - 1) / sfag::kBk;
      items += nblk * ((p->lens.lq[b] + sfag::kSegRows - 1) / sfag::kSegRows);
      maxblk = std::max(maxblk, nblk);
    }
    p->items = items;
    p->maxblk = maxblk;
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
    const uint64_t pairs = (uint64_t)p->rows * p->topk;
    p->off_sorted = off;
    off = align_up(off + pairs * 4);
    p->off_count = off;
    off = align_up(off + (uint64_t)p->rows * 4);
    p->off_maxdup = off;
    off = align_up(off + (uint64_t)p->rows * 4);
    p->off_offs = off;
    off = align_up(off + (uint64_t)p->rows * (maxblk + 1) * 4);
    p->off_kpos = off;
    off = align_up(off + (uint64_t)p->rows * maxblk * sfag::kBk * 2);
    p->off_dsp = off;
    off = align_up(off + pairs * p->hg_count * 128 * 2);
    p->off_part = off;
    off = align_up(off + (uint64_t)p->hg_count * citems * sfag::kBk * kDacc * 4);
    p->off_flag = off;
    off = align_up(off + (uint64_t)p->hg_count * std::max<int64_t>(citems, 1) * 4);
    p->off_ilist = off;
    off = align_up(off + (uint64_t)std::max<int64_t>(citems, 1) * 4);
    p->off_imap = off;
    off = align_up(off + (uint64_t)std::max<int64_t>(items, 1) * 4);
    p->off_zero = off;
    off = align_up(off + 576 * 2);
    p->off_trash = off;                 // write-only sink for the records of invalid slots
    off = align_up(off + 128 * 2);
    p->off_bt = off;                    // Q | QRope | dO, heads innermost (key-major B operand)
    off = align_up(off + (uint64_t)p->rows * p->hg_count * kDacc * 64 * 2);
    p->bytes = off;
    return SFAG_OK;
  }
  p->off_acc = off;
  off = align_up(off + (uint64_t)p->keys * kDacc * sizeof(float));
  if (det) {
    const uint64_t per_row = (uint64_t)p->hg_count * p->topk * kDacc * sizeof(float);
    int64_t r = (int64_t)(kPartialBudget / per_row);
    if (r < 1) r = 1;
    if (r > p->rows) r = p->rows;
    // the sort takes an int item count
    while (r > 1 && r * p->topk > (int64_t)INT32_MAX / 2) r /= 2;
    p->det_rows = r;
    p->off_partial = off;
    off = align_up(off + (uint64_t)r * per_row);
    const uint64_t npairs = (uint64_t)r * p->topk;
    p->off_keys0 = off;
    off = align_up(off + npairs * sizeof(uint64_t));
    p->off_keys1 = off;
    off = align_up(off + npairs * sizeof(uint64_t));
    int bits = 1;
    while (((int64_t)1 << bits) < p->keys + 1) ++bits;
    p->end_bit = 32 + bits;
    p->sort_tmp_bytes = sfag::sort_temp_bytes((int64_t)npairs, p->end_bit);
    p->off_sorttmp = off;
    off = align_up(off + p->sort_tmp_bytes);
  }
  p->bytes = off;
  return SFAG_OK;
}

sfag_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(SFAG_ERR_PARAM_NULLPTR, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(SFAG_ERR_PARAM_INVALID, "%s must be 16-byte aligned", name);
  return SFAG_OK;
}

std::once_flag g_attr_once;
hipError_t g_attr_err = hipSuccess;

sfag_status init_device() {
  std::call_once(g_attr_once, [] {
    g_attr_err = sfag::set_bwd_attributes();
    if (g_attr_err == hipSuccess) g_attr_err = sfag::set_fwd_attributes();
    if (g_attr_err == hipSuccess) g_attr_err = sfag::set_dense_attributes();
    if (g_attr_err == hipSuccess) g_attr_err = sfag::set_q_attributes();
  });
  if (g_attr_err != hipSuccess)
    return fail(SFAG_ERR_DEVICE, "kernel attribute setup failed: %s", hipGetErrorString(g_attr_err));
  return SFAG_OK;
}

#define SFAG_HIP(call)                                                                    \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(SFAG_ERR_DEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

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
  if (workspace_size < p.bytes || (p.bytes > 0 && !workspace))
    return fail(SFAG_ERR_WORKSPACE, "workspace of %llu bytes needed, got %llu%s", (unsigned long long)p.bytes,
                (unsigned long long)workspace_size, workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(SFAG_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if ((st = init_device()) != SFAG_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* acc = reinterpret_cast<float*>(ws + p.off_acc);
  if (!p.dense) SFAG_HIP(sfag::launch_fill_zero(acc, p.keys * kDacc, s));

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
  a.acc = acc;
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
  a.scale = scale_value;

  if (p.dense) {
    sfag::DenseArgs da{};
    da.q = a.q;
    da.qr = a.qr;
    da.dout = a.dout;
    da.idx = sparse_indices;
    da.sorted = reinterpret_cast<int32_t*>(ws + p.off_sorted);
    da.count = reinterpret_cast<int32_t*>(ws + p.off_count);
    da.maxdup = reinterpret_cast<int32_t*>(ws + p.off_maxdup);
    da.offs = reinterpret_cast<int32_t*>(ws + p.off_offs);
    da.kpos = reinterpret_cast<int16_t*>(ws + p.off_kpos);
    da.kstride = (int)(p.maxblk * sfag::kBk);
    da.dsp = reinterpret_cast<uint16_t*>(ws + p.off_dsp);
    da.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
    da.part = reinterpret_cast<float*>(ws + p.off_part);
    da.flag = reinterpret_cast<int32_t*>(ws + p.off_flag);
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
    da.items = (int)p.items;
    da.citems = (int)p.citems;
    da.ilist = reinterpret_cast<int32_t*>(ws + p.off_ilist);
    da.imap = reinterpret_cast<int32_t*>(ws + p.off_imap);
    da.scale = scale_value;
    a.sorted = da.sorted;
    a.count = da.count;
    a.dsp = reinterpret_cast<uint16_t*>(ws + p.off_dsp);
    a.zero_row = da.zero_row;
    a.trash = reinterpret_cast<uint16_t*>(ws + p.off_trash);
    a.bt = reinterpret_cast<uint16_t*>(ws + p.off_bt);
    a.row_begin = 0;
    a.pairs_per_launch = 0;
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

  if (g_ev[0]) SFAG_HIP(hipEventRecord(g_ev[0], s));
  if (!p.det) {
    a.row_begin = 0;
    a.pairs_per_launch = 0;
    SFAG_HIP(sfag::launch_bwd_main(a, p.rows, p.hg_count, 0, s));
  } else {
    a.partial = reinterpret_cast<float*>(ws + p.off_partial);
    uint64_t* k0 = reinterpret_cast<uint64_t*>(ws + p.off_keys0);
    uint64_t* k1 = reinterpret_cast<uint64_t*>(ws + p.off_keys1);
    void* tmp = ws + p.off_sorttmp;
    for (int64_t r0 = 0; r0 < p.rows; r0 += p.det_rows) {
      const int64_t nr = std::min<int64_t>(p.det_rows, p.rows - r0);
      a.row_begin = r0;
      a.pairs_per_launch = nr * p.topk;
      SFAG_HIP(sfag::launch_bwd_main(a, nr, p.hg_count, 1, s));
      SFAG_HIP(sfag::launch_pair_keys(a, k0, nr, s));
      SFAG_HIP(sfag::sort_pair_keys(tmp, p.sort_tmp_bytes, k0, k1, nr * p.topk, p.end_bit, s));
      SFAG_HIP(sfag::launch_det_reduce(k1, nr * p.topk, a.partial, nr * p.topk, p.hg_count, acc, p.keys, s));
    }
  }
  if (g_ev[1]) SFAG_HIP(hipEventRecord(g_ev[1], s));
  SFAG_HIP(sfag::launch_cast(acc, static_cast<uint16_t*>(d_key), static_cast<uint16_t*>(d_key_rope),
                             static_cast<uint16_t*>(d_value), p.keys, s));
  g_last_path = 1;
  return ok();
}

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
  if ((st = init_device()) != SFAG_OK) return st;
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
  SFAG_HIP(sfag::launch_fwd(a, p.rows, p.hg_count, s));
  return ok();
}

}  // extern "C"
