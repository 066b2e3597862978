// host_driver.cpp -- drives every host-side path of the C ABI (argument checks, workspace
// planning for the large workloads, the error paths of the compute entry points) so that a build
// of the host library with AddressSanitizer and UndefinedBehaviorSanitizer can check them on a
// machine without a GPU.  The kernel launchers are stand-ins that report "no device", so no call
// ever reaches a kernel; device pointers passed here are never dereferenced by host code.
//
// Exit status 0 when every expectation held; the sanitizers abort the process on their own
// findings.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sfag.h"

namespace {

int g_fail = 0;

void expect(bool ok, const char* what, sfag_status st) {
  if (!ok) {
    std::printf("FAIL %s: status %d (%s)\n", what, (int)st, sfag_last_error());
    ++g_fail;
  }
}

// a status that is not OK must leave a message behind
void expect_err(sfag_status st, sfag_status want, const char* what) {
  expect(st == want && std::strlen(sfag_last_error()) > 0, what, st);
}

sfag_dims dims(int64_t B, int64_t S1, int64_t S2, int64_t N1, int64_t topk, int64_t dtype = SFAG_DTYPE_BF16) {
  sfag_dims d{};
  d.B = B;
  d.S1 = S1;
  d.S2 = S2;
  d.N1 = N1;
  d.N2 = 1;
  d.D = 512;
  d.Drope = 64;
  d.topk = topk;
  d.dtype = dtype;
  return d;
}

sfag_status ws(const sfag_dims& d, const int32_t* sq, const int32_t* skv, int64_t bs, const char* layout,
               int64_t mode, int32_t det, uint64_t* out) {
  return sfag_get_workspace_size(&d, sq, skv, 0.04f, bs, layout, mode, 65536, 65536, det, out);
}

// a fake, 256-byte aligned device address: host code only checks it for NULL and alignment
void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + 4096 * i); }

sfag_status grad(const sfag_dims& d, const int32_t* sq, const int32_t* skv, const char* layout, bool rope,
                 void* workspace, uint64_t wsize, bool noalloc, int null_at = -1) {
  void* p[16];
  for (int i = 0; i < 16; ++i) p[i] = i == null_at ? nullptr : fake(i + 1);
  const void* qr = rope ? p[8] : nullptr;
  const void* kr = rope ? p[9] : nullptr;
  if (noalloc)
    return sfag_sparse_flash_attention_grad_noalloc(
        p[0], p[1], p[1], static_cast<const int32_t*>(p[2]), p[3], p[4], static_cast<const float*>(p[5]),
        static_cast<const float*>(p[6]), sq, skv, qr, kr, &d, 0.04f, 1, layout, 3, 65536, 0, 0, p[10], p[11],
        p[12], p[13], p[14], nullptr);
  return sfag_sparse_flash_attention_grad(
      p[0], p[1], p[1], static_cast<const int32_t*>(p[2]), p[3], p[4], static_cast<const float*>(p[5]),
      static_cast<const float*>(p[6]), sq, skv, qr, kr, &d, 0.04f, 1, layout, 3, 65536, 0, 0, p[10], p[11], p[12],
      p[13], p[14], workspace, wsize, nullptr);
}

void backward_cases() {
  uint64_t w = 0, w2 = 0;
  // the benchmark workloads: BSND 8K x 8K, N1 = 64, topk = 2048, causal, both dtypes and modes
  sfag_dims d = dims(1, 8192, 8192, 64, 2048);
  expect(ws(d, nullptr, nullptr, 1, "BSND", 3, 0, &w) == SFAG_OK && w > 0, "bsnd 8k", SFAG_OK);
  expect(ws(d, nullptr, nullptr, 1, "BSND", 3, 1, &w2) == SFAG_OK && w2 == w, "bsnd 8k deterministic", SFAG_OK);
  sfag_dims d16 = dims(1, 8192, 8192, 64, 2048, SFAG_DTYPE_FP16);
  expect(ws(d16, nullptr, nullptr, 1, "BSND", 3, 0, &w2) == SFAG_OK && w2 == w, "bsnd 8k fp16", SFAG_OK);
  // 128K keys, 2048 of them per row (per-pair path)
  d = dims(1, 4096, 131072, 64, 2048);
  expect(ws(d, nullptr, nullptr, 1, "BSND", 3, 0, &w) == SFAG_OK && w > 0, "bsnd 128k keys", SFAG_OK);
  // TND, N1 = 128 (two head groups), sequences of different lengths
  const int32_t tq[4] = {2048, 4096, 8192, 16384};
  d = dims(4, 30720, 30720, 128, 2048);
  expect(ws(d, tq, tq, 1, "TND", 3, 0, &w) == SFAG_OK && w > 0, "tnd n1 128", SFAG_OK);
  // block selection: 32 blocks of 64 keys
  d = dims(1, 8192, 8192, 64, 32);
  expect(ws(d, nullptr, nullptr, 64, "BSND", 3, 0, &w) == SFAG_OK && w > 0, "block selection", SFAG_OK);
  // every admitted head count, B up to 256, ragged lengths, mode 0
  const int64_t heads[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 128};
  std::vector<int32_t> lq(256), lkv(256);
  for (int b = 0; b < 256; ++b) {
    lq[b] = (b * 37) % 65;
    lkv[b] = 1 + (b * 53) % 300;
  }
  for (int64_t n : heads) {
    d = dims(256, 64, 300, n, 96);
    expect(ws(d, lq.data(), lkv.data(), 1, "BSND", n % 2 ? 0 : 3, 0, &w) == SFAG_OK, "heads / B 256", SFAG_OK);
  }
  // argument errors
  d = dims(1, 128, 256, 16, 64);
  expect_err(sfag_get_workspace_size(nullptr, nullptr, nullptr, 0.04f, 1, "BSND", 3, 0, 0, 0, &w),
             SFAG_ERR_PARAM_NULLPTR, "dims NULL");
  expect_err(ws(d, nullptr, nullptr, 1, "BSND", 3, 0, nullptr), SFAG_ERR_PARAM_NULLPTR, "size NULL");
  expect_err(ws(d, nullptr, nullptr, 1, nullptr, 3, 0, &w), SFAG_ERR_PARAM_NULLPTR, "layout NULL");
  expect_err(ws(d, nullptr, nullptr, 1, "BNSD", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "layout");
  expect_err(ws(d, nullptr, nullptr, 1, "BSND", 1, 0, &w), SFAG_ERR_PARAM_INVALID, "sparse mode");
  expect_err(ws(d, nullptr, nullptr, 0, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "block size 0");
  expect_err(ws(d, nullptr, nullptr, (int64_t)1 << 62, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID,
             "block size overflowing topk * block");
  expect_err(ws(d, nullptr, nullptr, INT64_MAX, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "block size max");
  expect_err(ws(d, nullptr, nullptr, 1, "BSND", 3, 2, &w), SFAG_ERR_PARAM_INVALID, "deterministic 2");
  expect_err(sfag_get_workspace_size(&d, nullptr, nullptr, 1.0f / 0.0f, 1, "BSND", 3, 0, 0, 0, &w),
             SFAG_ERR_PARAM_INVALID, "scale inf");
  struct Bad { int field; int64_t value; const char* what; } bad[] = {
      {0, 0, "B 0"}, {0, 257, "B 257"}, {1, 0, "S1 0"}, {1, 131073, "S1 too long"}, {2, 131073, "S2 too long"},
      {3, 5, "N1 5"}, {3, 256, "N1 256"}, {4, 2, "N2 2"}, {5, 256, "D 256"}, {6, 32, "Drope 32"},
      {7, 0, "topk 0"}, {7, 131073, "topk too large"}, {7, INT64_MAX, "topk max"}, {8, 2, "dtype 2"},
      {0, INT64_MAX, "B max"}, {1, -1, "S1 negative"}};
  for (const Bad& b : bad) {
    sfag_dims e = d;
    int64_t* f[] = {&e.B, &e.S1, &e.S2, &e.N1, &e.N2, &e.D, &e.Drope, &e.topk, &e.dtype};
    *f[b.field] = b.value;
    expect_err(ws(e, nullptr, nullptr, 1, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, b.what);
  }
  const int32_t long_q[1] = {129}, neg[1] = {-1}, ok_len[1] = {128};
  expect_err(ws(d, long_q, nullptr, 1, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "seq q > S1");
  expect_err(ws(d, nullptr, neg, 1, "BSND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "seq kv negative");
  // TND: lengths required, must sum to the totals, each within range
  d = dims(4, 30720, 30720, 128, 2048);
  expect_err(ws(d, nullptr, tq, 1, "TND", 3, 0, &w), SFAG_ERR_PARAM_NULLPTR, "tnd without q lengths");
  const int32_t tbad[4] = {2048, 4096, 8192, 16383};
  expect_err(ws(d, tq, tbad, 1, "TND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "tnd sum mismatch");
  const int32_t tneg[4] = {-2048, 4096, 8192, 20480};
  expect_err(ws(d, tneg, tq, 1, "TND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "tnd negative length");
  const int32_t thuge[2] = {131073, 1};
  sfag_dims d2 = dims(2, 131074, 131074, 8, 64);
  expect_err(ws(d2, thuge, thuge, 1, "TND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "tnd sequence too long");
  const int32_t tzero[2] = {0, 0};
  d2 = dims(2, 0, 0, 8, 64);
  expect_err(ws(d2, tzero, tzero, 1, "TND", 3, 0, &w), SFAG_ERR_PARAM_INVALID, "tnd empty");

  // compute entry points: pointer checks, workspace checks, then device set-up fails (no device)
  d = dims(1, 128, 256, 16, 64);
  expect(ws(d, ok_len, nullptr, 1, "BSND", 3, 0, &w) == SFAG_OK, "small size", SFAG_OK);
  for (int i = 0; i < 15; ++i) {
    if (i == 7) continue;   // unused slot
    expect_err(grad(d, ok_len, nullptr, "BSND", true, fake(64), w, false, i), SFAG_ERR_PARAM_NULLPTR,
               "grad NULL pointer");
  }
  expect_err(grad(d, ok_len, nullptr, "BSND", true, fake(64), w - 1, false), SFAG_ERR_WORKSPACE, "small workspace");
  expect_err(grad(d, ok_len, nullptr, "BSND", true, nullptr, w, false), SFAG_ERR_WORKSPACE, "NULL workspace");
  expect_err(grad(d, ok_len, nullptr, "BSND", true, (char*)fake(64) + 16, w, false), SFAG_ERR_WORKSPACE,
             "misaligned workspace");
  expect_err(grad(d, ok_len, nullptr, "BSND", true, fake(64), w, false), SFAG_ERR_DEVICE, "grad reaches device");
  expect_err(grad(d, ok_len, nullptr, "BSND", false, fake(64), w, false), SFAG_ERR_DEVICE, "rope-less grad");
  sfag_dims bigd = dims(1, 8192, 8192, 64, 2048);
  expect_err(grad(bigd, nullptr, nullptr, "BSND", true, nullptr, 0, true), SFAG_ERR_WORKSPACE,
             "no-alloc entry rejects a problem beyond its scratch");
  const sfag_status na = grad(d, ok_len, nullptr, "BSND", true, nullptr, 0, true);
  expect(na != SFAG_OK && std::strlen(sfag_last_error()) > 0, "no-alloc entry without device", na);
  // forward
  void* f[8];
  for (int i = 0; i < 8; ++i) f[i] = fake(100 + i);
  expect_err(sfag_sparse_flash_attention_forward(f[0], f[1], f[1], static_cast<const int32_t*>(f[2]), ok_len,
                                                 nullptr, f[3], nullptr, &d, 0.04f, 1, "BSND", 3, 0, 0, f[5],
                                                 static_cast<float*>(f[6]), static_cast<float*>(f[7]), nullptr),
             SFAG_ERR_PARAM_NULLPTR, "forward with one rope input");
  expect_err(sfag_sparse_flash_attention_forward(f[0], f[1], f[1], static_cast<const int32_t*>(f[2]), ok_len,
                                                 nullptr, f[3], f[4], &d, 0.04f, 1, "BSND", 3, 0, 0, nullptr,
                                                 static_cast<float*>(f[6]), static_cast<float*>(f[7]), nullptr),
             SFAG_ERR_PARAM_NULLPTR, "forward without out");
  expect_err(sfag_sparse_flash_attention_forward(f[0], f[1], f[1], static_cast<const int32_t*>(f[2]), ok_len,
                                                 nullptr, f[3], f[4], &d, 0.04f, 1, "BSND", 3, 0, 0, f[5],
                                                 static_cast<float*>(f[6]), static_cast<float*>(f[7]), nullptr),
             SFAG_ERR_DEVICE, "forward reaches device");
}

sfag_indexer_dims ixdims(int64_t B, int64_t S1, int64_t S2, int64_t N1, int64_t G) {
  sfag_indexer_dims d{};
  d.B = B;
  d.S1 = S1;
  d.S2 = S2;
  d.N1 = N1;
  d.G = G;
  d.D = 512;
  d.Drope = 64;
  d.Di = 128;
  d.dtype = SFAG_DTYPE_BF16;
  return d;
}

void indexer_cases() {
  uint64_t w = 0;
  sfag_indexer_dims d = ixdims(1, 8192, 8192, 128, 64);
  expect(sfag_lightning_indexer_grad_get_workspace_size(&d, nullptr, nullptr, "BSND", 3, &w) == SFAG_OK && w > 0,
         "indexer bsnd", SFAG_OK);
  const int64_t tq[3] = {100, 3000, 1};
  d = ixdims(3, 3101, 3101, 64, 64);
  expect(sfag_lightning_indexer_grad_get_workspace_size(&d, tq, tq, "TND", 0, &w) == SFAG_OK, "indexer tnd", SFAG_OK);
  expect_err(sfag_lightning_indexer_grad_get_workspace_size(&d, tq, nullptr, "TND", 0, &w), SFAG_ERR_PARAM_NULLPTR,
             "indexer tnd lengths");
  const int64_t tneg[3] = {-1, 3101, 1};
  expect_err(sfag_lightning_indexer_grad_get_workspace_size(&d, tneg, tq, "TND", 0, &w), SFAG_ERR_PARAM_INVALID,
             "indexer negative length");
  const int64_t thuge[3] = {(int64_t)1 << 40, 1, 1};
  expect_err(sfag_lightning_indexer_grad_get_workspace_size(&d, thuge, tq, "TND", 0, &w), SFAG_ERR_PARAM_INVALID,
             "indexer huge length");
  struct Bad { int field; int64_t value; const char* what; } bad[] = {
      {0, 0, "B 0"}, {1, 131073, "S1"}, {3, 129, "N1"}, {4, 65, "G"}, {5, 256, "D"}, {6, 0, "Drope"},
      {7, 64, "Di"}, {8, -1, "dtype"}};
  for (const Bad& b : bad) {
    sfag_indexer_dims e = ixdims(1, 64, 64, 8, 8);
    int64_t* f[] = {&e.B, &e.S1, &e.S2, &e.N1, &e.G, &e.D, &e.Drope, &e.Di, &e.dtype};
    *f[b.field] = b.value;
    expect_err(sfag_lightning_indexer_grad_get_workspace_size(&e, nullptr, nullptr, "BSND", 3, &w),
               SFAG_ERR_PARAM_INVALID, b.what);
  }
  d = ixdims(1, 64, 128, 8, 8);
  expect(sfag_lightning_indexer_grad_get_workspace_size(&d, nullptr, nullptr, "BSND", 3, &w) == SFAG_OK, "ix small",
         SFAG_OK);
  void* p[16];
  for (int i = 0; i < 16; ++i) p[i] = fake(200 + i);
  auto call = [&](void* q, void* qr, void* kr, void* wsp, uint64_t wsz) {
    return sfag_dense_lightning_indexer_grad_kl_loss(
        q, p[1], p[2], p[3], p[4], static_cast<const float*>(p[5]), static_cast<const float*>(p[6]),
        static_cast<const float*>(p[7]), static_cast<const float*>(p[8]), qr, kr, nullptr, nullptr, &d, 0.04, "BSND",
        3, 0, 0, p[11], p[12], p[13], static_cast<float*>(p[14]), wsp, wsz, nullptr);
  };
  expect_err(call(nullptr, p[9], p[10], p[15], w), SFAG_ERR_PARAM_NULLPTR, "indexer NULL query");
  expect_err(call(p[0], p[9], nullptr, p[15], w), SFAG_ERR_PARAM_INVALID, "indexer one rope input");
  expect_err(call(p[0], p[9], p[10], p[15], w - 1), SFAG_ERR_WORKSPACE, "indexer small workspace");
  expect_err(call(p[0], p[9], p[10], p[15], w), SFAG_ERR_DEVICE, "indexer reaches device");
}

}  // namespace

int main() {
  expect(std::strlen(sfag_version()) > 0, "version", SFAG_OK);
  backward_cases();
  indexer_cases();
  std::printf("%s: %d failed expectations\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
