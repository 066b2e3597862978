/*
 * oracle_driver.c -- runs the fp64 oracle (forward, dQ and dK / dV, whole and for row / key
 * subsets) on small seeded problems that reach every branch of its slot rules: invalid and
 * duplicate indices, ragged lengths, both layouts, both masks and block selection.  Built once
 * plainly and once with AddressSanitizer and UndefinedBehaviorSanitizer; the test compares the
 * printed checksums of the two builds and relies on the sanitizers to abort on a finding.
 * Test infrastructure only, like the oracle it drives.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "sfag_oracle.h"

static uint64_t g_state;

/* splitmix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number generators") */
static uint64_t next_u64(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * (2.0 / 9007199254740992.0) - 1.0; }

static double* rand_array(int64_t n) {
  double* a = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) a[i] = uniform();
  return a;
}

static double* zeros(int64_t n) { return (double*)calloc((size_t)(n > 0 ? n : 1), sizeof(double)); }

static void checksum(const char* name, const double* a, int64_t n) {
  double s = 0.0, w = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    s += fabs(a[i]);
    w += a[i] * (double)((i % 97) + 1);
  }
  printf("%s %.17g %.17g\n", name, s, w);
}

/* One problem: forward over all rows, then the backward for all rows / keys and for subsets. */
static void run(const char* tag, sfag_oracle_problem* pb, int64_t idx_hi) {
  const int64_t rows = pb->layout == 0 ? pb->B * pb->S1 : pb->S1;
  const int64_t keys = pb->layout == 0 ? pb->B * pb->S2 : pb->S2;
  const int64_t N1 = pb->N1, D = pb->D, Dr = pb->Dr;
  double* q = rand_array(rows * N1 * D);
  double* qr = rand_array(rows * N1 * Dr);
  double* k = rand_array(keys * D);
  double* kr = rand_array(keys * Dr);
  double* dout = rand_array(rows * N1 * D);
  int32_t* idx = (int32_t*)malloc((size_t)(rows * pb->topk) * sizeof(int32_t));
  /* indices from -2 to idx_hi: some negative, some past the key length, some repeated */
  for (int64_t i = 0; i < rows * pb->topk; ++i) idx[i] = (int32_t)((int64_t)(next_u64() % (uint64_t)(idx_hi + 3)) - 2);
  double* out = zeros(rows * N1 * D);
  double* smax = zeros(N1 * rows);
  double* ssum = zeros(N1 * rows);
  if (sfag_oracle_forward(pb, q, k, k, qr, kr, idx, NULL, 0, out, smax, ssum) != 0) {
    printf("%s forward failed\n", tag);
    exit(2);
  }
  printf("== %s\n", tag);
  checksum("out", out, rows * N1 * D);
  checksum("max", smax, N1 * rows);
  checksum("sum", ssum, N1 * rows);

  double* dq = zeros(rows * N1 * D);
  double* dqr = zeros(rows * N1 * Dr);
  sfag_oracle_backward_dq(pb, q, k, k, qr, kr, idx, dout, out, smax, ssum, NULL, 0, dq, dqr);
  checksum("dq", dq, rows * N1 * D);
  checksum("dqr", dqr, rows * N1 * Dr);
  const int64_t sub_rows[3] = {rows - 1, 0, rows / 2};
  sfag_oracle_backward_dq(pb, q, k, k, qr, kr, idx, dout, out, smax, ssum, sub_rows, 3, dq, dqr);
  checksum("dq_rows", dq, 3 * N1 * D);

  double* dk = zeros(keys * D);
  double* dkr = zeros(keys * Dr);
  double* dv = zeros(keys * D);
  sfag_oracle_backward_dkv(pb, q, k, k, qr, kr, idx, dout, out, smax, ssum, NULL, 0, 0, rows, dk, dkr, dv);
  checksum("dk", dk, keys * D);
  checksum("dkr", dkr, keys * Dr);
  checksum("dv", dv, keys * D);
  const int64_t sub_keys[3] = {keys - 1, 1, keys / 3};
  sfag_oracle_backward_dkv(pb, q, k, k, qr, kr, idx, dout, out, smax, ssum, sub_keys, 3, rows / 3, rows - 1, dk,
                           dkr, dv);
  checksum("dk_keys", dk, 3 * D);
  checksum("dv_keys", dv, 3 * D);

  free(q);
  free(qr);
  free(k);
  free(kr);
  free(dout);
  free(idx);
  free(out);
  free(smax);
  free(ssum);
  free(dq);
  free(dqr);
  free(dk);
  free(dkr);
  free(dv);
}

int main(void) {
  g_state = 20240611u;
  {
    /* BSND, causal, ragged lengths, one head group of 3 heads */
    const int32_t sq[2] = {6, 4}, skv[2] = {21, 13};
    sfag_oracle_problem pb = {2, 6, 21, 3, 16, 8, 9, 0, 3, sq, skv, 0.125, 1};
    run("bsnd causal", &pb, 23);
  }
  {
    /* BSND, no mask, full lengths (NULL length arrays) */
    sfag_oracle_problem pb = {1, 5, 9, 2, 8, 4, 12, 0, 0, NULL, NULL, 0.3, 1};
    run("bsnd full", &pb, 10);
  }
  {
    /* TND, no mask, block selection of 3 keys per index */
    const int32_t sq[2] = {5, 3}, skv[2] = {11, 7};
    sfag_oracle_problem pb = {2, 8, 18, 2, 8, 4, 4, 1, 0, sq, skv, 0.2, 3};
    run("tnd blocks", &pb, 4);
  }
  {
    /* TND, causal, an empty query sequence and a key-less one */
    const int32_t sq[3] = {4, 0, 3}, skv[3] = {6, 5, 0};
    sfag_oracle_problem pb = {3, 7, 11, 4, 8, 4, 5, 1, 3, sq, skv, 0.25, 2};
    run("tnd causal empty", &pb, 4);
  }
  return 0;
}
