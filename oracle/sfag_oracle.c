/*
 * sfag_oracle.c -- fp64 CPU oracle for SparseFlashAttentionGrad (test
 * infrastructure only; see sfag_oracle.h for what is computed and the layouts).
 *
 * Every loop follows the per-slot definition written on the SparseFlashAttentionGrad
 * README ("function description": gather, stage 1, stage 2, stage 3) with no
 * blocking or fusion.  Readings taken where the page is silent or garbled:
 *   - the "@" between P and (dP - FlashSoftmaxGrad) in stage 2 is an
 *     elementwise product (the only shape-consistent reading);
 *   - the left-hand sides missing from the dV and dK lines are scatter-adds into
 *     the selected rows u;
 *   - every "/sqrt(d)" is the scaleValue attribute, also used in the logits;
 *   - FlashSoftmaxGrad(dO, O) = rowsum(dO * out) using the given out;
 *   - p = exp(z - softmaxMax) / softmaxSum, with p = 0 when softmaxSum <= 0;
 *   - invalid, out-of-range and causally masked slots are skipped.
 */
#include "sfag_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Geometry of one query row. */
typedef struct {
  int64_t b, i;      /* batch/sequence and position inside it */
  int64_t lq, lkv;   /* valid query / key lengths of that batch */
  int64_t kbase;     /* global key row of key position 0 of that batch */
  int64_t stat;      /* offset of head 0 in max/sum; head stride is hstride */
  int64_t hstride;
  int active;        /* 0 for padded rows */
} row_geo;

static int64_t total_rows(const sfag_oracle_problem* pb) {
  return pb->layout == 0 ? pb->B * pb->S1 : pb->S1;
}
static int64_t total_keys(const sfag_oracle_problem* pb) {
  return pb->layout == 0 ? pb->B * pb->S2 : pb->S2;
}

static row_geo geo_of(const sfag_oracle_problem* pb, int64_t g) {
  row_geo r;
  if (pb->layout == 0) {
    r.b = g / pb->S1;
    r.i = g % pb->S1;
    r.lq = pb->seq_q ? pb->seq_q[r.b] : pb->S1;
    r.lkv = pb->seq_kv ? pb->seq_kv[r.b] : pb->S2;
    r.kbase = r.b * pb->S2;
    r.stat = r.b * pb->N1 * pb->S1 + r.i;
    r.hstride = pb->S1;
  } else {
    int64_t cq = 0, ckv = 0, b = 0;
    while (b < pb->B && g >= cq + pb->seq_q[b]) {
      cq += pb->seq_q[b];
      ckv += pb->seq_kv[b];
      ++b;
    }
    r.b = b;
    r.i = g - cq;
    r.lq = b < pb->B ? pb->seq_q[b] : 0;
    r.lkv = b < pb->B ? pb->seq_kv[b] : 0;
    r.kbase = ckv;
    r.stat = g;
    r.hstride = pb->S1;
  }
  r.active = r.i < r.lq;
  return r;
}

static int64_t block_of(const sfag_oracle_problem* pb) { return pb->block > 1 ? pb->block : 1; }

/* Slots per query row: one per key of every selected block. */
static int64_t nslots(const sfag_oracle_problem* pb) { return pb->topk * block_of(pb); }

/* Key position selected by slot s of row g, or -1 when the slot is skipped.  Slot s is key
 * s % bs of the block named by index s / bs of the row. */
static int64_t slot_key(const sfag_oracle_problem* pb, const row_geo* r, const int32_t* idx,
                        int64_t g, int64_t s) {
  if (!r->active) return -1;
  const int64_t bs = block_of(pb);
  const int64_t jb = idx[g * pb->topk + s / bs];
  if (jb < 0) return -1;
  const int64_t j = jb * bs + s % bs;
  if (j >= r->lkv) return -1;
  if (pb->sparse_mode == 3 && j > r->i + r->lkv - r->lq) return -1;
  return j;
}

static double dot(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t d = 0; d < n; ++d) acc += a[d] * b[d];
  return acc;
}

/* Scaled logit z = scale * (q.k + qRope.kRope) for head h of row g and key row kr_row. */
static double logit(const sfag_oracle_problem* pb, const double* q, const double* k,
                    const double* qr, const double* kr, int64_t g, int64_t h, int64_t key_row) {
  const double* qh = q + (g * pb->N1 + h) * pb->D;
  const double* qrh = qr + (g * pb->N1 + h) * pb->Dr;
  return pb->scale * (dot(qh, k + key_row * pb->D, pb->D) +
                      dot(qrh, kr + key_row * pb->Dr, pb->Dr));
}

/* p = exp(z - max) / sum, the softmax recomputed from the forward statistics. */
static double prob(double z, double m, double l) { return l > 0.0 ? exp(z - m) / l : 0.0; }

int sfag_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int sfag_oracle_forward(const sfag_oracle_problem* pb, const double* q, const double* k,
                        const double* v, const double* qr, const double* kr, const int32_t* idx,
                        const int64_t* rows, int64_t nrows, double* out, double* smax,
                        double* ssum) {
  const int64_t n = rows ? nrows : total_rows(pb);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n; ++it) {
    const int64_t g = rows ? rows[it] : it;
    const row_geo r = geo_of(pb, g);
    const int64_t tk = nslots(pb) > 0 ? nslots(pb) : 1;
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)tk);
    double* z = (double*)malloc(sizeof(double) * (size_t)(tk * pb->N1));  /* z[a*N1 + h] */
    double* mh = (double*)malloc(sizeof(double) * (size_t)pb->N1);
    double* lh = (double*)malloc(sizeof(double) * (size_t)pb->N1);
    int64_t nv = 0;
    for (int64_t s = 0; s < nslots(pb); ++s) {
      const int64_t j = slot_key(pb, &r, idx, g, s);
      if (j >= 0) key[nv++] = r.kbase + j;
    }
    for (int64_t a = 0; a < nv; ++a)
      for (int64_t h = 0; h < pb->N1; ++h) z[a * pb->N1 + h] = logit(pb, q, k, qr, kr, g, h, key[a]);
    for (int64_t h = 0; h < pb->N1; ++h) {
      double m = -INFINITY, l = 0.0;
      for (int64_t a = 0; a < nv; ++a)
        if (z[a * pb->N1 + h] > m) m = z[a * pb->N1 + h];
      for (int64_t a = 0; a < nv; ++a) l += exp(z[a * pb->N1 + h] - m);
      mh[h] = nv > 0 ? m : 0.0;
      lh[h] = l;
      double* o = out + (g * pb->N1 + h) * pb->D;
      for (int64_t d = 0; d < pb->D; ++d) o[d] = 0.0;
    }
    /* out = sum over slots of p * v[j] */
    for (int64_t a = 0; a < nv; ++a) {
      const double* vr = v + key[a] * pb->D;
      for (int64_t h = 0; h < pb->N1; ++h) {
        const double p = exp(z[a * pb->N1 + h] - mh[h]) / lh[h];
        double* o = out + (g * pb->N1 + h) * pb->D;
        for (int64_t d = 0; d < pb->D; ++d) o[d] += p * vr[d];
      }
    }
    for (int64_t h = 0; h < pb->N1; ++h) {
      smax[r.stat + h * r.hstride] = mh[h];
      ssum[r.stat + h * r.hstride] = lh[h];
    }
    free(key);
    free(z);
    free(mh);
    free(lh);
  }
  return 0;
}

int sfag_oracle_backward_dq(const sfag_oracle_problem* pb, const double* q, const double* k,
                            const double* v, const double* qr, const double* kr,
                            const int32_t* idx, const double* dout, const double* out,
                            const double* smax, const double* ssum, const int64_t* rows,
                            int64_t nrows, double* dq, double* dqr) {
  const int64_t n = rows ? nrows : total_rows(pb);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t it = 0; it < n; ++it) {
    const int64_t g = rows ? rows[it] : it;
    const row_geo r = geo_of(pb, g);
    double* Dt = (double*)malloc(sizeof(double) * (size_t)pb->N1);
    for (int64_t h = 0; h < pb->N1; ++h) {
      /* FlashSoftmaxGrad(dO, O) = rowsum(dO * out) */
      Dt[h] = dot(dout + (g * pb->N1 + h) * pb->D, out + (g * pb->N1 + h) * pb->D, pb->D);
      double* dqh = dq + (it * pb->N1 + h) * pb->D;
      double* dqrh = dqr + (it * pb->N1 + h) * pb->Dr;
      for (int64_t d = 0; d < pb->D; ++d) dqh[d] = 0.0;
      for (int64_t d = 0; d < pb->Dr; ++d) dqrh[d] = 0.0;
    }
    for (int64_t s = 0; s < nslots(pb); ++s) {
      const int64_t j = slot_key(pb, &r, idx, g, s);
      if (j < 0) continue;
      const int64_t key_row = r.kbase + j;
      const double* kk = k + key_row * pb->D;
      const double* kkr = kr + key_row * pb->Dr;
      for (int64_t h = 0; h < pb->N1; ++h) {
        const double* doh = dout + (g * pb->N1 + h) * pb->D;
        const double m = smax[r.stat + h * r.hstride];
        const double l = ssum[r.stat + h * r.hstride];
        const double p = prob(logit(pb, q, k, qr, kr, g, h, key_row), m, l);
        const double dp = dot(doh, v + key_row * pb->D, pb->D);  /* stage 1: dP = dO V^T */
        const double ds = p * (dp - Dt[h]);                     /* stage 2 */
        const double c = pb->scale * ds;                        /* stage 3: dQ = dS K scale */
        double* dqh = dq + (it * pb->N1 + h) * pb->D;
        double* dqrh = dqr + (it * pb->N1 + h) * pb->Dr;
        for (int64_t d = 0; d < pb->D; ++d) dqh[d] += c * kk[d];
        for (int64_t d = 0; d < pb->Dr; ++d) dqrh[d] += c * kkr[d];
      }
    }
    free(Dt);
  }
  return 0;
}

int sfag_oracle_backward_dkv(const sfag_oracle_problem* pb, const double* q, const double* k,
                             const double* v, const double* qr, const double* kr,
                             const int32_t* idx, const double* dout, const double* out,
                             const double* smax, const double* ssum, const int64_t* keys,
                             int64_t nkeys, int64_t row_lo, int64_t row_hi, double* dk,
                             double* dkr, double* dv) {
  const int64_t nk = keys ? nkeys : total_keys(pb);
  const int64_t nall = total_keys(pb);
  const int64_t nrow = total_rows(pb);
  if (row_lo < 0) row_lo = 0;
  if (row_hi > nrow) row_hi = nrow;
  /* position of each global key row in the output list (-1 = not requested) */
  int64_t* where = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nall > 0 ? nall : 1));
  for (int64_t a = 0; a < nall; ++a) where[a] = keys ? -1 : a;
  if (keys)
    for (int64_t a = 0; a < nk; ++a)
      if (keys[a] >= 0 && keys[a] < nall) where[keys[a]] = a;
  /* (row, slot) pairs per requested key, in ascending (row, slot) order */
  int64_t* cnt = (int64_t*)calloc((size_t)nk + 1, sizeof(int64_t));
  for (int64_t g = row_lo; g < row_hi; ++g) {
    const row_geo r = geo_of(pb, g);
    for (int64_t s = 0; s < nslots(pb); ++s) {
      const int64_t j = slot_key(pb, &r, idx, g, s);
      if (j >= 0 && where[r.kbase + j] >= 0) cnt[where[r.kbase + j] + 1]++;
    }
  }
  for (int64_t a = 0; a < nk; ++a) cnt[a + 1] += cnt[a];
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nk > 0 ? nk : 1));
  for (int64_t a = 0; a < nk; ++a) fill[a] = cnt[a];
  int64_t* pr = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cnt[nk] > 0 ? cnt[nk] : 1));
  for (int64_t g = row_lo; g < row_hi; ++g) {
    const row_geo r = geo_of(pb, g);
    for (int64_t s = 0; s < nslots(pb); ++s) {
      const int64_t j = slot_key(pb, &r, idx, g, s);
      if (j >= 0 && where[r.kbase + j] >= 0) pr[fill[where[r.kbase + j]]++] = g * nslots(pb) + s;
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t a = 0; a < nk; ++a) {
    const int64_t key_row = keys ? keys[a] : a;
    double* dka = dk + a * pb->D;
    double* dkra = dkr + a * pb->Dr;
    double* dva = dv + a * pb->D;
    for (int64_t d = 0; d < pb->D; ++d) dka[d] = dva[d] = 0.0;
    for (int64_t d = 0; d < pb->Dr; ++d) dkra[d] = 0.0;
    for (int64_t e = cnt[a]; e < cnt[a + 1]; ++e) {
      const int64_t g = pr[e] / nslots(pb);
      const row_geo r = geo_of(pb, g);
      for (int64_t h = 0; h < pb->N1; ++h) {
        const double* doh = dout + (g * pb->N1 + h) * pb->D;
        const double* oh = out + (g * pb->N1 + h) * pb->D;
        const double* qh = q + (g * pb->N1 + h) * pb->D;
        const double* qrh = qr + (g * pb->N1 + h) * pb->Dr;
        const double m = smax[r.stat + h * r.hstride];
        const double l = ssum[r.stat + h * r.hstride];
        const double p = prob(logit(pb, q, k, qr, kr, g, h, key_row), m, l);
        const double dp = dot(doh, v + key_row * pb->D, pb->D);
        const double ds = p * (dp - dot(doh, oh, pb->D));
        const double c = pb->scale * ds;
        for (int64_t d = 0; d < pb->D; ++d) dka[d] += c * qh[d];     /* dK[u] += dS^T Q scale */
        for (int64_t d = 0; d < pb->Dr; ++d) dkra[d] += c * qrh[d];
        for (int64_t d = 0; d < pb->D; ++d) dva[d] += p * doh[d];    /* dV[u] += P^T dO */
      }
    }
  }
  free(where);
  free(cnt);
  free(fill);
  free(pr);
  return 0;
}
