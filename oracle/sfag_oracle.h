/*
 * sfag_oracle.h -- plain, slow, fp64 CPU oracle for SparseFlashAttentionGrad.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (SparseFlashAttentionGrad README, "function description"
 * section, and its "parameters" / "constraints" sections):
 *   - per query token, the key/value rows named by sparseIndices are gathered;
 *   - forward (used only to build consistent inputs): the scaled logit of a
 *     slot is scale*(q.k + qRope.kRope); softmaxMax is the maximum logit over
 *     valid slots, softmaxSum the sum of exp(logit - max), out the
 *     probability-weighted sum of the gathered value rows (SparseAttnSharedkv
 *     README, "function description": O = softmax(Q K~^T scale) V~ with K~ = V~);
 *   - backward, stages 1-3 of the SparseFlashAttentionGrad formulas:
 *     dP = dO V^T, dV[u] += P^T dO, D = rowsum(dO * out) (FlashSoftmaxGrad),
 *     dS = P * (dP - D) (elementwise), dQ = dS K[u] * scale,
 *     dK[u] += dS^T Q * scale, and the same split for the rope part.
 *
 * Layouts (row-major, all arrays double precision):
 *   BSND: q,dO,out,dq [B,S1,N1,D]; qr,dqr [B,S1,N1,Dr]; k,v,dk,dv [B,S2,D];
 *         kr,dkr [B,S2,Dr]; idx [B,S1,topk]; max,sum [B,N1,S1].
 *   TND:  q.. [T1,N1,D]; k.. [T2,D]; idx [T1,topk]; max,sum [N1,T1]; S1=T1,
 *         S2=T2 and seq_q/seq_kv (B entries) are required.
 * A slot of query row i of batch b is valid iff its key position j satisfies
 * 0 <= j < Lkv_b and, for sparse_mode 3, j <= i + Lkv_b - Lq_b.  Rows i >= Lq_b
 * are padding.  Invalid slots are skipped.
 * Block selection (README "function description": topk blocks of sparseBlockSize
 * keys each are gathered): with block = bs > 1 a row has topk * bs slots, and
 * index idx[row][a] >= 0 gives the slots of key positions idx*bs .. idx*bs + bs - 1,
 * each checked on its own as above; a negative index skips its bs slots.
 */
#ifndef SFAG_ORACLE_H
#define SFAG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t B, S1, S2;      /* BSND: padded lengths; TND: S1 = T1, S2 = T2 totals */
  int64_t N1, D, Dr, topk;
  int32_t layout;         /* 0 = BSND, 1 = TND */
  int32_t sparse_mode;    /* 0 = no mask, 3 = causal, bottom-right aligned */
  const int32_t* seq_q;   /* B query lengths (NULL: S1 each, BSND only) */
  const int32_t* seq_kv;  /* B key lengths   (NULL: S2 each, BSND only) */
  double scale;
  int64_t block;          /* sparseBlockSize (<= 1: each index is one key position) */
} sfag_oracle_problem;

/* Forward for the listed query rows (global row ids, NULL = all rows).
 * Writes out/max/sum at their full-layout positions. */
int sfag_oracle_forward(const sfag_oracle_problem* pb, const double* q, const double* k,
                        const double* v, const double* qr, const double* kr, const int32_t* idx,
                        const int64_t* rows, int64_t nrows,
                        double* out, double* smax, double* ssum);

/* dQ / dQRope for the listed query rows (NULL = all rows); results are written
 * compactly in list order: dq[n,N1,D], dqr[n,N1,Dr]. */
int sfag_oracle_backward_dq(const sfag_oracle_problem* pb, const double* q, const double* k,
                            const double* v, const double* qr, const double* kr,
                            const int32_t* idx, const double* dout, const double* out,
                            const double* smax, const double* ssum,
                            const int64_t* rows, int64_t nrows, double* dq, double* dqr);

/* dK / dKRope / dV for the listed key rows (global key row ids, NULL = all),
 * counting only query rows in [row_lo, row_hi).  Written compactly in list
 * order: dk[n,D], dkr[n,Dr], dv[n,D].  Each key row sums its contributions in
 * ascending (query row, slot, head) order, independent of the thread count. */
int sfag_oracle_backward_dkv(const sfag_oracle_problem* pb, const double* q, const double* k,
                             const double* v, const double* qr, const double* kr,
                             const int32_t* idx, const double* dout, const double* out,
                             const double* smax, const double* ssum,
                             const int64_t* keys, int64_t nkeys, int64_t row_lo, int64_t row_hi,
                             double* dk, double* dkr, double* dv);

/* Number of OpenMP threads the oracle runs with. */
int sfag_oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
