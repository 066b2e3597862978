/*
 * sfag.h -- C ABI of the MI355X (gfx950) SparseFlashAttentionGrad library.
 *
 * The operation is the one defined on the SparseFlashAttentionGrad README
 * (gitcode ops-transformer, attention/sparse_flash_attention_grad):
 *   "function description": for every query token the key/value rows named by
 *   sparseIndices are gathered, then
 *     stage 1: dP = dO V^T,  dV[u] += P^T dO
 *     stage 2: dS = P * (dP - FlashSoftmaxGrad(dO, out)),  FlashSoftmaxGrad = rowsum(dO * out)
 *     stage 3: dQ = dS K[u] * scale,  dK[u] += dS^T Q * scale
 *   with P rebuilt from the forward statistics softmaxMax / softmaxSum
 *   ("parameters": both are intermediate outputs of the forward pass) and the
 *   MLA split of every head into a 512-wide part and a 64-wide rope part
 *   (queryRope / keyRope in, dQueryRope / dKeyRope out).
 * The argument list mirrors the page's parameter table; the two-call pattern
 * (size the workspace, then run on a stream) mirrors the workspace-query /
 * execute pair of the CANN FlashAttention backward page ("function prototype").
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous.  Pointers named *_host are
 *     host memory read during the call only; every other pointer is device
 *     memory owned by the caller.  Device pointers of the sparse operator's
 *     tensors, and of the indexer's query / key / index rows and dQueryIndex,
 *     must be 16-byte aligned (SFAG_ERR_PARAM_INVALID otherwise).  The library allocates no device memory and
 *     keeps no pointer after a call returns; the one exception is the fixed
 *     scratch array of the no-allocation entry point (SFAG_NOALLOC_SCRATCH_BYTES
 *     per GPU, created with the library's code on that device).
 *   - Every 16-bit tensor of a call (query, key, value, dOut, out, the rope
 *     tensors and all gradients) has one element type, sfag_dims.dtype: bfloat16
 *     (SFAG_DTYPE_BF16) or IEEE half (SFAG_DTYPE_FP16), the two dtypes of the
 *     README's "parameters" table.  Statistics are fp32.  Products run on the
 *     matching MFMA (bf16 or fp16 operands, fp32 accumulation); the dS / P
 *     operands of the key-side contractions are rounded to that same type.
 *   - Layout "BSND": query-side [B, S1, N1, W], key-side [B, S2, 1, W],
 *     sparseIndices [B, S1, 1, topk], statistics [B, N1, S1].
 *     Layout "TND": query-side [T1, N1, W], key-side [T2, 1, W],
 *     sparseIndices [T1, 1, topk], statistics [N1, T1]; sfag_dims.S1 = T1 and
 *     .S2 = T2, and the per-sequence lengths are required.  (W = 512 or 64.)
 *   - sparseIndices hold key positions relative to the start of the query's own
 *     batch / sequence.  A slot is skipped (not an error) when its index is
 *     negative, >= the sequence's key length, or, for sparseMode 3, greater than
 *     i + Lkv - Lq for query position i (causal mask aligned at the bottom-right
 *     vertex).  Query rows at or beyond the sequence's query length are padding.
 *   - Block selection (sparseBlockSize = bs > 1; the README's "function description"
 *     selects topk blocks of sparseBlockSize keys): index j names the block of key
 *     positions j*bs .. j*bs + bs - 1, and each of those keys is a slot of its own,
 *     skipped by the rules above (so a block may be cut by the key length or the
 *     causal mask).  A negative index skips its whole block.  topk * bs <= 131072.
 *   - sparseMode 0 (no mask) and 3 (causal, bottom-right) are supported, as the
 *     page's constraint section states; preTokens / nextTokens are accepted and
 *     ignored in both modes.
 *   - Outputs are overwritten completely: key rows selected by no query get
 *     dK = dKRope = dV = 0, padded / empty query rows get dQ = dQRope = 0.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t, NULL = the
 *     default stream) and the call returns; inputs must stay valid until the
 *     stream reaches that point.
 *   - Errors: every argument check runs before anything is enqueued; on a
 *     non-OK status nothing was launched and outputs are untouched.  The text of
 *     the last error of the calling thread is available from sfag_last_error().
 *     Status codes 161001 / 161002 mirror the CANN null-pointer / invalid-
 *     parameter codes (CANN FlashAttention backward page, "return codes").
 *   - Determinism: the page calls the operator non-deterministic by default and
 *     lets deterministic = 1 ask for reproducible results ("constraints").  Here
 *     every key gradient is summed in a fixed order in both modes (per-key partial
 *     sums added in row-segment or (row, position) order; no atomics), so results
 *     are bit-identical across runs for the same inputs, shape and device whatever
 *     the flag; it is accepted and validated.
 */
#ifndef SFAG_H
#define SFAG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFAG_OK = 0,
  SFAG_ERR_PARAM_NULLPTR = 161001, /* a required pointer is NULL */
  SFAG_ERR_PARAM_INVALID = 161002, /* a shape, attribute or layout violates the constraints */
  SFAG_ERR_UNSUPPORTED = 161901,   /* legal on the page but not built here */
  SFAG_ERR_WORKSPACE = 161902,     /* workspace NULL or smaller than sfag_get_workspace_size() */
  SFAG_ERR_DEVICE = 161903         /* a HIP runtime / launch error */
} sfag_status;

typedef struct {
  int64_t B;      /* batches (BSND) or sequences (TND), 1..256 */
  int64_t S1;     /* BSND: padded query length; TND: total query tokens T1 (1..131072 per sequence) */
  int64_t S2;     /* BSND: padded key length; TND: total key tokens T2 */
  int64_t N1;     /* query heads: 1,2,3,4,6,8,12,16,24,32,48,64,128 */
  int64_t N2;     /* key heads: must be 1 */
  int64_t D;      /* head width: must be 512 */
  int64_t Drope;  /* rope width: must be 64 */
  int64_t topk;   /* indices per query token (>= 1; the page lists 1024..8192 step 1024) */
  int64_t dtype;  /* element type of the 16-bit tensors: SFAG_DTYPE_BF16 (0) or SFAG_DTYPE_FP16 (1) */
} sfag_dims;

#define SFAG_DTYPE_BF16 0
#define SFAG_DTYPE_FP16 1

/*
 * Bytes of device workspace the backward call needs for these arguments.
 * Validates every argument that does not need device pointers; returns the
 * same status the backward call would return for them.
 *   seq_len_q_host / seq_len_kv_host: B valid lengths (actualSeqLengthsQuery /
 *     actualSeqLengthsKv); NULL means full S1 / S2 (BSND only).
 *   sparse_block_size: sparseBlockSize >= 1, with topk * sparse_block_size <= 131072
 *     (PARAM_INVALID otherwise).
 *   layout: "BSND" or "TND".
 */
sfag_status sfag_get_workspace_size(const sfag_dims* dims, const int32_t* seq_len_q_host,
                                    const int32_t* seq_len_kv_host, float scale_value,
                                    int64_t sparse_block_size, const char* layout,
                                    int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
                                    int32_t deterministic, uint64_t* workspace_size);

/*
 * SparseFlashAttentionGrad backward.
 *   query [..,N1,512], key / value [..,1,512], query_rope [..,N1,64], key_rope [..,1,64],
 *   d_out / out [..,N1,512]: bf16.  value must equal key (page constraint); it is
 *   checked for NULL but never read, key supplies both roles.
 *   sparse_indices: int32 [..,1,topk].
 *   softmax_max / softmax_sum: fp32 statistics of the forward pass (layout above).
 *   d_query, d_key, d_value, d_query_rope, d_key_rope: bf16 outputs shaped like
 *   query, key, value, query_rope, key_rope.
 *   query_rope / key_rope are optional (queryRopeOptional / keyRopeOptional): give
 *   both, with both rope gradients, or neither; then the logits have no rope term
 *   and d_query_rope / d_key_rope are ignored.  Exactly one of them NULL, or a rope
 *   gradient NULL while the rope inputs are given -> PARAM_NULLPTR.
 *   workspace: device buffer of at least sfag_get_workspace_size() bytes, 256-byte
 *   aligned; its contents on entry are ignored.
 */
sfag_status sfag_sparse_flash_attention_grad(
    const void* query, const void* key, const void* value, const int32_t* sparse_indices,
    const void* d_out, const void* out, const float* softmax_max, const float* softmax_sum,
    const int32_t* seq_len_q_host, const int32_t* seq_len_kv_host, const void* query_rope,
    const void* key_rope, const sfag_dims* dims, float scale_value, int64_t sparse_block_size,
    const char* layout, int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
    int32_t deterministic, void* d_query, void* d_key, void* d_value, void* d_query_rope,
    void* d_key_rope, void* workspace, uint64_t workspace_size, void* stream);

/*
 * Largest workspace (bytes) the no-allocation entry point below can serve from its built-in
 * scratch.
 */
#define SFAG_NOALLOC_SCRATCH_BYTES (256ull << 20)

/*
 * No-allocation variant of sfag_sparse_flash_attention_grad, for callers that cannot call
 * hipMalloc or take a caller-sized workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Arguments and results are those of
 * sfag_sparse_flash_attention_grad without workspace / workspace_size; inputs and outputs
 * are still the caller's device buffers.  Instead of a workspace the call uses a scratch array
 * built into the library (SFAG_NOALLOC_SCRATCH_BYTES per GPU, allocated with the library's
 * code on each device it runs on and held until the process ends).  Problems whose
 * sfag_get_workspace_size() exceeds that size are rejected with SFAG_ERR_WORKSPACE before
 * anything is enqueued.  The call allocates no device or pinned host memory.
 * Every call on one GPU shares that GPU's scratch and leaves its contents behind (the kernels
 * clear whatever must start at zero themselves), so calls on one GPU that overlap in time
 * (different streams or threads without ordering between them) race: order them on one
 * stream or serialise them.
 */
sfag_status sfag_sparse_flash_attention_grad_noalloc(
    const void* query, const void* key, const void* value, const int32_t* sparse_indices,
    const void* d_out, const void* out, const float* softmax_max, const float* softmax_sum,
    const int32_t* seq_len_q_host, const int32_t* seq_len_kv_host, const void* query_rope,
    const void* key_rope, const sfag_dims* dims, float scale_value, int64_t sparse_block_size,
    const char* layout, int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens,
    int32_t deterministic, void* d_query, void* d_key, void* d_value, void* d_query_rope,
    void* d_key_rope, void* stream);

/*
 * Sparse forward over the same selection (the step that produces the inputs
 * `out`, softmaxMax and softmaxSum of the backward; SparseAttnSharedkv README,
 * "function description": O = softmax(Q K~^T scale) V~ with K~ = V~, and the
 * statistics described on the SparseFlashAttentionGrad page).  out [..,N1,512]
 * bf16; softmax_max = maximum scaled logit over valid slots, softmax_sum =
 * sum of exp(logit - max); rows without a valid slot get out = 0, max = sum = 0.
 * Needs no workspace.  Same conventions and checks as the backward.
 */
sfag_status sfag_sparse_flash_attention_forward(
    const void* query, const void* key, const void* value, const int32_t* sparse_indices,
    const int32_t* seq_len_q_host, const int32_t* seq_len_kv_host, const void* query_rope,
    const void* key_rope, const sfag_dims* dims, float scale_value, int64_t sparse_block_size,
    const char* layout, int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens, void* out,
    float* softmax_max, float* softmax_sum, void* stream);

/*
 * Instrumentation: until called again, every backward call made by this thread records
 * the given hipEvent_t handles on its stream around its two main stages, so that a caller
 * can time them with hipEventElapsedTime:
 *   stage 1 (`s1_begin`, `s1_end`): key-major path: the query-major kernel (scores, dS, P,
 *     dQ); per-pair path: the whole chunk loop (query-major kernel, slot sort, partials and
 *     per-key sums of every chunk);
 *   stage 2 (`s2_begin`, `s2_end`): key-major path only: the key-major dK / dV kernel.
 * A NULL handle is not recorded.  All NULL (the default) disables recording.  The events
 * stay owned by the caller.  Always returns SFAG_OK.
 */
sfag_status sfag_set_profile_events(void* s1_begin, void* s1_end, void* s2_begin, void* s2_end);

/*
 * dK / dV path taken by the calling thread's last successful backward call: 0 = key-major
 * dense-masked kernels, 1 = per-pair partials, -1 = no call yet.  The
 * path follows from the shapes alone (see sfag_sparse_flash_attention_grad).
 */
int32_t sfag_last_path(void);

/*
 * Lightning-indexer backward with KL loss (DenseLightningIndexerGradKLLoss README,
 * "function description" and "parameters"): per query token t over the keys its mask admits,
 *   S[g, s] = queryIndex[t, g] . keyIndex[s],  I[s] = sum_g weights[t, g] ReLU(S[g, s]);
 *   p[s] = sum over the N1 main heads of exp(scale (q . k + qRope . kRope) - softmaxMax) /
 *          softmaxSum, L1-normalised over s (the head-summed main attention);
 *   loss = sum_t KL(p || Softmax(I)) with Softmax(I)[s] = exp(I[s] - softmaxMaxIndex[t]) /
 *          softmaxSumIndex[t];
 *   dI = Softmax(I) - p;  dWeights[t, g] = sum_s dI[s] ReLU(S[g, s]);
 *   dS = dI weights [S > 0];  dQueryIndex[t, g] = sum_s dS[g, s] keyIndex[s];
 *   dKeyIndex[s] = sum_t sum_g dS[g, s] queryIndex[t, g].
 * Layouts follow the sparse operator: BSND query [B, S1, N1, 512], key [B, S2, 1, 512], rope
 * [.., 64], queryIndex [B, S1, G, 128], keyIndex [B, S2, 1, 128], weights [B, S1, G], main
 * statistics [B, N1, S1], index statistics [B, S1]; TND the same without B ([T, ...], main
 * statistics [N1, T1], index statistics [T1]).  The mask is the sparse operator's (sparseMode 3:
 * keys s <= t + Lkv - Lq; mode 0: all keys of the sequence); pre/nextTokens are accepted and
 * ignored.  The 16-bit tensors share sfag_indexer_dims.dtype; statistics and the loss are fp32.
 * The actual sequence lengths are int64 host arrays (the page's INT64), optional for BSND and
 * required for TND.  queryRope / keyRope may both be NULL (no rope terms).
 * Outputs are overwritten completely (tokens or keys without admitted pairs get zeros); `loss`
 * is one fp32 value on the device.  Summation orders are fixed: results are bit-reproducible.
 * Errors and asynchrony as for the backward above; workspace from the size query below.
 */
typedef struct {
  int64_t B, S1, S2;   /* as in sfag_dims */
  int64_t N1;          /* main query heads, 1..128 */
  int64_t G;           /* index heads of queryIndex / weights, 1..64 */
  int64_t D;           /* 512 */
  int64_t Drope;       /* 64 */
  int64_t Di;          /* index head width: 128 */
  int64_t dtype;       /* SFAG_DTYPE_BF16 or SFAG_DTYPE_FP16 */
} sfag_indexer_dims;

sfag_status sfag_lightning_indexer_grad_get_workspace_size(const sfag_indexer_dims* dims,
                                                         const int64_t* seq_len_q_host,
                                                         const int64_t* seq_len_kv_host, const char* layout,
                                                         int64_t sparse_mode, uint64_t* workspace_size);

sfag_status sfag_dense_lightning_indexer_grad_kl_loss(
    const void* query, const void* key, const void* query_index, const void* key_index, const void* weights,
    const float* softmax_max, const float* softmax_sum, const float* softmax_max_index,
    const float* softmax_sum_index, const void* query_rope, const void* key_rope, const int64_t* seq_len_q_host,
    const int64_t* seq_len_kv_host, const sfag_indexer_dims* dims, double scale_value, const char* layout,
    int64_t sparse_mode, int64_t pre_tokens, int64_t next_tokens, void* d_query_index, void* d_key_index,
    void* d_weights, float* loss, void* workspace, uint64_t workspace_size, void* stream);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* sfag_last_error(void);

/* Library version string. */
const char* sfag_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SFAG_H */
