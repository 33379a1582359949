/*
 * infllm2.h -- C ABI of an MI355X (gfx950) library for InfLLM v2 block-sparse attention.
 *
 * The method (MiniCPM4 paper summary, section 2.1 "InfLLM v2"; arXiv abstract of MiniCPM4):
 * the key/value cache is divided into fixed-size blocks, each block is represented through
 * fine-grained "semantic kernels" pooled from its keys, every query token scores the blocks
 * through those kernels, the query heads of one GQA group share the highest-scoring blocks,
 * and attention runs only over the chosen blocks, both when prefilling and when decoding.
 *
 * The five compute calls below are the steps of that path, in order:
 *   infllm2_compress_kernels    keys                      -> semantic kernels
 *   infllm2_block_scores        queries, kernels          -> per-block relevance scores
 *   infllm2_topk_select         scores                    -> selected block indices
 *   infllm2_sparse_attn_prefill queries, keys, values, idx-> attention output (+ LSE)
 *   infllm2_sparse_attn_decode  the same for a few query rows per sequence, split over the
 *                               selected blocks and merged by log-sum-exp
 * and, for training, infllm2_sparse_attn_backward (gradients of the prefill attention), and
 * infllm2_sliding_window_attn (dense attention over a window of recent tokens).
 *
 * Conventions shared by every call
 * --------------------------------
 * Layouts (all row-major, contiguous, device memory, 16-byte aligned base pointers):
 *   Q, O      [q_rows,  Hq,  d]       dtype of params->dtype
 *   K, V      [kv_rows, Hkv, d]       dtype of params->dtype
 *   kernels   [kc_rows, Hkv, d]       dtype of params->dtype
 *   scores    [q_rows,  Hkv, nb_stride]  float32
 *   block_idx [q_rows,  Hkv, topk]    int32, ascending, padded with -1
 *   lse       [q_rows,  Hq]           float32, natural log of the softmax denominator
 * Query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups).
 *
 * Sequences (infllm2_seqs): sequence b owns query rows q_start[b] .. q_start[b]+q_len[b]-1,
 * whose positions in the sequence are q_pos0[b]+j; its keys/values are rows kv_start[b] ..
 * kv_start[b]+kv_len[b]-1 (position t at row kv_start+t); its semantic kernels are rows
 * kc_start[b] + c, c < floor((kv_len-w)/s)+1.  A packed prefill uses q_start = kv_start =
 * cu_seqlens and q_pos0 = 0; a decode batch over a padded cache uses kv_start = b*max_len,
 * q_len = 1, q_pos0 = kv_len-1 (the new token's K/V already stored).  Every query must see its
 * own key: q_pos0 + q_len <= kv_len.  The per-sequence arrays live in DEVICE memory and are read
 * by the kernels when they run; a call reads only the host bounds of the struct.  So a call, or
 * a captured graph of calls, may be replayed after the caller rewrites the arrays on the device
 * (the next decoding step's lengths), as long as the host bounds still hold.
 *
 * Ownership and errors: the caller allocates every buffer; the library never allocates,
 * frees or synchronises.  Calls only enqueue kernels on `stream` (a hipStream_t; NULL = the
 * default stream) and return.  Arguments are validated on the host before anything is
 * enqueued; a failed check returns a non-zero status, enqueues nothing and records a message
 * for infllm2_last_error() (thread-local).  A failed launch returns INFLLM2_ERR_HIP.  Device
 * contents (values, indices and the per-sequence arrays) are trusted: metadata that breaks the
 * rules above or the host bounds, and non-finite inputs, give undefined results.
 */
#ifndef INFLLM2_H
#define INFLLM2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INFLLM2_OK = 0,
  INFLLM2_ERR_NULL = 1,        /* a required pointer is NULL */
  INFLLM2_ERR_SHAPE = 2,       /* inconsistent sizes or sequence metadata */
  INFLLM2_ERR_UNSUPPORTED = 3, /* valid but not implemented (dtype, head_dim, ...) */
  INFLLM2_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  INFLLM2_ERR_WORKSPACE = 5,   /* workspace smaller than the matching *_workspace_size() */
  INFLLM2_ERR_HIP = 6          /* the HIP runtime reported an error */
} infllm2_status;

typedef enum { INFLLM2_F32 = 0, INFLLM2_BF16 = 1 } infllm2_dtype;

/* Method constants of one attention layer.  The pages fix none of them; the measured
 * configurations use block 64, kernel window 32, kernel stride 16. */
typedef struct {
  int32_t num_q_heads;      /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;     /* Hkv */
  int32_t head_dim;         /* d: 64 or 128 (bf16); multiple of 8 up to 256 (f32) */
  int32_t block_size;       /* B: tokens per KV block, multiple of kernel_stride, <= 256 */
  int32_t kernel_size;      /* w: tokens pooled into one semantic kernel, multiple of s */
  int32_t kernel_stride;    /* s: distance between consecutive kernels */
  int32_t topk;             /* blocks per (query token, KV head), forced blocks included */
  int32_t num_init_blocks;  /* leading blocks always selected (>= 0) */
  int32_t num_local_blocks; /* blocks ending at the query's own block always selected (>= 1) */
  float softmax_scale;      /* <= 0 selects 1/sqrt(head_dim) */
  int32_t dtype;            /* infllm2_dtype of Q, K, V, O and the kernels */
  int32_t score_mode;       /* relevance score of infllm2_block_scores: 0 = group sum of scaled
                               dot products, 1 = group sum of per-head softmax probabilities
                               over the visible kernels (see there) */
} infllm2_params;

/* Per-sequence metadata.  The host bounds size the launches and are checked on the host; the
 * six arrays (num_seqs entries each) are DEVICE memory, read only by the kernels and trusted
 * (every q_len[b] <= max_q_len, kv_len[b] <= max_kv_len, q_start[b] + q_len[b] <= q_rows,
 * row indices below 2^31).  kc_start may be NULL for calls without semantic kernels (top-k,
 * attention). */
typedef struct {
  int32_t num_seqs;        /* host: number of sequences, >= 1 (no upper limit) */
  int32_t max_q_len;       /* host: bound on every q_len[b] */
  int32_t max_kv_len;      /* host: bound on every kv_len[b] */
  int32_t q_rows;          /* host: rows of q / out / scores / block_idx / lse (a bound on
                              every q_start[b] + q_len[b]) */
  const int64_t* q_start;  /* device arrays */
  const int32_t* q_len;
  const int32_t* q_pos0;
  const int64_t* kv_start;
  const int32_t* kv_len;
  const int64_t* kc_start;
} infllm2_seqs;

/* Semantic kernels (paper summary section 2.1.2: fine-grained semantic kernels represent each
 * KV block).  Kernel c of a sequence is the mean of the keys of its tokens s*c .. s*c+w-1,
 * summed in float64 and rounded once, to nearest even, to the key dtype.  The float64 sum is
 * exact, so the kernel is the exactly rounded mean, whenever the window's nonzero keys differ in
 * binary exponent by at most 53 - p - ceil(log2 w) (p = 8 significant bits for bf16, 24 for
 * float32: 40 and 24 binades for w = 32), which keys of ordinary magnitude always meet; a window
 * spread wider may round once more in the sum and land one unit in the last place away.
 * prev_kv_len (device array of num_seqs entries, may be NULL = all zeros) makes the call
 * incremental: only kernels with prev_kv_len[b] < s*c + w <= kv_len[b] are written; other rows
 * of `kernels` are left untouched.  Reads k, writes kernels. */
infllm2_status infllm2_compress_kernels(const infllm2_params* params, const infllm2_seqs* seqs,
                                        const void* k, const int32_t* prev_kv_len,
                                        void* kernels, void* stream);

/* Query-block relevance (section 2.1.2: the relevance of each query token to each KV block,
 * shared by the query heads of one group).  For query row at position i and KV head g:
 *   u[c]  = scale * sum over heads h of group g of  q[h] . kernel[c, g]   for kernels c whose
 *           last token s*c+w-1 <= i,
 *   S[b]  = max of u[c] over the kernels overlapping block b ([s*c, s*c+w) meets
 *           [B*b, B*b+B)), or -inf if none is visible,
 * written for blocks b = 0 .. floor(i/B) at scores[row, g, b]; entries after floor(i/B) are
 * not written.  nb_stride >= ceil(max_kv_len / B) (every reachable block).  bf16 scores use
 * the group-summed query in float32 split into two bf16 parts on the matrix cores (relative
 * error about 2^-16 of sum |q . kernel|); f32 scores use float32 arithmetic.
 * params->score_mode = 1 takes the other reading of the same passage: each head's scores are
 * normalised first, u[c] = sum over h of exp(scale q[h] . kernel[c, g] - lse_h), lse_h the
 * log-sum-exp of that head's scores over the visible kernels, so u[c] lies in [0, G] and sums
 * to G over the visible kernels; S[b] as above.  Computed in float32 from the exact bf16
 * products (two passes over the kernels). */
infllm2_status infllm2_block_scores(const infllm2_params* params, const infllm2_seqs* seqs,
                                    const void* q, const void* kernels, float* scores,
                                    int32_t nb_stride, void* stream);

/* Group-shared top-k (section 2.1.1: each query token picks the highest-scoring blocks;
 * section 2.1.2: one set per query-head group).  For query row at position i and KV head g,
 * with E = {0 .. floor(i/B)} the reachable blocks: all of E if |E| <= topk; otherwise the
 * forced blocks F = {0 .. n_init-1} U {floor(i/B)-n_local+1 .. floor(i/B)} plus the
 * topk-|F| best other blocks by (score descending, block index ascending; -0 equals +0).
 * Written ascending to block_idx[row, g, 0..topk-1], padded with -1.  Scores are read for
 * b <= floor(i/B) only.  Supported up to ceil(max_kv_len / B) = 4096 reachable blocks. */
infllm2_status infllm2_topk_select(const infllm2_params* params, const infllm2_seqs* seqs,
                                   const float* scores, int32_t nb_stride, int32_t* block_idx,
                                   void* stream);

/* Block-sparse attention (section 2.1.3: each token attends only to its most relevant KV
 * blocks).  For query row at position i, head h, KV head g = h / (Hq/Hkv):
 *   O[row, h] = sum_j softmax_j(scale * q[h] . k[j, g]) v[j, g]
 * over the tokens j <= i of the blocks listed in block_idx[row, g] (-1 entries end the list),
 * and lse[row, h] = log sum_j exp(scale * q . k_j).  lse may be NULL.  Indices must be
 * ascending, distinct, and within the sequence's blocks. */
infllm2_status infllm2_sparse_attn_prefill(const infllm2_params* params,
                                           const infllm2_seqs* seqs, const void* q,
                                           const void* k, const void* v,
                                           const int32_t* block_idx, void* out, float* lse,
                                           void* stream);

/* Sliding-window attention, the second attention workload the pages name (paper summary,
 * section 4.1.3: the speculative draft model uses sliding-window attention to keep the first
 * token's latency low).  For query row at position i, head h, KV head g = h / (Hq/Hkv):
 *   O[row, h] = sum_j softmax_j(scale * q[h] . k[j, g]) v[j, g]  over i - window < j <= i,
 * and lse[row, h] = log sum_j exp(scale * q . k_j) (may be NULL).  No block selection and no
 * block_idx: the window is given in tokens (>= 1; window >= i + 1 is causal attention).  Same
 * layouts as infllm2_sparse_attn_prefill; params->topk and the kernel constants are validated
 * but unused.  Supported: bf16, block_size 64, head_dim 64 or 128, Hq/Hkv 8 or 16 and
 * max_kv_len <= 2048 * 64 (else INFLLM2_ERR_UNSUPPORTED). */
infllm2_status infllm2_sliding_window_attn(const infllm2_params* params,
                                           const infllm2_seqs* seqs, int32_t window,
                                           const void* q, const void* k, const void* v,
                                           void* out, float* lse, void* stream);

/* Bytes of device workspace infllm2_sparse_attn_backward needs for these sequences (0 if the
 * arguments are invalid or the geometry is unsupported).  It holds delta, the reverse block
 * index, its offsets and a work counter of the key/value gradient pass; its contents need no
 * initialisation (the call zeroes what must start at zero) and are scratch between calls. */
size_t infllm2_backward_workspace_size(const infllm2_params* params, const infllm2_seqs* seqs);

/* Gradients of infllm2_sparse_attn_prefill (model card "Efficient Model Architecture" and
 * paper summary section 2.1: the sparse attention is trainable), with block_idx held fixed
 * (the selection is piecewise constant in q and k).  For query row at position i, head h,
 * KV head g, over the same attended tokens j, with P_j the softmax weights,
 * delta = dout[row, h] . out[row, h] and dS_j = P_j (dout[row, h] . v[j, g] - delta):
 *   dq[row, h] = scale * sum_j dS_j k[j, g]
 *   dk[j, g]  += scale * dS_j q[row, h],   dv[j, g] += P_j dout[row, h]
 * Inputs are the forward's: q, k, v, block_idx, out and lse (natural log, not NULL) exactly
 * as infllm2_sparse_attn_prefill wrote them, plus dout [q_rows, Hq, d] (bf16).  Outputs are
 * float32: dq [q_rows, Hq, d] (every row of every sequence written), dk and dv
 * [kv_rows, Hkv, d] (every key row of every sequence overwritten; keys no row attends to get
 * 0).  Supported: bf16, block_size 64, head_dim 64 or 128, Hq/Hkv 8 or 16 and max_kv_len <=
 * 2048 * 64 (else INFLLM2_ERR_UNSUPPORTED).  dk and dv are summed with
 * atomic float32 additions, so their last bits may differ between calls; sequences that
 * share key rows receive the sum of their gradients. */
infllm2_status infllm2_sparse_attn_backward(const infllm2_params* params,
                                            const infllm2_seqs* seqs, const void* q,
                                            const void* k, const void* v,
                                            const int32_t* block_idx, const void* out,
                                            const float* lse, const void* dout, float* dq,
                                            float* dk, float* dv, void* workspace,
                                            size_t workspace_bytes, void* stream);

/* Bytes of device workspace infllm2_sparse_attn_decode and infllm2_decode_step need for
 * `total_q_rows` rows of q (the q_rows of the calls' infllm2_seqs) split `num_splits` ways (0 =
 * the automatic choice of each call).  The workspace holds per-(row, KV head) counters, indexed
 * by the query row, then the per-split partial
 * results: it must be zero-filled before its first use, and every call leaves the counters
 * zero again.  Calls that share a workspace must not overlap
 * (enqueue them on one stream). */
size_t infllm2_decode_workspace_size(const infllm2_params* params, int32_t total_q_rows,
                                     int32_t num_splits);

/* The same attention for decoding (arXiv abstract: the sparse attention accelerates both
 * prefilling and decoding): each row's selected blocks are split into num_splits contiguous
 * parts (0 = automatic) computed in parallel into `workspace`, then merged by log-sum-exp.
 * The result does not depend on num_splits beyond float32 rounding. */
infllm2_status infllm2_sparse_attn_decode(const infllm2_params* params, const infllm2_seqs* seqs,
                                          const void* q, const void* k, const void* v,
                                          const int32_t* block_idx, int32_t num_splits,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          float* lse, void* stream);

/* One decoding step in the method's order (csdn summary 2.1.1-2.1.3): semantic kernels
 * completed since prev_kv_len (device array, may be NULL), block scores into `scores` (nb_stride
 * floats per (row, KV head)), top-k into block_idx, then split-KV attention.  Arguments mean
 * what they mean in the separate calls, and the same checks apply; `workspace` is always
 * required here.  For bf16, block 64, kernels 32/16, d 64 or 128, groups of 8 or 16 and score
 * mode 0 (and at most 256 selected blocks per split), the kernels completed since prev_kv_len
 * and the scores run as one launch (new kernels are computed from k_cache where they are scored
 * and stored into `kernels`), the top-k and the attention as a second (every split workgroup of
 * a (row, KV head) selects the pair's blocks itself; the first writes them to block_idx); the
 * results equal those of the separate calls (kernels, scores and indices exactly, outputs to
 * float32 rounding).  Otherwise the
 * separate calls are chained on `stream`; the first failing call's status is returned and
 * nothing after it is enqueued. */
infllm2_status infllm2_decode_step(const infllm2_params* params, const infllm2_seqs* seqs,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  void* kernels, const int32_t* prev_kv_len, float* scores,
                                  int32_t nb_stride, int32_t* block_idx, int32_t num_splits,
                                  void* workspace, size_t workspace_bytes, void* out, float* lse,
                                  void* stream);

/* infllm2_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture that may not call hipMalloc, tight serving loops, harnesses that forbid allocation):
 * the same step, arguments and results, without the workspace arguments.  Its workspace is a
 * buffer the library keeps in device memory, 16 MiB on each GPU it runs on (held until the
 * process ends); a step whose workspace (infllm2_decode_workspace_size for seqs->q_rows rows and
 * num_splits) exceeds it returns INFLLM2_ERR_WORKSPACE and enqueues nothing.  The call allocates
 * nothing; a kernel clears the buffer's completion counters before the step's attention.  Every
 * call on one GPU shares that GPU's buffer, so calls that overlap on one GPU (other streams,
 * other host threads) race: the caller must serialise them. */
infllm2_status infllm2_decode_step_noalloc(const infllm2_params* params, const infllm2_seqs* seqs,
                                          const void* q, const void* k_cache,
                                          const void* v_cache, void* kernels,
                                          const int32_t* prev_kv_len, float* scores,
                                          int32_t nb_stride, int32_t* block_idx,
                                          int32_t num_splits, void* out, float* lse,
                                          void* stream);

/* Static text for a status code. */
const char* infllm2_status_string(infllm2_status status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* infllm2_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t infllm2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* INFLLM2_H */
