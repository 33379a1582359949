// C ABI of libinfllm2: host-side validation, work decomposition and kernel dispatch.
// Every check runs before anything is enqueued; the library keeps no global state other
// than the thread-local text of the last error.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "internal.h"

using infllm2::Geom;
using infllm2::SeqTable;

namespace {

thread_local std::string g_last_error;

infllm2_status fail(infllm2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

infllm2_status ok() {
  g_last_error.clear();
  return INFLLM2_OK;
}

infllm2_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(INFLLM2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

infllm2_status check_params(const infllm2_params* p, Geom* g) {
  if (p == nullptr) return fail(INFLLM2_ERR_NULL, "params is NULL");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(INFLLM2_ERR_SHAPE, "head counts must be positive (Hq=%d, Hkv=%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(INFLLM2_ERR_SHAPE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->dtype != INFLLM2_F32 && p->dtype != INFLLM2_BF16)
    return fail(INFLLM2_ERR_UNSUPPORTED, "unknown dtype %d", p->dtype);
  const int G = p->num_q_heads / p->num_kv_heads;
  const int d = p->head_dim;
  if (d < 8 || d > 256 || d % 8 != 0)
    return fail(INFLLM2_ERR_UNSUPPORTED, "head_dim %d unsupported (multiple of 8, 8..256)", d);
  if (G > 16 || G * d > 4096)
    return fail(INFLLM2_ERR_UNSUPPORTED, "group size %d with head_dim %d unsupported (G<=16, G*d<=4096)",
                G, d);
  if (p->kernel_stride <= 0 || p->kernel_size <= 0 || p->block_size <= 0)
    return fail(INFLLM2_ERR_SHAPE, "block_size, kernel_size and kernel_stride must be positive");
  if (p->kernel_size % p->kernel_stride != 0)
    return fail(INFLLM2_ERR_SHAPE, "kernel_size (%d) must be a multiple of kernel_stride (%d)",
                p->kernel_size, p->kernel_stride);
  if (p->block_size % p->kernel_stride != 0)
    return fail(INFLLM2_ERR_SHAPE, "block_size (%d) must be a multiple of kernel_stride (%d)",
                p->block_size, p->kernel_stride);
  if (p->block_size > 256)
    return fail(INFLLM2_ERR_UNSUPPORTED, "block_size %d above 256", p->block_size);
  if (p->topk <= 0 || p->topk > 4096)
    return fail(INFLLM2_ERR_SHAPE, "topk %d outside 1..4096", p->topk);
  if (p->num_init_blocks < 0 || p->num_local_blocks < 1)
    return fail(INFLLM2_ERR_SHAPE, "need num_init_blocks >= 0 and num_local_blocks >= 1 (%d, %d)",
                p->num_init_blocks, p->num_local_blocks);
  if (p->num_init_blocks + p->num_local_blocks > p->topk)
    return fail(INFLLM2_ERR_SHAPE, "forced blocks (%d + %d) exceed topk %d", p->num_init_blocks,
                p->num_local_blocks, p->topk);
  if (!isfinite(p->softmax_scale))
    return fail(INFLLM2_ERR_SHAPE, "softmax_scale is not finite");
  g->Hq = p->num_q_heads;
  g->Hkv = p->num_kv_heads;
  g->G = G;
  g->d = d;
  g->B = p->block_size;
  g->w = p->kernel_size;
  g->s = p->kernel_stride;
  g->topk = p->topk;
  g->n_init = p->num_init_blocks;
  g->n_local = p->num_local_blocks;
  g->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf(static_cast<float>(d));
  g->window = 0;
  if (p->score_mode != 0 && p->score_mode != 1)
    return fail(INFLLM2_ERR_SHAPE, "score_mode %d is neither 0 nor 1", p->score_mode);
  g->score_mode = p->score_mode;
  return INFLLM2_OK;
}

// Checks the host bounds and the presence of the device arrays (their contents are the
// kernels' to read).  need_kc: kc_start is required.
infllm2_status build_table(const infllm2_seqs* s, const Geom& g, bool need_kc, SeqTable* t) {
  (void)g;
  if (s == nullptr) return fail(INFLLM2_ERR_NULL, "seqs is NULL");
  if (s->num_seqs < 1) return fail(INFLLM2_ERR_SHAPE, "num_seqs %d below 1", s->num_seqs);
  if (s->max_q_len < 0 || s->max_kv_len < 0 || s->q_rows < 0)
    return fail(INFLLM2_ERR_SHAPE, "negative bound (max_q_len %d, max_kv_len %d, q_rows %d)",
                s->max_q_len, s->max_kv_len, s->q_rows);
  if (s->max_q_len > s->max_kv_len)
    return fail(INFLLM2_ERR_SHAPE, "max_q_len %d exceeds max_kv_len %d (every query sees its own key)",
                s->max_q_len, s->max_kv_len);
  if (!s->q_start || !s->q_len || !s->q_pos0 || !s->kv_start || !s->kv_len)
    return fail(INFLLM2_ERR_NULL, "a sequence metadata array is NULL");
  if (need_kc && !s->kc_start) return fail(INFLLM2_ERR_NULL, "kc_start is NULL");
  t->n = s->num_seqs;
  t->max_q_len = s->max_q_len;
  t->max_kv_len = s->max_kv_len;
  t->q_rows = s->q_rows;
  t->q_start = s->q_start;
  t->q_len = s->q_len;
  t->q_pos0 = s->q_pos0;
  t->kv_start = s->kv_start;
  t->kv_len = s->kv_len;
  t->kc_start = s->kc_start;
  t->prev_kv_len = nullptr;
  return INFLLM2_OK;
}

int auto_splits(const Geom& g, int rows) {
  if (rows <= 0) return 1;
  long long target = 512;
  long long s = (target + static_cast<long long>(rows) * g.Hkv - 1) / (static_cast<long long>(rows) * g.Hkv);
  if (s < 1) s = 1;
  if (s > g.topk) s = g.topk;
  return static_cast<int>(s);
}

}  // namespace

extern "C" {

const char* infllm2_status_string(infllm2_status st) {
  switch (st) {
    case INFLLM2_OK: return "ok";
    case INFLLM2_ERR_NULL: return "null pointer";
    case INFLLM2_ERR_SHAPE: return "invalid shape or metadata";
    case INFLLM2_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFLLM2_ERR_ALIGN: return "misaligned pointer";
    case INFLLM2_ERR_WORKSPACE: return "workspace too small";
    case INFLLM2_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* infllm2_last_error(void) { return g_last_error.c_str(); }

int32_t infllm2_version(void) { return 100; }

infllm2_status infllm2_compress_kernels(const infllm2_params* params, const infllm2_seqs* seqs,
                                        const void* k, const int32_t* prev_kv_len,
                                        void* kernels, void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, g, true, &t)) != INFLLM2_OK) return st;
  if (k == nullptr || kernels == nullptr) return fail(INFLLM2_ERR_NULL, "k or kernels is NULL");
  if (!aligned16(k) || !aligned16(kernels))
    return fail(INFLLM2_ERR_ALIGN, "k and kernels must be 16-byte aligned");
  t.prev_kv_len = prev_kv_len;
  return hip_status(infllm2::launch_compress(g, params->dtype, t, k, kernels,
                                             static_cast<hipStream_t>(stream)),
                    "compress_kernels launch");
}

infllm2_status infllm2_block_scores(const infllm2_params* params, const infllm2_seqs* seqs,
                                    const void* q, const void* kernels, float* scores,
                                    int32_t nb_stride, void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, g, true, &t)) != INFLLM2_OK) return st;
  if (q == nullptr || kernels == nullptr || scores == nullptr)
    return fail(INFLLM2_ERR_NULL, "q, kernels or scores is NULL");
  if (!aligned16(q) || !aligned16(kernels) || !aligned16(scores))
    return fail(INFLLM2_ERR_ALIGN, "q, kernels and scores must be 16-byte aligned");
  const int need = infllm2::bound_blocks(t, g.B);
  if (nb_stride < need)
    return fail(INFLLM2_ERR_SHAPE, "nb_stride %d below the %d reachable blocks", nb_stride, need);
  if (g.score_mode == 1)
    return hip_status(infllm2::launch_scores_softmax(g, params->dtype, t, q, kernels, scores,
                                                     nb_stride, static_cast<hipStream_t>(stream)),
                      "block_scores launch");
  return hip_status(infllm2::launch_scores(g, params->dtype, t, q, kernels, scores, nb_stride,
                                           static_cast<hipStream_t>(stream)),
                    "block_scores launch");
}

infllm2_status infllm2_topk_select(const infllm2_params* params, const infllm2_seqs* seqs,
                                   const float* scores, int32_t nb_stride, int32_t* block_idx,
                                   void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, g, false, &t)) != INFLLM2_OK) return st;
  if (scores == nullptr || block_idx == nullptr)
    return fail(INFLLM2_ERR_NULL, "scores or block_idx is NULL");
  if (!aligned16(scores) || !aligned16(block_idx))
    return fail(INFLLM2_ERR_ALIGN, "scores and block_idx must be 16-byte aligned");
  const int need = infllm2::bound_blocks(t, g.B);
  if (nb_stride < need)
    return fail(INFLLM2_ERR_SHAPE, "nb_stride %d below the %d reachable blocks", nb_stride, need);
  if (need > 4096)
    return fail(INFLLM2_ERR_UNSUPPORTED, "%d reachable blocks exceed 4096", need);
  return hip_status(infllm2::launch_topk(g, t, scores, nb_stride, block_idx,
                                         static_cast<hipStream_t>(stream)),
                    "topk_select launch");
}

static infllm2_status attn_common(const infllm2_params* params, const infllm2_seqs* seqs,
                                  const void* q, const void* k, const void* v,
                                  const int32_t* block_idx, void* out, float* lse, Geom* g,
                                  SeqTable* t) {
  infllm2_status st = check_params(params, g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, *g, false, t)) != INFLLM2_OK) return st;
  if (!q || !k || !v || !block_idx || !out)
    return fail(INFLLM2_ERR_NULL, "q, k, v, block_idx or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return fail(INFLLM2_ERR_ALIGN, "attention buffers must be 16-byte aligned");
  return INFLLM2_OK;
}

infllm2_status infllm2_sparse_attn_prefill(const infllm2_params* params,
                                           const infllm2_seqs* seqs, const void* q,
                                           const void* k, const void* v,
                                           const int32_t* block_idx, void* out, float* lse,
                                           void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = attn_common(params, seqs, q, k, v, block_idx, out, lse, &g, &t);
  if (st != INFLLM2_OK) return st;
  if (infllm2::attn_tile_supported(g, params->dtype, t)) {
    return hip_status(infllm2::launch_attn_tile(g, t, q, k, v, block_idx, out, lse,
                                                static_cast<hipStream_t>(stream)),
                      "sparse_attn_prefill launch");
  }
  return hip_status(infllm2::launch_attn(g, params->dtype, t, q, k, v, block_idx, 1, out, lse,
                                         nullptr, static_cast<hipStream_t>(stream)),
                    "sparse_attn_prefill launch");
}

infllm2_status infllm2_sliding_window_attn(const infllm2_params* params,
                                           const infllm2_seqs* seqs, int32_t window,
                                           const void* q, const void* k, const void* v,
                                           void* out, float* lse, void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, g, false, &t)) != INFLLM2_OK) return st;
  if (window < 1) return fail(INFLLM2_ERR_SHAPE, "window %d must be at least 1", window);
  if (!q || !k || !v || !out) return fail(INFLLM2_ERR_NULL, "q, k, v or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && !aligned16(lse)))
    return fail(INFLLM2_ERR_ALIGN, "attention buffers must be 16-byte aligned");
  if (!infllm2::attn_tile_supported(g, params->dtype, t))
    return fail(INFLLM2_ERR_UNSUPPORTED,
                "sliding-window attention needs bf16, block_size 64, head_dim 64 or 128, group "
                "size 8 or 16 and max_kv_len at most 2048 * 64");
  g.window = window;
  return hip_status(infllm2::launch_attn_tile_window(g, t, q, k, v, out, lse,
                                                     static_cast<hipStream_t>(stream)),
                    "sliding_window_attn launch");
}

static int decode_splits(const Geom& g, int dtype, int rows, int num_splits) {
  if (num_splits > 0) return num_splits;
  if (infllm2::attn_decode_supported(g, dtype)) return (g.topk + 3) / 4;
  return auto_splits(g, rows);
}

size_t infllm2_decode_workspace_size(const infllm2_params* params, int32_t total_q_rows,
                                     int32_t num_splits) {
  Geom g;
  if (check_params(params, &g) != INFLLM2_OK || total_q_rows < 0 || num_splits < 0) return 0;
  // enough for infllm2_sparse_attn_decode and for the two-launch form of infllm2_decode_step
  const int step = num_splits > 0 ? num_splits : infllm2::decode_step_splits(g, total_q_rows);
  const int splits = std::max(decode_splits(g, params->dtype, total_q_rows, num_splits), step);
  return infllm2::decode_workspace(g, total_q_rows, splits);
}

infllm2_status infllm2_sparse_attn_decode(const infllm2_params* params, const infllm2_seqs* seqs,
                                          const void* q, const void* k, const void* v,
                                          const int32_t* block_idx, int32_t num_splits,
                                          void* workspace, size_t workspace_bytes, void* out,
                                          float* lse, void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = attn_common(params, seqs, q, k, v, block_idx, out, lse, &g, &t);
  if (st != INFLLM2_OK) return st;
  if (num_splits < 0 || num_splits > g.topk)
    return fail(INFLLM2_ERR_SHAPE, "num_splits %d outside 0..topk", num_splits);
  const int rows = t.q_rows;
  const int splits = decode_splits(g, params->dtype, rows, num_splits);
  const size_t need = infllm2::decode_workspace(g, rows, splits);
  if (splits > 1) {
    if (workspace == nullptr) return fail(INFLLM2_ERR_NULL, "workspace is NULL");
    if (!aligned16(workspace)) return fail(INFLLM2_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(INFLLM2_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (infllm2::attn_decode_supported(g, params->dtype))
    return hip_status(infllm2::launch_attn_decode(g, t, q, k, v, block_idx, splits, workspace, out,
                                                  lse, s),
                      "sparse_attn_decode launch");
  // generic kernels: partials after the counter area of the common layout
  float* part = splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                      infllm2::decode_layout(rows * g.Hkv).part)
                           : nullptr;
  hipError_t e = infllm2::launch_attn(g, params->dtype, t, q, k, v, block_idx, splits, out, lse,
                                      part, s);
  if (e != hipSuccess || splits == 1) return hip_status(e, "sparse_attn_decode launch");
  return hip_status(infllm2::launch_attn_combine(g, params->dtype, t, splits, part, out, lse, s),
                    "sparse_attn_decode combine launch");
}

static infllm2_status bwd_common(const infllm2_params* params, const infllm2_seqs* seqs, Geom* g,
                                 SeqTable* t) {
  infllm2_status st = check_params(params, g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, *g, false, t)) != INFLLM2_OK) return st;
  if (!infllm2::attn_tile_supported(*g, params->dtype, *t))
    return fail(INFLLM2_ERR_UNSUPPORTED,
                "backward needs bf16, block_size 64, head_dim 64 or 128, group size 8 or 16 and "
                "max_kv_len at most 2048 * 64");
  const long long lim = (1LL << 31) - 1;
  const long long nb = static_cast<long long>(t->n) * infllm2::bound_blocks(*t, 64);
  if (nb * g->Hkv > lim || static_cast<long long>(infllm2::bound_rows(*t)) * g->Hkv * g->topk > lim)
    return fail(INFLLM2_ERR_SHAPE, "backward index beyond 2^31 entries");
  if (infllm2::bwd_segments(*g, *t) > lim)
    return fail(INFLLM2_ERR_SHAPE, "backward index beyond 2^31 segments");
  return INFLLM2_OK;
}

size_t infllm2_backward_workspace_size(const infllm2_params* params, const infllm2_seqs* seqs) {
  Geom g;
  SeqTable t;
  if (bwd_common(params, seqs, &g, &t) != INFLLM2_OK) return 0;
  return infllm2::bwd_workspace(g, t);
}

infllm2_status infllm2_sparse_attn_backward(const infllm2_params* params,
                                            const infllm2_seqs* seqs, const void* q,
                                            const void* k, const void* v,
                                            const int32_t* block_idx, const void* out,
                                            const float* lse, const void* dout, float* dq,
                                            float* dk, float* dv, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  Geom g;
  SeqTable t;
  infllm2_status st = bwd_common(params, seqs, &g, &t);
  if (st != INFLLM2_OK) return st;
  if (!q || !k || !v || !block_idx || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(INFLLM2_ERR_NULL, "a backward tensor or the workspace is NULL");
  const void* ptrs[] = {q, k, v, block_idx, out, lse, dout, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(INFLLM2_ERR_ALIGN, "backward buffers must be 16-byte aligned");
  const size_t need = infllm2::bwd_workspace(g, t);
  if (workspace_bytes < need)
    return fail(INFLLM2_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  return hip_status(infllm2::launch_attn_bwd(g, t, q, k, v, block_idx, out, lse, dout, dq, dk, dv,
                                             workspace, static_cast<hipStream_t>(stream)),
                    "sparse_attn_backward launch");
}

}  // extern "C"

namespace {

static infllm2_status decode_step_impl(const infllm2_params* params, const infllm2_seqs* seqs,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  void* kernels, const int32_t* prev_kv_len, float* scores,
                                  int32_t nb_stride, int32_t* block_idx, int32_t num_splits,
                                  void* workspace, size_t workspace_bytes, void* out, float* lse,
                                  void* stream, bool noalloc) {
  Geom g;
  SeqTable t;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if ((st = build_table(seqs, g, true, &t)) != INFLLM2_OK) return st;
  if (num_splits < 0 || num_splits > g.topk)
    return fail(INFLLM2_ERR_SHAPE, "num_splits %d outside 0..topk", num_splits);
  const int splits = num_splits > 0 ? num_splits : infllm2::decode_step_splits(g, t.q_rows);
  if (!infllm2::decode_step_supported(g, params->dtype, t, splits)) {
    st = infllm2_compress_kernels(params, seqs, k_cache, prev_kv_len, kernels, stream);
    if (st != INFLLM2_OK) return st;
    st = infllm2_block_scores(params, seqs, q, kernels, scores, nb_stride, stream);
    if (st != INFLLM2_OK) return st;
    st = infllm2_topk_select(params, seqs, scores, nb_stride, block_idx, stream);
    if (st != INFLLM2_OK) return st;
    if (noalloc) {   // the attention's completion counters start at zero (see below)
      const hipError_t e = infllm2::launch_fill_zero(
          workspace, infllm2::decode_layout(t.q_rows * g.Hkv).part, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_status(e, "decode_step_noalloc clear");
    }
    return infllm2_sparse_attn_decode(params, seqs, q, k_cache, v_cache, block_idx, num_splits,
                                      workspace, workspace_bytes, out, lse, stream);
  }
  // Fused form: the arguments are checked as the separate calls check them; one launch computes
  // the kernels completed since prev_kv_len (storing them into `kernels`) and the scores, one
  // the top-k and the attention.
  if (!q || !k_cache || !v_cache || !kernels || !scores || !block_idx || !out)
    return fail(INFLLM2_ERR_NULL, "q, k_cache, v_cache, kernels, scores, block_idx or out is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(kernels) ||
      !aligned16(scores) || !aligned16(block_idx) || !aligned16(out) || (lse && !aligned16(lse)))
    return fail(INFLLM2_ERR_ALIGN, "decode step buffers must be 16-byte aligned");
  const int need_nb = infllm2::bound_blocks(t, g.B);
  if (nb_stride < need_nb)
    return fail(INFLLM2_ERR_SHAPE, "nb_stride %d below the %d reachable blocks", nb_stride, need_nb);
  if (need_nb > 4096)
    return fail(INFLLM2_ERR_UNSUPPORTED, "%d reachable blocks exceed 4096", need_nb);
  const size_t need = infllm2::decode_workspace(g, t.q_rows, splits);
  if (workspace == nullptr) return fail(INFLLM2_ERR_NULL, "workspace is NULL");
  if (!aligned16(workspace)) return fail(INFLLM2_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(INFLLM2_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (noalloc) {
    // the completion counters must start at zero: a kernel clears them (every call leaves them
    // zero, but the buffer is shared by every call on this GPU and outlives failed ones)
    const hipError_t e = infllm2::launch_fill_zero(
        workspace, infllm2::decode_layout(t.q_rows * g.Hkv).part, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, "decode_step_noalloc clear");
  }
  t.prev_kv_len = prev_kv_len;
  return hip_status(infllm2::launch_decode_step(g, t, q, kernels, k_cache, v_cache, scores,
                                                 nb_stride, block_idx, splits, workspace, out,
                                                 lse, static_cast<hipStream_t>(stream)),
                    "decode_step launch");
}

}  // namespace

extern "C" {

infllm2_status infllm2_decode_step(const infllm2_params* params, const infllm2_seqs* seqs,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  void* kernels, const int32_t* prev_kv_len, float* scores,
                                  int32_t nb_stride, int32_t* block_idx, int32_t num_splits,
                                  void* workspace, size_t workspace_bytes, void* out, float* lse,
                                  void* stream) {
  return decode_step_impl(params, seqs, q, k_cache, v_cache, kernels, prev_kv_len, scores,
                          nb_stride, block_idx, num_splits, workspace, workspace_bytes, out, lse,
                          stream, false);
}

infllm2_status infllm2_decode_step_noalloc(const infllm2_params* params, const infllm2_seqs* seqs,
                                          const void* q, const void* k_cache,
                                          const void* v_cache, void* kernels,
                                          const int32_t* prev_kv_len, float* scores,
                                          int32_t nb_stride, int32_t* block_idx,
                                          int32_t num_splits, void* out, float* lse,
                                          void* stream) {
  Geom g;
  infllm2_status st = check_params(params, &g);
  if (st != INFLLM2_OK) return st;
  if (seqs == nullptr) return fail(INFLLM2_ERR_NULL, "seqs is NULL");
  if (seqs->q_rows < 0) return fail(INFLLM2_ERR_SHAPE, "negative bound q_rows %d", seqs->q_rows);
  const int splits = num_splits > 0 ? num_splits : infllm2::decode_step_splits(g, seqs->q_rows);
  const size_t need = infllm2::decode_workspace(g, seqs->q_rows, std::max(splits,
                                                decode_splits(g, params->dtype, seqs->q_rows,
                                                              num_splits)));
  if (need > infllm2::kNoAllocScratchBytes)
    return fail(INFLLM2_ERR_WORKSPACE,
                "decode step needs %zu bytes of workspace, above the %zu-byte static buffer of "
                "infllm2_decode_step_noalloc (fewer rows or splits, or infllm2_decode_step with "
                "a workspace)", need, infllm2::kNoAllocScratchBytes);
  void* ws = nullptr;
  const hipError_t e = infllm2::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "decode_step_noalloc scratch lookup");
  return decode_step_impl(params, seqs, q, k_cache, v_cache, kernels, prev_kv_len, scores,
                          nb_stride, block_idx, num_splits, ws, infllm2::kNoAllocScratchBytes, out,
                          lse, stream, true);
}

}  // extern "C"
