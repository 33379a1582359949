// Internal declarations shared by the HIP translation units of libinfllm2 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "infllm2.h"

namespace infllm2 {

constexpr int kMaxSeqs = INFLLM2_MAX_SEQS;

// Sequence metadata passed by value as a kernel argument (no device-side metadata buffers).
// work_prefix[b] is the first work item of sequence b for the launch at hand; work_prefix[n]
// is the total.  Its meaning (tiles, rows, ...) is defined by each launch.
struct SeqTable {
  int32_t n;
  int32_t q_start[kMaxSeqs];
  int32_t q_len[kMaxSeqs];
  int32_t q_pos0[kMaxSeqs];
  int32_t kv_start[kMaxSeqs];
  int32_t kv_len[kMaxSeqs];
  int32_t kc_start[kMaxSeqs];
  int32_t aux[kMaxSeqs];          // per-launch extra (e.g. first kernel of an incremental pass)
  int32_t work_prefix[kMaxSeqs + 1];
};

struct Geom {
  int32_t Hq, Hkv, G, d;
  int32_t B, w, s;
  int32_t topk, n_init, n_local;
  float scale;
  int32_t window;       // sliding-window attention: keys pos - window < j <= pos (0 = unused)
  int32_t score_mode;   // 0: group sum of scaled dot products; 1: of per-head softmaxes
};

// Sequence owning work item `item` (linear scan; at most kMaxSeqs entries).
__device__ __forceinline__ int find_seq(const SeqTable& t, int item) {
  int b = 0;
  while (b + 1 < t.n && t.work_prefix[b + 1] <= item) ++b;
  return b;
}

__host__ __device__ __forceinline__ int num_kernels(int len, int w, int s) {
  return len < w ? 0 : (len - w) / s + 1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Number of compute units of the current device (cached per device; 256 if the query fails).
int device_cus();

// Decode workspace, shared by the split-KV decode attention and the decoding step: two int
// arrays over the (row, KV head) pairs (completed attention splits, completed score chunks),
// each padded to 256 bytes, then the float32 partials: outputs [pair][split][G][d], then
// (max, sum) [pair][split][G][2].  Byte offsets:
struct DecodeLayout {
  size_t split_done, score_done, part;
};
__host__ __device__ inline DecodeLayout decode_layout(int pairs) {
  const size_t arr = (static_cast<size_t>(pairs) * 4 + 255) / 256 * 256;
  DecodeLayout L;
  L.split_done = 0;
  L.score_done = arr;
  L.part = 2 * arr;
  return L;
}

// Launch entry points (one per translation unit).  All return hipSuccess or the launch error.
hipError_t launch_compress(const Geom& g, int dtype, const SeqTable& t, const void* k,
                           void* kernels, hipStream_t stream);
hipError_t launch_scores(const Geom& g, int dtype, const SeqTable& t, const void* q,
                         const void* kernels, float* scores, int nb_stride, int range_tiles,
                         hipStream_t stream);
// Score mode 1 (per-head softmax over the visible kernels before the group sum).
bool scores_softmax_mfma_supported(const Geom& g, int dtype);
int scores_softmax_rows(const Geom& g, bool split);
hipError_t launch_scores_softmax(const Geom& g, int dtype, const SeqTable& t, const void* q,
                                 const void* kernels, float* scores, int nb_stride, bool split,
                                 hipStream_t stream);
hipError_t launch_topk(const Geom& g, const SeqTable& t, const float* scores, int nb_stride,
                       int max_blocks, int32_t* idx, hipStream_t stream);
// Attention over blocks idx[row, g, k0 .. k1) for split `sp` of `splits`.  With splits == 1
// the kernels write O and lse; otherwise they write partials to `part` and
// launch_attn_combine merges them.
hipError_t launch_attn(const Geom& g, int dtype, const SeqTable& t, const void* q,
                       const void* k, const void* v, const int32_t* idx, int splits,
                       void* out, float* lse, float* part, hipStream_t stream);
// Tiled prefill attention (tiles of consecutive query rows sharing staged K/V blocks).  The
// three tile launchers take work_prefix over query rows and form their own tiles.
bool attn_tile_supported(const Geom& g, int dtype, const SeqTable& t);
hipError_t launch_attn_tile(const Geom& g, const SeqTable& t, const void* q, const void* k,
                            const void* v, const int32_t* idx, void* out, float* lse,
                            hipStream_t stream);
// Sliding-window attention by the tile kernel (g.window >= 1):
// the blocks each tile needs follow from the positions, no index array.
hipError_t launch_attn_tile_window(const Geom& g, const SeqTable& t, const void* q, const void* k,
                                   const void* v, void* out, float* lse, hipStream_t stream);
// Gradient of the queries by the tile kernel; delta[row, h]
// = dout . out.  Writes dq as float32 [row, Hq, d].
hipError_t launch_attn_tile_dq(const Geom& g, const SeqTable& t, const void* q, const void* k,
                               const void* v, const int32_t* idx, const void* dout,
                               const float* lse, const float* delta, float* dq,
                               hipStream_t stream);
// Whole backward (dq, dk, dv as float32).  t: work_prefix over query rows, aux[b] the first
// global KV block of sequence b, n_blocks their total; q_rows bounds every row index + 1.
size_t bwd_workspace(const Geom& g, const SeqTable& t, int n_blocks, int q_rows);
long long bwd_segments(const Geom& g, const SeqTable& t, int n_blocks);
hipError_t launch_attn_bwd(const Geom& g, const SeqTable& t, int n_blocks, int q_rows,
                           const void* q, const void* k, const void* v, const int32_t* idx,
                           const void* out, const float* lse, const void* dout, float* dq,
                           float* dk, float* dv, void* workspace, hipStream_t stream);
// Split-KV decoding attention with the merge done by the last workgroup of each (row, kv head);
// its workspace follows decode_layout.
bool attn_decode_supported(const Geom& g, int dtype);
size_t decode_workspace(const Geom& g, int rows, int nsplit);
hipError_t launch_attn_decode(const Geom& g, const SeqTable& t, const void* q, const void* k,
                              const void* v, const int32_t* idx, int nsplit, void* workspace,
                              void* out, float* lse, hipStream_t stream);
// One decoding step after the kernels are compressed: block scores and top-k in one launch
// (decode_select), then the split-KV attention; work_prefix of `t` counts query rows.
bool decode_step_supported(const Geom& g, int dtype, const SeqTable& t);
int decode_step_splits(const Geom& g);
hipError_t launch_decode_step(const Geom& g, const SeqTable& t, const void* q,
                               const void* kernels, const void* k, const void* v, float* scores,
                               int nb_stride, int32_t* idx, int nsplit, void* workspace,
                               void* out, float* lse, hipStream_t stream);
hipError_t launch_attn_combine(const Geom& g, int dtype, const SeqTable& t, int splits,
                               const float* part, void* out, float* lse, hipStream_t stream);

}  // namespace infllm2
