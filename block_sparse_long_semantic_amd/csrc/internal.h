// Internal declarations shared by the HIP translation units of libinfllm2 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "infllm2.h"

namespace infllm2 {

// Sequence metadata as the kernels see it: the caller's device arrays (read when a kernel runs,
// never on the host) and the host bounds that size the grids.  Kernels map a dense work item to
// its sequence with locate() below; what an item is (a query row, a tile of rows, a tile of
// kernels, ...) is defined by each launch.
struct SeqTable {
  int32_t n;            // sequences
  int32_t max_q_len;    // bound on every q_len[b]
  int32_t max_kv_len;   // bound on every kv_len[b]
  int32_t q_rows;       // bound on every q_start[b] + q_len[b]
  const int64_t* q_start;
  const int32_t* q_len;
  const int32_t* q_pos0;
  const int64_t* kv_start;
  const int32_t* kv_len;
  const int64_t* kc_start;      // may be null where the call has no kernels
  const int32_t* prev_kv_len;   // incremental compression only (null: all zeros)
};

// A wave-uniform value as the compiler should see it (scalar registers): values loaded from the
// metadata arrays at a uniform index are uniform, but the compiler cannot prove it, and would
// otherwise build addresses and buffer descriptors from them in vector registers.
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// One sequence's metadata, loaded from the device arrays (row indices fit in 32 bits); b must be
// wave-uniform.
struct Seq {
  int32_t q_start, q_len, q_pos0, kv_start, kv_len, kc_start;
};

__device__ __forceinline__ Seq load_seq(const SeqTable& t, int b) {
  Seq s;
  s.q_start = uniform(static_cast<int32_t>(t.q_start[b]));
  s.q_len = uniform(t.q_len[b]);
  s.q_pos0 = uniform(t.q_pos0[b]);
  s.kv_start = uniform(static_cast<int32_t>(t.kv_start[b]));
  s.kv_len = uniform(t.kv_len[b]);
  s.kc_start = t.kc_start != nullptr ? uniform(static_cast<int32_t>(t.kc_start[b])) : 0;
  return s;
}

// Sequence b owns count(b) consecutive work items, in sequence order.  locate() finds the
// sequence owning dense item `item` and the item's index within it; false once item is past
// the last sequence's items.  Every active lane of the calling wave must call it with the same
// item (a wave-wide prefix sum over as many sequences at a time as the wave has lanes; a
// partial wave, lanes 0 .. nl-1, works too); the results are wave-uniform.
template <typename F>
__device__ __forceinline__ bool locate(const SeqTable& t, int item, F count, int& b, int& local) {
  const int lane = threadIdx.x & 63;
  const int nl = 64 - __builtin_clzll(static_cast<unsigned long long>(__ballot(1)));
  int acc = 0;
  for (int base = 0; base < t.n; base += nl) {
    const int c = base + lane < t.n ? count(base + lane) : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int tot = uniform(__shfl(incl, nl - 1));
    if (item < acc + tot) {
      const int L = __ffsll(static_cast<unsigned long long>(__ballot(incl > item - acc))) - 1;
      b = uniform(base + L);
      local = uniform(item - acc - __shfl(incl - c, L));
      return true;
    }
    acc += tot;
  }
  return false;
}

// Total of count(b) over all sequences (same calling rule as locate).
template <typename F>
__device__ __forceinline__ int count_items(const SeqTable& t, F count) {
  const int lane = threadIdx.x & 63;
  const int nl = 64 - __builtin_clzll(static_cast<unsigned long long>(__ballot(1)));
  int acc = 0;
  for (int base = 0; base < t.n; base += nl) {
    int c = base + lane < t.n ? count(base + lane) : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(c, off);
      if (lane >= off) c += y;
    }
    acc += uniform(__shfl(c, nl - 1));
  }
  return acc;
}

// Host-side bounds on the number of work items of a launch (the grid), from the host bounds of
// the table: query rows, and tiles of `rows` query rows per sequence.
inline int bound_rows(const SeqTable& t) {
  const long long a = static_cast<long long>(t.n) * t.max_q_len;
  return static_cast<int>(a < t.q_rows ? a : t.q_rows);
}
inline int bound_tiles(const SeqTable& t, int rows) {
  const long long a = static_cast<long long>(t.n) * ((t.max_q_len + rows - 1) / rows);
  const long long c = (static_cast<long long>(t.q_rows) + rows - 1) / rows + t.n;
  return static_cast<int>(a < c ? a : c);
}
// Reachable blocks of the longest sequence (query positions are below max_kv_len).
__host__ __device__ inline int bound_blocks(const SeqTable& t, int B) {
  return t.max_kv_len > 0 ? (t.max_kv_len - 1) / B + 1 : 0;
}

struct Geom {
  int32_t Hq, Hkv, G, d;
  int32_t B, w, s;
  int32_t topk, n_init, n_local;
  float scale;
  int32_t window;       // sliding-window attention: keys pos - window < j <= pos (0 = unused)
  int32_t score_mode;   // 0: group sum of scaled dot products; 1: of per-head softmaxes
};

__host__ __device__ __forceinline__ int num_kernels(int len, int w, int s) {
  return len < w ? 0 : (len - w) / s + 1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float64 -> bf16 bits, round to nearest even, in one step (no float32 double rounding).
// Keeps sign, 11 exponent bits and 7 fraction bits of the binary64 encoding; the rounded
// binary64 value then converts exactly to float32, whose top half is the bf16 encoding.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const unsigned long long lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;            // 2^44 - 1 + lsb
  u &= ~((1ull << 45) - 1ull);
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// One semantic kernel's 8 consecutive bf16 columns: the mean of w key rows starting at p (row
// stride `rs` elements), summed in float64 in row order and rounded once to bf16.  Every
// kernel the library writes in bf16 comes from here (the compression launch and the decode
// step's scoring launch), so both write the same bits.
__device__ __forceinline__ uint4 window_mean_bf16x8(const uint16_t* __restrict__ p, size_t rs,
                                                   int w) {
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll 8
  for (int r = 0; r < w; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + static_cast<size_t>(r) * rs);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += static_cast<double>(__uint_as_float(w4[e] << 16));
      acc[2 * e + 1] += static_cast<double>(__uint_as_float(w4[e] & 0xFFFF0000u));
    }
  }
  const bool pow2 = (w & (w - 1)) == 0;
  const double inv_w = 1.0 / static_cast<double>(w);
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double m0 = pow2 ? acc[2 * e] * inv_w : acc[2 * e] / w;
    const double m1 = pow2 ? acc[2 * e + 1] * inv_w : acc[2 * e + 1] / w;
    o[e] = static_cast<uint32_t>(f64_to_bf16_rne(m0)) |
           (static_cast<uint32_t>(f64_to_bf16_rne(m1)) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
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

// The allocation-free decoding step's workspace: a file-scope device array (noalloc.hip) of this
// many bytes per GPU; noalloc_scratch() gives its device address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// Launch entry points (one per translation unit).  All return hipSuccess or the launch error.
hipError_t launch_compress(const Geom& g, int dtype, const SeqTable& t, const void* k,
                           void* kernels, hipStream_t stream);
hipError_t launch_scores(const Geom& g, int dtype, const SeqTable& t, const void* q,
                         const void* kernels, float* scores, int nb_stride, hipStream_t stream);
// Score mode 1 (per-head softmax over the visible kernels before the group sum).
bool scores_softmax_mfma_supported(const Geom& g, int dtype);
hipError_t launch_scores_softmax(const Geom& g, int dtype, const SeqTable& t, const void* q,
                                 const void* kernels, float* scores, int nb_stride,
                                 hipStream_t stream);
hipError_t launch_topk(const Geom& g, const SeqTable& t, const float* scores, int nb_stride,
                       int32_t* idx, hipStream_t stream);
// Attention over blocks idx[row, g, k0 .. k1) for split `sp` of `splits`.  With splits == 1
// the kernels write O and lse; otherwise they write partials to `part` and
// launch_attn_combine merges them.
hipError_t launch_attn(const Geom& g, int dtype, const SeqTable& t, const void* q,
                       const void* k, const void* v, const int32_t* idx, int splits,
                       void* out, float* lse, float* part, hipStream_t stream);
// Tiled prefill attention (tiles of consecutive query rows sharing staged K/V blocks).
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
// Whole backward (dq, dk, dv as float32).  KV blocks are numbered per sequence slot: block j of
// sequence b is global block b * bound_blocks(t, 64) + j.
size_t bwd_workspace(const Geom& g, const SeqTable& t);
long long bwd_segments(const Geom& g, const SeqTable& t);
hipError_t launch_attn_bwd(const Geom& g, const SeqTable& t, const void* q, const void* k,
                           const void* v, const int32_t* idx, const void* out, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, void* workspace,
                           hipStream_t stream);
// Split-KV decoding attention with the merge done by the last workgroup of each (row, kv head);
// its workspace follows decode_layout.
bool attn_decode_supported(const Geom& g, int dtype);
size_t decode_workspace(const Geom& g, int rows, int nsplit);
hipError_t launch_attn_decode(const Geom& g, const SeqTable& t, const void* q, const void* k,
                              const void* v, const int32_t* idx, int nsplit, void* workspace,
                              void* out, float* lse, hipStream_t stream);
// The fused decode step: block scores in one launch (decode_scores, which also computes and
// stores the kernels completed since t.prev_kv_len), then the split-KV attention in its
// selecting form (each split workgroup runs the pair's top-k itself; the first writes it out).
bool decode_step_supported(const Geom& g, int dtype, const SeqTable& t, int nsplit);
int decode_step_splits(const Geom& g, int rows);
hipError_t launch_decode_step(const Geom& g, const SeqTable& t, const void* q,
                               void* kernels, const void* k, const void* v, float* scores,
                               int nb_stride, int32_t* idx, int nsplit, void* workspace,
                               void* out, float* lse, hipStream_t stream);
hipError_t launch_attn_combine(const Geom& g, int dtype, const SeqTable& t, int splits,
                               const float* part, void* out, float* lse, hipStream_t stream);

}  // namespace infllm2
