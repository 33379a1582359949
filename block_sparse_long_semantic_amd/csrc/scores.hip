// Query-block relevance scores (MiniCPM4 paper summary, section 2.1.2: the relevance between
// query tokens and KV blocks, computed through semantic kernels, shared by one query-head
// group).  For a query at position i and KV head g:
//   u[c] = scale * (sum_{h in g} q[h]) . kernel[c]      for kernels whose last token <= i
//   S[b] = max over kernels overlapping block b of u[c]  (-inf if none is visible)
// Two implementations:
//   * scores_mfma  bf16, block 64 / window 32 / stride 16, d in {64, 128}.  The group-summed
//                  query (float32) is split into bf16 hi + lo parts and both are contracted
//                  with the bf16 kernels on v_mfma_f32_16x16x32_bf16 (A = 16 kernels x 32
//                  dims, B = 32 dims x 16 query rows).  The 4x4 output fragment a lane holds
//                  is exactly one block's four contained kernels for one query row; the
//                  fifth (halo) kernel 4b-1 comes from the neighbouring lane group.
//   * scores_simple any dtype and geometry, plain float32 dot products.
// Score mode 1 (the softmax-normalised reading of the same passage): each head's scaled dot
// products are turned into a softmax over the kernels the query can see before the group sum,
//   u[c] = sum_{h in g} exp(scale q[h] . kernel[c] - lse_h),  lse_h over the visible kernels,
// and S[b] is the max of u over the visible kernels overlapping b.  Per-head products cannot be
// pre-summed, so this runs as two passes over the kernels (lse, then u):
//   * scores_softmax_mfma  bf16, 64 / 32 / 16, d in {64, 128}, G in {8, 16}
//   * scores_softmax_simple any dtype and geometry.
#include <algorithm>

#include "dpp.h"
#include "internal.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ------------------------------------------------------------------------------ simple path
// One workgroup per (query row, KV head).
template <typename T>
__global__ void __launch_bounds__(kThreads)
scores_simple(Geom g, SeqTable t, const T* __restrict__ q, const T* __restrict__ kern,
              float* __restrict__ scores, int nb_stride) {
  __shared__ float qs[256];
  const int kvh = blockIdx.y;
  int b, j;
  if (!locate(t, static_cast<int>(blockIdx.x), [&](int s) { return t.q_len[s]; }, b, j)) return;
  const Seq sq = load_seq(t, b);
  const int row = sq.q_start + j;
  const int pos = sq.q_pos0 + j;
  for (int e = threadIdx.x; e < g.d; e += kThreads) {
    float acc = 0.f;
    for (int h = 0; h < g.G; ++h)
      acc += load_elem(q, (static_cast<size_t>(row) * g.Hq + kvh * g.G + h) * g.d + e);
    qs[e] = acc;
  }
  __syncthreads();
  const int C = num_kernels(sq.kv_len, g.w, g.s);
  const int nb = pos / g.B + 1;
  float* out = scores + (static_cast<size_t>(row) * g.Hkv + kvh) * nb_stride;
  for (int blk = threadIdx.x; blk < nb; blk += kThreads) {
    const int lo_num = g.B * blk - g.w + 1;
    const int lo = lo_num <= 0 ? 0 : (lo_num + g.s - 1) / g.s;
    const int hi = min(C, (g.B * (blk + 1) + g.s - 1) / g.s);
    float best = -INFINITY;
    for (int c = lo; c < hi; ++c) {
      if (g.s * c + g.w - 1 > pos) break;
      const size_t base = (static_cast<size_t>(sq.kc_start) + c) * g.Hkv * g.d +
                          static_cast<size_t>(kvh) * g.d;
      float dot = 0.f;
      for (int e = 0; e < g.d; ++e) dot += qs[e] * load_elem(kern, base + e);
      best = fmaxf(best, dot);
    }
    out[blk] = best * g.scale;
  }
}

// ------------------------------------------------------------------------------ MFMA path
// Work item = (sequence, tile of 64 query rows, KV head).  Every wave holds the group-summed
// queries of all 64 rows as MFMA B operands (4 row groups of 16; float32 sums split into hi and
// lo bf16 parts; wave w sums row group w and the groups are exchanged through LDS) and streams
// a quarter of the kernel tiles the rows can see (a kernel tile is 16 kernels = 4 blocks), so
// each kernel fragment it loads feeds 8 MFMAs.  Block scores are max-pooled in registers: a lane
// holds 4 consecutive kernels of one row, and the kernel before them (shared with the previous
// block) comes from the lane 16 below, or from the previous tile.  Each kernel tile's fragment
// is loaded while the previous tile's MFMAs run.  Scores are collected per wave in LDS for 16
// kernel tiles (64 blocks) and written out four blocks per lane, four rows per instruction.
constexpr int kChunkTiles = 16;                  // kernel tiles per staged chunk (64 blocks)
constexpr int kStageRow = 4 * kChunkTiles + 4;   // floats per staged row (16-byte rows)

template <int D>
__global__ void __launch_bounds__(kThreads)
scores_mfma(Geom g, SeqTable t, const uint16_t* __restrict__ q,
            const uint16_t* __restrict__ kern, float* __restrict__ scores, int nb_stride) {
  constexpr int KS = D / 32;
  constexpr int RG = 4;                                        // row groups of 16 per wave
  constexpr int QOP_BYTES = RG * KS * 2 * 64 * 16;             // exchanged B operands
  constexpr int STAGE_BYTES = 4 * 64 * kStageRow * 4;          // per-wave score staging
  __shared__ __attribute__((aligned(16))) unsigned char smem[QOP_BYTES > STAGE_BYTES ? QOP_BYTES : STAGE_BYTES];
  auto tiles64 = [&](int s) { return (t.q_len[s] + 63) / 64; };
  const int total = count_items(t, tiles64);
  const int item = total - 1 - static_cast<int>(blockIdx.x);   // heaviest (latest) rows first
  if (item < 0) return;
  const int kvh = blockIdx.y;
  int b, lt;
  locate(t, item, tiles64, b, lt);
  const Seq sq = load_seq(t, b);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int q_len = sq.q_len;
  const int r0 = lt * 64;
  const int r_last = min(r0 + 63, q_len - 1);
  const int nbt = ((sq.q_pos0 + r_last) / 64 + 1 + 3) / 4;  // kernel tiles of the last row
  const int per = (nbt + 3) / 4;
  const int t_begin = wave * per;
  const int t_end = min(nbt, t_begin + per);

  // ---- B operands: wave w sums row group w (rows r0 + 16w + c16, dims 32ks + 8q4 + 0..7)
  uint4* qop = reinterpret_cast<uint4*>(smem);                 // [rg][ks][hi/lo][lane]
  {
    const int r = r0 + 16 * wave + c16;
    const size_t row = static_cast<size_t>(sq.q_start) + (r < q_len ? r : q_len - 1);
#pragma unroll
    for (int ks2 = 0; ks2 < KS; ks2 += 2) {
      // every head of the group (at most 16) over two dimension slices is loaded before the
      // first addition, so a slice pair waits for one round trip; indices past the group repeat
      // its last head and are not added (the sum runs over the heads in order)
      const uint16_t* qrow = q + (row * g.Hq + kvh * g.G) * D + 32 * ks2 + 8 * q4;
      uint4 v[2][16];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int h = 0; h < 16; ++h)
          v[j][h] = *reinterpret_cast<const uint4*>(qrow + 32 * j +
                                                    static_cast<size_t>(min(h, g.G - 1)) * D);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = ks2 + j;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
          const uint32_t w4[4] = {v[j][h].x, v[j][h].y, v[j][h].z, v[j][h].w};
          if (h < g.G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] += __uint_as_float(w4[e] << 16);
              acc[2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
            }
          }
        }
        uint32_t hi4[4], lo4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t h0 = f32_to_bf16(acc[2 * e]), h1 = f32_to_bf16(acc[2 * e + 1]);
          const uint16_t l0 = f32_to_bf16(acc[2 * e] - bf16_to_f32(h0));
          const uint16_t l1 = f32_to_bf16(acc[2 * e + 1] - bf16_to_f32(h1));
          hi4[e] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
          lo4[e] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
        }
        qop[((wave * KS + ks) * 2 + 0) * 64 + lane] = make_uint4(hi4[0], hi4[1], hi4[2], hi4[3]);
        qop[((wave * KS + ks) * 2 + 1) * 64 + lane] = make_uint4(lo4[0], lo4[1], lo4[2], lo4[3]);
      }
    }
  }
  __syncthreads();
  bf16x8 bhi[RG][KS], blo[RG][KS];
  int pos[RG];
  bool row_ok[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int r = r0 + 16 * rg + c16;
    row_ok[rg] = r < q_len;
    pos[rg] = sq.q_pos0 + (row_ok[rg] ? r : q_len - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bhi[rg][ks] = __builtin_bit_cast(bf16x8, qop[((rg * KS + ks) * 2 + 0) * 64 + lane]);
      blo[rg][ks] = __builtin_bit_cast(bf16x8, qop[((rg * KS + ks) * 2 + 1) * 64 + lane]);
    }
  }
  __syncthreads();                                             // smem becomes score staging
  if (t_begin >= t_end) return;
  float* stage = reinterpret_cast<float*>(smem) + wave * 64 * kStageRow;   // [row][block]

  const int C = num_kernels(sq.kv_len, g.w, g.s);
  const size_t kbase = static_cast<size_t>(sq.kc_start) * g.Hkv * D + static_cast<size_t>(kvh) * D;
  const unsigned src_lane = static_cast<unsigned>((lane + 48) & 63);   // lane - 16 (mod 64)
  // whole float4 stores need 16-byte aligned output rows
  const bool vec_out = (nb_stride & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  float carry[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) carry[rg] = -INFINITY;
  // A operands of kernel tile tt (16 kernels x D dims; kernel index clamped into the sequence)
  auto load_tile = [&](int tt, bf16x8 (&a)[KS]) {
    const int ck_c = min(16 * tt + c16, C - 1 > 0 ? C - 1 : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[ks] = C > 0 ? *reinterpret_cast<const bf16x8*>(kern + kbase +
                                                      static_cast<size_t>(ck_c) * g.Hkv * D +
                                                      32 * ks + 8 * q4)
                    : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  };
  bf16x8 a_next[KS];                     // the next tile's operands, loaded one tile ahead
  load_tile(t_begin > 0 ? t_begin - 1 : t_begin, a_next);
  for (int c0 = t_begin; c0 < t_end; c0 += kChunkTiles) {
    const int c1 = min(t_end, c0 + kChunkTiles);
    // the first chunk starts one tile early (not staged) for the halo kernel of its first block
    for (int tt = (c0 == t_begin && t_begin > 0) ? t_begin - 1 : c0; tt < c1; ++tt) {
      bf16x8 a[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[ks] = a_next[ks];
      if (tt + 1 < t_end) load_tile(tt + 1, a_next);
      f32x4 acc[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bhi[rg][ks], acc[rg], 0, 0, 0);
          acc[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], blo[rg][ks], acc[rg], 0, 0, 0);
        }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        // lane holds u[kernel 16*tt + 4*q4 + i][row 16*rg + c16]
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 16 * tt + 4 * q4 + i;
          u[i] = (c < C && 16 * c + 31 <= pos[rg]) ? acc[rg][i] : -INFINITY;
        }
        const float h = __shfl(u[3], src_lane);
        const float halo = (q4 == 0) ? carry[rg] : h;
        carry[rg] = h;
        const float best = fmaxf(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])), halo);
        if (tt >= c0) stage[(16 * rg + c16) * kStageRow + 4 * (tt - c0) + q4] = best * g.scale;
      }
    }
    asm volatile("" ::: "memory");
    // write the chunk: four rows per instruction, four consecutive blocks per lane (blocks
    // 4*c0 .. 4*c1 - 1, up to the row's own block)
    const int j4 = 4 * c16;
    const int blk = 4 * c0 + j4;
    for (int rr0 = 0; rr0 < 64 && r0 + rr0 < q_len; rr0 += 4) {
      const int rr = rr0 + q4;
      const int r = r0 + rr;
      const int own = (sq.q_pos0 + r) / 64;
      if (r < q_len && j4 < 4 * (c1 - c0) && blk <= own) {
        const float4 s4 = *reinterpret_cast<const float4*>(stage + rr * kStageRow + j4);
        float* dst = scores + (static_cast<size_t>(sq.q_start) + r) * g.Hkv * nb_stride +
                     static_cast<size_t>(kvh) * nb_stride + blk;
        if (vec_out && blk + 3 <= own) {
          *reinterpret_cast<float4*>(dst) = s4;
        } else {
          dst[0] = s4.x;
          if (blk + 1 <= own) dst[1] = s4.y;
          if (blk + 2 <= own) dst[2] = s4.z;
          if (blk + 3 <= own) dst[3] = s4.w;
        }
      }
    }
    asm volatile("" ::: "memory");
  }
}


// ------------------------------------------------------------------------------ decode path
// Few query rows (decoding): the work is streaming every semantic kernel of the sequence once,
// so it is spread over chunks of 64 blocks (256 kernels + the halo kernel before them) per
// workgroup.  The group-summed query stays in float32; each kernel row is read by D/8 lanes
// (16 bytes each, one coalesced row per lane group), dotted with float32 FMAs and reduced across
// the lanes by DPP moves.  Kernel scores go to LDS, then 64 threads max-pool them onto the chunk's
// blocks and write one coalesced row segment.
template <int D>
__global__ void __launch_bounds__(kThreads)
scores_decode(Geom g, SeqTable t, const uint16_t* __restrict__ q,
              const uint16_t* __restrict__ kern, float* __restrict__ scores, int nb_stride) {
  constexpr int LPR = D / 8;              // lanes per kernel row
  constexpr int RPI = 64 / LPR;           // rows per wave instruction
  constexpr int NROW = 257;               // kernels c0-1 .. c0+255
  __shared__ float qs[D];
  __shared__ float u[NROW + 3];
  const int chunk = blockIdx.x;
  const int kvh = blockIdx.y;
  int b, j;
  if (!locate(t, static_cast<int>(blockIdx.z), [&](int s) { return t.q_len[s]; }, b, j)) return;
  const Seq sq = load_seq(t, b);
  const int row = sq.q_start + j;
  const int pos = sq.q_pos0 + j;
  const int own = pos / 64;
  const int blk0 = chunk * 64;
  if (blk0 > own) return;                 // whole workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int C = num_kernels(sq.kv_len, g.w, g.s);
  const int c0 = 4 * blk0;
  const int col = (lane % LPR) * 8;
  const size_t kbase = static_cast<size_t>(sq.kc_start) * g.Hkv * D + static_cast<size_t>(kvh) * D;
  constexpr int NIT = (NROW + RPI - 1) / RPI;
  constexpr int NW = kThreads / 64;
  constexpr int PER = (NIT + NW - 1) / NW;                // row groups per wave
  // the kernel rows do not depend on the query: every load is issued before the query sum
  uint4 kv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = w + NW * i;
    const int r = it * RPI + lane / LPR;                   // 0 .. NROW-1 (+ padding)
    const int c = c0 - 1 + r;
    const bool ok = it < NIT && r < NROW && c >= 0 && c < C && 16 * c + 31 <= pos;
    kv[i] = ok ? *reinterpret_cast<const uint4*>(kern + kbase + static_cast<size_t>(c) * g.Hkv * D + col)
               : make_uint4(0u, 0u, 0u, 0u);
  }
  for (int e = tid; e < D; e += kThreads) {
    float acc = 0.f;
    for (int h0 = 0; h0 < g.G; h0 += 16) {
      float qh[16];                                     // 16 heads' loads in flight at once
#pragma unroll
      for (int j = 0; j < 16; ++j)
        qh[j] = bf16_to_f32(q[(static_cast<size_t>(row) * g.Hq + kvh * g.G + min(h0 + j, g.G - 1)) * D + e]);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (h0 + j < g.G) acc += qh[j];
    }
    qs[e] = acc;
  }
  __syncthreads();
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[col + e];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = w + NW * i;
    const int r = it * RPI + lane / LPR;
    const int c = c0 - 1 + r;
    const bool ok = it < NIT && r < NROW && c >= 0 && c < C && 16 * c + 31 <= pos;
    const uint32_t w4[4] = {kv[i].x, kv[i].y, kv[i].z, kv[i].w};
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot = fmaf(__uint_as_float(w4[e] << 16), qv[2 * e], dot);
      dot = fmaf(__uint_as_float(w4[e] & 0xFFFF0000u), qv[2 * e + 1], dot);
    }
    dot = group_sum<LPR>(dot);
    if (lane % LPR == 0 && it < NIT && r < NROW) u[r] = ok ? dot : -INFINITY;
  }
  __syncthreads();
  if (tid < 64) {
    const int blk = blk0 + tid;
    if (blk <= own) {
      // block blk's kernels 4blk-1 .. 4blk+3 sit at u[4*tid .. 4*tid+4]
      float best = u[4 * tid];
#pragma unroll
      for (int e = 1; e < 5; ++e) best = fmaxf(best, u[4 * tid + e]);
      scores[(static_cast<size_t>(row) * g.Hkv + kvh) * nb_stride + blk] = best * g.scale;
    }
  }
}


// ------------------------------------------------------------------------------ score mode 1
constexpr float kLog2eS = 1.4426950408889634f;
constexpr float kLazyS = 8.f;        // log2 headroom before a running max is moved

// One workgroup per (query row, KV head).  Thread-strided over
// the visible kernels: per head, a block-wide max and sum give lse; then every thread takes
// whole blocks and sums the heads' probabilities of their overlapping kernels.
template <typename T>
__global__ void __launch_bounds__(kThreads)
scores_softmax_simple(Geom g, SeqTable t, const T* __restrict__ q, const T* __restrict__ kern,
                      float* __restrict__ scores, int nb_stride) {
  __shared__ float qh[16][256];
  __shared__ float lse[16];
  __shared__ float red[kThreads / 64];
  const int kvh = blockIdx.y;
  int b, j;
  if (!locate(t, static_cast<int>(blockIdx.x), [&](int s) { return t.q_len[s]; }, b, j)) return;
  const Seq sq = load_seq(t, b);
  const int row = sq.q_start + j;
  const int pos = sq.q_pos0 + j;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < g.G * g.d; e += kThreads)
    qh[e / g.d][e % g.d] = load_elem(q, (static_cast<size_t>(row) * g.Hq + kvh * g.G) * g.d + e);
  __syncthreads();
  const int C = num_kernels(sq.kv_len, g.w, g.s);
  const int nvis = pos - g.w + 1 < 0 ? 0 : min(C, (pos - g.w + 1) / g.s + 1);
  const size_t kbase = static_cast<size_t>(sq.kc_start) * g.Hkv * g.d + static_cast<size_t>(kvh) * g.d;
  auto dot = [&](int h, int c) {
    float acc = 0.f;
    const size_t base = kbase + static_cast<size_t>(c) * g.Hkv * g.d;
    for (int e = 0; e < g.d; ++e) acc += qh[h][e] * load_elem(kern, base + e);
    return acc * g.scale;
  };
  for (int h = 0; h < g.G; ++h) {
    float m = -INFINITY;
    for (int c = tid; c < nvis; c += kThreads) m = fmaxf(m, dot(h, c));
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) red[w] = m;
    __syncthreads();
    m = red[0];
    for (int ww = 1; ww < kThreads / 64; ++ww) m = fmaxf(m, red[ww]);
    __syncthreads();
    float sum = 0.f;
    for (int c = tid; c < nvis; c += kThreads) sum += expf(dot(h, c) - m);
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) red[w] = sum;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int ww = 0; ww < kThreads / 64; ++ww) tot += red[ww];
      lse[h] = m + logf(tot);
    }
    __syncthreads();
  }
  const int nb = pos / g.B + 1;
  float* out = scores + (static_cast<size_t>(row) * g.Hkv + kvh) * nb_stride;
  for (int blk = tid; blk < nb; blk += kThreads) {
    const int lo_num = g.B * blk - g.w + 1;
    const int lo = lo_num <= 0 ? 0 : (lo_num + g.s - 1) / g.s;
    const int hi = min(nvis, (g.B * (blk + 1) + g.s - 1) / g.s);
    float best = -INFINITY;
    for (int c = lo; c < hi; ++c) {
      float u = 0.f;
      for (int h = 0; h < g.G; ++h) u += expf(dot(h, c) - lse[h]);
      best = fmaxf(best, u);
    }
    out[blk] = best;
  }
}

// Work item = rows of one sequence x one KV head.  A wave holds NCT column tiles of 16
// (row, head) columns as MFMA A operands (its queries, 16 heads of one row or 8 heads of two)
// and streams kernel tiles of 16 as B operands from L2 (v_mfma_f32_16x16x32_bf16), so a lane's
// accumulator holds 4 heads of one row against one kernel.  Pass 1 keeps, per column, a running
// max (moved lazily, by ballot) and sum of exp2; the 16 kernel lanes are then merged, giving
// each head's lse.  Pass 2 recomputes the products, turns them into probabilities, sums the
// group's heads (4 in the lane, the rest across the 16-lane rows by the gfx950 row swaps) and
// max-pools kernels onto blocks (a block is the 4 kernels of a lane quad, by DPP quad moves,
// plus the one before, from the neighbouring lane by a DPP row rotation or from the previous
// tile).  SPLIT (few rows, e.g. decoding): every wave holds the same columns and takes a
// quarter of the kernel tiles; the waves' partial maxima and sums are merged through LDS.
template <int D, int G, bool SPLIT>
__global__ void __launch_bounds__(kThreads)
scores_softmax_mfma(Geom g, SeqTable t, const uint16_t* __restrict__ q,
                    const uint16_t* __restrict__ kern, float* __restrict__ scores,
                    int nb_stride) {
  constexpr int KS = D / 32;
  constexpr int NCT = 4;                          // column tiles per wave
  constexpr int RPC = 16 / G;                     // rows per column tile
  constexpr int RPW = NCT * RPC;                  // rows per wave
  constexpr int ROWS = SPLIT ? RPW : 4 * RPW;     // rows per work item
  __shared__ float xm[4][NCT][4][4][2];           // SPLIT: [wave][ct][q4][i][m, l]
  auto tiles_of = [&](int s) { return (t.q_len[s] + ROWS - 1) / ROWS; };
  const int total = count_items(t, tiles_of);
  const int item = total - 1 - static_cast<int>(blockIdx.x);   // latest rows first
  if (item < 0) return;
  const int kvh = blockIdx.y;
  int b, lt;
  locate(t, item, tiles_of, b, lt);
  const Seq sq = load_seq(t, b);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int q_len = sq.q_len;
  const int r0 = lt * ROWS;
  const int r_last = min(r0 + ROWS - 1, q_len - 1);
  const int own_last = (sq.q_pos0 + r_last) / 64;
  const int nt = (own_last + 1 + 3) / 4;                        // kernel tiles (4 blocks each)
  const int C = num_kernels(sq.kv_len, g.w, g.s);
  const size_t kbase = static_cast<size_t>(sq.kc_start) * g.Hkv * D + static_cast<size_t>(kvh) * D;
  const float qscale = g.scale * kLog2eS;
  const int wrow0 = r0 + (SPLIT ? 0 : wave * RPW);              // first row of the wave

  // A operands: column c16 of tile ct = row wrow0 + ct*RPC + c16/G, head c16 % G
  bf16x8 aq[NCT][KS];
  int pos_l[NCT];          // position of the row of the lane's accumulator columns (4q4..4q4+3)
  bool row_ok[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int ra = wrow0 + ct * RPC + c16 / G;
    const size_t rowa = static_cast<size_t>(sq.q_start) + min(ra, q_len - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      aq[ct][ks] = *reinterpret_cast<const bf16x8*>(
          q + (rowa * g.Hq + kvh * G + c16 % G) * D + 32 * ks + 8 * q4);
    const int rc = wrow0 + ct * RPC + (4 * q4) / G;
    row_ok[ct] = rc < q_len;
    pos_l[ct] = sq.q_pos0 + min(rc, q_len - 1);
  }
  int t_begin = 0, t_end = nt;
  if constexpr (SPLIT) {
    const int per = (nt + 3) / 4;
    t_begin = min(nt, wave * per);
    t_end = min(nt, t_begin + per);
  }
  auto load_b = [&](int tt, bf16x8 (&kb)[KS]) {
    const int c = min(16 * tt + c16, C > 0 ? C - 1 : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kb[ks] = C > 0 ? *reinterpret_cast<const bf16x8*>(kern + kbase + static_cast<size_t>(c) * g.Hkv * D +
                                                       32 * ks + 8 * q4)
                     : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  };
  auto visible = [&](int c, int pos) { return c < C && g.s * c + g.w - 1 <= pos; };

  // ---- pass 1: per column, max and sum of exp2 over the visible kernels
  float m[NCT][4], l[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[ct][i] = -INFINITY;
      l[ct][i] = 0.f;
    }
  if (t_begin < t_end) {
    bf16x8 kb[KS];
    load_b(t_begin, kb);
    for (int tt = t_begin; tt < t_end; ++tt) {
      bf16x8 kn[KS];
      load_b(min(tt + 1, t_end - 1), kn);
      const int c = 16 * tt + c16;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ct][ks], kb[ks], acc, 0, 0, 0);
        const bool vis = visible(c, pos_l[ct]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = vis ? acc[i] * qscale : -INFINITY;
          if (__ballot(x > m[ct][i] + kLazyS) != 0ull) {
            const float mn = fmaxf(m[ct][i], x);
            l[ct][i] *= mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[ct][i] - mn);
            m[ct][i] = mn;
          }
          if (vis) l[ct][i] += __builtin_amdgcn_exp2f(x - m[ct][i]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[ks] = kn[ks];
    }
  }
  // merge the 16 kernel lanes of every column (and, SPLIT, the 4 waves)
  auto merge = [](float& ma, float& la, float mb, float lb) {
    const float mn = fmaxf(ma, mb);
    if (mn == -INFINITY) return;
    la = la * __builtin_amdgcn_exp2f(ma - mn) + lb * __builtin_amdgcn_exp2f(mb - mn);
    ma = mn;
  };
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float mo = __shfl_xor(m[ct][i], off);
        const float lo = __shfl_xor(l[ct][i], off);
        merge(m[ct][i], l[ct][i], mo, lo);
      }
  if constexpr (SPLIT) {
    if (c16 == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xm[wave][ct][q4][i][0] = m[ct][i];
          xm[wave][ct][q4][i][1] = l[ct][i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mm = -INFINITY, ll = 0.f;
        for (int ww = 0; ww < 4; ++ww) merge(mm, ll, xm[ww][ct][q4][i][0], xm[ww][ct][q4][i][1]);
        m[ct][i] = mm;
        l[ct][i] = ll;
      }
  }
  float lse2[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) lse2[ct][i] = l[ct][i] > 0.f ? m[ct][i] + log2f(l[ct][i]) : INFINITY;

  // ---- pass 2: probabilities, group sum, block max-pool
  // with SPLIT a wave starts one tile early (not written) for its first block's halo kernel
  const int t_first = (SPLIT && t_begin > 0) ? t_begin - 1 : t_begin;
  if (t_first >= t_end) return;
  float carry[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) carry[ct] = -INFINITY;
  bf16x8 kb[KS];
  load_b(t_first, kb);
  for (int tt = t_first; tt < t_end; ++tt) {
    bf16x8 kn[KS];
    load_b(min(tt + 1, t_end - 1), kn);
    const int c = 16 * tt + c16;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ct][ks], kb[ks], acc, 0, 0, 0);
      const bool vis = visible(c, pos_l[ct]);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sum += vis ? __builtin_amdgcn_exp2f(acc[i] * qscale - lse2[ct][i]) : 0.f;
      sum = xor16_sum(sum);                                       // heads of 8 (G = 8: a row)
      if constexpr (G == 16) sum = xor32_sum(sum);                // all 16 heads
      const float u = vis ? sum : -INFINITY;
      float qm = fmaxf(u, dpp_f32<kDppXor1>(u));
      qm = fmaxf(qm, dpp_f32<kDppXor2>(qm));
      // lane c16 takes kernel c16 - 1 of the tile; lane 0 gets kernel 15 of this tile, which is
      // its previous kernel in the next tile (carried)
      const float prev = dpp_f32<kDppRowRor1>(u);
      const float best = fmaxf(qm, c16 == 0 ? carry[ct] : prev);
      carry[ct] = prev;
      const int blk = 4 * tt + c16 / 4;
      const bool writer = (c16 & 3) == 0 && (G == 16 ? q4 == 0 : (q4 & 1) == 0);
      if (writer && tt >= t_begin && row_ok[ct] && blk <= pos_l[ct] / 64) {
        const int rc = wrow0 + ct * RPC + (4 * q4) / G;
        scores[(static_cast<size_t>(sq.q_start) + rc) * g.Hkv * nb_stride +
               static_cast<size_t>(kvh) * nb_stride + blk] = best;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = kn[ks];
  }
}

}  // namespace

bool scores_softmax_mfma_supported(const Geom& g, int dtype) {
  return dtype == INFLLM2_BF16 && g.B == 64 && g.w == 32 && g.s == 16 && (g.d == 64 || g.d == 128) &&
         (g.G == 8 || g.G == 16);
}

int scores_softmax_rows(const Geom& g, bool split) { return (split ? 64 : 256) / g.G; }

// Score mode 1: one workgroup per query row (generic path) or per tile of
// scores_softmax_rows(g, split) rows (matrix cores; the split form when the tiles of the full
// form would not fill the GPU).
hipError_t launch_scores_softmax(const Geom& g, int dtype, const SeqTable& t, const void* q,
                                 const void* kernels, float* scores, int nb_stride,
                                 hipStream_t stream) {
  if (!scores_softmax_mfma_supported(g, dtype)) {
    const int rows = bound_rows(t);
    if (rows == 0) return hipSuccess;
    if (g.G > 16 || g.d > 256) return hipErrorInvalidValue;
    const dim3 grid(rows, g.Hkv);
    if (dtype == INFLLM2_BF16)
      hipLaunchKernelGGL(scores_softmax_simple<uint16_t>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kernels),
                         scores, nb_stride);
    else
      hipLaunchKernelGGL(scores_softmax_simple<float>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const float*>(q), static_cast<const float*>(kernels), scores,
                         nb_stride);
    return hipGetLastError();
  }
  const bool split = static_cast<long long>(bound_tiles(t, scores_softmax_rows(g, false))) * g.Hkv < 128;
  const int items = bound_tiles(t, scores_softmax_rows(g, split));
  if (items == 0) return hipSuccess;
  const dim3 grid(items, g.Hkv);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kernels);
#define INFLLM2_SOFTMAX_CASE(DD, GG)                                                            \
  if (g.d == DD && g.G == GG) {                                                                 \
    if (split)                                                                                  \
      hipLaunchKernelGGL((scores_softmax_mfma<DD, GG, true>), grid, dim3(kThreads), 0, stream, g, \
                         t, qq, kk, scores, nb_stride);                                         \
    else                                                                                        \
      hipLaunchKernelGGL((scores_softmax_mfma<DD, GG, false>), grid, dim3(kThreads), 0, stream,   \
                         g, t, qq, kk, scores, nb_stride);                                      \
    return hipGetLastError();                                                                   \
  }
  INFLLM2_SOFTMAX_CASE(128, 16)
  INFLLM2_SOFTMAX_CASE(128, 8)
  INFLLM2_SOFTMAX_CASE(64, 16)
  INFLLM2_SOFTMAX_CASE(64, 8)
#undef INFLLM2_SOFTMAX_CASE
  return hipErrorInvalidValue;
}

// Score mode 0: generic path one workgroup per (query row, KV head); matrix cores either per
// tile of 64 rows, or, when those tiles would not fill the GPU (decoding), per (64-block chunk,
// KV head, row).
hipError_t launch_scores(const Geom& g, int dtype, const SeqTable& t, const void* q,
                         const void* kernels, float* scores, int nb_stride, hipStream_t stream) {
  const bool mfma = dtype == INFLLM2_BF16 && g.B == 64 && g.w == 32 && g.s == 16 &&
                    (g.d == 64 || g.d == 128);
  if (!mfma) {
    const int rows = bound_rows(t);
    if (rows == 0) return hipSuccess;
    const dim3 grid(rows, g.Hkv);
    if (dtype == INFLLM2_BF16)
      hipLaunchKernelGGL(scores_simple<uint16_t>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kernels),
                         scores, nb_stride);
    else
      hipLaunchKernelGGL(scores_simple<float>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const float*>(q), static_cast<const float*>(kernels), scores,
                         nb_stride);
    return hipGetLastError();
  }
  const int items = bound_tiles(t, 64);
  if (items == 0) return hipSuccess;
  if (static_cast<long long>(items) * g.Hkv < 512) {
    const int rows = bound_rows(t);
    const dim3 grid((bound_blocks(t, 64) + 63) / 64, g.Hkv, rows);
    if (g.d == 128)
      hipLaunchKernelGGL(scores_decode<128>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kernels),
                         scores, nb_stride);
    else
      hipLaunchKernelGGL(scores_decode<64>, grid, dim3(kThreads), 0, stream, g, t,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kernels),
                         scores, nb_stride);
    return hipGetLastError();
  }
  const dim3 grid(items, g.Hkv);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(kernels);
  if (g.d == 128)
    hipLaunchKernelGGL(scores_mfma<128>, grid, dim3(kThreads), 0, stream, g, t, qq, kk, scores,
                       nb_stride);
  else
    hipLaunchKernelGGL(scores_mfma<64>, grid, dim3(kThreads), 0, stream, g, t, qq, kk, scores,
                       nb_stride);
  return hipGetLastError();
}

}  // namespace infllm2
