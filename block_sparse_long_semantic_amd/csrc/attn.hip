// Block-sparse attention over the selected KV blocks (MiniCPM4 paper summary, section 2.1.3:
// each token computes attention only with its most relevant KV blocks; arXiv abstract: used
// for both prefilling and decoding), with FlashAttention-style online softmax (the technique
// of "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness", cited by
// the paper).
//
//   attn_mfma     bf16, block 64, d in {64, 128}, group size 8 or 16.  The G query heads of a
//                 GQA group share the block list, so they are stacked as the 16-wide MFMA
//                 dimension (group 8 is padded).  Per selected block the wave computes
//                 S^T = K Q^T (16 keys x 16 heads per v_mfma_f32_16x16x32_bf16) and then
//                 O += P V (16 heads x 16 dims).  The key order inside each 32-key step is
//                 permuted so that the S^T fragment a lane holds is directly the P operand
//                 of the second product: no cross-lane shuffle of probabilities.  K is
//                 staged in LDS row-major (padded rows) and V transposed (key-contiguous).
//   attn_simple   any dtype / shape: float32 CUDA-core style reference path.
//   combine       log-sum-exp merge of split-KV partials (decode).
#include "internal.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The query row of dense work item `item` (query rows counted over the sequences in order);
// false past the last row.  Every lane of the calling wave must call it.  Split-KV partials are
// indexed by the query row itself (vrow == row).
struct RowInfo {
  int vrow, row, pos, kv0, kv_len;
};

__device__ __forceinline__ bool row_info(const SeqTable& t, int item, RowInfo& r) {
  int b, j;
  if (!locate(t, item, [&](int s) { return t.q_len[s]; }, b, j)) return false;
  const Seq sq = load_seq(t, b);
  r.row = sq.q_start + j;
  r.vrow = r.row;
  r.pos = sq.q_pos0 + j;
  r.kv0 = sq.kv_start;
  r.kv_len = sq.kv_len;
  return true;
}

// Number of valid (non -1) entries of an ascending, -1 padded index row.
__device__ __forceinline__ int count_selected(const int32_t* sel, int topk) {
  int lo = 0, hi = topk;        // first -1 by bisection (entries are >= 0 then -1)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sel[mid] >= 0) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Partials layout (split-KV): ml[(vrow*Hq + h)*splits + sp] = {m (log2 units), l}, and
// o[((vrow*Hq + h)*splits + sp)*d + e] = unnormalised output.
struct Partials {
  float* ml;
  float* o;
};

__device__ __forceinline__ Partials partials_of(float* part, const Geom& g, int total_rows,
                                                int splits) {
  Partials p;
  p.ml = part;
  p.o = part + static_cast<size_t>(total_rows) * g.Hq * splits * 2;
  return p;
}

// ------------------------------------------------------------------------------ simple path
template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float x) {
  p[i] = f32_to_bf16(x);
}

constexpr int kSimpleThreads = 256;
constexpr int kSimpleMaxItems = 16;   // (G*d) / 256 output elements per thread

template <typename T>
__global__ void __launch_bounds__(kSimpleThreads)
attn_simple(Geom g, SeqTable t, const T* __restrict__ q, const T* __restrict__ k,
            const T* __restrict__ v, const int32_t* __restrict__ idx, int splits,
            T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part) {
  __shared__ float qs[4096];
  __shared__ float z[16 * 64];
  __shared__ float m_s[16], l_s[16], a_s[16];
  RowInfo ri;
  if (!row_info(t, static_cast<int>(blockIdx.x), ri)) return;
  const int kvh = blockIdx.y;
  const int sp = blockIdx.z;
  const int G = g.G, d = g.d;
  const float qscale = g.scale * kLog2e;
  for (int e = threadIdx.x; e < G * d; e += kSimpleThreads)
    qs[e] = ld(q, (static_cast<size_t>(ri.row) * g.Hq + kvh * G) * d + e) * qscale;
  if (threadIdx.x < G) {
    m_s[threadIdx.x] = -INFINITY;
    l_s[threadIdx.x] = 0.f;
  }
  float acc[kSimpleMaxItems];
#pragma unroll
  for (int i = 0; i < kSimpleMaxItems; ++i) acc[i] = 0.f;
  const int32_t* sel = idx + (static_cast<size_t>(ri.row) * g.Hkv + kvh) * g.topk;
  const int nsel = count_selected(sel, g.topk);
  const int k0 = static_cast<int>(static_cast<long long>(sp) * nsel / splits);
  const int k1 = static_cast<int>(static_cast<long long>(sp + 1) * nsel / splits);
  __syncthreads();
  for (int kk = k0; kk < k1; ++kk) {
    const int blk = sel[kk];
    const int j_end = min(min((blk + 1) * g.B, ri.kv_len), ri.pos + 1);
    for (int jc = blk * g.B; jc < j_end; jc += 64) {
      const int nk = min(64, j_end - jc);
      for (int pr = threadIdx.x; pr < G * 64; pr += kSimpleThreads) {
        const int h = pr / 64, jj = pr % 64;
        float dot = -INFINITY;
        if (jj < nk) {
          const size_t kb = (static_cast<size_t>(ri.kv0 + jc + jj) * g.Hkv + kvh) * d;
          dot = 0.f;
          for (int e = 0; e < d; ++e) dot += qs[h * d + e] * ld(k, kb + e);
        }
        z[pr] = dot;
      }
      __syncthreads();
      if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float mx = -INFINITY;
        for (int jj = 0; jj < nk; ++jj) mx = fmaxf(mx, z[h * 64 + jj]);
        const float m_new = fmaxf(m_s[h], mx);
        const float alpha = exp2f(m_s[h] - m_new);
        float sum = 0.f;
        for (int jj = 0; jj < 64; ++jj) {
          const float p = jj < nk ? exp2f(z[h * 64 + jj] - m_new) : 0.f;
          z[h * 64 + jj] = p;
          sum += p;
        }
        l_s[h] = l_s[h] * alpha + sum;
        m_s[h] = m_new;
        a_s[h] = alpha;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSimpleMaxItems; ++i) {
        const int it = threadIdx.x + i * kSimpleThreads;
        if (it < G * d) {
          const int h = it / d, e = it % d;
          float o = acc[i] * a_s[h];
          for (int jj = 0; jj < nk; ++jj)
            o += z[h * 64 + jj] * ld(v, (static_cast<size_t>(ri.kv0 + jc + jj) * g.Hkv + kvh) * d + e);
          acc[i] = o;
        }
      }
      __syncthreads();
    }
  }
  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < kSimpleMaxItems; ++i) {
      const int it = threadIdx.x + i * kSimpleThreads;
      if (it < G * d) {
        const int h = it / d, e = it % d;
        st(out, (static_cast<size_t>(ri.row) * g.Hq + kvh * G + h) * d + e, acc[i] / l_s[h]);
      }
    }
    if (lse != nullptr && threadIdx.x < G)
      lse[static_cast<size_t>(ri.row) * g.Hq + kvh * G + threadIdx.x] =
          (m_s[threadIdx.x] + log2f(l_s[threadIdx.x])) * kLn2;
  } else {
    const Partials pp = partials_of(part, g, t.q_rows, splits);
#pragma unroll
    for (int i = 0; i < kSimpleMaxItems; ++i) {
      const int it = threadIdx.x + i * kSimpleThreads;
      if (it < G * d) {
        const int h = it / d, e = it % d;
        const size_t slot = (static_cast<size_t>(ri.vrow) * g.Hq + kvh * G + h) * splits + sp;
        pp.o[slot * d + e] = acc[i];
      }
    }
    if (threadIdx.x < G) {
      const size_t slot =
          (static_cast<size_t>(ri.vrow) * g.Hq + kvh * G + threadIdx.x) * splits + sp;
      pp.ml[2 * slot] = m_s[threadIdx.x];
      pp.ml[2 * slot + 1] = l_s[threadIdx.x];
    }
  }
}

// ------------------------------------------------------------------------------ MFMA path
// One wave per (query row, KV head, split).
template <int D, int G>
__global__ void __launch_bounds__(64)
attn_mfma(Geom g, SeqTable t, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
          const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int splits,
          uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part) {
  constexpr int KS = D / 32;        // 32-dim steps of Q.K
  constexpr int NT = D / 16;        // 16-dim output tiles
  constexpr int KP = D + 8;         // padded K row in LDS (elements)
  constexpr int VP = 64 + 8;        // padded V^T row in LDS (elements)
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  RowInfo ri;
  if (!row_info(t, static_cast<int>(blockIdx.x), ri)) return;
  const int kvh = blockIdx.y;
  const int sp = blockIdx.z;
  const int lane = threadIdx.x;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int Hq = g.Hq, Hkv = g.Hkv;

  // Q^T operand: column = head c16, dims 32*ks + 8*q4 .. +7
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (c16 < G)
      qf[ks] = *reinterpret_cast<const bf16x8*>(
          q + (static_cast<size_t>(ri.row) * Hq + kvh * G + c16) * D + 32 * ks + 8 * q4);
    else
      qf[ks] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;      // for head c16, log2 units
  const float qscale = g.scale * kLog2e;

  const int32_t* sel = idx + (static_cast<size_t>(ri.row) * Hkv + kvh) * g.topk;
  const int nsel = count_selected(sel, g.topk);
  const int k0 = static_cast<int>(static_cast<long long>(sp) * nsel / splits);
  const int k1 = static_cast<int>(static_cast<long long>(sp + 1) * nsel / splits);

  for (int kk = k0; kk < k1; ++kk) {
    const int blk = sel[kk];
    const int key0 = blk * 64;
    __syncthreads();
    // stage K (row-major) and V (transposed) of this block for KV head kvh
    for (int c = lane; c < 64 * CPR; c += 64) {
      const int r = c / CPR, cc = c % CPR;
      const int src = ri.kv0 + min(key0 + r, ri.kv_len - 1);
      const uint4 kv = *reinterpret_cast<const uint4*>(
          k + (static_cast<size_t>(src) * Hkv + kvh) * D + 8 * cc);
      *reinterpret_cast<uint4*>(&Ks[r * KP + 8 * cc]) = kv;
    }
    for (int c = lane; c < 64 * CPR; c += 64) {
      const int r = c % 64, cc = c / 64;
      const int src = ri.kv0 + min(key0 + r, ri.kv_len - 1);
      const uint4 vv = *reinterpret_cast<const uint4*>(
          v + (static_cast<size_t>(src) * Hkv + kvh) * D + 8 * cc);
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(8 * cc + 2 * e) * VP + r] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
        Vt[(8 * cc + 2 * e + 1) * VP + r] = static_cast<uint16_t>(w4[e] >> 16);
      }
    }
    __syncthreads();

    // S^T: tile (s, tp) row r -> key 32*s + 8*(r/4) + 4*tp + (r%4); the lane then holds keys
    // 32*s + 8*q4 + 4*tp + i (i = 0..3) for head c16.
    float sv[2][2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        const int key_r = 32 * s + 8 * (c16 >> 2) + 4 * tp + (c16 & 3);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[key_r * KP + 32 * ks + 8 * q4]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kp = key0 + 32 * s + 8 * q4 + 4 * tp + i;     // key position
          sv[s][tp][i] = (kp <= ri.pos && kp < ri.kv_len) ? acc[i] * qscale : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[s][tp][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(sv[s][tp][i] - m_new);
          sv[s][tp][i] = p;
          psum += p;
        }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale O rows (heads 4*q4 + i) by their alpha, held by lane 4*q4 + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a_i = __shfl(alpha, 4 * q4 + i);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n][i] *= a_i;
    }
    // O += P V: A = P (head c16, keys 32*s + 8*q4 + 0..7), B = V (keys x dims)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pw[e] = static_cast<uint32_t>(f32_to_bf16(sv[s][0][2 * e])) |
                (static_cast<uint32_t>(f32_to_bf16(sv[s][0][2 * e + 1])) << 16);
        pw[2 + e] = static_cast<uint32_t>(f32_to_bf16(sv[s][1][2 * e])) |
                    (static_cast<uint32_t>(f32_to_bf16(sv[s][1][2 * e + 1])) << 16);
      }
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const bf16x8 vb =
            *reinterpret_cast<const bf16x8*>(&Vt[(16 * n + c16) * VP + 32 * s + 8 * q4]);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[n], 0, 0, 0);
      }
    }
  }

  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q4 + i;
      const float l_i = __shfl(l_run, h);
      const float inv = 1.f / l_i;
      if (h < G) {
        uint16_t* orow = out + (static_cast<size_t>(ri.row) * Hq + kvh * G + h) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) orow[16 * n + c16] = f32_to_bf16(o[n][i] * inv);
      }
    }
    if (lse != nullptr && q4 == 0 && c16 < G)
      lse[static_cast<size_t>(ri.row) * Hq + kvh * G + c16] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const Partials pp = partials_of(part, g, t.q_rows, splits);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q4 + i;
      if (h < G) {
        const size_t slot = (static_cast<size_t>(ri.vrow) * Hq + kvh * G + h) * splits + sp;
#pragma unroll
        for (int n = 0; n < NT; ++n) pp.o[slot * D + 16 * n + c16] = o[n][i];
      }
    }
    if (q4 == 0 && c16 < G) {
      const size_t slot = (static_cast<size_t>(ri.vrow) * Hq + kvh * G + c16) * splits + sp;
      pp.ml[2 * slot] = m_run;
      pp.ml[2 * slot + 1] = l_run;
    }
  }
}

// ------------------------------------------------------------------------------ combine
// One workgroup of d threads per (row, head).
template <typename T>
__global__ void __launch_bounds__(256)
attn_combine(Geom g, SeqTable t, int splits, const float* __restrict__ part, T* __restrict__ out,
             float* __restrict__ lse) {
  RowInfo ri;
  if (!row_info(t, static_cast<int>(blockIdx.x), ri)) return;
  const int h = blockIdx.y;
  const Partials pp = partials_of(const_cast<float*>(part), g, t.q_rows, splits);
  const size_t slot0 = (static_cast<size_t>(ri.vrow) * g.Hq + h) * splits;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pp.ml[2 * (slot0 + s)]);
  float L = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float m = pp.ml[2 * (slot0 + s)];
    if (m != -INFINITY) L += pp.ml[2 * (slot0 + s) + 1] * exp2f(m - M);
  }
  const float inv = 1.f / L;
  for (int e = threadIdx.x; e < g.d; e += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float m = pp.ml[2 * (slot0 + s)];
      if (m != -INFINITY) acc += pp.o[(slot0 + s) * g.d + e] * exp2f(m - M);
    }
    st(out, (static_cast<size_t>(ri.row) * g.Hq + h) * g.d + e, acc * inv);
  }
  if (lse != nullptr && threadIdx.x == 0)
    lse[static_cast<size_t>(ri.row) * g.Hq + h] = (M + log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_attn(const Geom& g, int dtype, const SeqTable& t, const void* q,
                       const void* k, const void* v, const int32_t* idx, int splits,
                       void* out, float* lse, float* part, hipStream_t stream) {
  const int rows = bound_rows(t);
  if (rows == 0) return hipSuccess;
  const dim3 grid(rows, g.Hkv, splits);
  const bool mfma = dtype == INFLLM2_BF16 && g.B == 64 && (g.d == 64 || g.d == 128) &&
                    (g.G == 8 || g.G == 16);
  if (mfma) {
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const uint16_t* vv = static_cast<const uint16_t*>(v);
    uint16_t* oo = static_cast<uint16_t*>(out);
#define INFLLM2_ATTN_CASE(DD, GG)                                                            \
  if (g.d == DD && g.G == GG) {                                                              \
    hipLaunchKernelGGL((attn_mfma<DD, GG>), grid, dim3(64), 0, stream, g, t, qq, kk, vv, idx, \
                       splits, oo, lse, part);                                               \
    return hipGetLastError();                                                                \
  }
    INFLLM2_ATTN_CASE(128, 16)
    INFLLM2_ATTN_CASE(128, 8)
    INFLLM2_ATTN_CASE(64, 16)
    INFLLM2_ATTN_CASE(64, 8)
#undef INFLLM2_ATTN_CASE
  }
  if (dtype == INFLLM2_BF16)
    hipLaunchKernelGGL(attn_simple<uint16_t>, grid, dim3(kSimpleThreads), 0, stream, g, t,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), idx, splits,
                       static_cast<uint16_t*>(out), lse, part);
  else
    hipLaunchKernelGGL(attn_simple<float>, grid, dim3(kSimpleThreads), 0, stream, g, t,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), idx, splits, static_cast<float*>(out), lse,
                       part);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const Geom& g, int dtype, const SeqTable& t, int splits,
                               const float* part, void* out, float* lse, hipStream_t stream) {
  const int rows = bound_rows(t);
  if (rows == 0) return hipSuccess;
  const dim3 grid(rows, g.Hq);
  const dim3 block(g.d < 256 ? g.d : 256);
  if (dtype == INFLLM2_BF16)
    hipLaunchKernelGGL(attn_combine<uint16_t>, grid, block, 0, stream, g, t, splits, part,
                       static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL(attn_combine<float>, grid, block, 0, stream, g, t, splits, part,
                       static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace infllm2
