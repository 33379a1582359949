// Split-KV block-sparse attention for decoding (arXiv abstract of MiniCPM4: the sparse
// attention accelerates decoding as well as prefilling; paper summary section 2.1.3).
//
// A decoding batch has one (or a few) query rows per sequence, so the selected blocks of a
// row are spread over many workgroups: workgroup (row, kv head, split) owns a contiguous range
// of the row's block list, and each of its 4 waves takes every 4th block of that range.  A wave
// loads its block's K straight into registers, already in MFMA A-operand order (16 bytes per
// lane per step), and its block's V into its own LDS slot with global_load_lds, in the order the
// transposing LDS reads need; it folds the block into a running (max, sum, output) for the 16
// stacked heads of the group.  The 4 waves then merge through LDS, and the workgroup writes its
// partial.  The last workgroup of a
// (row, kv head) to finish -- counted with an agent-scope atomic in the workspace -- merges all
// partials by log-sum-exp and writes the output, so no separate combine launch is needed.  It
// resets the counter, leaving the workspace ready for the next call.
#include "internal.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 8 transposing reads at immediate offsets 512*(2n + h); waited for inside the statement.
__device__ __forceinline__ void read_v8(uint32_t addr, uint64_t (&vt)[4][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %8 offset:512\n"
      "ds_read_b64_tr_b16 %2, %8 offset:1024\n"
      "ds_read_b64_tr_b16 %3, %8 offset:1536\n"
      "ds_read_b64_tr_b16 %4, %8 offset:2048\n"
      "ds_read_b64_tr_b16 %5, %8 offset:2560\n"
      "ds_read_b64_tr_b16 %6, %8 offset:3072\n"
      "ds_read_b64_tr_b16 %7, %8 offset:3584\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(vt[0][0]), "=&v"(vt[0][1]), "=&v"(vt[1][0]), "=&v"(vt[1][1]),
        "=&v"(vt[2][0]), "=&v"(vt[2][1]), "=&v"(vt[3][0]), "=&v"(vt[3][1])
      : "v"(addr)
      : "memory");
}

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return static_cast<uint64_t>(__float_as_uint(a)) | (static_cast<uint64_t>(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float lo_f32(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v)); }
__device__ __forceinline__ float hi_f32(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v >> 32)); }
__device__ __forceinline__ void agent_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t agent_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace: partial outputs O[d] per (row, kv head, split, head of group), then the partial
// (max, sum) pairs in the same order, then one counter per (row, kv head).
struct DecodeWs {
  float* part_o;
  float* part_ml;
  int* count;
};

__device__ __forceinline__ DecodeWs ws_of(void* ws, int rows, int Hkv, int nsplit, int G, int D) {
  DecodeWs w;
  const size_t n = static_cast<size_t>(rows) * Hkv * nsplit * G;
  w.part_o = static_cast<float*>(ws);
  w.part_ml = w.part_o + n * D;
  w.count = reinterpret_cast<int*>(w.part_ml + n * 2);
  return w;
}

template <int D, int G>
__global__ void __launch_bounds__(64 * kWaves)
attn_decode(Geom g, SeqTable t, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int nsplit,
            void* __restrict__ workspace, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int CPR = D / 8;
  constexpr int MAT = 64 * D * 2;                          // one block of V
  __shared__ __attribute__((aligned(16))) unsigned char ring[kWaves][MAT];
  __shared__ float wm_s[kWaves][16], wl_s[kWaves][16];
  __shared__ int s_last;

  const int vrow = blockIdx.x;
  const int kvh = blockIdx.y;
  const int sp = blockIdx.z;
  const int rows = t.work_prefix[t.n];
  const int b = find_seq(t, vrow);
  const int j = vrow - t.work_prefix[b];
  const int row = t.q_start[b] + j;
  const int pos = t.q_pos0[b] + j;
  const int kv0 = t.kv_start[b];
  const int kv_len = t.kv_len[b];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int Hq = g.Hq, Hkv = g.Hkv;
  const int rowstride = Hkv * D;

  const int32_t* sel = idx + (static_cast<size_t>(row) * Hkv + kvh) * g.topk;
  // the valid entries form a prefix (ascending, then -1): count them with ballots
  int nsel = 0;
  for (int base = 0; base < g.topk; base += 128) {
    const int e0 = base + lane, e1 = base + 64 + lane;
    const bool v0 = e0 < g.topk && sel[e0] >= 0;
    const bool v1 = e1 < g.topk && sel[e1] >= 0;
    const unsigned long long m1 = __ballot(v1);
    nsel += __popcll(__ballot(v0)) + __popcll(m1);
    if (~m1 != 0ull) break;
  }
  const int per = (nsel + nsplit - 1) / nsplit;
  const int k_begin = min(nsel, sp * per);
  const int k_end = min(nsel, k_begin + per);

  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (c16 < G)
      qf[ks] = *reinterpret_cast<const bf16x8*>(
          q + (static_cast<size_t>(row) * Hq + kvh * G + c16) * D + 32 * ks + 8 * q4);
    else
      qf[ks] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;   // head c16; l_run is this lane's partial sum
  const float qscale = g.scale * kLog2e;

  const int k_lrow = 8 * (c16 >> 2) + (c16 & 3);
  const int v_lrow = 8 * ((lane & 31) >> 3) + 4 * (lane >> 5) + ((lane >> 1) & 3);
  const int k_lane_off = k_lrow * rowstride + 8 * q4;
  const int v_lane_off = v_lrow * rowstride + 8 * (lane & 1);
  const uint16_t* kbase = k + static_cast<size_t>(kv0) * rowstride + static_cast<size_t>(kvh) * D;
  const uint16_t* vbase = v + static_cast<size_t>(kv0) * rowstride + static_cast<size_t>(kvh) * D;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&ring[w][0]));
  const uint32_t vaddr = ring_lds + 16 * (8 * q4 + 2 * (c16 >> 2) + ((c16 & 3) >> 1)) + 8 * (c16 & 1);

  for (int kk = k_begin + w; kk < k_end; kk += kWaves) {
    const int key0 = sel[kk] * 64;
    const bool tail = key0 + 64 > kv_len;
    const int last = kv_len - 1 - key0;
    const uint16_t* kb = kbase + static_cast<size_t>(key0) * rowstride;
    const uint16_t* vb = vbase + static_cast<size_t>(key0) * rowstride;
    bf16x8 kr[CPR];                 // A operand of MFMA step J = (2s + tp) * KS + ks
#pragma unroll
    for (int J = 0; J < CPR; ++J) {
      const int krow0 = 32 * (J / (2 * KS)) + 4 * ((J / KS) % 2);
      const int vrow0 = 32 * (J / NT);
      int ko = k_lane_off + krow0 * rowstride + 32 * (J % KS);
      int vo = v_lane_off + vrow0 * rowstride + 16 * (J % NT);
      if (tail) {                   // rows past the cache end repeat its last row (masked)
        const int kr0 = krow0 + k_lrow, vr = vrow0 + v_lrow;
        ko += ((kr0 < last ? kr0 : last) - kr0) * rowstride;
        vo += ((vr < last ? vr : last) - vr) * rowstride;
      }
      const uint16_t* gv = vb + vo;
      kr[J] = *reinterpret_cast<const bf16x8*>(kb + ko);
      __builtin_amdgcn_global_load_lds(gv, (lds_void*)(&ring[w][J * 1024]), 16, 0, 0);
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    float sv[2][2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[(2 * s + tp) * KS + ks], qf[ks], acc,
                                                        0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[s][tp][i] = acc[i];
      }
    }
    if (key0 + 63 > pos || tail) {
      const int lim = min(pos, kv_len - 1) - key0;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * s + 8 * q4 + 4 * tp + i > lim) sv[s][tp][i] = -INFINITY;
    }
    float mx = sv[0][0][0];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[s][tp][i]);
    mx *= qscale;
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a_i = __shfl(alpha, 4 * q4 + i);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n][i] *= a_i;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sv[s][tp][i], qscale, -m_run));
          sv[s][tp][i] = p;
          l_run += p;
        }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x2 pp[4] = {__builtin_convertvector((f32x2){sv[s][0][0], sv[s][0][1]}, bf16x2),
                            __builtin_convertvector((f32x2){sv[s][0][2], sv[s][0][3]}, bf16x2),
                            __builtin_convertvector((f32x2){sv[s][1][0], sv[s][1][1]}, bf16x2),
                            __builtin_convertvector((f32x2){sv[s][1][2], sv[s][1][3]}, bf16x2)};
      const bf16x8 pa = __builtin_bit_cast(bf16x8, pp);
#pragma unroll
      for (int hh = 0; hh < NT / 4; ++hh) {
        uint64_t vt[4][2];
        read_v8(vaddr + 512u * (2 * NT * s + 8 * hh), vt);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const uint64_t both[2] = {vt[n][0], vt[n][1]};
          o[hh * 4 + n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              pa, __builtin_bit_cast(bf16x8, both), o[hh * 4 + n], 0, 0, 0);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot reads done before its refill
  }

  // ---- merge the 4 waves through LDS (their slots are free now)
  float l = l_run;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (q4 == 0) {
    wm_s[w][c16] = m_run;
    wl_s[w][c16] = l;
  }
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(&ring[0][0]);               // [wave][16][D] floats
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, wm_s[ww][h]);
    const float scale = wm_s[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm_s[w][h] - M);
#pragma unroll
    for (int n = 0; n < NT; ++n) obuf[(w * 16 + h) * D + 16 * n + c16] = o[n][i] * scale;
  }
  __syncthreads();
  // thread -> (head h, 8 dims); 256 threads cover 16 heads x 128 dims (d = 64: half idle)
  const int h = tid >> 4;
  const int d0 = (tid & 15) * 8;
  float M = -INFINITY, L = 0.f;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, wm_s[ww][h]);
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww)
    if (wm_s[ww][h] != -INFINITY) L += wl_s[ww][h] * __builtin_amdgcn_exp2f(wm_s[ww][h] - M);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (d0 < D) {
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += obuf[(ww * 16 + h) * D + d0 + e];
  }

  if (nsplit == 1) {
    if (h < G && d0 < D) {
      uint16_t* op = out + (static_cast<size_t>(row) * Hq + kvh * G + h) * D + d0;
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < 8; ++e) op[e] = f32_to_bf16(acc[e] * inv);
      if (lse != nullptr && d0 == 0) lse[static_cast<size_t>(row) * Hq + kvh * G + h] = (M + log2f(L)) * kLn2;
    }
    return;
  }

  // ---- partial of this split, then the last split of (row, kv head) merges all of them
  DecodeWs ws = ws_of(workspace, rows, Hkv, nsplit, G, D);
  const size_t ebase = (static_cast<size_t>(vrow) * Hkv + kvh) * nsplit * G;   // entry of split 0
  // Partials cross workgroups (and XCDs, whose L2s are not coherent with each other) through
  // agent-scope atomic stores and loads, which are coherent at that scope by themselves; a
  // fence would instead write back and invalidate the whole L2 of the XCD.
  if (h < G && d0 < D) {
    const size_t e = ebase + static_cast<size_t>(sp) * G + h;
    uint64_t* po = reinterpret_cast<uint64_t*>(ws.part_o + e * D + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      agent_store(po + i, pack2(acc[2 * i], acc[2 * i + 1]));
    if (d0 == 0) agent_store(reinterpret_cast<uint64_t*>(ws.part_ml + e * 2), pack2(M, L));
  }
  wait_vmcnt<0>();                                   // this wave's stores are complete
  __syncthreads();
  int* cnt = ws.count + static_cast<size_t>(vrow) * Hkv + kvh;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  if (h < G && d0 < D) {
    // online log-sum-exp merge; the loads of 8 splits are issued before any is used
    float MM = -INFINITY, LL = 0.f;
    float a2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a2[e] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      uint64_t ml[8], ov[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const size_t e = ebase + static_cast<size_t>(min(s0 + u, nsplit - 1)) * G + h;
        ml[u] = agent_load(reinterpret_cast<const uint64_t*>(ws.part_ml + e * 2));
        const uint64_t* po = reinterpret_cast<const uint64_t*>(ws.part_o + e * D + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[u][i] = agent_load(po + i);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float ms = lo_f32(ml[u]);
        if (s0 + u >= nsplit || ms == -INFINITY) continue;      // duplicate or empty split
        const float Mn = fmaxf(MM, ms);
        const float fo = __builtin_amdgcn_exp2f(MM - Mn);
        const float fn = __builtin_amdgcn_exp2f(ms - Mn);
        LL = LL * fo + hi_f32(ml[u]) * fn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a2[2 * i] = a2[2 * i] * fo + lo_f32(ov[u][i]) * fn;
          a2[2 * i + 1] = a2[2 * i + 1] * fo + hi_f32(ov[u][i]) * fn;
        }
        MM = Mn;
      }
    }
    uint16_t* op = out + (static_cast<size_t>(row) * Hq + kvh * G + h) * D + d0;
    const float inv = 1.f / LL;
#pragma unroll
    for (int e = 0; e < 8; ++e) op[e] = f32_to_bf16(a2[e] * inv);
    if (lse != nullptr && d0 == 0) lse[static_cast<size_t>(row) * Hq + kvh * G + h] = (MM + log2f(LL)) * kLn2;
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
}

}  // namespace

bool attn_decode_supported(const Geom& g, int dtype) {
  return dtype == INFLLM2_BF16 && g.B == 64 && (g.d == 64 || g.d == 128) && (g.G == 8 || g.G == 16);
}

size_t attn_decode_workspace(const Geom& g, int rows, int nsplit) {
  return static_cast<size_t>(rows) * g.Hkv * nsplit * g.G * (g.d + 2) * sizeof(float) +
         static_cast<size_t>(rows) * g.Hkv * sizeof(int);
}

// work_prefix of `t` counts query rows.
hipError_t launch_attn_decode(const Geom& g, const SeqTable& t, const void* q, const void* k,
                              const void* v, const int32_t* idx, int nsplit, void* workspace,
                              void* out, float* lse, hipStream_t stream) {
  const int rows = t.work_prefix[t.n];
  if (rows == 0) return hipSuccess;
  if (nsplit < 1 || nsplit > 65535 || g.Hkv > 65535) return hipErrorInvalidValue;
  const dim3 grid(rows, g.Hkv, nsplit);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(out);
#define INFLLM2_DEC_CASE(DD, GG)                                                                \
  if (g.d == DD && g.G == GG) {                                                                 \
    hipLaunchKernelGGL((attn_decode<DD, GG>), grid, dim3(64 * kWaves), 0, stream, g, t, qq, kk, \
                       vv, idx, nsplit, workspace, oo, lse);                                    \
    return hipGetLastError();                                                                   \
  }
  INFLLM2_DEC_CASE(128, 16)
  INFLLM2_DEC_CASE(128, 8)
  INFLLM2_DEC_CASE(64, 16)
  INFLLM2_DEC_CASE(64, 8)
#undef INFLLM2_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllm2
