// Decoding (arXiv abstract of MiniCPM4: the sparse attention accelerates decoding as well as
// prefilling), in two forms that share the per-block arithmetic:
//
// attn_decode -- split-KV block-sparse attention over a given selection (paper summary, section
// 2.1.3).  A decoding batch has one (or a few) query rows per sequence, so the selected blocks of
// a row are spread over many workgroups: workgroup (row, kv head, split) owns a contiguous range
// of the row's block list, and each of its waves takes every NW-th block of that range.  A wave
// loads its block's K straight into registers, already in MFMA A-operand order (16 bytes per
// lane per step), and its block's V into its own LDS slot with global_load_lds, in the order the
// transposing LDS reads need; it folds the block into a running (max, sum, output) for the 16
// stacked heads of the group.  The waves then merge through LDS, and the workgroup writes its
// partial.  The last workgroup of a (row, kv head) to finish -- counted with an agent-scope
// atomic in the workspace -- merges all partials by log-sum-exp and writes the output, so no
// separate combine launch is needed.  It resets the counter, leaving the workspace ready for the
// next call.
//
// The decode step (infllm2_decode_step) is two launches.  decode_scores: block scores (section
// 2.1.2: the group-summed query against every semantic kernel, max-pooled onto blocks), one
// workgroup per chunk of 64 blocks of a (row, kv head); the kernels completed since the last
// compression are computed there from the keys and stored.  Then attn_decode in its selecting
// form: every split workgroup of a (row, kv head) first runs the group-shared top-k (2.1.1-2.1.2)
// of the pair itself, from the stored scores (a radix select over the order-preserving score
// keys, in LDS), keeps the part of the selection its split folds, and the first split writes the
// whole selection out.  The selection is computed once per split instead of once per pair, but
// no workgroup waits for another's and the indices never make a round trip through memory
// before the fold.
//
// Data crossing workgroups of one launch (partials, counters) moves through agent-scope atomic
// stores and loads, which are coherent across the XCDs' separate L2s by themselves; a fence
// would instead write back and invalidate a whole L2.
#include <algorithm>

#include "dpp.h"
#include "internal.h"
#include "select.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxKeysPerThread = 8;      // the decode step's selection: at most 8 * 512 blocks
constexpr int kMaxSplitBlocks = 256;      // ... and at most 256 selected blocks per split

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

// Row-major V slot (d = 128): 4 x 2 transposing reads, tile n from its own address a_n, the two
// 4-key halves at +0 and +1024 bytes (+8192 for the second 32-key half of the block); waited
// for inside the statement.
#define INFLLM2_TR4X2(NAME, O0, O1)                                                            \
  __device__ __forceinline__ void NAME(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,    \
                                       uint64_t(&vt)[4][2]) {                                 \
    asm volatile("ds_read_b64_tr_b16 %0, %8 offset:" #O0 "\n"                                 \
                 "ds_read_b64_tr_b16 %1, %8 offset:" #O1 "\n"                                 \
                 "ds_read_b64_tr_b16 %2, %9 offset:" #O0 "\n"                                 \
                 "ds_read_b64_tr_b16 %3, %9 offset:" #O1 "\n"                                 \
                 "ds_read_b64_tr_b16 %4, %10 offset:" #O0 "\n"                                \
                 "ds_read_b64_tr_b16 %5, %10 offset:" #O1 "\n"                                \
                 "ds_read_b64_tr_b16 %6, %11 offset:" #O0 "\n"                                \
                 "ds_read_b64_tr_b16 %7, %11 offset:" #O1 "\n"                                \
                 "s_waitcnt lgkmcnt(0)"                                                        \
                 : "=&v"(vt[0][0]), "=&v"(vt[0][1]), "=&v"(vt[1][0]), "=&v"(vt[1][1]),         \
                   "=&v"(vt[2][0]), "=&v"(vt[2][1]), "=&v"(vt[3][0]), "=&v"(vt[3][1])          \
                 : "v"(a0), "v"(a1), "v"(a2), "v"(a3)                                          \
                 : "memory");                                                                  \
  }
INFLLM2_TR4X2(read_tr_half0, 0, 1024)
INFLLM2_TR4X2(read_tr_half1, 8192, 9216)
#undef INFLLM2_TR4X2

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return static_cast<uint64_t>(__float_as_uint(a)) | (static_cast<uint64_t>(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float lo_f32(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v)); }
__device__ __forceinline__ float hi_f32(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v >> 32)); }
template <typename T>
__device__ __forceinline__ void agent_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T agent_load(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int agent_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The query row of dense work item `item` (query rows counted over the sequences in order);
// false past the last row.  Every lane of the calling wave must call it.  Per-(row, KV head)
// workspace entries are indexed by the query row itself.
struct DecRow {
  int row, pos, kv0, kv_len, kc0;
  int seq;        // the row's sequence
  bool last;      // the sequence's last query row
};
__device__ __forceinline__ bool dec_row(const SeqTable& t, int item, DecRow& r) {
  int b, j;
  if (!locate(t, item, [&](int s) { return t.q_len[s]; }, b, j)) return false;
  const Seq sq = load_seq(t, b);
  r.row = sq.q_start + j;
  r.pos = sq.q_pos0 + j;
  r.kv0 = sq.kv_start;
  r.kv_len = sq.kv_len;
  r.kc0 = sq.kc_start;
  r.seq = b;
  r.last = j == sq.q_len - 1;
  return true;
}

// ------------------------------------------------------------------ attention over selected blocks
// A wave's running state for the 16 stacked heads of a group: O (accumulator tiles, head = row
// 4*(lane/16) + i of tile n), the running max (log2 domain) and this lane's partial sum, both
// for head lane % 16.
template <int D>
struct WaveAcc {
  f32x4 o[D / 16];
  float m, l;
};

// Per-lane constants of a wave's block fold for one (row, kv head).  d = 128: V goes to the
// wave's LDS slot as whole rows (4 rows of 256 bytes per load instruction), row r's 16-byte
// chunk c stored at position c ^ vswz(r), vswz(r) = 2 ((r & 3) + 4 ((r >> 3) & 1)), which
// spreads every transposing read over all 64 banks (each chunk position read by 2 of its 16
// rows); lane addresses of the 8 column tiles in vt_addr.  d = 64: V in the order of the
// transposing reads (one base address, immediate offsets).
template <int D, int G>
struct FoldCtx {
  bf16x8 qf[D / 32];
  const uint16_t* kbase;
  const uint16_t* vbase;
  int rowstride, k_lane_off, v_lane_off, k_lrow, v_lrow, pos, kv_len;
  int v_col0, v_col1;
  uint32_t vaddr;
  uint32_t vt_addr[D == 128 ? 8 : 1];
  lds_u8* slot;
  float qscale;
};

template <int D, int G>
__device__ __forceinline__ void fold_init(FoldCtx<D, G>& c, WaveAcc<D>& a, const Geom& g,
                                          const uint16_t* q, const uint16_t* k,
                                          const uint16_t* v, const DecRow& r, int kvh,
                                          lds_u8* slot, int lane) {
  constexpr int KS = D / 32;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (c16 < G)
      c.qf[ks] = *reinterpret_cast<const bf16x8*>(
          q + (static_cast<size_t>(r.row) * g.Hq + kvh * G + c16) * D + 32 * ks + 8 * q4);
    else
      c.qf[ks] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  c.rowstride = g.Hkv * D;
  c.k_lrow = 8 * (c16 >> 2) + (c16 & 3);
  c.v_lrow = 8 * ((lane & 31) >> 3) + 4 * (lane >> 5) + ((lane >> 1) & 3);
  c.k_lane_off = c.k_lrow * c.rowstride + 8 * q4;
  c.v_lane_off = c.v_lrow * c.rowstride + 8 * (lane & 1);
  c.kbase = k + static_cast<size_t>(r.kv0) * c.rowstride + static_cast<size_t>(kvh) * D;
  c.vbase = v + static_cast<size_t>(r.kv0) * c.rowstride + static_cast<size_t>(kvh) * D;
  c.slot = slot;
  const uint32_t slot_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(slot));
  c.vaddr = slot_addr + 16 * (8 * q4 + 2 * (c16 >> 2) + ((c16 & 3) >> 1)) + 8 * (c16 & 1);
  if constexpr (D == 128) {
    // load instruction J: lane -> row 4J + lane/16, global chunk (lane % 16) ^ vswz(row), where
    // vswz(row) = 2 (lane/16) + 8 ((J >> 1) & 1)
    c.v_col0 = 8 * ((lane & 15) ^ (2 * (lane >> 4)));
    c.v_col1 = c.v_col0 ^ 64;
    // transposing reads: lane (L = lane % 16, kq = lane / 16) addresses row 8 kq + L/4 (+4 for
    // the second 4-key half), columns 16 n + 4 (L % 4) .. + 3
    const int L = lane & 15;
    const int sw = 2 * ((L >> 2) + 4 * (q4 & 1));
#pragma unroll
    for (int n = 0; n < 8; ++n)
      c.vt_addr[n] = slot_addr + (8 * q4 + (L >> 2)) * 256 + (((2 * n) ^ sw) + ((L & 3) >> 1)) * 16 +
                     8 * (L & 1);
  } else {
    c.v_col0 = c.v_col1 = 0;
    c.vt_addr[0] = 0;
  }
  c.pos = r.pos;
  c.kv_len = r.kv_len;
  c.qscale = g.scale * kLog2e;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) a.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  a.m = -INFINITY;
  a.l = 0.f;
}

// Folds the block starting at key key0 into the wave's state: S^T = K Q^T (keys as rows, in the
// permuted order that makes the accumulator the P operand), keys past the query position or the
// cache end masked, online softmax in the exp2 domain, O += P V.
template <int D, int G>
__device__ __forceinline__ void fold_block(const FoldCtx<D, G>& c, WaveAcc<D>& a, int key0,
                                           int lane) {
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int CPR = D / 8;
  const int q4 = lane >> 4;
  const bool tail = key0 + 64 > c.kv_len;
  const int last = c.kv_len - 1 - key0;
  const uint16_t* kb = c.kbase + static_cast<size_t>(key0) * c.rowstride;
  const uint16_t* vb = c.vbase + static_cast<size_t>(key0) * c.rowstride;
  bf16x8 kr[CPR];                 // A operand of MFMA step J = (2s + tp) * KS + ks
#pragma unroll
  for (int J = 0; J < CPR; ++J) {
    const int krow0 = 32 * (J / (2 * KS)) + 4 * ((J / KS) % 2);
    const int vrow0 = 32 * (J / NT);
    int ko = c.k_lane_off + krow0 * c.rowstride + 32 * (J % KS);
    int vo;
    if constexpr (D == 128) {
      const int vr = 4 * J + (lane >> 4);
      vo = (tail && vr > last ? last : vr) * c.rowstride + (((J >> 1) & 1) ? c.v_col1 : c.v_col0);
    } else {
      vo = c.v_lane_off + vrow0 * c.rowstride + 16 * (J % NT);
      if (tail) {
        const int vr = vrow0 + c.v_lrow;
        vo += ((vr < last ? vr : last) - vr) * c.rowstride;
      }
    }
    if (tail) {                   // rows past the cache end repeat its last row (masked)
      const int kr0 = krow0 + c.k_lrow;
      ko += ((kr0 < last ? kr0 : last) - kr0) * c.rowstride;
    }
    kr[J] = *reinterpret_cast<const bf16x8*>(kb + ko);
    __builtin_amdgcn_global_load_lds(vb + vo, (lds_void*)(c.slot + J * 1024), 16, 0, 0);
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
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[(2 * s + tp) * KS + ks], c.qf[ks], acc,
                                                      0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[s][tp][i] = acc[i];
    }
  }
  if (key0 + 63 > c.pos || tail) {
    const int lim = min(c.pos, c.kv_len - 1) - key0;
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
  mx *= c.qscale;
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(a.m, mx);
  const float alpha = __builtin_amdgcn_exp2f(a.m - m_new);
  a.l *= alpha;
  a.m = m_new;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a_i = __shfl(alpha, 4 * q4 + i);
#pragma unroll
    for (int n = 0; n < NT; ++n) a.o[n][i] *= a_i;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sv[s][tp][i], c.qscale, -a.m));
        sv[s][tp][i] = p;
        a.l += p;
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
      if constexpr (D == 128) {
        if (s == 0)
          read_tr_half0(c.vt_addr[4 * hh], c.vt_addr[4 * hh + 1], c.vt_addr[4 * hh + 2],
                        c.vt_addr[4 * hh + 3], vt);
        else
          read_tr_half1(c.vt_addr[4 * hh], c.vt_addr[4 * hh + 1], c.vt_addr[4 * hh + 2],
                        c.vt_addr[4 * hh + 3], vt);
      } else {
        read_v8(c.vaddr + 512u * (2 * NT * s + 8 * hh), vt);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint64_t both[2] = {vt[n][0], vt[n][1]};
        a.o[hh * 4 + n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pa, __builtin_bit_cast(bf16x8, both), a.o[hh * 4 + n], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot reads done before its refill
}

// Merges the NW waves' states through LDS (`ring`, whose slots are free by now; every thread
// must call it).  Thread tid ends with head h = tid / (T/16) and DPT = 16 D / T consecutive
// dims from d0: unnormalised sums acc[], the workgroup max M (log2 domain) and sum L of head h.
template <int D, int NW>
__device__ __forceinline__ void merge_waves(const WaveAcc<D>& a, unsigned char* ring,
                                            float (*wm_s)[16], float (*wl_s)[16], int tid,
                                            float (&acc)[16 * D / (64 * NW)], float& M,
                                            float& L) {
  constexpr int NT = D / 16;
  constexpr int T = 64 * NW;
  constexpr int DPT = 16 * D / T;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  float l = a.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (q4 == 0) {
    wm_s[w][c16] = a.m;
    wl_s[w][c16] = l;
  }
  __syncthreads();
  float* obuf = reinterpret_cast<float*>(ring);               // [wave][16][D] floats
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * q4 + i;
    float Mh = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) Mh = fmaxf(Mh, wm_s[ww][h]);
    const float scale = wm_s[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wm_s[w][h] - Mh);
#pragma unroll
    for (int n = 0; n < NT; ++n) obuf[(w * 16 + h) * D + 16 * n + c16] = a.o[n][i] * scale;
  }
  __syncthreads();
  const int h = tid / (T / 16);
  const int d0 = (tid % (T / 16)) * DPT;
  M = -INFINITY;
  L = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, wm_s[ww][h]);
#pragma unroll
  for (int ww = 0; ww < NW; ++ww)
    if (wm_s[ww][h] != -INFINITY) L += wl_s[ww][h] * __builtin_amdgcn_exp2f(wm_s[ww][h] - M);
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww)
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] += obuf[(ww * 16 + h) * D + d0 + e];
}

// Writes the merged workgroup result of (row, kv head) straight to the output (single split),
// or its partial; then the last split of the pair to finish merges all partials by log-sum-exp
// and writes the output.  Every thread must call it (thread mapping of merge_waves).
template <int D, int G, int NW>
__device__ __forceinline__ void finish_split(const Geom& g, int row, int kvh, int pair, int sp,
                                             int nsplit, const float (&acc)[16 * D / (64 * NW)],
                                             float M, float L, int* split_done, float* part,
                                             int pairs, int tid, int* s_last,
                                             uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int T = 64 * NW;
  constexpr int DPT = 16 * D / T;
  constexpr int NP = DPT / 2;                 // 8-byte pieces per thread
  constexpr int R = DPT >= 8 ? 8 : 16;        // partials merged per round of loads
  const int h = tid / (T / 16);
  const int d0 = (tid % (T / 16)) * DPT;
  const int Hq = g.Hq;
  if (nsplit == 1) {
    if (h < G) {
      uint16_t* op = out + (static_cast<size_t>(row) * Hq + kvh * G + h) * D + d0;
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < DPT; ++e) op[e] = f32_to_bf16(acc[e] * inv);
      if (lse != nullptr && d0 == 0) lse[static_cast<size_t>(row) * Hq + kvh * G + h] = (M + log2f(L)) * kLn2;
    }
    return;
  }
  const size_t n_ent = static_cast<size_t>(pairs) * nsplit * G;
  float* part_o = part;
  float* part_ml = part + n_ent * D;
  const size_t ebase = static_cast<size_t>(pair) * nsplit * G;        // entry of split 0
  if (h < G) {
    const size_t e = ebase + static_cast<size_t>(sp) * G + h;
    uint64_t* po = reinterpret_cast<uint64_t*>(part_o + e * D + d0);
#pragma unroll
    for (int i = 0; i < NP; ++i) agent_store(po + i, pack2(acc[2 * i], acc[2 * i + 1]));
    if (d0 == 0) agent_store(reinterpret_cast<uint64_t*>(part_ml + e * 2), pack2(M, L));
  }
  wait_vmcnt<0>();                                   // this wave's stores are complete
  __syncthreads();
  if (tid == 0) *s_last = agent_add(split_done + pair, 1) == nsplit - 1;
  __syncthreads();
  if (!*s_last) return;
  if (h < G) {
    // online log-sum-exp merge; the loads of R splits are issued before any is used
    float MM = -INFINITY, LL = 0.f;
    float a2[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) a2[e] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += R) {
      uint64_t ml[R], ov[R][NP];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const size_t e = ebase + static_cast<size_t>(min(s0 + u, nsplit - 1)) * G + h;
        ml[u] = agent_load(reinterpret_cast<const uint64_t*>(part_ml + e * 2));
        const uint64_t* po = reinterpret_cast<const uint64_t*>(part_o + e * D + d0);
#pragma unroll
        for (int i = 0; i < NP; ++i) ov[u][i] = agent_load(po + i);
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const float ms = lo_f32(ml[u]);
        if (s0 + u >= nsplit || ms == -INFINITY) continue;      // duplicate or empty split
        const float Mn = fmaxf(MM, ms);
        const float fo = __builtin_amdgcn_exp2f(MM - Mn);
        const float fn = __builtin_amdgcn_exp2f(ms - Mn);
        LL = LL * fo + hi_f32(ml[u]) * fn;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          a2[2 * i] = a2[2 * i] * fo + lo_f32(ov[u][i]) * fn;
          a2[2 * i + 1] = a2[2 * i + 1] * fo + hi_f32(ov[u][i]) * fn;
        }
        MM = Mn;
      }
    }
    uint16_t* op = out + (static_cast<size_t>(row) * Hq + kvh * G + h) * D + d0;
    const float inv = 1.f / LL;
#pragma unroll
    for (int e = 0; e < DPT; ++e) op[e] = f32_to_bf16(a2[e] * inv);
    if (lse != nullptr && d0 == 0) lse[static_cast<size_t>(row) * Hq + kvh * G + h] = (MM + log2f(LL)) * kLn2;
  }
  if (tid == 0) agent_store(split_done + pair, 0);   // ready for the next call
}

// SEL: the selecting form of the decode step -- the workgroup selects the pair's blocks from
// `scores` (nb_stride floats per (row, kv head)) and writes the selection to idx when it is the
// pair's first split; otherwise idx is the given selection.
template <int D, int G, int NW, bool SEL>
__global__ void __launch_bounds__(64 * NW)
attn_decode(Geom g, SeqTable t, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
            const uint16_t* __restrict__ v, int32_t* __restrict__ idx,
            const float* __restrict__ scores, int nb_stride, int nsplit,
            void* __restrict__ workspace, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int MAT = 64 * D * 2;                          // one block of V
  static_assert(!SEL || NW * MAT >= kMaxKeysPerThread * 64 * NW * 4, "selection keys fit the ring");
  __shared__ __attribute__((aligned(16))) unsigned char ring[NW][MAT];
  __shared__ float wm_s[NW][16], wl_s[NW][16];
  __shared__ int s_last;

  const int kvh = blockIdx.y;
  const int sp = blockIdx.z;
  DecRow r;
  if (!dec_row(t, static_cast<int>(blockIdx.x), r)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  // split sp takes entries sp*per .. sp*per + per - 1 of the selection (per from topk, so no
  // wave waits to count the valid entries first); the valid entries form a prefix (ascending,
  // then -1), so a wave stops at its first -1
  const int per = (g.topk + nsplit - 1) / nsplit;
  const int k_begin = min(g.topk, sp * per);
  const int k_end = min(g.topk, k_begin + per);
  int32_t* const pair_idx = idx + (static_cast<size_t>(r.row) * g.Hkv + kvh) * g.topk;
  const int32_t* sel = pair_idx;
  if constexpr (SEL) {
    // the pair's selection, in LDS: its keys in the ring's first bytes (the ring is unused
    // until the fold), this split's entries in s_sel
    __shared__ WgSelectLds<NW> sm;
    __shared__ int32_t s_sel[kMaxSplitBlocks];
    for (int e = tid; e < per; e += 64 * NW) s_sel[e] = -1;
    const bool first = sp == 0;
    wg_select<NW, kMaxKeysPerThread>(
        g, r.pos / 64, scores + (static_cast<size_t>(r.row) * g.Hkv + kvh) * nb_stride,
        [&](int e, int blk) {
          if (first) pair_idx[e] = blk;
          if (e >= k_begin && e < k_end) s_sel[e - k_begin] = blk;
        },
        reinterpret_cast<uint32_t*>(&ring[0][0]), sm, tid);
    __syncthreads();                                  // s_sel written, the ring free again
    sel = s_sel - k_begin;
  }

  FoldCtx<D, G> c;
  WaveAcc<D> a;
  fold_init(c, a, g, q, k, v, r, kvh, (lds_u8*)&ring[w][0], lane);
  const int own = r.pos / 64;                       // indices past the row's own block: clamped
  for (int kk = k_begin + w; kk < k_end; kk += NW) {
    const int blk = uniform(sel[kk]);
    if (blk < 0) break;
    fold_block(c, a, min(blk, own) * 64, lane);
  }

  float acc[16 * D / (64 * NW)], M, L;
  merge_waves<D, NW>(a, &ring[0][0], wm_s, wl_s, tid, acc, M, L);
  const int pairs = t.q_rows * g.Hkv;
  const DecodeLayout lay = decode_layout(pairs);
  char* ws = static_cast<char*>(workspace);
  finish_split<D, G, NW>(g, r.row, kvh, r.row * g.Hkv + kvh, sp, nsplit, acc, M, L,
                         reinterpret_cast<int*>(ws + lay.split_done),
                         reinterpret_cast<float*>(ws + lay.part), pairs, tid, &s_last, out, lse);
}

// waves of the attention workgroups: alone (given indices), and in the decode step
constexpr int kSplitWaves = 4;
constexpr int kStepWaves = 8;

// ------------------------------------------------------------------------------ block scores
constexpr int kScoreWaves = 8;
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kChunkBlocks = 64;                // blocks per score work item

// A kernel row's 8 bf16 columns dotted with the group-summed query's (float32 FMAs in column
// order; the row total is the DPP group sum over the row's lanes).
__device__ __forceinline__ float kernel_dot8(const uint4 k, const float (&qv)[8]) {
  const uint32_t w4[4] = {k.x, k.y, k.z, k.w};
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dot = fmaf(__uint_as_float(w4[e] << 16), qv[2 * e], dot);
    dot = fmaf(__uint_as_float(w4[e] & 0xFFFF0000u), qv[2 * e + 1], dot);
  }
  return dot;
}

// Block scores of one chunk: blocks blk0 .. blk0+127 (those <= own) of query row `r`, kv head
// kvh, from kernels 4*blk0-1 .. 4*blk0+511 (the first one is the halo of block blk0).  The
// group-summed query stays in float32; each kernel row is read by D/8 lanes (16 bytes each),
// dotted with float32 FMAs and reduced across the lanes by DPP moves; every kernel load is
// issued before the query sum.  Kernel scores go to LDS, then 128 threads max-pool them onto the blocks.
// Kernels c >= c_new are not in the cache yet (completed since the last compression): after the
// cached rows are scored, they are computed from the keys (window_mean_bf16x8, the compression's
// own arithmetic) and scored, and stored by the chunk that owns them (not the halo) when
// `writer` is set.
template <int D, int G>
__device__ __forceinline__ void score_chunk(const Geom& g, const SeqTable& t, const DecRow& r,
                                            int kvh, int blk0, int own,
                                            const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ keys,
                                            uint16_t* __restrict__ kern, int c_new, bool writer,
                                            float* srow, float* qs, float* u, int tid) {
  constexpr int LPR = D / 8;              // lanes per kernel row
  constexpr int RPI = 64 / LPR;           // rows per wave instruction
  constexpr int NROW = 4 * kChunkBlocks + 1;
  constexpr int NIT = (NROW + RPI - 1) / RPI;
  constexpr int NW = kScoreWaves;
  constexpr int PER = (NIT + NW - 1) / NW;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int C = num_kernels(r.kv_len, g.w, g.s);
  const int c0 = 4 * blk0;
  const int col = (lane % LPR) * 8;
  const size_t kbase = static_cast<size_t>(r.kc0) * g.Hkv * D + static_cast<size_t>(kvh) * D;
  uint4 kv[PER];
  unsigned fresh = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = w + NW * i;
    const int rr = it * RPI + lane / LPR;
    const int cc = c0 - 1 + rr;
    const bool ok = it < NIT && rr < NROW && cc >= 0 && cc < C && 16 * cc + 31 <= r.pos;
    kv[i] = ok && cc < c_new
                ? *reinterpret_cast<const uint4*>(kern + kbase + static_cast<size_t>(cc) * g.Hkv * D + col)
                : make_uint4(0u, 0u, 0u, 0u);
    fresh |= static_cast<unsigned>(ok && cc >= c_new) << i;
  }
  for (int e = tid; e < D; e += kScoreThreads) {
    float qh[G];                                        // all heads' loads in flight at once
#pragma unroll
    for (int h = 0; h < G; ++h) qh[h] = bf16_to_f32(q[(static_cast<size_t>(r.row) * g.Hq + kvh * G + h) * D + e]);
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) s += qh[h];
    qs[e] = s;
  }
  __syncthreads();
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[col + e];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = w + NW * i;
    const int rr = it * RPI + lane / LPR;
    const int cc = c0 - 1 + rr;
    const bool ok = it < NIT && rr < NROW && cc >= 0 && cc < C && 16 * cc + 31 <= r.pos;
    const float dot = group_sum<LPR>(kernel_dot8(kv[i], qv));
    if (lane % LPR == 0 && it < NIT && rr < NROW) u[rr] = ok ? dot : -INFINITY;
  }
  if (fresh != 0) {   // rare (a new kernel every 16 decoded tokens); whole rows of lanes
    const size_t rs = static_cast<size_t>(g.Hkv) * D;
#pragma unroll 1
    for (int i = 0; i < PER; ++i) {
      if ((fresh >> i) & 1u) {
        const int rr = (w + NW * i) * RPI + lane / LPR;
        const int cc = c0 - 1 + rr;
        const uint4 kf = window_mean_bf16x8(
            keys + (static_cast<size_t>(r.kv0) + static_cast<size_t>(g.s) * cc) * rs +
                static_cast<size_t>(kvh) * D + col,
            rs, g.w);
        if (writer && rr >= 1)
          *reinterpret_cast<uint4*>(kern + kbase + static_cast<size_t>(cc) * rs + col) = kf;
        const float dot = group_sum<LPR>(kernel_dot8(kf, qv));
        if (lane % LPR == 0) u[rr] = dot;
      }
    }
  }
  __syncthreads();
  if (tid < kChunkBlocks) {
    const int blk = blk0 + tid;
    if (blk <= own) {
      // block blk's kernels 4blk-1 .. 4blk+3 sit at u[4*tid .. 4*tid+4]
      float best = u[4 * tid];
#pragma unroll
      for (int e = 1; e < 5; ++e) best = fmaxf(best, u[4 * tid + e]);
      srow[blk] = best * g.scale;
    }
  }
}

// The new kernels of chunk `chunk` (its 4 kChunkBlocks kernels, from 4 kChunkBlocks chunk on)
// that no query row scores (the cache runs past the sequence's last query position), computed
// and stored by the sequence's last row's workgroup of that chunk.
template <int D>
__device__ __forceinline__ void compress_unscored(const Geom& g, const DecRow& r, int kvh,
                                                  int chunk, int c_new,
                                                  const uint16_t* __restrict__ keys,
                                                  uint16_t* __restrict__ kern, int tid) {
  const int c0 = 4 * kChunkBlocks * chunk;
  const int lo = max(max(c0, c_new), num_kernels(r.pos + 1, g.w, g.s));
  const int hi = min(c0 + 4 * kChunkBlocks, num_kernels(r.kv_len, g.w, g.s));
  const size_t rs = static_cast<size_t>(g.Hkv) * D;
  for (int it = tid; it < (hi - lo) * (D / 8); it += kScoreThreads) {
    const int cc = lo + it / (D / 8);
    const int col = (it % (D / 8)) * 8;
    *reinterpret_cast<uint4*>(kern + (static_cast<size_t>(r.kc0) + cc) * rs +
                              static_cast<size_t>(kvh) * D + col) =
        window_mean_bf16x8(keys + (static_cast<size_t>(r.kv0) + static_cast<size_t>(g.s) * cc) * rs +
                               static_cast<size_t>(kvh) * D + col,
                           rs, g.w);
  }
}

template <int D, int G>
__global__ void __launch_bounds__(kScoreThreads)
decode_scores(Geom g, SeqTable t, const uint16_t* __restrict__ q,
              const uint16_t* __restrict__ keys, uint16_t* __restrict__ kern,
              float* __restrict__ scores, int nb_stride) {
  __shared__ __attribute__((aligned(16))) float u[4 * kChunkBlocks + 4];
  __shared__ float qs[D];

  const int tid = threadIdx.x;
  const int chunk = blockIdx.x;
  const int kvh = static_cast<int>(blockIdx.y) % g.Hkv;
  DecRow r;
  if (!dec_row(t, static_cast<int>(blockIdx.y) / g.Hkv, r)) return;
  const int own = r.pos / 64;
  const int n_chunks = own / kChunkBlocks + 1;
  // kernels below c_new are in the cache; the sequence's last row stores the others
  const int c_new = t.prev_kv_len != nullptr
                        ? num_kernels(min(uniform(t.prev_kv_len[r.seq]), r.kv_len), g.w, g.s)
                        : 0;
  if (r.last) compress_unscored<D>(g, r, kvh, chunk, c_new, keys, kern, tid);
  if (chunk >= n_chunks) return;                       // whole workgroup
  float* srow = scores + (static_cast<size_t>(r.row) * g.Hkv + kvh) * nb_stride;
  score_chunk<D, G>(g, t, r, kvh, chunk * kChunkBlocks, own, q, keys, kern, c_new, r.last, srow,
                    qs, u, tid);
}

}  // namespace

bool attn_decode_supported(const Geom& g, int dtype) {
  return dtype == INFLLM2_BF16 && g.B == 64 && (g.d == 64 || g.d == 128) && (g.G == 8 || g.G == 16);
}

size_t decode_workspace(const Geom& g, int rows, int nsplit) {
  const int pairs = rows * g.Hkv;
  return decode_layout(pairs).part +
         static_cast<size_t>(pairs) * nsplit * g.G * (g.d + 2) * sizeof(float);
}

// Splits of the decode step's attention: at least one selected block per wave, and up to twice
// that many splits while the (row, KV head) pairs leave compute units without a workgroup (at
// batch 8 x 2 KV heads: 16 splits, one workgroup per compute unit).
int decode_step_splits(const Geom& g, int rows) {
  const long long base = (g.topk + kStepWaves - 1) / kStepWaves;
  const long long pairs = std::max<long long>(1, static_cast<long long>(rows) * g.Hkv);
  const long long fill = device_cus() / pairs;
  return static_cast<int>(std::min<long long>(std::min(std::max(fill, base), 2 * base), g.topk));
}

bool decode_step_supported(const Geom& g, int dtype, const SeqTable& t, int nsplit) {
  if (!attn_decode_supported(g, dtype) || g.w != 32 || g.s != 16 || g.score_mode != 0) return false;
  if (static_cast<long long>(bound_rows(t)) * g.Hkv > 65535) return false;  // a grid row per pair
  if (nsplit < 1 || (g.topk + nsplit - 1) / nsplit > kMaxSplitBlocks) return false;
  return bound_blocks(t, 64) <= kMaxKeysPerThread * 64 * kStepWaves;
}

template <int NW, bool SEL>
static hipError_t launch_split_attention(const Geom& g, const SeqTable& t, const void* q,
                                         const void* k, const void* v, int32_t* idx,
                                         const float* scores, int nb_stride, int nsplit,
                                         void* workspace, void* out, float* lse,
                                         hipStream_t stream) {
  const int rows = bound_rows(t);
  if (rows == 0) return hipSuccess;
  if (nsplit < 1 || nsplit > 65535 || g.Hkv > 65535) return hipErrorInvalidValue;
  const dim3 grid(rows, g.Hkv, nsplit);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(out);
#define INFLLM2_DEC_CASE(DD, GG)                                                                \
  if (g.d == DD && g.G == GG) {                                                                 \
    hipLaunchKernelGGL((attn_decode<DD, GG, NW, SEL>), grid, dim3(64 * NW), 0, stream, g, t, qq, \
                       kk, vv, idx, scores, nb_stride, nsplit, workspace, oo, lse);             \
    return hipGetLastError();                                                                   \
  }
  INFLLM2_DEC_CASE(128, 16)
  INFLLM2_DEC_CASE(128, 8)
  INFLLM2_DEC_CASE(64, 16)
  INFLLM2_DEC_CASE(64, 8)
#undef INFLLM2_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_decode(const Geom& g, const SeqTable& t, const void* q, const void* k,
                              const void* v, const int32_t* idx, int nsplit, void* workspace,
                              void* out, float* lse, hipStream_t stream) {
  return launch_split_attention<kSplitWaves, false>(g, t, q, k, v, const_cast<int32_t*>(idx),
                                                    nullptr, 0, nsplit, workspace, out, lse,
                                                    stream);
}

// kernels must hold every kernel completed by t.prev_kv_len (null: none); the scoring launch
// computes and stores the rest.  The attention launch selects the blocks (and writes idx).
hipError_t launch_decode_step(const Geom& g, const SeqTable& t, const void* q,
                               void* kernels, const void* k, const void* v, float* scores,
                               int nb_stride, int32_t* idx, int nsplit, void* workspace,
                               void* out, float* lse, hipStream_t stream) {
  const int rows = bound_rows(t);
  if (rows == 0) return hipSuccess;
  const int max_blocks = std::max(1, bound_blocks(t, 64));
  const int max_chunks = (max_blocks + kChunkBlocks - 1) / kChunkBlocks;
  if (static_cast<long long>(rows) * g.Hkv > 65535) return hipErrorInvalidValue;
  const dim3 grid(max_chunks, rows * g.Hkv);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  uint16_t* kc = static_cast<uint16_t*>(kernels);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  bool launched = false;
#define INFLLM2_SEL_CASE(DD, GG)                                                                \
  if (!launched && g.d == DD && g.G == GG) {                                                    \
    hipLaunchKernelGGL((decode_scores<DD, GG>), grid, dim3(kScoreThreads), 0, stream, g, t, qq, \
                       kk, kc, scores, nb_stride);                                              \
    launched = true;                                                                            \
  }
  INFLLM2_SEL_CASE(128, 16)
  INFLLM2_SEL_CASE(128, 8)
  INFLLM2_SEL_CASE(64, 16)
  INFLLM2_SEL_CASE(64, 8)
#undef INFLLM2_SEL_CASE
  if (!launched) return hipErrorInvalidValue;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_split_attention<kStepWaves, true>(g, t, q, k, v, idx, scores, nb_stride, nsplit,
                                                  workspace, out, lse, stream);
}

}  // namespace infllm2
