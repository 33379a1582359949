// Backward of the block-sparse attention for gfx950, with the block selection held fixed (the
// selection is piecewise constant in Q and K; MiniCPM4 model card "Efficient Model
// Architecture" and paper summary section 2.1 describe the sparse attention as trainable).
//
// For every query row and head, with P the forward's softmax over the attended tokens j,
// delta = dO . O and dS_j = P_j (dO . v_j - delta):
//   dQ  = scale * sum_j dS_j k_j           (tile kernel in attn_tile.hip, query-major)
//   dK_j += scale * dS_j q,  dV_j += P_j dO  (this file, key-block-major)
//
// The key/value gradients are accumulated per KV block: a reverse index lists, for every
// (KV head, block), the query rows that selected it (count, scan, scatter), and one workgroup
// per chunk of such a list keeps the block's K and V in registers, streams the rows' Q, dO,
// lse and delta through an LDS ring and accumulates dK and dV on the matrix cores.  Chunks of
// one block add their float32 results atomically, so dK and dV are summed in an order that
// may differ between calls (results agree to float32 rounding).
#include <algorithm>

#include "internal.h"

namespace infllm2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 512;       // query rows per dK/dV work item (one KV block's list slice)
constexpr int kRows = 32;         // (token, head) rows per step: two 16-row MFMA tiles
constexpr int kSlots = 4;         // LDS ring depth of the dK/dV kernel
// The reverse index is split into windows of query rows whose q and dO together take about
// this many bytes, processed one window after the other, so that the rows a window's blocks
// stream stay in the last-level cache instead of being fetched from HBM once per block.
constexpr long long kWindowBytes = 64LL << 20;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `later` steps of PER loads each are still in flight (later <= MAXL).
template <int PER, int MAXL>
__device__ __forceinline__ void wait_steps(int later) {
  if constexpr (MAXL > 0) {
    if (later >= MAXL) {
      wait_vmcnt<MAXL * PER>();
      return;
    }
    wait_steps<PER, MAXL - 1>(later);
  } else {
    wait_vmcnt<0>();
  }
}

__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Global KV block numbering: block j of sequence b is b * bound_blocks(t, 64) + j (a slot of
// the longest sequence's block count per sequence).

// Transposing LDS reads for the B operands of one step: for each 16-dim tile nd, two reads (row
// tiles u = 0, 1) at addresses a0[nd], a1[nd], waited for in the same statement (the compiler
// does not track loads it cannot see).
template <int NT>
__device__ __forceinline__ void read_tr(const uint32_t (&a0)[NT], const uint32_t (&a1)[NT],
                                        uint64_t (&r)[NT][2]);

template <>
__device__ __forceinline__ void read_tr<8>(const uint32_t (&a0)[8], const uint32_t (&a1)[8],
                                           uint64_t (&r)[8][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n"
      "ds_read_b64_tr_b16 %1, %17\n"
      "ds_read_b64_tr_b16 %2, %18\n"
      "ds_read_b64_tr_b16 %3, %19\n"
      "ds_read_b64_tr_b16 %4, %20\n"
      "ds_read_b64_tr_b16 %5, %21\n"
      "ds_read_b64_tr_b16 %6, %22\n"
      "ds_read_b64_tr_b16 %7, %23\n"
      "ds_read_b64_tr_b16 %8, %24\n"
      "ds_read_b64_tr_b16 %9, %25\n"
      "ds_read_b64_tr_b16 %10, %26\n"
      "ds_read_b64_tr_b16 %11, %27\n"
      "ds_read_b64_tr_b16 %12, %28\n"
      "ds_read_b64_tr_b16 %13, %29\n"
      "ds_read_b64_tr_b16 %14, %30\n"
      "ds_read_b64_tr_b16 %15, %31\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]),
        "=&v"(r[2][1]), "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[4][0]), "=&v"(r[4][1]),
        "=&v"(r[5][0]), "=&v"(r[5][1]), "=&v"(r[6][0]), "=&v"(r[6][1]), "=&v"(r[7][0]),
        "=&v"(r[7][1])
      : "v"(a0[0]), "v"(a1[0]), "v"(a0[1]), "v"(a1[1]), "v"(a0[2]), "v"(a1[2]), "v"(a0[3]),
        "v"(a1[3]), "v"(a0[4]), "v"(a1[4]), "v"(a0[5]), "v"(a1[5]), "v"(a0[6]), "v"(a1[6]),
        "v"(a0[7]), "v"(a1[7])
      : "memory");
}

template <>
__device__ __forceinline__ void read_tr<4>(const uint32_t (&a0)[4], const uint32_t (&a1)[4],
                                           uint64_t (&r)[4][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]),
        "=&v"(r[2][1]), "=&v"(r[3][0]), "=&v"(r[3][1])
      : "v"(a0[0]), "v"(a1[0]), "v"(a0[1]), "v"(a1[1]), "v"(a0[2]), "v"(a1[2]), "v"(a0[3]),
        "v"(a1[3])
      : "memory");
}

// LDS reads of the dK/dV kernel's ring and row list.  Written as asm statements that wait for
// their own results: a plain LDS load would make the compiler first wait for every LDS-DMA
// load in flight, which would stall the ring's prefetch on every step.

// N 4-byte reads at independent addresses, one wait.
template <int N>
__device__ __forceinline__ void lds_read_i32s(const uint32_t (&a)[N], int (&r)[N]);

template <>
__device__ __forceinline__ void lds_read_i32s<5>(const uint32_t (&a)[5], int (&r)[5]) {
  asm volatile(
      "ds_read_b32 %0, %5\n"
      "ds_read_b32 %1, %6\n"
      "ds_read_b32 %2, %7\n"
      "ds_read_b32 %3, %8\n"
      "ds_read_b32 %4, %9\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_i32s<3>(const uint32_t (&a)[3], int (&r)[3]) {
  asm volatile(
      "ds_read_b32 %0, %3\n"
      "ds_read_b32 %1, %4\n"
      "ds_read_b32 %2, %5\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2])
      : "v"(a[0]), "v"(a[1]), "v"(a[2])
      : "memory");
}

// First reads of a step: A operands of row tile 0 (q[ks] at a[ks], dout[ks] at a[ks] + OFF),
// the lse and delta of both row tiles (ld[0..3] at la + 0, 64, 128, 192) and the rows of the
// two tiles' tokens (p0 at e0, p1 at e1).
template <int KS, int OFF>
__device__ __forceinline__ void read_first(const uint32_t (&a)[KS], uint32_t la, uint32_t e0,
                                           uint32_t e1, bf16x8 (&qa)[KS], bf16x8 (&da)[KS],
                                           f32x4 (&ld)[4], int& p0, int& p1);

template <>
__device__ __forceinline__ void read_first<4, 8192>(const uint32_t (&a)[4], uint32_t la,
                                                    uint32_t e0, uint32_t e1, bf16x8 (&qa)[4],
                                                    bf16x8 (&da)[4], f32x4 (&ld)[4], int& p0,
                                                    int& p1) {
  asm volatile(
      "ds_read_b128 %0, %14\n"
      "ds_read_b128 %1, %14 offset:8192\n"
      "ds_read_b128 %2, %15\n"
      "ds_read_b128 %3, %15 offset:8192\n"
      "ds_read_b128 %4, %16\n"
      "ds_read_b128 %5, %16 offset:8192\n"
      "ds_read_b128 %6, %17\n"
      "ds_read_b128 %7, %17 offset:8192\n"
      "ds_read_b128 %8, %18\n"
      "ds_read_b128 %9, %18 offset:64\n"
      "ds_read_b128 %10, %18 offset:128\n"
      "ds_read_b128 %11, %18 offset:192\n"
      "ds_read_b32 %12, %19\n"
      "ds_read_b32 %13, %20\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qa[0]), "=&v"(da[0]), "=&v"(qa[1]), "=&v"(da[1]), "=&v"(qa[2]), "=&v"(da[2]),
        "=&v"(qa[3]), "=&v"(da[3]), "=&v"(ld[0]), "=&v"(ld[1]), "=&v"(ld[2]), "=&v"(ld[3]),
        "=&v"(p0), "=&v"(p1)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(la), "v"(e0), "v"(e1)
      : "memory");
}

template <>
__device__ __forceinline__ void read_first<2, 4096>(const uint32_t (&a)[2], uint32_t la,
                                                    uint32_t e0, uint32_t e1, bf16x8 (&qa)[2],
                                                    bf16x8 (&da)[2], f32x4 (&ld)[4], int& p0,
                                                    int& p1) {
  asm volatile(
      "ds_read_b128 %0, %10\n"
      "ds_read_b128 %1, %10 offset:4096\n"
      "ds_read_b128 %2, %11\n"
      "ds_read_b128 %3, %11 offset:4096\n"
      "ds_read_b128 %4, %12\n"
      "ds_read_b128 %5, %12 offset:64\n"
      "ds_read_b128 %6, %12 offset:128\n"
      "ds_read_b128 %7, %12 offset:192\n"
      "ds_read_b32 %8, %13\n"
      "ds_read_b32 %9, %14\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qa[0]), "=&v"(da[0]), "=&v"(qa[1]), "=&v"(da[1]), "=&v"(ld[0]), "=&v"(ld[1]),
        "=&v"(ld[2]), "=&v"(ld[3]), "=&v"(p0), "=&v"(p1)
      : "v"(a[0]), "v"(a[1]), "v"(la), "v"(e0), "v"(e1)
      : "memory");
}

// A operands of one row tile: q[ks] at a[ks], dout[ks] at a[ks] + OFF (the dO matrix).
template <int KS, int OFF>
__device__ __forceinline__ void read_a(const uint32_t (&a)[KS], bf16x8 (&qa)[KS], bf16x8 (&da)[KS]);

template <>
__device__ __forceinline__ void read_a<4, 8192>(const uint32_t (&a)[4], bf16x8 (&qa)[4],
                                                bf16x8 (&da)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:8192\n"
      "ds_read_b128 %2, %9\n"
      "ds_read_b128 %3, %9 offset:8192\n"
      "ds_read_b128 %4, %10\n"
      "ds_read_b128 %5, %10 offset:8192\n"
      "ds_read_b128 %6, %11\n"
      "ds_read_b128 %7, %11 offset:8192\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qa[0]), "=&v"(da[0]), "=&v"(qa[1]), "=&v"(da[1]), "=&v"(qa[2]), "=&v"(da[2]),
        "=&v"(qa[3]), "=&v"(da[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

template <>
__device__ __forceinline__ void read_a<2, 4096>(const uint32_t (&a)[2], bf16x8 (&qa)[2],
                                                bf16x8 (&da)[2]) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:4096\n"
      "ds_read_b128 %2, %5\n"
      "ds_read_b128 %3, %5 offset:4096\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(qa[0]), "=&v"(da[0]), "=&v"(qa[1]), "=&v"(da[1])
      : "v"(a[0]), "v"(a[1])
      : "memory");
}

// ---------------------------------------------------------------------------------------------
// Fill float32 ranges with zeros: sequence b's KV rows of dk and dv (sequences strided over
// grid.y).
__global__ void __launch_bounds__(256) zero_kv_grads(SeqTable t, int row_elems, float* dk,
                                                      float* dv) {
  for (int b = blockIdx.y; b < t.n; b += gridDim.y) {
    const size_t n4 = static_cast<size_t>(uniform(t.kv_len[b])) * row_elems / 4;
    const size_t base4 = static_cast<size_t>(uniform(static_cast<int32_t>(t.kv_start[b]))) * row_elems / 4;
    f32x4* k4 = reinterpret_cast<f32x4*>(dk) + base4;
    f32x4* v4 = reinterpret_cast<f32x4*>(dv) + base4;
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * 256) {
      k4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      v4[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

__global__ void __launch_bounds__(256) zero_ints(int* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// One workgroup per query row (r = dense row item): delta[row, h] = dO[row, h] . O[row, h]
// in float32 from the stored bf16 tensors, and the row's selected blocks counted per
// (KV head, global block) segment.
template <int D>
__global__ void __launch_bounds__(256) bwd_prep(Geom g, SeqTable t, const uint16_t* __restrict__ out,
                                                const uint16_t* __restrict__ dout,
                                                const int32_t* __restrict__ idx,
                                                float* __restrict__ delta, int* __restrict__ cnt,
                                                int n_blocks, int win_rows) {
  const int r = blockIdx.x;
  int b, j;
  if (!locate(t, r, [&](int s) { return t.q_len[s]; }, b, j)) return;
  const Seq sq = load_seq(t, b);
  const int row = sq.q_start + j;
  const int gb0 = b * bound_blocks(t, 64);
  constexpr int CPH = D / 8;  // 16-byte chunks per head
  const int n = g.Hq * CPH;   // a multiple of 64: whole waves only
  for (int c = threadIdx.x; c < n; c += 256) {
    const size_t off = static_cast<size_t>(row) * g.Hq * D + 8 * static_cast<size_t>(c);
    const uint4 o8 = *reinterpret_cast<const uint4*>(out + off);
    const uint4 d8 = *reinterpret_cast<const uint4*>(dout + off);
    const uint32_t ow[4] = {o8.x, o8.y, o8.z, o8.w};
    const uint32_t dw[4] = {d8.x, d8.y, d8.z, d8.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(ow[i] << 16), __uint_as_float(dw[i] << 16), s);
      s = fmaf(__uint_as_float(ow[i] & 0xFFFF0000u), __uint_as_float(dw[i] & 0xFFFF0000u), s);
    }
#pragma unroll
    for (int m = 1; m < CPH; m <<= 1) s += __shfl_xor(s, m);
    if ((c & (CPH - 1)) == 0) delta[static_cast<size_t>(row) * g.Hq + c / CPH] = s;
  }
  const int per_row = g.Hkv * g.topk;
  const int nb = (sq.kv_len + 63) / 64;      // entries outside the sequence are ignored
  for (int e = threadIdx.x; e < per_row; e += 256) {
    const int blk = idx[static_cast<size_t>(row) * per_row + e];
    if (blk >= 0 && blk < nb)
      atomicAdd(&cnt[((r / win_rows) * g.Hkv + e / g.topk) * n_blocks + gb0 + blk], 1);
  }
}

// Single workgroup: exclusive scans of the segment sizes (seg_off) and of their work items of
// up to kChunk rows (item_off); both end with the totals.  cnt is reset to zero for the scatter.
__global__ void __launch_bounds__(1024) bwd_scan(int* __restrict__ cnt, int* __restrict__ seg_off,
                                                 int* __restrict__ item_off, int n_seg) {
  __shared__ int wsum[2][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (n_seg + 1023) / 1024;
  const int s0 = min(n_seg, tid * per), s1 = min(n_seg, s0 + per);
  int c_tot = 0, i_tot = 0;
  for (int s = s0; s < s1; ++s) {
    const int c = cnt[s];
    c_tot += c;
    i_tot += (c + kChunk - 1) / kChunk;
  }
  int ci = c_tot, ii = i_tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int yc = __shfl_up(ci, off), yi = __shfl_up(ii, off);
    if (lane >= off) {
      ci += yc;
      ii += yi;
    }
  }
  if (lane == 63) {
    wsum[0][w] = ci;
    wsum[1][w] = ii;
  }
  __syncthreads();
  int cb = ci - c_tot, ib = ii - i_tot;
  for (int ww = 0; ww < w; ++ww) {
    cb += wsum[0][ww];
    ib += wsum[1][ww];
  }
  for (int s = s0; s < s1; ++s) {
    const int c = cnt[s];
    seg_off[s] = cb;
    item_off[s] = ib;
    cb += c;
    ib += (c + kChunk - 1) / kChunk;
    cnt[s] = 0;
  }
  if (tid == 1023) {
    seg_off[n_seg] = cb;
    item_off[n_seg] = ib;
  }
}

// One workgroup per query row: the row index appended to the list of every segment it selected.
__global__ void __launch_bounds__(256) bwd_scatter(Geom g, SeqTable t, const int32_t* __restrict__ idx,
                                                   int* __restrict__ fill,
                                                   const int* __restrict__ seg_off,
                                                   int* __restrict__ list, int n_blocks,
                                                   int win_rows) {
  const int r = blockIdx.x;
  int b, j;
  if (!locate(t, r, [&](int s) { return t.q_len[s]; }, b, j)) return;
  const Seq sq = load_seq(t, b);
  const int row = sq.q_start + j;
  const int gb0 = b * bound_blocks(t, 64);
  const int per_row = g.Hkv * g.topk;
  const int nb = (sq.kv_len + 63) / 64;
  for (int e = threadIdx.x; e < per_row; e += 256) {
    const int blk = idx[static_cast<size_t>(row) * per_row + e];
    if (blk >= 0 && blk < nb) {
      const int seg = ((r / win_rows) * g.Hkv + e / g.topk) * n_blocks + gb0 + blk;
      list[seg_off[seg] + atomicAdd(&fill[seg], 1)] = row;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV.  A work item is up to kChunk rows of one segment (KV head kvh, block blk of sequence
// b).  Wave w owns keys 16w .. 16w+15 of the block, with their K and V rows as the B operand of
//   S  = Q K^T     (16 (token, head) rows x 16 keys per v_mfma_f32_16x16x32_bf16)
//   dP = dO V^T
// The accumulators hold S[row 4*q4+i][key c16] per lane, which is exactly the A operand (keys x
// rows) of the products over rows:
//   dV[key][dim] += sum_rows P[row][key]  dO[row][dim]
//   dK[key][dim] += sum_rows dS[row][key] Q[row][dim]
// taken 32 rows (two row tiles) per MFMA; the B operands are read from LDS with transposing
// reads.  A step stages 32 (token, head) rows: Q and dO (row-major, 16-byte chunks XOR-swizzled
// by row) and the rows' lse and delta, all by global_load_lds.
template <int D, int G>
__global__ void __launch_bounds__(256, 2)
bwd_dkv(Geom g, SeqTable t, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
        const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
        const float* __restrict__ lse, const float* __restrict__ delta,
        const int* __restrict__ seg_off, const int* __restrict__ item_off,
        const int* __restrict__ list, int n_seg, int n_blocks, float* __restrict__ dk,
        float* __restrict__ dv, int* __restrict__ work) {
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int TPS = kRows / G;           // tokens per step
  constexpr int MATB = kRows * D * 2;      // bytes of Q (or dO) per step
  constexpr int SLOT = 2 * MATB + 256;     // + lse[32], delta[32]
  constexpr int PER = CPR / 4 + 1;         // global_load_lds per thread per step
  static_assert(G == 8 || G == 16, "group size");
  __shared__ __attribute__((aligned(16))) unsigned char ring[kSlots][SLOT];
  __shared__ int ents[kChunk];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c16 = lane & 15;
  const int q4 = lane >> 4;
  const int Hq = g.Hq, Hkv = g.Hkv;
  const float qscale = g.scale * kLog2e;
  const int n_items = item_off[n_seg];
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&ring[0][0]));
  const uint32_t ents_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)&ents[0]));

  // per-lane LDS offsets within a slot's matrix
  //   A operand (rows 16u + c16, chunk 4ks + q4):  arow + 16 * ((4ks + q4) ^ ax)
  //   transposing read (rows 16u + 4q4 + c16/4, dims 16nd + 4(c16%4)):
  //       trow + 32 * (nd ^ (tx >> 1)) + 16 * (((c16 & 3) >> 1) ^ (tx & 1)) + 8 * (c16 & 1)
  const int ax = c16 & (CPR - 1);
  const uint32_t arow = static_cast<uint32_t>(c16 * D * 2);
  const int trr = 4 * q4 + (c16 >> 2);
  const int tx = trr & (CPR - 1);
  const uint32_t trow = static_cast<uint32_t>(trr * D * 2) +
                        16u * static_cast<uint32_t>(((c16 & 3) >> 1) ^ (tx & 1)) +
                        8u * static_cast<uint32_t>(c16 & 1);

  // Work items are taken in order from a shared counter (zero at launch), kGrab at a time: they
  // still run row window by row window, and a workgroup that finishes early takes more, so the
  // last workgroups end within an item or two of each other (a fixed item-to-workgroup assignment
  // leaves the slowest of the persistent workgroups well behind the mean; at 128K the backward
  // call measured 78.1 / 78.3 / 79.0 / 79.8 ms with 1 / 2 / 4 / 8 items per update)
  constexpr int kGrab = 1;
  __shared__ int s_item;
  for (int item = 0, item_end = 0;; ++item) {
    if (item == item_end) {
      __syncthreads();                                   // every thread has read s_item
      if (tid == 0) s_item = atomicAdd(work, kGrab);
      __syncthreads();
      item = uniform(s_item);
      item_end = item + kGrab;
    }
    if (item >= n_items) break;
    // segment of the item: the last s with item_off[s] <= item
    int lo = 0, hi = n_seg;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (item_off[mid] <= item) lo = mid;
      else hi = mid;
    }
    const int seg = lo;
    const int kvh = (seg / n_blocks) % Hkv;       // segment = (row window, KV head, block)
    const int gb = seg % n_blocks;
    const int nbs = bound_blocks(t, 64);
    const int b = gb / nbs;
    const Seq sq = load_seq(t, b);
    const int key0 = 64 * (gb - b * nbs);
    const int e0 = seg_off[seg] + (item - item_off[seg]) * kChunk;
    const int ne = min(kChunk, seg_off[seg + 1] - e0);
    const int kv_len = sq.kv_len;
    const int pos_shift = sq.q_pos0 - sq.q_start;   // position = row + pos_shift

    __syncthreads();                                     // previous item's reads of ents done
    for (int e = tid; e < ne; e += 256) ents[e] = list[e0 + e];

    // the wave's 16 keys (clamped to the sequence; keys past its end get P = 0)
    bf16x8 kf[KS], vf[KS];
    {
      const int key = min(key0 + 16 * w + c16, kv_len - 1);
      const size_t off = (static_cast<size_t>(sq.kv_start + key) * Hkv + kvh) * D + 8 * q4;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = *reinterpret_cast<const bf16x8*>(k + off + 32 * ks);
        vf[ks] = *reinterpret_cast<const bf16x8*>(v + off + 32 * ks);
      }
    }
    f32x4 adv[NT], adk[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      adv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      adk[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();                                     // ents visible

    const int nsteps = (ne + TPS - 1) / TPS;
    // Loads of step j into slot sl: unit U = 256J + 64w + lane of the Q|dO matrices holds row
    // (U / CPR) % 32 (token j*TPS + row/G, head row%G), stored chunk U % CPR = source chunk
    // XOR (row % CPR); lanes 0-3 of each wave then load 4 rows of lse (waves 0, 1) or delta
    // (waves 2, 3).
    auto issue = [&](int j, int sl) {
      unsigned char* base = &ring[sl][0];
      constexpr int NJ = CPR / 4;
      // the rows of every load of this lane (entries past the chunk repeat entry 0)
      uint32_t ea[NJ + 1];
#pragma unroll
      for (int J = 0; J <= NJ; ++J) {
        const int U = 256 * J + 64 * w + lane;
        const int row = J < NJ ? (U / CPR) % 32 : 4 * ((4 * w + lane) & 7);
        const int e = j * TPS + row / G;
        ea[J] = ents_lds + 4u * static_cast<uint32_t>(e < ne ? e : 0);
      }
      int grow[NJ + 1];
      lds_read_i32s<NJ + 1>(ea, grow);
#pragma unroll
      for (int J = 0; J < NJ; ++J) {
        const int U = 256 * J + 64 * w + lane;
        const int mat = U / (32 * CPR);
        const int row = (U / CPR) % 32;
        const int ch = (U % CPR) ^ (row & (CPR - 1));
        const uint16_t* src = (mat ? dout : q) +
                              (static_cast<size_t>(grow[J]) * Hq + kvh * G + row % G) * D + 8 * ch;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + (256 * J + 64 * w) * 16), 16, 0, 0);
      }
      if (lane < 4) {
        const int vv = 4 * w + lane;               // 16-byte unit of the lse|delta area
        const int row = 4 * (vv & 7);
        const float* src =
            (vv >> 3 ? delta : lse) + static_cast<size_t>(grow[NJ]) * Hq + kvh * G + row % G;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + 2 * MATB + 64 * w), 16, 0, 0);
      }
    };

    for (int j = 0; j < kSlots - 1 && j < nsteps; ++j) issue(j, j);
    for (int j = 0; j < nsteps; ++j) {
      wait_steps<PER, kSlots - 2>(min(kSlots - 2, nsteps - 1 - j));
      raw_barrier();                                     // step j landed for every wave
      const uint32_t slot = ring_lds + static_cast<uint32_t>((j % kSlots) * SLOT);
      // S and dP for the two row tiles
      f32x4 sacc[2], pacc[2];
      f32x4 ld[4];                                       // lse u0, lse u1, delta u0, delta u1
      int prow[2];                                       // the tiles' query rows
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        pacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint32_t aa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          aa[ks] = slot + static_cast<uint32_t>(u * 16 * D * 2) + arow +
                   16u * static_cast<uint32_t>((4 * ks + q4) ^ ax);
        bf16x8 qa[KS], da[KS];
        if (u == 0) {
          const int e0 = min(j * TPS + (4 * q4) / G, kChunk - 1);
          const int e1 = min(j * TPS + (16 + 4 * q4) / G, kChunk - 1);
          read_first<KS, MATB>(aa, slot + 2 * MATB + 16 * q4, ents_lds + 4u * e0, ents_lds + 4u * e1,
                               qa, da, ld, prow[0], prow[1]);
        } else {
          read_a<KS, MATB>(aa, qa, da);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          sacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kf[ks], sacc[u], 0, 0, 0);
          pacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[ks], vf[ks], pacc[u], 0, 0, 0);
        }
      }
      // P and dS; rows 16u + 4q4 + i belong to token j*TPS + (16u + 4q4)/G
      const int key = key0 + 16 * w + c16;
      float pv[2][4], dsv[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = j * TPS + (16 * u + 4 * q4) / G;
        const int pos = e < ne ? prow[u] + pos_shift : -1;
        const f32x4 l4 = ld[u];
        const f32x4 d4 = ld[2 + u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = key > pos ? 0.f
                                    : __builtin_amdgcn_exp2f(fmaf(sacc[u][i], qscale, -l4[i] * kLog2e));
          pv[u][i] = p;
          dsv[u][i] = p * (pacc[u][i] - d4[i]);
        }
      }
      const bf16x8 pa = bf16x8{(__bf16)pv[0][0], (__bf16)pv[0][1], (__bf16)pv[0][2], (__bf16)pv[0][3],
                               (__bf16)pv[1][0], (__bf16)pv[1][1], (__bf16)pv[1][2], (__bf16)pv[1][3]};
      const bf16x8 sa = bf16x8{(__bf16)dsv[0][0], (__bf16)dsv[0][1], (__bf16)dsv[0][2], (__bf16)dsv[0][3],
                               (__bf16)dsv[1][0], (__bf16)dsv[1][1], (__bf16)dsv[1][2], (__bf16)dsv[1][3]};
      // dV += P^T dO, dK += dS^T Q: B operands by transposing reads of the two row tiles
      uint32_t a0[NT], a1[NT];
      uint64_t tr[NT][2];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        a0[n] = slot + MATB + trow + 32u * static_cast<uint32_t>(n ^ (tx >> 1));
        a1[n] = a0[n] + 16 * D * 2;
      }
      read_tr<NT>(a0, a1, tr);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint64_t both[2] = {tr[n][0], tr[n][1]};
        adv[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, both), adv[n], 0, 0, 0);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        a0[n] -= MATB;
        a1[n] -= MATB;
      }
      read_tr<NT>(a0, a1, tr);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint64_t both[2] = {tr[n][0], tr[n][1]};
        adk[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, __builtin_bit_cast(bf16x8, both), adk[n], 0, 0, 0);
      }
      // refill the slot every wave finished with before this step's barrier
      if (j + kSlots - 1 < nsteps) issue(j + kSlots - 1, (j + kSlots - 1) % kSlots);
    }
    // accumulate: lane holds dV/dK[key 16w + 4q4 + i][dim 16n + c16]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + 16 * w + 4 * q4 + i;
      if (key < kv_len) {
        const size_t off = (static_cast<size_t>(sq.kv_start + key) * Hkv + kvh) * D + c16;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          unsafeAtomicAdd(dv + off + 16 * n, adv[n][i]);
          unsafeAtomicAdd(dk + off + 16 * n, adk[n][i] * g.scale);
        }
      }
    }
  }
}

}  // namespace

// Query rows per window of the reverse index (at least 1024).
int bwd_window_rows(const Geom& g) {
  const long long per_row = 2LL * g.Hq * g.d * 2;          // q and dO, bf16
  return static_cast<int>(std::max<long long>(1024, kWindowBytes / per_row));
}

static int bwd_blocks(const SeqTable& t) { return t.n * bound_blocks(t, 64); }

long long bwd_segments(const Geom& g, const SeqTable& t) {
  const int w = bwd_window_rows(g);
  const long long n_win = std::max(1, (bound_rows(t) + w - 1) / w);
  return n_win * g.Hkv * bwd_blocks(t);
}

size_t bwd_workspace(const Geom& g, const SeqTable& t) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t n_seg = static_cast<size_t>(bwd_segments(g, t));
  const size_t entries = static_cast<size_t>(bound_rows(t)) * g.Hkv * g.topk;
  return al(static_cast<size_t>(t.q_rows) * g.Hq * 4) + 3 * al((n_seg + 1) * 4) +
         al(std::max<size_t>(entries, 1) * 4);
}

// The workspace must be bwd_workspace() bytes.
hipError_t launch_attn_bwd(const Geom& g, const SeqTable& t, const void* q, const void* k,
                           const void* v, const int32_t* idx, const void* out, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, void* workspace,
                           hipStream_t stream) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const int n_blocks = bwd_blocks(t);
  const int n_seg = static_cast<int>(bwd_segments(g, t));
  const int win_rows = bwd_window_rows(g);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* delta = reinterpret_cast<float*>(ws);
  ws += al(static_cast<size_t>(t.q_rows) * g.Hq * 4);
  int* cnt = reinterpret_cast<int*>(ws);               // n_seg counts, then the dK/dV work counter
  ws += al((static_cast<size_t>(n_seg) + 1) * 4);
  int* seg_off = reinterpret_cast<int*>(ws);
  ws += al((static_cast<size_t>(n_seg) + 1) * 4);
  int* item_off = reinterpret_cast<int*>(ws);
  ws += al((static_cast<size_t>(n_seg) + 1) * 4);
  int* list = reinterpret_cast<int*>(ws);

  const int rows = bound_rows(t);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  const uint16_t* oo = static_cast<const uint16_t*>(out);
  const uint16_t* dd = static_cast<const uint16_t*>(dout);
  hipError_t e;

  if (t.max_kv_len > 0) {
    const int row_elems = g.Hkv * g.d;
    const long long n4 = static_cast<long long>(t.max_kv_len) * row_elems / 4;
    const int gx = static_cast<int>(std::min<long long>((n4 + 255) / 256, 1024));
    hipLaunchKernelGGL(zero_kv_grads, dim3(gx, std::min(t.n, 65535)), dim3(256), 0, stream, t,
                       row_elems, dk, dv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_ints, dim3(std::min((n_seg + 256) / 256, 1024)), dim3(256), 0, stream,
                     cnt, n_seg + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.d == 128) {
    hipLaunchKernelGGL(bwd_prep<128>, dim3(rows), dim3(256), 0, stream, g, t, oo, dd, idx,
                       delta, cnt, n_blocks, win_rows);
  } else {
    hipLaunchKernelGGL(bwd_prep<64>, dim3(rows), dim3(256), 0, stream, g, t, oo, dd, idx,
                       delta, cnt, n_blocks, win_rows);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scan, dim3(1), dim3(1024), 0, stream, cnt, seg_off, item_off, n_seg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scatter, dim3(rows), dim3(256), 0, stream, g, t, idx, cnt, seg_off,
                     list, n_blocks, win_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // dQ: the forward's tile kernel in its gradient form (it forms its own tiles from the rows)
  if ((e = launch_attn_tile_dq(g, t, q, k, v, idx, dout, lse, delta, dq, stream)) != hipSuccess)
    return e;

  // dK, dV: persistent grid over the work items (their count is known on the device only),
  // taken from the counter after the segment counts
  const long long bound = static_cast<long long>(rows) * g.Hkv * g.topk / kChunk + n_seg;
  const int cus = device_cus();
  const int grid = static_cast<int>(std::max<long long>(1, std::min<long long>(bound, 2LL * cus)));
#define INFLLM2_DKV_CASE(DD, GG)                                                                \
  if (g.d == DD && g.G == GG) {                                                                 \
    hipLaunchKernelGGL((bwd_dkv<DD, GG>), dim3(grid), dim3(256), 0, stream, g, t, qq, kk, vv, dd, \
                       lse, delta, seg_off, item_off, list, n_seg, n_blocks, dk, dv,            \
                       cnt + n_seg);                                                            \
    return hipGetLastError();                                                                   \
  }
  INFLLM2_DKV_CASE(128, 16)
  INFLLM2_DKV_CASE(128, 8)
  INFLLM2_DKV_CASE(64, 16)
  INFLLM2_DKV_CASE(64, 8)
#undef INFLLM2_DKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllm2
