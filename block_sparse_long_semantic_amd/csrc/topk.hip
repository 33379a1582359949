// Group-shared top-k block selection (MiniCPM4 paper summary, section 2.1.1: each query token
// selects the KV blocks with the highest relevance; section 2.1.2: the query heads of a group
// share the same top blocks).  One wavefront per (query row, KV head):
//   * the row's reachable scores live in registers, block b = 64*e + lane;
//   * forced blocks (initial and local) are set aside;
//   * the (topk - |forced|)-th largest score is found by a bitwise search over order-preserving
//     32-bit keys, each step counting "key >= candidate" with wave ballots, stopping as soon as
//     exactly the wanted number of keys lies above the threshold;
//   * keys equal to the threshold are taken in ascending block order (ties -> lower index);
//   * the selection is written in ascending block order with ballot prefix counts.
#include "internal.h"

namespace infllm2 {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.f) x = 0.f;                          // -0 ranks as +0
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int prefix_count(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Sum over the wave of a small per-lane count (< 128): one ballot per bit of the count.
__device__ __forceinline__ int wave_count(int c) {
  int tot = 0;
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) tot += __popcll(__ballot((c >> bit) & 1)) << bit;
  return tot;
}

// work_prefix counts query rows.
template <int NPL>
__global__ void __launch_bounds__(64 * kWaves)
topk_kernel(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
            int32_t* __restrict__ idx) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int total = t.work_prefix[t.n] * g.Hkv;
  if (item >= total) return;
  const int vrow = item / g.Hkv;
  const int kvh = item % g.Hkv;
  const int b = find_seq(t, vrow);
  const int j = vrow - t.work_prefix[b];
  const int row = t.q_start[b] + j;
  const int pos = t.q_pos0[b] + j;
  const int own = pos / g.B;
  const int nb = own + 1;
  int32_t* out = idx + (static_cast<size_t>(row) * g.Hkv + kvh) * g.topk;
  if (nb <= g.topk) {
    for (int e = lane; e < g.topk; e += 64) out[e] = e < nb ? e : -1;
    return;
  }
  const float* srow = scores + (static_cast<size_t>(row) * g.Hkv + kvh) * nb_stride;
  const int local_lo = max(0, own - g.n_local + 1);
  const int init_end = min(g.n_init, nb);
  const int n_forced = init_end + (own - local_lo + 1) - max(0, init_end - local_lo);
  const int want = g.topk - n_forced;

  // every load is issued (index clamped into the row) before any is used
  float sc[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) sc[e] = srow[min(64 * e + lane, nb - 1)];
  uint32_t key[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int blk = 64 * e + lane;
    const bool forced = blk < g.n_init || blk >= local_lo;
    key[e] = (blk < nb && !forced) ? order_key(sc[e]) : 0u;     // 0: not a candidate
  }

  // bitwise search: each lane counts its keys >= the candidate, the wave sums the counts
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) c += key[e] >= cand ? 1 : 0;
    const int cnt = wave_count(c);
    if (cnt >= want) {
      thr = cand;
      if (cnt == want) break;
    }
  }
  int c_gt = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) c_gt += key[e] > thr ? 1 : 0;
  const int need_eq = want - wave_count(c_gt);

  int base_eq = 0, base = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int blk = 64 * e + lane;
    const bool eq = key[e] == thr && key[e] != 0u;
    const unsigned long long meq = __ballot(eq);
    const bool take_eq = eq && (base_eq + prefix_count(meq)) < need_eq;
    base_eq += __popcll(meq);
    const bool forced = blk < nb && (blk < g.n_init || blk >= local_lo);
    const bool sel = forced || key[e] > thr || take_eq;
    const unsigned long long ms = __ballot(sel);
    if (sel) out[base + prefix_count(ms)] = blk;
    base += __popcll(ms);
  }
  for (int p = base + lane; p < g.topk; p += 64) out[p] = -1;
}

// The same selection with one workgroup of 16 waves per (query row, KV head), for launches
// with few rows (decoding): block b = 1024*e + thread, counts summed across the waves in LDS.
constexpr int kWideWaves = 16;
constexpr int kWideThreads = 64 * kWideWaves;

__device__ __forceinline__ int wide_sum(int (*buf)[kWideWaves], int slot, int w, int lane, int v,
                                        int* before) {
  if (lane == 0) buf[slot][w] = v;
  __syncthreads();
  int tot = 0, pre = 0;
#pragma unroll
  for (int i = 0; i < kWideWaves; ++i) {
    const int c = buf[slot][i];
    tot += c;
    pre += i < w ? c : 0;
  }
  if (before) *before = pre;
  return tot;
}

template <int NPT>
__global__ void __launch_bounds__(kWideThreads)
topk_wide(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
          int32_t* __restrict__ idx) {
  __shared__ int cnt[2 + 2 * NPT][kWideWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int item = blockIdx.x;
  const int vrow = item / g.Hkv;
  const int kvh = item % g.Hkv;
  const int b = find_seq(t, vrow);
  const int j = vrow - t.work_prefix[b];
  const int row = t.q_start[b] + j;
  const int pos = t.q_pos0[b] + j;
  const int own = pos / g.B;
  const int nb = own + 1;
  int32_t* out = idx + (static_cast<size_t>(row) * g.Hkv + kvh) * g.topk;
  if (nb <= g.topk) {                                       // uniform over the workgroup
    for (int e = tid; e < g.topk; e += kWideThreads) out[e] = e < nb ? e : -1;
    return;
  }
  const float* srow = scores + (static_cast<size_t>(row) * g.Hkv + kvh) * nb_stride;
  const int local_lo = max(0, own - g.n_local + 1);
  const int init_end = min(g.n_init, nb);
  const int n_forced = init_end + (own - local_lo + 1) - max(0, init_end - local_lo);
  const int want = g.topk - n_forced;

  uint32_t key[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int blk = kWideThreads * e + tid;
    const bool forced = blk < g.n_init || blk >= local_lo;
    key[e] = (blk < nb && !forced) ? order_key(srow[blk]) : 0u;
  }

  // bitwise search for the threshold; buffers alternate so one barrier per step suffices
  uint32_t thr = 0u;
  int step = 0;
  for (int bit = 31; bit >= 0; --bit, ++step) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < NPT; ++e) c += __popcll(__ballot(key[e] >= cand));
    const int tot = wide_sum(cnt, step & 1, w, lane, c, nullptr);
    if (tot >= want) {
      thr = cand;
      if (tot == want) break;                              // same decision in every wave
    }
  }
  __syncthreads();                                         // the last step's counts are read
  int c_gt = 0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) c_gt += __popcll(__ballot(key[e] > thr));
  const int need_eq = want - wide_sum(cnt, 0, w, lane, c_gt, nullptr);

  int base_eq = 0, base = 0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int blk = kWideThreads * e + tid;
    const bool eq = key[e] == thr && key[e] != 0u;
    const unsigned long long meq = __ballot(eq);
    int eq_before;
    const int eq_tot = wide_sum(cnt, 2 + 2 * e, w, lane, __popcll(meq), &eq_before);
    const bool take_eq = eq && (base_eq + eq_before + prefix_count(meq)) < need_eq;
    base_eq += eq_tot;
    const bool forced = blk < nb && (blk < g.n_init || blk >= local_lo);
    const bool sel = forced || key[e] > thr || take_eq;
    const unsigned long long ms = __ballot(sel);
    int sel_before;
    const int sel_tot = wide_sum(cnt, 3 + 2 * e, w, lane, __popcll(ms), &sel_before);
    if (sel) out[base + sel_before + prefix_count(ms)] = blk;
    base += sel_tot;
  }
  for (int p = base + tid; p < g.topk; p += kWideThreads) out[p] = -1;
}

}  // namespace

hipError_t launch_topk(const Geom& g, const SeqTable& t, const float* scores, int nb_stride,
                       int max_blocks, int32_t* idx, hipStream_t stream) {
  const int items = t.work_prefix[t.n] * g.Hkv;
  if (items == 0) return hipSuccess;
  if (items <= 1024 && max_blocks <= 4 * kWideThreads) {
    const int npt = (max_blocks + kWideThreads - 1) / kWideThreads;
#define INFLLM2_TOPK_WIDE(N)                                                                  \
    if (npt <= N) {                                                                           \
      hipLaunchKernelGGL(topk_wide<N>, dim3(items), dim3(kWideThreads), 0, stream, g, t,     \
                         scores, nb_stride, idx);                                             \
      return hipGetLastError();                                                               \
    }
    INFLLM2_TOPK_WIDE(1)
    INFLLM2_TOPK_WIDE(2)
    INFLLM2_TOPK_WIDE(4)
#undef INFLLM2_TOPK_WIDE
  }
  const dim3 grid((items + kWaves - 1) / kWaves);
  const dim3 block(64 * kWaves);
  const int npl = (max_blocks + 63) / 64;
#define INFLLM2_TOPK_CASE(N)                                                                  \
  if (npl <= N) {                                                                             \
    hipLaunchKernelGGL(topk_kernel<N>, grid, block, 0, stream, g, t, scores, nb_stride, idx); \
    return hipGetLastError();                                                                 \
  }
  INFLLM2_TOPK_CASE(1)
  INFLLM2_TOPK_CASE(2)
  INFLLM2_TOPK_CASE(4)
  INFLLM2_TOPK_CASE(8)
  INFLLM2_TOPK_CASE(16)
  INFLLM2_TOPK_CASE(32)
  INFLLM2_TOPK_CASE(64)
#undef INFLLM2_TOPK_CASE
  return hipErrorInvalidValue;
}

}  // namespace infllm2
