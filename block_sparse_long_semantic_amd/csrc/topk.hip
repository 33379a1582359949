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
#include "select.h"

namespace infllm2 {
namespace {

constexpr int kWaves = 4;

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
// with few rows (decoding): block b = 1024*e + thread.
constexpr int kWideWaves = 16;
constexpr int kWideThreads = 64 * kWideWaves;

template <int NPT>
__global__ void __launch_bounds__(kWideThreads)
topk_wide(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
          int32_t* __restrict__ idx) {
  __shared__ SelectScratch<kWideWaves, NPT> sm;
  const int tid = threadIdx.x;
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
  uint32_t key[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int blk = kWideThreads * e + tid;
    const float sc = srow[min(blk, nb - 1)];
    const bool forced = blk < g.n_init || blk >= local_lo;
    key[e] = (blk < nb && !forced) ? order_key(sc) : 0u;
  }
  wg_select<kWideWaves, NPT>(key, own, g.topk, g.n_init, g.n_local, out, sm);
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
