// Group-shared top-k block selection (MiniCPM4 paper summary, section 2.1.1: each query token
// selects the KV blocks with the highest relevance; section 2.1.2: the query heads of a group
// share the same top blocks).  One wavefront (a workgroup of its own) per (query row, KV head):
//   * the row's reachable scores live in registers as order-preserving 32-bit keys, block
//     b = 64*e + lane in register e; forced blocks (initial and local) are set aside;
//   * the (topk - |forced|)-th largest key is located by a radix select over the keys' actual
//     range: the first pass bins (key - min) >> s into 256 LDS counters (s the smallest shift
//     that fits max - min), later passes split the chosen bin 256 ways; it stops when the
//     whole bin is wanted, or the bin holds one key value, or at most 64 keys, which are then
//     gathered in block order and ranked exactly;
//   * keys above the threshold are taken, keys equal to it in ascending block order (ties ->
//     lower index) as far as wanted; the selection is written ascending with ballot prefix
//     counts.
#include "dpp.h"
#include "internal.h"
#include "select.h"

namespace infllm2 {
namespace {

struct WaveSelectLds {
  int hist[256];
  uint32_t bin_key[64];
};

// work_prefix counts query rows.
template <int NPL>
__global__ void __launch_bounds__(64)
topk_kernel(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
            int32_t* __restrict__ idx) {
  __shared__ WaveSelectLds sm;
  const int lane = threadIdx.x;
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
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int blk = 64 * e + lane;
    const bool forced = blk < g.n_init || blk >= local_lo;
    key[e] = (blk < nb && !forced) ? order_key(sc[e]) : 0u;     // 0: not a candidate
    if (key[e] != 0u) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }

  // Threshold: keys above thr are taken; of the keys equal to it, the first n_eq in block order
  // (n_eq < 0: all of them).
  uint32_t thr = 0xFFFFFFFFu;
  int n_eq = 0;
  if (want > 0) {
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.hist[4 * lane + i] = 0;
    uint32_t blo = kmin;                                 // the current bin is [blo, bin_hi)
    uint64_t bin_hi = static_cast<uint64_t>(kmax) + 1;
    const uint32_t span = kmax - kmin;
    int s = span == 0u ? 0 : max(0, 32 - __clz(static_cast<int>(span)) - 8);
    const uint64_t above_lane = ~((2ull << lane) - 1);   // lanes over this one (none for 63)
    int w = want;                                        // still wanted within the bin
    for (;;) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const uint32_t k = key[e];
        if (k != 0u && k >= blo && k < bin_hi) atomicAdd(&sm.hist[(k - blo) >> s], 1);
      }
      __syncthreads();
      // lane L holds bins 4L .. 4L+3 (zeroed again for the next pass); the count of the bins
      // above them is summed from the lanes above by one ballot per bit (counts < 2^13)
      int c[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = sm.hist[4 * lane + i];
        sm.hist[4 * lane + i] = 0;
        tot += c[i];
      }
      int above = masked_count<13>(tot, above_lane);
      int digit = -1, d_above = 0, d_count = 0;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        if (above < w && above + c[i] >= w) {
          digit = 4 * lane + i;
          d_above = above;
          d_count = c[i];
        }
        above += c[i];
      }
      const int src = __ffsll(static_cast<unsigned long long>(__ballot(digit >= 0))) - 1;
      digit = __builtin_amdgcn_readlane(digit, src);
      d_above = __builtin_amdgcn_readlane(d_above, src);
      d_count = __builtin_amdgcn_readlane(d_count, src);
      blo += static_cast<uint32_t>(digit) << s;
      bin_hi = static_cast<uint64_t>(blo) + (uint64_t{1} << s);
      w -= d_above;
      if (d_count == w) {                                // every key of the bin is wanted
        thr = blo;
        n_eq = -1;
        break;
      }
      if (s == 0) {                                      // one key value, more keys than wanted
        thr = blo;
        n_eq = w;
        break;
      }
      if (d_count <= 64) {
        // gather the bin's keys in block order, rank them: thr is the key with fewer than w
        // keys above it and at least w at or above it
        int base = 0;
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
          const uint32_t k = key[e];
          const bool in = k != 0u && k >= blo && k < bin_hi;
          const unsigned long long m = __ballot(in);
          if (in) sm.bin_key[base + prefix_count(m)] = k;
          base += __popcll(m);
        }
        __syncthreads();
        const uint32_t ki = lane < d_count ? sm.bin_key[lane] : 0u;
        int gt = 0, ge = 0;
        for (int jj = 0; jj < d_count; ++jj) {
          const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ki), jj));
          gt += kj > ki ? 1 : 0;
          ge += kj >= ki ? 1 : 0;
        }
        const bool is_thr = lane < d_count && gt < w && w <= ge;
        const int t_src = __ffsll(static_cast<unsigned long long>(__ballot(is_thr))) - 1;
        thr = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ki), t_src));
        const int t_gt = __builtin_amdgcn_readlane(gt, t_src);
        const int t_ge = __builtin_amdgcn_readlane(ge, t_src);
        n_eq = (t_ge == w) ? -1 : w - t_gt;
        break;
      }
      s = max(0, s - 8);
    }
  }

  int base = 0;
  if (n_eq < 0) {
    // every key at or above thr is taken (thr >= the smallest candidate key, so thr > 0)
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      const int blk = 64 * e + lane;
      const bool forced = blk < nb && (blk < g.n_init || blk >= local_lo);
      const bool sel = forced || key[e] >= thr;
      const unsigned long long ms = __ballot(sel);
      if (sel) out[base + prefix_count(ms)] = blk;
      base += __popcll(ms);
    }
  } else {
    int seen_eq = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) {
      const int blk = 64 * e + lane;
      const bool eq = key[e] == thr && key[e] != 0u;
      const unsigned long long meq = __ballot(eq);
      const bool take_eq = eq && (seen_eq + prefix_count(meq)) < n_eq;
      seen_eq += __popcll(meq);
      const bool forced = blk < nb && (blk < g.n_init || blk >= local_lo);
      const bool sel = forced || key[e] > thr || take_eq;
      const unsigned long long ms = __ballot(sel);
      if (sel) out[base + prefix_count(ms)] = blk;
      base += __popcll(ms);
    }
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
  const dim3 grid(items);
  const dim3 block(64);
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
