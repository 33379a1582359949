// Group-shared top-k block selection (MiniCPM4 paper summary, section 2.1.1: each query token
// selects the KV blocks with the highest relevance; section 2.1.2: the query heads of a group
// share the same top blocks).  One wavefront (a workgroup of its own) per (query row, KV head):
//   * the row's reachable scores live in registers as order-preserving 32-bit keys, block
//     b = 64*e + lane in register e; forced blocks (initial and local) are set aside;
//   * the (topk - |forced|)-th largest key is located by a radix select over the keys' actual
//     range, from the smallest key or, for topk - |forced| <= 128, from a lower bound of the
//     wanted key (the smallest of the lanes' second-largest keys): the first pass bins
//     (key - lo) >> s into 256 LDS counters (s the smallest shift that fits max - lo), later
//     passes split the chosen bin 256 ways; it stops when the whole bin is wanted, or the bin
//     holds one key value, or at most 64 keys, which are then gathered one per lane and
//     finished by a bitwise search over their offsets in the bin;
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

// One wave per (query row, KV head).
template <int NPL>
__global__ void __launch_bounds__(64)
topk_kernel(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
            int32_t* __restrict__ idx) {
  __shared__ WaveSelectLds sm;
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const int kvh = item % g.Hkv;
  int b, j;
  if (!locate(t, item / g.Hkv, [&](int s) { return t.q_len[s]; }, b, j)) return;
  const int row = uniform(static_cast<int>(t.q_start[b])) + j;
  const int pos = uniform(t.q_pos0[b]) + j;
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
  uint32_t kmin1 = 0xFFFFFFFFu;                            // smallest key - 1
  uint32_t m1 = 0u, m2 = 0u;                               // the lane's two largest keys
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int blk = 64 * e + lane;
    const bool forced = blk < g.n_init || blk >= local_lo;
    key[e] = (blk < nb && !forced) ? order_key(sc[e]) : 0u;     // 0: not a candidate
    kmin1 = min(kmin1, key[e] - 1u);                             // 0 wraps past every key
    m2 = max(m2, min(m1, key[e]));
    m1 = max(m1, key[e]);
  }

  // Threshold: keys above thr are taken; of the keys equal to it, the first n_eq in block order
  // (n_eq < 0: all of them).
  uint32_t thr = 0xFFFFFFFFu;
  int n_eq = 0;
  if (want > 0) {
    uint32_t kmin = wave_min_u32(kmin1) + 1u;
    const uint32_t kmax = wave_max_u32(m1);
    // every lane holds two keys at or above the smallest lane's second largest, so at least 128
    // keys lie at or above it: for want <= 128 so does the wanted key, and the first pass can
    // start there (over the 128K scores: 1.05 passes per row instead of 1.9)
    if (want <= 128) kmin = max(kmin, wave_min_u32(m2));
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.hist[4 * lane + i] = 0;
    // the current bin is [blo, blo + span]; since blo >= kmin > 0, the single unsigned test
    // (k - blo) <= span also rejects the non-candidates (k = 0 wraps past it)
    uint32_t blo = kmin;
    uint32_t span = kmax - kmin;
    int s = span == 0u ? 0 : max(0, 32 - __clz(static_cast<int>(span)) - 8);
    const uint64_t above_lane = ~((2ull << lane) - 1);   // lanes over this one (none for 63)
    int w = want;                                        // still wanted within the bin
    for (;;) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const uint32_t r = key[e] - blo;
        if (r <= span) atomicAdd(&sm.hist[r >> s], 1);
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
      span = (1u << s) - 1u;                             // s <= 24
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
        // gather the bin's keys (one per lane, as offsets from blo) and finish with a bitwise
        // search over the s offset bits: t is the largest offset with at least w keys at or
        // above it (lanes past the bin hold 0, never counted: every candidate offset is > 0)
        int base = 0;
#pragma unroll
        for (int e = 0; e < NPL; ++e) {
          const uint32_t r = key[e] - blo;
          const bool in = r <= span;
          const unsigned long long m = __ballot(in);
          if (in) sm.bin_key[base + prefix_count(m)] = r;
          base += __popcll(m);
        }
        __syncthreads();
        const uint32_t ri = lane < d_count ? sm.bin_key[lane] : 0u;
        uint32_t t = 0u;
        int n_ge = d_count;
        for (int bit = s - 1; bit >= 0; --bit) {
          const uint32_t cand = t | (1u << bit);
          const int c = __popcll(__ballot(ri >= cand));
          if (c >= w) {
            t = cand;
            n_ge = c;
            if (c == w) break;
          }
        }
        thr = blo + t;
        n_eq = n_ge == w ? -1 : w - __popcll(__ballot(lane < d_count && ri > t));
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

// The same selection by one workgroup of 8 waves per (query row, KV head), for launches with
// few rows (decoding): the radix select of select.h, up to 8 blocks per thread.
constexpr int kWideWaves = 8;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kWideKeys = 8;

__global__ void __launch_bounds__(kWideThreads)
topk_wide(Geom g, SeqTable t, const float* __restrict__ scores, int nb_stride,
          int32_t* __restrict__ idx) {
  __shared__ uint32_t keys[kWideKeys * kWideThreads];
  __shared__ WgSelectLds<kWideWaves> sm;
  const int item = blockIdx.x;
  const int kvh = item % g.Hkv;
  int b, j;
  if (!locate(t, item / g.Hkv, [&](int s) { return t.q_len[s]; }, b, j)) return;
  const int row = uniform(static_cast<int>(t.q_start[b])) + j;
  const int pos = uniform(t.q_pos0[b]) + j;
  const size_t pair = static_cast<size_t>(row) * g.Hkv + kvh;
  int32_t* out = idx + pair * g.topk;
  wg_select<kWideWaves, kWideKeys>(g, pos / g.B, scores + pair * nb_stride,
                                   [&](int e, int blk) { out[e] = blk; }, keys, sm,
                                   static_cast<int>(threadIdx.x));
}

}  // namespace

hipError_t launch_topk(const Geom& g, const SeqTable& t, const float* scores, int nb_stride,
                       int32_t* idx, hipStream_t stream) {
  const int max_blocks = bound_blocks(t, g.B);
  const int items = bound_rows(t) * g.Hkv;
  if (items == 0) return hipSuccess;
  if (items <= 1024 && max_blocks <= kWideKeys * kWideThreads) {
    hipLaunchKernelGGL(topk_wide, dim3(items), dim3(kWideThreads), 0, stream, g, t, scores,
                       nb_stride, idx);
    return hipGetLastError();
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
