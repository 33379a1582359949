// Group-shared top-k selection of one (query row, KV head) by a whole workgroup (MiniCPM4 paper
// summary, section 2.1.1: each query token selects its most relevant KV blocks; section 2.1.2:
// one selection per query-head group), for launches with few rows (decoding): the selection
// kernel's small-batch form, and the decode step's attention launch, where every split
// workgroup of a (row, KV head) selects the pair's blocks itself.
//
// Scores map to order-preserving unsigned keys (-0 ranks as +0).  Forced blocks (the first
// n_init and the n_local ending at the query's own block) are always taken; among the others
// the best by (score descending, block ascending) fill the rest of topk; the selection is
// written ascending, padded with -1.
#pragma once

#include "dpp.h"
#include "internal.h"

namespace infllm2 {

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x == 0.f) x = 0.f;                          // -0 ranks as +0
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int prefix_count(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// LDS of wg_select.
template <int NW>
struct WgSelectLds {
  int hist[2][256];
  int wsum[NW][2];
  uint32_t wmin[NW], wmax[NW], wlow[NW];
  int wquads[NW];
  uint32_t bin_key[64];
  int bin_blk[64];
  int nbin;
  int digit, above, count;
};

// Group-shared top-k of one (row, kv head) by a workgroup of NW waves, from its stored block
// scores srow[0 .. own] (up to KPT per thread); the p-th entry of the ascending selection goes
// out as emit(p, block) (p < topk; -1 for the padding of a row with at most topk blocks).  The
// (topk - forced)-th largest order-preserving key among the non-forced blocks is located by a
// radix select over the keys' actual range: the first pass bins (key - min) >> s into 256 LDS
// counters (s the smallest shift that fits max - min), each later pass splits the chosen bin 256
// ways.  It stops when every key of the chosen bin is wanted, or the bin holds a single key value
// (taken in block order), or the bin holds at most 64 keys: then one wave ranks those keys
// exactly (key descending, block ascending) and marks the wanted ones.  `keys` (LDS, one word
// per block) holds the keys for the ordered output.  The scores must come from an earlier launch
// (plain loads).  Every thread of the workgroup must call it.
template <int NW, int KPT, typename Emit>
__device__ __forceinline__ void wg_select(const Geom& g, int own, const float* srow, Emit emit,
                                          uint32_t* keys, WgSelectLds<NW>& sm, int tid) {
  constexpr int T = 64 * NW;
  constexpr uint32_t kTaken = 0xFFFFFFFFu;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nb = own + 1;
  if (nb <= g.topk) {
    for (int e = tid; e < g.topk; e += T) emit(e, e < nb ? e : -1);
    return;
  }
  const int local_lo = max(0, own - g.n_local + 1);
  const int init_end = min(g.n_init, nb);
  const int n_forced = init_end + (own - local_lo + 1) - max(0, init_end - local_lo);
  const int npt = (nb + T - 1) / T;
  // every score load is issued before any is used
  float sc[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    sc[e] = e < npt ? srow[min(e * T + tid, nb - 1)] : 0.f;
  uint32_t kr[KPT];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int blk = e * T + tid;
    const bool forced = blk < g.n_init || blk >= local_lo;
    kr[e] = (e < npt && blk < nb && !forced) ? order_key(sc[e]) : 0u;   // 0: not a candidate
    if (e < npt && blk < nb) keys[blk] = kr[e];
    if (kr[e] != 0u) {
      kmin = min(kmin, kr[e]);
      kmax = max(kmax, kr[e]);
    }
  }
  // A lower bound of the wanted key: the smallest of the thread quads' largest candidate keys.
  // Every quad that holds a candidate has one at or above it, so once at least `want` quads do,
  // the wanted key (the want-th largest) is at or above it too, and the first pass bins only the
  // keys from there up.
  uint32_t qmax = 0u;
#pragma unroll
  for (int e = 0; e < KPT; ++e) qmax = max(qmax, kr[e]);
  qmax = max(qmax, dpp_u32<kDppXor1>(qmax));
  qmax = max(qmax, dpp_u32<kDppXor2>(qmax));
  const uint32_t qlow = wave_min_u32(qmax != 0u ? qmax : 0xFFFFFFFFu);
  const int nquads = __popcll(__ballot(qmax != 0u && (lane & 3) == 0));
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sm.wmin[w] = kmin;
    sm.wmax[w] = kmax;
    sm.wlow[w] = qlow;
    sm.wquads[w] = nquads;
  }
  if (tid < 256) {
    sm.hist[0][tid] = 0;
    sm.hist[1][tid] = 0;
  }
  if (tid == 0) sm.nbin = 0;
  __syncthreads();
  uint32_t low = 0xFFFFFFFFu;
  int quads = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    kmin = min(kmin, sm.wmin[ww]);
    kmax = max(kmax, sm.wmax[ww]);
    low = min(low, sm.wlow[ww]);
    quads += sm.wquads[ww];
  }
  int want = g.topk - n_forced;                         // still wanted in the current bin
  if (quads >= want) kmin = max(kmin, low);             // keys below cannot be the wanted one
  // keys >= hi are taken, keys in [lo, hi) in block order until `want` are (want == 0: none)
  uint64_t lo = uint64_t{1} << 32, hi = uint64_t{1} << 32;
  if (want > 0) {
    uint32_t blo = kmin;                                // the current bin is [blo, bin_hi)
    uint64_t bin_hi = static_cast<uint64_t>(kmax) + 1;
    const uint32_t span = kmax - kmin;
    int s = span == 0u ? 0 : max(0, 32 - __clz(static_cast<int>(span)) - 8);
    const uint64_t above_lane = ~((2ull << lane) - 1);  // lanes over this one (none for 63)
    for (int pass = 0;; ++pass) {
      int* hist = sm.hist[pass & 1];
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t key = kr[e];
        if (key != 0u && key >= blo && key < bin_hi) atomicAdd(&hist[(key - blo) >> s], 1);
      }
      __syncthreads();
      if (w == 0) {
        // lane L holds bins 4L .. 4L+3 (zeroed again for the pass after next); the count over
        // them is summed from the lanes above by one ballot per bit (counts < 2^13)
        int c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[4 * lane + j];
          hist[4 * lane + j] = 0;
          tot += c[j];
        }
        int above = masked_count<13>(tot, above_lane);
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (above < want && above + c[j] >= want) {
            sm.digit = 4 * lane + j;
            sm.above = above;
            sm.count = c[j];
          }
          above += c[j];
        }
      }
      __syncthreads();
      blo += static_cast<uint32_t>(sm.digit) << s;
      bin_hi = static_cast<uint64_t>(blo) + (uint64_t{1} << s);
      want -= sm.above;
      const int count = sm.count;
      lo = blo;
      hi = bin_hi;
      if (count == want || s == 0) break;               // the whole bin is wanted, or one value
      if (count <= 64) {
        // rank the bin's keys in one wave and mark the wanted ones taken, the others dropped
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          const uint32_t key = kr[e];
          if (key != 0u && key >= blo && key < bin_hi) {
            const int slot = atomicAdd(&sm.nbin, 1);
            sm.bin_key[slot] = key;
            sm.bin_blk[slot] = e * T + tid;
          }
        }
        __syncthreads();
        if (w == 0) {
          const uint32_t ki = lane < count ? sm.bin_key[lane] : 0u;
          const int bi = lane < count ? sm.bin_blk[lane] : 0x7FFFFFFF;
          int rank = 0;
          for (int j = 0; j < count; ++j) {
            const uint32_t kj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ki), j));
            const int bj = __builtin_amdgcn_readlane(bi, j);
            rank += (kj > ki || (kj == ki && bj < bi)) ? 1 : 0;
          }
          if (lane < count) keys[bi] = rank < want ? kTaken : 0u;
        }
        __syncthreads();
        want = 0;                                       // the bin is decided: marks only
        hi = min(bin_hi, static_cast<uint64_t>(kTaken));
        lo = hi;
        break;
      }
      s = max(0, s - 8);
    }
  }
  // over the bin: taken; in the bin: taken in block order until `want` are.  Thread tid
  // writes blocks npt*tid .. npt*tid + npt - 1.
  const int blk_lo = npt * tid;
  const int blk_hi = min(nb, blk_lo + npt);
  int fixed = 0, eq = 0;
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const uint32_t key = keys[blk];
    const bool forced = blk < g.n_init || blk >= local_lo;
    fixed += (forced || (key != 0u && key >= hi)) ? 1 : 0;
    eq += (!forced && key != 0u && key >= lo && key < hi) ? 1 : 0;
  }
  // exclusive prefix counts over the workgroup: bit ballots within the wave, then wave totals
  const uint64_t below = (1ull << lane) - 1;
  int fixed_before = masked_count<4>(fixed, below);
  int eq_before = masked_count<4>(eq, below);
  const int fixed_wave = masked_count<4>(fixed, ~0ull);    // ballots: the whole wave takes part
  const int eq_wave = masked_count<4>(eq, ~0ull);
  if (lane == 0) {
    sm.wsum[w][0] = fixed_wave;
    sm.wsum[w][1] = eq_wave;
  }
  __syncthreads();
  for (int ww = 0; ww < w; ++ww) {
    fixed_before += sm.wsum[ww][0];
    eq_before += sm.wsum[ww][1];
  }
  int eq_seen = eq_before;
  int p = fixed_before + min(eq_seen, want);
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const uint32_t key = keys[blk];
    const bool forced = blk < g.n_init || blk >= local_lo;
    bool take = forced || (key != 0u && key >= hi);
    if (!take && key != 0u && key >= lo && key < hi) {
      take = eq_seen < want;
      ++eq_seen;
    }
    if (take && p < g.topk) emit(p, blk);               // p < topk unless keys are NaN
    p += take ? 1 : 0;
  }
}

}  // namespace infllm2
