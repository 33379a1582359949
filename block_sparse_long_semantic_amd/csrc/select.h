// Group-shared top-k selection of one (query row, KV head) by a whole workgroup (MiniCPM4 paper
// summary, section 2.1.1: each query token selects its most relevant KV blocks; section 2.1.2:
// one selection per query-head group).  Used where few rows are selected at once (decoding).
//
// Scores map to order-preserving unsigned keys (-0 ranks as +0).  Forced blocks (the first
// n_init and the n_local ending at the query's own block) are set aside; the (topk - forced)-th
// largest key among the others is found by a bitwise search (each thread counts its keys at or
// above the candidate, waves sum with bit ballots, the workgroup through LDS); keys equal to
// the threshold are taken in ascending block order; the selection is written ascending,
// padded with -1.
#pragma once

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

// Sum over the wave of a small per-lane count (< 128): one ballot per bit of the count.
__device__ __forceinline__ int wave_count(int c) {
  int tot = 0;
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) tot += __popcll(__ballot((c >> bit) & 1)) << bit;
  return tot;
}

// Workgroup total of a per-wave value through LDS slot `slot` (one barrier); *before receives
// the sum over the waves below this one.
template <int NW>
__device__ __forceinline__ int wg_sum(int (*buf)[NW], int slot, int w, int lane, int v,
                                      int* before) {
  if (lane == 0) buf[slot][w] = v;
  __syncthreads();
  int tot = 0, pre = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int c = buf[slot][i];
    tot += c;
    pre += i < w ? c : 0;
  }
  if (before) *before = pre;
  return tot;
}

// LDS scratch of wg_select.
template <int NW, int NPT>
struct SelectScratch {
  int cnt[2 + 2 * NPT][NW];
};

// Selects among blocks 0 .. own (own = query position / B) with keys in registers: thread tid of
// the NW-wave workgroup holds block 64*NW*e + tid in key[e] (0 for forced blocks and for blocks
// past own, non-zero otherwise).  Writes topk entries of `out`.  Every thread must call it.
template <int NW, int NPT>
__device__ void wg_select(const uint32_t (&key)[NPT], int own, int topk, int n_init, int n_local,
                          int32_t* __restrict__ out, SelectScratch<NW, NPT>& sm) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nb = own + 1;
  const int local_lo = max(0, own - n_local + 1);
  const int init_end = min(n_init, nb);
  const int n_forced = init_end + (own - local_lo + 1) - max(0, init_end - local_lo);
  const int want = topk - n_forced;

  // bitwise search for the threshold; buffers alternate so one barrier per step suffices
  uint32_t thr = 0u;
  int step = 0;
  for (int bit = 31; bit >= 0; --bit, ++step) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < NPT; ++e) c += key[e] >= cand ? 1 : 0;
    const int tot = wg_sum<NW>(sm.cnt, step & 1, w, lane, wave_count(c), nullptr);
    if (tot >= want) {
      thr = cand;
      if (tot == want) break;                              // same decision in every wave
    }
  }
  __syncthreads();                                         // the last step's counts are read
  int c_gt = 0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) c_gt += key[e] > thr ? 1 : 0;
  const int need_eq = want - wg_sum<NW>(sm.cnt, 0, w, lane, wave_count(c_gt), nullptr);

  int base_eq = 0, base = 0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int blk = NT * e + tid;
    const bool eq = key[e] == thr && key[e] != 0u;
    const unsigned long long meq = __ballot(eq);
    int eq_before;
    const int eq_tot = wg_sum<NW>(sm.cnt, 2 + 2 * e, w, lane, __popcll(meq), &eq_before);
    const bool take_eq = eq && (base_eq + eq_before + prefix_count(meq)) < need_eq;
    base_eq += eq_tot;
    const bool forced = blk < nb && (blk < n_init || blk >= local_lo);
    const bool sel = forced || key[e] > thr || take_eq;
    const unsigned long long ms = __ballot(sel);
    int sel_before;
    const int sel_tot = wg_sum<NW>(sm.cnt, 3 + 2 * e, w, lane, __popcll(ms), &sel_before);
    if (sel) out[base + sel_before + prefix_count(ms)] = blk;
    base += sel_tot;
  }
  for (int p = base + tid; p < topk; p += NT) out[p] = -1;
}

}  // namespace infllm2
