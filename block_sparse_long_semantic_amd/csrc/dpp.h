// Cross-lane reductions of a wave by DPP moves (VALU, a few cycles each) instead of LDS-routed
// shuffles (ds_bpermute, whose latency chains up in a reduction tree).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infllm2 {

// DPP controls: quad permutations [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2), mirror within
// each 8-lane half row, mirror within each 16-lane row.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppRowRor1 = 0x121;       // lane i of a 16-lane row takes lane (i - 1) mod 16

// Sums of lanes l and l ^ 16 (rows 0+1 and 2+3), and of lanes l and l ^ 32 (the two halves), by
// the gfx950 row swaps: swapping a value with itself and adding the two results pairs every lane
// with its partner; both partners get the same sum (the operands in the same order).
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of N = 4, 8 or 16 lanes; every lane of a group gets the same value
// (the same additions in a commuted order).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  if (N >= 8) x += dpp_f32<kDppHalfMirror>(x);
  if (N >= 16) x += dpp_f32<kDppMirror>(x);
  return x;
}

// Minimum / maximum over the whole wave (the result is uniform).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<kDppXor1>(x));
  x = min(x, dpp_u32<kDppXor2>(x));
  x = min(x, dpp_u32<kDppHalfMirror>(x));
  x = min(x, dpp_u32<kDppMirror>(x));
  const uint32_t a = min(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 0)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 16)));
  const uint32_t b = min(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 32)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 48)));
  return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<kDppXor1>(x));
  x = max(x, dpp_u32<kDppXor2>(x));
  x = max(x, dpp_u32<kDppHalfMirror>(x));
  x = max(x, dpp_u32<kDppMirror>(x));
  const uint32_t a = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 0)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 16)));
  const uint32_t b = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 32)),
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 48)));
  return max(a, b);
}

// Count of a small per-lane value c (0 <= c < 2^BITS) summed over the lanes selected by `mask`,
// by one ballot per bit.
template <int BITS>
__device__ __forceinline__ int masked_count(int c, uint64_t mask) {
  int tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b)
    tot += __popcll(__ballot((c >> b) & 1) & mask) << b;
  return tot;
}

}  // namespace infllm2
