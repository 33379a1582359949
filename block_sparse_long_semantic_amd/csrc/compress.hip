// Semantic-kernel compression: mean-pool of keys over windows of w tokens every s tokens
// (MiniCPM4 paper summary, section 2.1.2: fine-grained semantic kernels represent each KV
// block).  HBM-bound: every key row is read once per window containing it (w/s = 2 times for
// the measured geometry; the second read hits L2) and each kernel row is written once.
//
// Exactness: window sums are accumulated in float64.  For bf16 (8 significant bits) or f32
// inputs of ordinary magnitude these sums are exact, so the single rounding to the storage
// dtype below (to nearest even, straight from float64) reproduces the exact mean's rounding.
#include "internal.h"

namespace infllm2 {
namespace {

constexpr int kTile = 16;        // kernels per workgroup
constexpr int kThreads = 256;

// float64 -> bf16 bits, round to nearest even, in one step (no float32 double rounding).
// Keeps sign, 11 exponent bits and 7 fraction bits of the binary64 encoding; the rounded
// binary64 value then converts exactly to float32, whose top half is the bf16 encoding.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(x));
  const unsigned long long lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;            // 2^44 - 1 + lsb
  u &= ~((1ull << 45) - 1ull);
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

template <bool kBf16>
__global__ void __launch_bounds__(kThreads)
compress_kernel(Geom g, SeqTable t, const void* __restrict__ k, void* __restrict__ out) {
  const int tile = blockIdx.x;
  const int b = find_seq(t, tile);
  const int c0 = t.aux[b] + (tile - t.work_prefix[b]) * kTile;
  const int c_hi = num_kernels(t.kv_len[b], g.w, g.s);
  const int cols = g.Hkv * g.d;
  const int ncg = cols / 8;
  const double inv_w = 1.0 / static_cast<double>(g.w);
  const bool pow2 = (g.w & (g.w - 1)) == 0;
  for (int it = threadIdx.x; it < kTile * ncg; it += kThreads) {
    const int c = c0 + it / ncg;
    const int cg = it % ncg;
    if (c >= c_hi) break;                      // items are ordered by kernel
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    const size_t row0 = static_cast<size_t>(t.kv_start[b]) + static_cast<size_t>(g.s) * c;
#pragma unroll 8
    for (int r = 0; r < g.w; ++r) {
      const size_t off = (row0 + r) * cols + static_cast<size_t>(cg) * 8;
      if constexpr (kBf16) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k) + off);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += static_cast<double>(__uint_as_float(w4[e] << 16));
          acc[2 * e + 1] += static_cast<double>(__uint_as_float(w4[e] & 0xFFFF0000u));
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(k) + off);
        const float4 a = p[0], c2 = p[1];
        const float f[8] = {a.x, a.y, a.z, a.w, c2.x, c2.y, c2.z, c2.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(f[e]);
      }
    }
    const size_t orow = static_cast<size_t>(t.kc_start[b]) + c;
    const size_t ooff = orow * cols + static_cast<size_t>(cg) * 8;
    double mean[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mean[e] = pow2 ? acc[e] * inv_w : acc[e] / g.w;
    if constexpr (kBf16) {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w4[e] = static_cast<uint32_t>(f64_to_bf16_rne(mean[2 * e])) |
                (static_cast<uint32_t>(f64_to_bf16_rne(mean[2 * e + 1])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + ooff) =
          make_uint4(w4[0], w4[1], w4[2], w4[3]);
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + ooff);
      p[0] = make_float4(static_cast<float>(mean[0]), static_cast<float>(mean[1]),
                         static_cast<float>(mean[2]), static_cast<float>(mean[3]));
      p[1] = make_float4(static_cast<float>(mean[4]), static_cast<float>(mean[5]),
                         static_cast<float>(mean[6]), static_cast<float>(mean[7]));
    }
  }
}

}  // namespace

hipError_t launch_compress(const Geom& g, int dtype, const SeqTable& t, const void* k,
                           void* kernels, hipStream_t stream) {
  const int tiles = t.work_prefix[t.n];
  if (tiles == 0) return hipSuccess;
  if (dtype == INFLLM2_BF16)
    hipLaunchKernelGGL(compress_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, g, t, k,
                       kernels);
  else
    hipLaunchKernelGGL(compress_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, g, t, k,
                       kernels);
  return hipGetLastError();
}

}  // namespace infllm2
