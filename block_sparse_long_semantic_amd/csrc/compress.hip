// Semantic-kernel compression: mean-pool of keys over windows of w tokens every s tokens
// (MiniCPM4 paper summary, section 2.1.2: fine-grained semantic kernels represent each KV
// block).  HBM-bound: every key row is read once per window containing it (w/s = 2 times for
// the measured geometry; the second read hits L2) and each kernel row is written once.
//
// Exactness: window sums are accumulated in float64.  With p significant bits per input (8 for
// bf16, 24 for f32) and w terms, no partial sum rounds while the window's nonzero inputs span at
// most 53 - p - ceil(log2 w) binary exponents (40 for bf16 at w = 32); then the single rounding
// to the storage dtype (to nearest even, straight from float64) is the exact mean's
// rounding.  Wider windows may round in the sum (at most one unit in the last place off).
#include <algorithm>

#include "internal.h"

namespace infllm2 {
namespace {

constexpr int kTile = 16;        // kernels per workgroup
constexpr int kThreads = 256;

// A persistent grid walks the tiles of 16 kernels of every sequence (the kernels completed
// after prev_kv_len[b]); the host knows only a bound on their number.
template <bool kBf16>
__global__ void __launch_bounds__(kThreads)
compress_kernel(Geom g, SeqTable t, const void* __restrict__ k, void* __restrict__ out) {
  auto first_kernel = [&](int b) {
    return t.prev_kv_len != nullptr ? num_kernels(min(t.prev_kv_len[b], t.kv_len[b]), g.w, g.s) : 0;
  };
  auto tiles_of = [&](int b) {
    return (num_kernels(t.kv_len[b], g.w, g.s) - first_kernel(b) + kTile - 1) / kTile;
  };
  const int total = count_items(t, tiles_of);
  const int cols = g.Hkv * g.d;
  const int ncg = cols / 8;
  const double inv_w = 1.0 / static_cast<double>(g.w);
  const bool pow2 = (g.w & (g.w - 1)) == 0;
  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int b, lt;
    locate(t, tile, tiles_of, b, lt);
    const Seq sq = load_seq(t, b);
    const int c0 = uniform(first_kernel(b)) + lt * kTile;
    const int c_hi = num_kernels(sq.kv_len, g.w, g.s);
    for (int it = threadIdx.x; it < kTile * ncg; it += kThreads) {
      const int c = c0 + it / ncg;
      const int cg = it % ncg;
      if (c >= c_hi) break;                    // items are ordered by kernel
      const size_t row0 = static_cast<size_t>(sq.kv_start) + static_cast<size_t>(g.s) * c;
      const size_t orow = static_cast<size_t>(sq.kc_start) + c;
      const size_t ooff = orow * cols + static_cast<size_t>(cg) * 8;
      if constexpr (kBf16) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + ooff) = window_mean_bf16x8(
            static_cast<const uint16_t*>(k) + row0 * cols + static_cast<size_t>(cg) * 8, cols, g.w);
      } else {
        double acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll 8
        for (int r = 0; r < g.w; ++r) {
          const size_t off = (row0 + r) * cols + static_cast<size_t>(cg) * 8;
          const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(k) + off);
          const float4 a = p[0], c2 = p[1];
          const float f[8] = {a.x, a.y, a.z, a.w, c2.x, c2.y, c2.z, c2.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(f[e]);
        }
        double mean[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) mean[e] = pow2 ? acc[e] * inv_w : acc[e] / g.w;
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + ooff);
        p[0] = make_float4(static_cast<float>(mean[0]), static_cast<float>(mean[1]),
                           static_cast<float>(mean[2]), static_cast<float>(mean[3]));
        p[1] = make_float4(static_cast<float>(mean[4]), static_cast<float>(mean[5]),
                           static_cast<float>(mean[6]), static_cast<float>(mean[7]));
      }
    }
  }
}

}  // namespace

hipError_t launch_compress(const Geom& g, int dtype, const SeqTable& t, const void* k,
                           void* kernels, hipStream_t stream) {
  const long long bound = static_cast<long long>(t.n) *
                          ((num_kernels(t.max_kv_len, g.w, g.s) + kTile - 1) / kTile);
  if (bound == 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<long long>(bound, 4LL * device_cus()));
  if (dtype == INFLLM2_BF16)
    hipLaunchKernelGGL(compress_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, g, t, k,
                       kernels);
  else
    hipLaunchKernelGGL(compress_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, g, t, k,
                       kernels);
  return hipGetLastError();
}

}  // namespace infllm2
