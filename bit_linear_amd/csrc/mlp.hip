// Intermediate of the gated MLP block around the layer, h = gelu(gate) * up,
// as a kernel of its own (the prefill form of the block, and decode shapes
// whose down projection runs the prefill path): gate and up are the two
// segments of the fused layer's bf16 output [M][2I]; geglu_bf16x2 gives the
// GELU and the single bf16 rounding that the decode kernels use when they
// form h in their input loads.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;

// eight consecutive intermediate values per thread (I is a multiple of 64)
__global__ __launch_bounds__(kThreads) void geglu_kernel(GegluArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= static_cast<int64_t>(a.M) * (a.I / 8)) return;
  const int64_t m = e / (a.I / 8);
  const int j = static_cast<int>(e - m * (a.I / 8)) * 8;
  const uint16_t *row = a.ygu + m * 2 * a.I;
  const u32x4 g = *reinterpret_cast<const u32x4 *>(row + j);
  const u32x4 u = *reinterpret_cast<const u32x4 *>(row + a.I + j);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = geglu_bf16x2(g[q], u[q]);
  *reinterpret_cast<u32x4 *>(a.h + m * a.I + j) = o;
}

}  // namespace

hipError_t launch_geglu(const GegluArgs &a, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.M) * (a.I / 8);
  return launch_kernel(reinterpret_cast<const void *>(geglu_kernel), dim3((n + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, s, a);
}

}  // namespace dvssq
