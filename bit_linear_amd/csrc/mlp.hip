// Intermediate of the gated MLP block around the layer: h = gelu(gate) * up
// (Spark-X2.5-4B GGUF page, "The model": a GELU feed-forward block; ASHQ1 page,
// Architecture: ffn_gate, ffn_up and ffn_down).  gate and up are the two
// segments of the fused layer's bf16 output [M][2I]; GELU is the exact
// v Phi(v) = v erfc(-v / sqrt 2) / 2; the product is rounded once to bf16,
// the input of the down projection.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;

// v Phi(v) with Phi(v) = erfc(-v / sqrt 2) / 2: relatively accurate in the
// negative tail, where 1 + erf(v / sqrt 2) would cancel
__device__ __forceinline__ float gelu(float v) { return 0.5f * v * erfcf(v * -0.70710678118654752f); }

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
  for (int q = 0; q < 4; ++q) {
    const float lo = gelu(bf16_to_f32(g[q] & 0xFFFFu)) * bf16_to_f32(u[q] & 0xFFFFu);
    const float hi = gelu(bf16_to_f32(g[q] >> 16)) * bf16_to_f32(u[q] >> 16);
    o[q] = pack_bf16x2(lo, hi);
  }
  *reinterpret_cast<u32x4 *>(a.h + m * a.I + j) = o;
}

}  // namespace

hipError_t launch_geglu(const GegluArgs &a, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.M) * (a.I / 8);
  return launch_kernel(reinterpret_cast<const void *>(geglu_kernel), dim3((n + kThreads - 1) / kThreads),
                       dim3(kThreads), 0, s, a);
}

}  // namespace dvssq
