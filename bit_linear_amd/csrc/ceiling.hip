// Achievable-bandwidth reference for the decode path: a plain streaming read of
// a device buffer with the access pattern that measured fastest for reads of a
// few tens of MB on MI355X (256-thread workgroups, each reading one contiguous
// 16 KB chunk with 16-byte nontemporal loads, all four issued before the
// first use).  Nothing of the layer is computed; the bytes are folded into an
// xor that is stored only if it equals a constant no realistic buffer gives,
// so that the loads cannot be removed.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;                                   // 16-byte loads per lane
constexpr int64_t kChunk = int64_t(kThreads) * kLoads * 16;  // bytes per workgroup

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *src, int64_t n16, uint32_t *sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kLoads + threadIdx.x;
  u32x4 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int64_t o = base + static_cast<int64_t>(i) * kThreads;
    v[i] = o < n16 ? __builtin_nontemporal_load(src + o) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, void *sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t grid = (bytes + kChunk - 1) / kChunk;
  return launch_kernel_args(reinterpret_cast<const void *>(stream_read_kernel), dim3(static_cast<unsigned>(grid)),
                            dim3(kThreads), 0, s, static_cast<const u32x4 *>(buf), n16,
                            static_cast<uint32_t *>(sink));
}

}  // namespace dvssq
