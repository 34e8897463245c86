// Dense materialization of a packed layer: the bf16 weight W = (W_hat + U V_seg) H^T
// in the original input domain, rows in original output order, so that
// x W^T is the layer's forward (Spark-X2.5-4B-Hadamard-GSQ model card,
// Quickstart & Inference Guide: materialize_weights() turns the quantized MLP
// weights into plain BF16; the layer itself: MiniCPM5-2B-Hadamard-GSQ model
// card, Mathematical Foundations 2, runtime equation).  H is symmetric, so
// each Hadamard block of a rotated row is transformed by H_b again.
//
// One wavefront per (1 to 16 packed rows, Hadamard block): each lane dequantizes VPL
// consecutive inputs (INT4 nibbles with the group scale, or INT8 codes with the
// row scale), adds the row's low-rank term U[p] . V_seg[:, k] in fp32, runs the
// register FWHT, scales by 1/sqrt(b) and rounds once to bf16.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;

// rows per wavefront: their loads are issued together
template <int VPL>
constexpr int rows_per_wave() { return VPL <= 4 ? 16 : VPL <= 8 ? 8 : VPL <= 16 ? 2 : 1; }

template <int VPL>
__global__ __launch_bounds__(kThreads) void materialize_kernel(DenseArgs a) {
  constexpr int B = 64 * VPL;
  constexpr int NR = rows_per_wave<VPL>();
  const int lane = threadIdx.x & 63;
  const int nblk = a.K / B;
  // wavefront-uniform row indices: idx, U and the INT8 scale come through scalar loads
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t ngrp = (static_cast<int64_t>(a.N) + NR - 1) / NR;
  if (wid >= ngrp * nblk) return;
  const int p0 = static_cast<int>(wid / nblk) * NR, bb = static_cast<int>(wid % nblk);
  const int k0 = bb * B + lane * VPL;
  float v[NR][VPL];
  int col[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int p = min(p0 + j, a.N - 1);   // rows past N repeat the last row and are not stored
    col[j] = a.idx[p];
    if (p < a.n4) {
      const uint8_t *row = a.q4 + static_cast<int64_t>(p) * (a.K / 2);
      const float s = bf16_to_f32(a.s4[static_cast<int64_t>(p) * (a.K / 64) + k0 / 64]);
      if constexpr (VPL >= 4) {
        // four inputs k .. k+3 (k % 4 == 0) share the 4 bytes of their run of 8:
        // the low nibbles for k % 8 == 0, the high ones for k % 8 == 4
#pragma unroll
        for (int h = 0; h < VPL / 4; ++h) {
          const int k = k0 + 4 * h;
          const uint32_t w = *reinterpret_cast<const uint32_t *>(row + 4 * (k >> 3));
          const int sh = (k & 4) ? 4 : 0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[j][4 * h + q] = static_cast<float>(static_cast<int>((w >> (8 * q + sh)) & 15u) - 8) * s;
        }
      } else {
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
          const int k = k0 + q, jj = k & 7;
          const uint32_t byte = row[4 * (k >> 3) + (jj & 3)];
          v[j][q] = static_cast<float>(static_cast<int>(jj < 4 ? (byte & 15u) : (byte >> 4)) - 8) * s;
        }
      }
    } else {
      const int8_t *row = a.q8 + static_cast<int64_t>(p - a.n4) * a.K + k0;
      const float s = a.s8[p - a.n4];
#pragma unroll
      for (int q = 0; q < VPL; ++q) v[j][q] = static_cast<float>(row[q]) * s;
    }
  }
  // low-rank term of each row: its segment's r rows of V, each loaded once per
  // wavefront for both segments and shared by the wavefront's rows
  const int seg_cols = a.N / a.n_seg;
  const uint16_t *v0 = a.V + k0;
  const uint16_t *v1 = a.V + static_cast<int64_t>(a.n_seg - 1) * a.r * a.K + k0;
  for (int i = 0; i < a.r; ++i) {
    float w0[VPL], w1[VPL];
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      w0[q] = bf16_to_f32(v0[static_cast<int64_t>(i) * a.K + q]);
      w1[q] = bf16_to_f32(v1[static_cast<int64_t>(i) * a.K + q]);
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int p = min(p0 + j, a.N - 1);
      const float ui = bf16_to_f32(a.U[static_cast<int64_t>(p) * a.r + i]);
      const bool s1 = col[j] >= seg_cols;
#pragma unroll
      for (int q = 0; q < VPL; ++q) v[j][q] = fmaf(ui, s1 ? w1[q] : w0[q], v[j][q]);
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    fwht_wave<VPL>(v[j], lane);
    if (p0 + j >= a.N) continue;
    uint16_t *out = a.w + static_cast<int64_t>(col[j]) * a.K + k0;
    if constexpr (VPL == 1) {
      out[0] = f32_to_bf16(v[j][0] * a.hscale);
    } else {
#pragma unroll
      for (int q = 0; q < VPL; q += 2)
        *reinterpret_cast<uint32_t *>(out + q) = pack_bf16x2(v[j][q] * a.hscale, v[j][q + 1] * a.hscale);
    }
  }
}

}  // namespace

hipError_t launch_materialize(const DenseArgs &a, int block, hipStream_t s) {
  const int nr = block <= 256 ? 16 : block <= 512 ? 8 : block <= 1024 ? 2 : 1;   // rows_per_wave<block / 64>
  const int64_t waves = (static_cast<int64_t>(a.N) + nr - 1) / nr * (a.K / block);
  const dim3 grid(static_cast<unsigned>((waves + kThreads / 64 - 1) / (kThreads / 64)));
  const void *fn;
  switch (block) {
    case 64: fn = reinterpret_cast<const void *>(materialize_kernel<1>); break;
    case 128: fn = reinterpret_cast<const void *>(materialize_kernel<2>); break;
    case 256: fn = reinterpret_cast<const void *>(materialize_kernel<4>); break;
    case 512: fn = reinterpret_cast<const void *>(materialize_kernel<8>); break;
    case 1024: fn = reinterpret_cast<const void *>(materialize_kernel<16>); break;
    case 2048: fn = reinterpret_cast<const void *>(materialize_kernel<32>); break;
    default: return hipErrorInvalidValue;
  }
  return launch_kernel(fn, grid, dim3(kThreads), 0, s, a);
}

}  // namespace dvssq
