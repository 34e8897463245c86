// Decode path (M <= 32) of y = (x H) W_hat^T + ((x H) V^T) U^T
// (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2, runtime
// equation), reading the packed tiers directly: INT4 groups of 64 with a bf16
// scale (same card, INT4 equation) and INT8 rows with an fp32 scale
// (Spark-X2.5-4B-Hadamard-GSQ model card, Tier A).
//
// Work unit = one wavefront = 32 packed rows x one 256-input chunk.  Codes
// stream from HBM as 16-byte loads per lane and become bf16 MFMA operands in
// registers:
//   INT4: (w & 0x000F000F) | 0x43004300 is the bf16 pair (128+n_a, 128+n_b);
//         since n = q + 8 the tile product is sum (q + 136) x, and 136 X_g
//         (X_g = sum of the rotated x over the group) is subtracted before the
//         group scale is applied in fp32.
//   INT8: q ^ 0x80 is the byte q + 128, converted exactly to fp32 and packed
//         to bf16; 128 X_chunk is subtracted and the row scale applied.
// The rotated activations (bf16, each 8-input run in the order 0,4,1,5,2,6,
// 3,7 to match the nibble extraction) are the other MFMA operand.  The
// low-rank term adds t(chunk) U^T as one more MFMA per 16 columns of t.
//
// Split-K: each unit writes its fp32 partial for its chunk; the last unit to
// finish a 32-row tile (arrival counter, cleared by the prologue kernel) sums
// the chunks in a fixed order, rounds to bf16 and scatters through idx.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 8 INT4 codes (one dword) -> 8 bf16 (128 + nibble), slot order k+0,4,1,5,2,6,3,7
__device__ __forceinline__ u32x4 int4_to_bf16(uint32_t w) {
  const uint32_t m = 0x000F000Fu, o = 0x43004300u;
  u32x4 r;
  r[0] = (w & m) | o;
  r[1] = ((w >> 4) & m) | o;
  r[2] = ((w >> 8) & m) | o;
  r[3] = ((w >> 12) & m) | o;
  return r;
}

// 8 INT8 codes (k+0..3 in lo, k+4..7 in hi) -> 8 bf16 (q + 128), slot order k+0,4,1,5,2,6,3,7
__device__ __forceinline__ u32x4 int8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_bf16x2(static_cast<float>((a >> (8 * i)) & 0xFFu),
                       static_cast<float>((b >> (8 * i)) & 0xFFu));
  return r;
}

template <int MV>  // accumulator entries per lane that hold real tokens: 4 (M<=8), 8 (M<=16), 16
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int n = lane & 31, h = lane >> 5;
  int unit = blockIdx.x;
  const bool t8 = unit >= a.n4_tiles * a.nchunk;
  if (t8) unit -= a.n4_tiles * a.nchunk;
  const int tile = unit / a.nchunk, c = unit % a.nchunk;
  const int rows = t8 ? a.n8 : a.n4;
  const int pl = tile * 32 + n;            // row inside the tier
  const bool row_ok = pl < rows;
  const int p = (t8 ? a.n4 : 0) + pl;      // packed row
  const int KG = a.K / kGroup;
  const int g0 = c * (kChunk / kGroup);
  const int ng = min(kChunk / kGroup, KG - g0);
  const bool m_ok = n < a.M;               // this lane's A-operand row (token) is real

  // ---- issue the weight loads first (the long-latency HBM stream)
  u32x4 cw[4][2];
  float sc[4];
  const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    cw[g][0] = z4;
    cw[g][1] = z4;
    sc[g] = 0.0f;
  }
  if (!t8) {
    const uint8_t *rowp = a.q4 + static_cast<int64_t>(pl) * (a.K / 2) + g0 * 32 + 16 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (row_ok && g < ng) cw[g][0] = load16(rowp + 32 * g);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (row_ok && g < ng) sc[g] = bf16_to_f32(a.s4[static_cast<int64_t>(pl) * KG + g0 + g]);
  } else {
    const int8_t *rowp = a.q8 + static_cast<int64_t>(pl) * a.K + g0 * 64 + 32 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (row_ok && g < ng) cw[g][s] = load16(rowp + 64 * g + 16 * s);
  }

  // ---- activation operand and group sums (L2-resident workspace)
  u32x4 xa[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int d = 0; d < 4; ++d)
      xa[g][d] = (m_ok && g < ng)
                     ? load16(a.xr + static_cast<int64_t>(n) * a.K + (g0 + g) * 64 + 32 * h + 8 * d)
                     : z4;
  float xs[4][MV];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q = 0; q < MV / 4; ++q) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (g < ng) v = *reinterpret_cast<const f32x4 *>(a.xs + (g0 + g) * kDecodeRows + 8 * q + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) xs[g][4 * q + e] = v[e];
    }

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  if (!t8) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x16 C;
#pragma unroll
      for (int v = 0; v < 16; ++v) C[v] = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) C = mfma32x32x16(xa[g][d], int4_to_bf16(cw[g][0][d]), C);
#pragma unroll
      for (int v = 0; v < MV; ++v) acc[v] = fmaf(sc[g], fmaf(-136.0f, xs[g][v], C[v]), acc[v]);
    }
  } else {
    f32x16 C;
#pragma unroll
    for (int v = 0; v < 16; ++v) C[v] = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          C = mfma32x32x16(xa[g][2 * s + e], int8_to_bf16(cw[g][s][2 * e], cw[g][s][2 * e + 1]), C);
    const float s8 = row_ok ? a.s8[pl] : 0.0f;
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      float xc = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) xc += xs[g][v];
      acc[v] = s8 * fmaf(-128.0f, xc, C[v]);
    }
  }

  // ---- low-rank term for the Hadamard blocks that start inside this chunk
  const int kc0 = c * kChunk, kc1 = min(a.K, kc0 + kChunk);
  const int bA = (kc0 + a.block - 1) / a.block, bB = (kc1 + a.block - 1) / a.block;
  if (bA < bB) {
    const int seg = row_ok ? a.idx[p] / (a.N / a.n_seg) : 0;
    for (int j = 0; j < a.nsr_pad / 16; ++j) {
      float tv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) tv[q] = 0.0f;
      if (m_ok)
        for (int bb = bA; bb < bB; ++bb) {
          const float *src = a.tp + (static_cast<int64_t>(bb) * kDecodeRows + n) * a.nsr_pad + 16 * j + 8 * h;
#pragma unroll
          for (int q = 0; q < 8; ++q) tv[q] += src[q];
        }
      u32x4 av, bv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = pack_bf16x2(tv[2 * q], tv[2 * q + 1]);
        uint32_t pair = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ig = 16 * j + 8 * h + 2 * q + e;
          const int il = ig - seg * a.r;
          uint32_t u = 0;
          if (row_ok && ig < a.nsr && il >= 0 && il < a.r) u = a.U[static_cast<int64_t>(p) * a.r + il];
          pair |= u << (16 * e);
        }
        bv[q] = pair;
      }
      acc = mfma32x32x16(av, bv, acc);
    }
  }

  // ---- publish the partial, count arrivals, last arrival reduces
#pragma unroll
  for (int v = 0; v < MV; ++v) {
    const int m = 8 * (v / 4) + 4 * h + (v % 4);
    if (m < a.M && row_ok)
      __hip_atomic_store(a.part + (static_cast<int64_t>(c) * kDecodeRows + m) * a.N + p, acc[v],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __threadfence();
  const int gtile = (t8 ? a.n4_tiles : 0) + tile;
  int old = 0;
  if (lane == 0) old = atomicAdd(a.cnt + gtile, 1);
  old = __shfl(old, 0, 64);
  if (old != a.nchunk - 1) return;
  __threadfence();
  const int base = (t8 ? a.n4 : 0) + tile * 32;
  const int nrows = min(32, rows - tile * 32);
  for (int e = lane; e < 32 * a.M; e += 64) {
    const int nn = e & 31, m = e >> 5;
    if (nn >= nrows) continue;
    const int pp = base + nn;
    float s = 0.0f;
    for (int cc = 0; cc < a.nchunk; ++cc)
      s += __hip_atomic_load(a.part + (static_cast<int64_t>(cc) * kDecodeRows + m) * a.N + pp,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.y[static_cast<int64_t>(m) * a.N + a.idx[pp]] = f32_to_bf16(s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  const int units = (a.n4_tiles + a.n8_tiles) * a.nchunk;
  if (a.M <= 8)
    hipLaunchKernelGGL(decode_kernel<4>, dim3(units), dim3(64), 0, s, a);
  else if (a.M <= 16)
    hipLaunchKernelGGL(decode_kernel<8>, dim3(units), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<16>, dim3(units), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace dvssq
