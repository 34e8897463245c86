// Prefill path (large M) of y = (x H) W_hat^T + ((x H) V^T) U^T
// (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2, runtime
// equation).  A tiled GEMM on the f16 matrix cores: x_rot tiles (f16, scaled
// by a power of two per row, from the prologue) and weight tiles dequantized
// into LDS as exact f16 values -- INT4 rows as (n - 8) s_g (same card, INT4
// equation), INT8 rows as the code q, whose fp32 row scale (Spark-X2.5-4B-
// Hadamard-GSQ model card, Tier A) is applied to the accumulator afterwards.
// Both operands hold each run of 8 inputs in the order 0,2,4,6,1,3,5,7, which
// leaves the K-reduction unchanged.  The epilogue undoes the row scale, then
// adds the low-rank term as one bf16 MFMA slab of t (bf16) times the U rows.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;          // padded LDS row, f16 elements
constexpr int kThreads = 256;

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t *As = lds;                       // [2][BM][LDK]
  uint16_t *Bs = lds + 2 * BM * LDK;        // [2][BN][LDK]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntile = blockIdx.x / a.m_tiles, mtile = blockIdx.x % a.m_tiles;
  const bool t8 = ntile >= a.n4_tiles;
  const int rows = t8 ? a.n8 : a.n4;
  const int p0l = (t8 ? ntile - a.n4_tiles : ntile) * BN;   // first tile row inside the tier
  const int m0 = mtile * BM;
  const int KG = a.K / kGroup;
  const int nk = KG;

  // global -> register staging assignment
  const int a_row = tid >> 3, a_seg = tid & 7;         // A: rows a_row + 32 i, 16-byte segment a_seg
  const int b_row = tid >> 1, b_half = tid & 1;        // B: one row, half of the 64-input step
  const bool b_ok = p0l + b_row < rows;

  u32x4 ra[4], rb[2];
  uint32_t rs = 0;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + a_row + 32 * i;
      ra[i] = (m < a.M) ? ld16(a.xr + static_cast<int64_t>(m) * a.K + k0 + 8 * a_seg) : z4;
    }
    if (!t8) {
      rb[0] = b_ok ? ld16(a.q4 + static_cast<int64_t>(p0l + b_row) * (a.K / 2) + k0 / 2 + 16 * b_half) : z4;
      rs = b_ok ? a.s4[static_cast<int64_t>(p0l + b_row) * KG + kt] : 0u;
    } else {
      const int8_t *src = a.q8 + static_cast<int64_t>(p0l + b_row) * a.K + k0 + 32 * b_half;
      rb[0] = b_ok ? ld16(src) : z4;
      rb[1] = b_ok ? ld16(src + 16) : z4;
    }
  };
  auto sstore = [&](int buf) {
    uint16_t *as = As + buf * BM * LDK;
    uint16_t *bs = Bs + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(as + (a_row + 32 * i) * LDK + 8 * a_seg) = ra[i];
    uint16_t *dst = bs + b_row * LDK + 32 * b_half;
    if (!t8) {
      const float s = bf16_to_f32(rs);
      const uint32_t s2 = pack_f16x2(s, s), c24 = pack_f16x2(-24.0f * s, -24.0f * s);
#pragma unroll
      for (int d = 0; d < 4; ++d) *reinterpret_cast<u32x4 *>(dst + 8 * d) = int4_to_f16(rb[0][d], s2, c24);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          *reinterpret_cast<u32x4 *>(dst + 16 * h + 8 * e) = int8_to_f16(rb[h][2 * e], rb[h][2 * e + 1]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fh = lane >> 5;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t *as = As + cur * BM * LDK + (64 * wm + fr) * LDK + 8 * fh;
    const uint16_t *bs = Bs + cur * BN * LDK + (64 * wn + fr) * LDK + 8 * fh;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *reinterpret_cast<const u32x4 *>(as + 32 * i * LDK + 16 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const u32x4 *>(bs + 32 * j * LDK + 16 * ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16_f16(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: row scale 2^e, INT8 row scale, low-rank slab, bf16 scatter through idx
  float rsc[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + 64 * wm + 32 * i + 8 * (v / 4) + 4 * fh + (v % 4);
      rsc[i][v] = (m < a.M) ? a.sc[m] : 0.0f;
    }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pl = p0l + 64 * wn + 32 * j + fr;
    const bool ok = pl < rows;
    const int p = (t8 ? a.n4 : 0) + pl;
    const float s8 = (t8 && ok) ? a.s8[pl] : 1.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] *= rsc[i][v] * s8;
    const int seg = ok ? a.idx[p] / (a.N / a.n_seg) : 0;
    for (int js = 0; js < a.nsr_pad / 16; ++js) {
      u32x4 bv;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t pair = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ig = 16 * js + 8 * fh + 2 * q + e;
          const int il = ig - seg * a.r;
          uint32_t u = 0;
          if (ok && ig < a.nsr && il >= 0 && il < a.r) u = a.U[static_cast<int64_t>(p) * a.r + il];
          pair |= u << (16 * e);
        }
        bv[q] = pair;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = m0 + 64 * wm + 32 * i + fr;
        u32x4 av = z4;
        if (m < a.M) {
          const float *src = a.t + static_cast<int64_t>(m) * a.nsr_pad + 16 * js + 8 * fh;
#pragma unroll
          for (int q = 0; q < 4; ++q) av[q] = pack_bf16x2(src[2 * q], src[2 * q + 1]);
        }
        acc[i][j] = mfma32x32x16(av, bv, acc[i][j]);
      }
    }
    if (!ok) continue;
    const int col = a.idx[p];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (v / 4) + 4 * fh + (v % 4);
        if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + col] = f32_to_bf16(acc[i][j][v]);
      }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(2) * (BM + BN) * LDK * 2;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = (a.n4_tiles + a.n8_tiles) * a.m_tiles;
  return launch_kernel(reinterpret_cast<const void *>(prefill_kernel), dim3(grid), dim3(kThreads), lds, s, a);
}

}  // namespace dvssq
