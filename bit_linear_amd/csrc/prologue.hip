// Activation side of the DV-SSQ layer for dvssq_fwht and the prefill path:
// x_rot = x H_K and t = x_rot V^T.
//
// Rotation: MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 1
// (X' = X H, Sylvester H) and Spark-X2.5-4B-Hadamard-GSQ model card, Tier B
// equation (block-diagonal H_K).  t: MiniCPM card, Mathematical Foundations 2,
// runtime equation (the X B^T factor).
//
// dvssq_fwht (fwht_kernel): one wavefront per (row, block), the register FWHT,
// bf16 stored in natural order straight from registers.
//
// Prefill (prologue_kernel): one workgroup = 4 wavefronts handles MT activation
// rows and a run of Hadamard blocks, each row of a block rotated by one
// wavefront (on the matrix cores for blocks of 256 and more, else with the
// register FWHT), staged in LDS and copied out as f16 scaled by a power of two
// per row, in the GEMM's tile layout, runs of 8 in the order 0,2,4,6,1,3,5,7
// (the order the weight decoder produces).  The row's exponent
// comes from the bound max|x H| <= sqrt(block) max|x| (rowscale_kernel), so the
// scaled values stay below 2^15.  For the prefill, t = x_rot V^T is then
// computed from those f16 tiles on the matrix cores (tgemm_kernel), its K-ranges
// summed in order by treduce_kernel.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;

template <int VPL>  // values per lane = block / 64
__device__ __forceinline__ void load_row(const uint16_t *src, float (&v)[VPL]) {
  if constexpr (VPL >= 8) {
#pragma unroll
    for (int q = 0; q < VPL / 8; ++q) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(src + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
        v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  } else if constexpr (VPL == 4) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(src);
    v[0] = __uint_as_float(w[0] << 16);
    v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
    v[2] = __uint_as_float(w[1] << 16);
    v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) v[j] = bf16_to_f32(src[j]);
  }
}

template <int VPL>
__device__ __forceinline__ void store_row(uint16_t *dst, const float (&v)[VPL]) {
  if constexpr (VPL >= 8) {
#pragma unroll
    for (int q = 0; q < VPL / 8; ++q) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[8 * q + 2 * e], v[8 * q + 2 * e + 1]);
      *reinterpret_cast<u32x4 *>(dst + 8 * q) = w;
    }
  } else if constexpr (VPL == 4) {
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2 *>(dst) = w;
  } else if constexpr (VPL == 2) {
    *reinterpret_cast<uint32_t *>(dst) = pack_bf16x2(v[0], v[1]);
  } else {
    dst[0] = f32_to_bf16(v[0]);
  }
}

// rows of one block that a wavefront rotates together: their loads are issued at once
template <int VPL>
constexpr int kRowBatch = VPL <= 4 ? 8 : VPL <= 8 ? 4 : VPL <= 16 ? 2 : 1;

// dvssq_fwht: [M][K] is M·K/B consecutive blocks of B values; wavefront w takes
// blocks w·RB .. w·RB + RB - 1, loads them all, then rotates and stores each
// (in place allowed: a wavefront reads its blocks before it writes them, and
// no other wavefront touches them).
template <int VPL>
__global__ __launch_bounds__(kThreads) void fwht_kernel(PrologueArgs a) {
  constexpr int B = 64 * VPL, RB = kRowBatch<VPL>;
  const int lane = threadIdx.x & 63;
  const int64_t nitem = static_cast<int64_t>(a.M) * (a.K / B);
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * RB;
  if (i0 >= nitem) return;
  float v[RB][VPL];
#pragma unroll
  for (int j = 0; j < RB; ++j) load_row<VPL>(a.x + min(i0 + j, nitem - 1) * B + lane * VPL, v[j]);
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    if (i0 + j < nitem) {
      fwht_wave<VPL>(v[j], lane);
#pragma unroll
      for (int q = 0; q < VPL; ++q) v[j][q] *= a.hscale;
      store_row<VPL>(a.xr + (i0 + j) * B + lane * VPL, v[j]);
    }
  }
}

template <int VPL>
hipError_t launch_fwht_vpl(const PrologueArgs &a, hipStream_t s) {
  constexpr int B = 64 * VPL;
  const int64_t waves = (static_cast<int64_t>(a.M) * (a.K / B) + kRowBatch<VPL> - 1) / kRowBatch<VPL>;
  const int64_t wgs = (waves + kThreads / 64 - 1) / (kThreads / 64);
  return launch_kernel(reinterpret_cast<const void *>(fwht_kernel<VPL>), dim3(static_cast<unsigned>(wgs)),
                       dim3(kThreads), 0, s, a);
}

template <int VPL, int MT>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueArgs a) {
  constexpr int B = 64 * VPL;
  constexpr int LDR = B + 4;  // padded LDS row (fp32)
  // blocks of 512 and more stage 16-bit values (the output format: f16 scaled
  // and permuted), so that two workgroups fit in LDS
  constexpr bool H16 = VPL >= 8;
  constexpr int LDH = B + 8;  // padded LDS row (16-bit)
  extern __shared__ __align__(16) float lds[];
  __shared__ int rowexp[MT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * MT;
  const int nblk = a.K / B;
  const int b0 = blockIdx.y * a.blocks_per_wg;
  const int b1 = min(nblk, b0 + a.blocks_per_wg);
  const int mrows = min(MT, a.M - m0);

  // 0. per-row power-of-two scale, written by rowscale_kernel (or, when a
  // block is the whole row, found below by the wavefront that rotates the row)
  if (!a.fuse_scale) {
    for (int ml = tid; ml < MT; ml += kThreads) rowexp[ml] = ml < mrows ? ilogbf(a.sc[m0 + ml]) : 0;
    __syncthreads();
  }

  constexpr int RB = kRowBatch<VPL>;

  for (int blk = b0; blk < b1; ++blk) {
    const int kb = blk * B;
    // 1. rotate each row of this block (one wavefront per row) and stage it in LDS
    for (int ml0 = wave; ml0 < MT; ml0 += 4 * RB) {
      if constexpr (B >= 256) {
        // on the matrix cores (rotate_blocks): lane (n, q) holds inputs
        // 256 c + 16 n + 4 q + j of the row's block
        constexpr int C = B / 256;
        const int n = lane & 15, q = lane >> 4;
        u32x2 xw[RB][C];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int ml = min(ml0 + 4 * j, mrows - 1);
          const uint16_t *src = a.x + static_cast<int64_t>(m0 + ml) * a.K + kb + 16 * n + 4 * q;
#pragma unroll
          for (int c = 0; c < C; ++c) xw[j][c] = *reinterpret_cast<const u32x2 *>(src + 256 * c);
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int ml = ml0 + 4 * j;
          if (ml >= MT) continue;
          const bool live = ml < mrows;
          int ex;   // the row's exponent e
          if (a.fuse_scale) {
            // as rowscale_kernel: e from max |x| of the row (this block)
            float mx = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int h = 0; h < 2; ++h)
                mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(xw[j][c][h] << 16)),
                                     fabsf(__uint_as_float(xw[j][c][h] & 0xFFFF0000u))));
#pragma unroll
            for (int sft = 1; sft < 64; sft <<= 1) mx = fmaxf(mx, __shfl_xor(mx, sft, 64));
            ex = 0;
            if (mx > 0.0f && mx <= 3.0e38f) ex = max(-120, min(120, ilogbf(mx) + a.exp_bias));
            if (lane == 0) {
              rowexp[ml] = live ? ex : 0;
              if (live) a.sc[m0 + ml] = ldexpf(1.0f, ex);
            }
          } else {
            ex = rowexp[ml];
          }
          float y[C][4];
          if (a.rotate) {
            rotate_blocks<C>(xw[j], y, B, a.hscale);
          } else {
#pragma unroll
            for (int c = 0; c < C; ++c) {
              y[c][0] = __uint_as_float(xw[j][c][0] << 16);
              y[c][1] = __uint_as_float(xw[j][c][0] & 0xFFFF0000u);
              y[c][2] = __uint_as_float(xw[j][c][1] << 16);
              y[c][3] = __uint_as_float(xw[j][c][1] & 0xFFFF0000u);
            }
          }
          if constexpr (H16) {
            // f16 x 2^-e; inputs 4 h + j (h = q % 2) of run r fill slots
            // (j even) h, ... and (j odd) 4 + h, ... of the order 0,2,4,6,1,3,5,7
            uint16_t *row = reinterpret_cast<uint16_t *>(lds) + ml * LDH;
            const float d = ldexpf(1.0f, -ex);
#pragma unroll
            for (int c = 0; c < C; ++c) {
              const int r = 32 * c + 2 * n + (q >> 1), h = q & 1;
              *reinterpret_cast<uint32_t *>(row + 8 * r + 2 * h) = live ? pack_f16x2(y[c][0] * d, y[c][2] * d) : 0u;
              *reinterpret_cast<uint32_t *>(row + 8 * r + 4 + 2 * h) = live ? pack_f16x2(y[c][1] * d, y[c][3] * d) : 0u;
            }
          } else {
            float *row = lds + ml * LDR;
#pragma unroll
            for (int c = 0; c < C; ++c) {
              const f32x4 o = {live ? y[c][0] : 0.0f, live ? y[c][1] : 0.0f, live ? y[c][2] : 0.0f,
                               live ? y[c][3] : 0.0f};
              *reinterpret_cast<f32x4 *>(row + 256 * c + 16 * n + 4 * q) = o;
            }
          }
        }
      } else {
        // blocks of 64 and 128: the register FWHT, fp32 in LDS
        float v[RB][VPL];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int ml = min(ml0 + 4 * j, mrows - 1);
          load_row<VPL>(a.x + static_cast<int64_t>(m0 + ml) * a.K + kb + lane * VPL, v[j]);
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int ml = ml0 + 4 * j;
          if (ml >= MT) continue;
          if (ml < mrows && a.rotate) {
            fwht_wave<VPL>(v[j], lane);
#pragma unroll
            for (int q = 0; q < VPL; ++q) v[j][q] *= a.hscale;
          }
          float *row = lds + ml * LDR + lane * VPL;
#pragma unroll
          for (int q = 0; q < VPL; ++q) row[q] = ml < mrows ? v[j][q] : 0.0f;
        }
      }
    }
    __syncthreads();
    // 2. copy out in runs of 8 into the GEMM's tiles (consecutive threads take
    // consecutive rows of one run): f16 as staged, or fp32 scaled by 2^-e and permuted
    constexpr int RUNS = B / 8;
    if constexpr (H16) {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(lds);
      for (int e = tid; e < mrows * RUNS; e += kThreads) {
        const int run = e / mrows, ml = e - run * mrows;
        *reinterpret_cast<u32x4 *>(a.xr + xr_tile_offset(m0 + ml, kb + run * 8, a.K)) =
            *reinterpret_cast<const u32x4 *>(h + ml * LDH + run * 8);
      }
    } else {
      for (int e = tid; e < mrows * RUNS; e += kThreads) {
        const int run = e / mrows, ml = e - run * mrows;
        const float *w = lds + ml * LDR + run * 8;
        const float d = ldexpf(1.0f, -rowexp[ml]);
        u32x4 o;
        o[0] = pack_f16x2(w[0] * d, w[2] * d);
        o[1] = pack_f16x2(w[4] * d, w[6] * d);
        o[2] = pack_f16x2(w[1] * d, w[3] * d);
        o[3] = pack_f16x2(w[5] * d, w[7] * d);
        *reinterpret_cast<u32x4 *>(a.xr + xr_tile_offset(m0 + ml, kb + run * 8, a.K)) = o;
      }
    }
    __syncthreads();
  }
}

// t = x_rot V^T for the prefill from the GEMM's f16 x_rot tiles: one workgroup
// per 128-row tile and K-range (grid y splits K), wavefront w on rows
// 32 w .. 32 w + 31, 32x32x16 f16 MFMAs against V converted to f16 in the
// tiles' input order (step s, chunk 2 ks + h: inputs 64 s + 32 h + 8 ks + 0,2,4,6,1,3,5,7);
// each row's partial is scaled back by its 2^e.  One K-range writes t directly,
// several write partials that treduce_kernel sums in range order.
template <int NI>   // column tiles of 32 in t (nsr_pad / 32)
__global__ __launch_bounds__(kThreads) void tgemm_kernel(PrologueArgs a, int spw) {
  const int lane = threadIdx.x & 63, fr = lane & 31, fh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int KG = a.K / kGroup;
  const int mt = blockIdx.x, s0 = blockIdx.y * spw, s1 = min(KG, s0 + spw);
  const uint16_t *tile0 = a.xr + static_cast<int64_t>(mt) * KG * (kPfTileM * kGroup) + (2 * 0 + fh) * 1024 +
                          (32 * wave + fr) * 8;
  const auto rv = make_rsrc(a.V, static_cast<uint32_t>(a.nsr) * a.K * 2);
  f32x16 acc[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[ni][e] = 0.0f;
  auto f16of = [](uint32_t bf) { return static_cast<_Float16>(__uint_as_float(bf << 16)); };
  for (int s = s0; s < s1; ++s) {
    u32x4 af[4], vb[4][NI];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      af[ks] = *reinterpret_cast<const u32x4 *>(tile0 + static_cast<int64_t>(s) * (kPfTileM * kGroup) + ks * 2048);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int i = 32 * ni + fr;
        const uint32_t off = i < a.nsr ? (static_cast<uint32_t>(i) * a.K + 64 * s + 32 * fh + 8 * ks) * 2 : kOutOfRange;
        vb[ks][ni] = buf_load16(rv, off);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        // natural-order bf16 pairs (k0,k1) .. (k6,k7) -> f16 in the order 0,2,4,6,1,3,5,7
        const u32x4 w = vb[ks][ni];
        f16x8 h;
        h[0] = f16of(w[0] & 0xFFFFu); h[1] = f16of(w[1] & 0xFFFFu);
        h[2] = f16of(w[2] & 0xFFFFu); h[3] = f16of(w[3] & 0xFFFFu);
        h[4] = f16of(w[0] >> 16);     h[5] = f16of(w[1] >> 16);
        h[6] = f16of(w[2] >> 16);     h[7] = f16of(w[3] >> 16);
        acc[ni] = mfma32x32x16_f16(af[ks], __builtin_bit_cast(u32x4, h), acc[ni]);
      }
  }
  // lane (fr, fh), acc[ni][v]: row 32 w + 8 (v / 4) + 4 fh + v % 4, column 32 ni + fr
  float *dst = gridDim.y == 1 ? a.t : a.tpart + static_cast<int64_t>(blockIdx.y) * a.M * a.nsr_pad;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = mt * kPfTileM + 32 * wave + 8 * (v / 4) + 4 * fh + (v % 4);
    if (m >= a.M) continue;
    const float sc = a.sc[m];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) dst[static_cast<int64_t>(m) * a.nsr_pad + 32 * ni + fr] = acc[ni][v] * sc;
  }
}

// t = sum over the K-ranges of their partial t, in range order; four
// consecutive t values per thread.
__global__ __launch_bounds__(kThreads) void treduce_kernel(PrologueArgs a, int ncol) {
  const int64_t n4 = static_cast<int64_t>(a.M) * a.nsr_pad / 4;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= n4) return;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(a.tpart) + e;
  constexpr int kB = 8;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < ncol; c0 += kB) {
    f32x4 v[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) v[j] = c0 + j < ncol ? src[(c0 + j) * n4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kB; ++j) s += v[j];
  }
  reinterpret_cast<f32x4 *>(a.t)[e] = s;
}

// INT4 row shifts of the prefill GEMM, one wavefront per packed INT4 row: the
// GEMM enters group g of row p as the exact f16 values (n - 8) s4[p][g] 2^-c
// and multiplies the row's fp32 result by 2^c.  c puts the row's largest
// scale in [2^10, 2^11), so that every scale within 2^27 of it is an exact f16
// of at least 2^-17 (whose multiples by n - 8 and -24 stay exact) and
// (16 + n) s 2^-c stays below the f16 maximum.  An all-zero row keeps c = 0.
__device__ void row_shift(const PrologueArgs &a, int p) {
  const int lane = threadIdx.x & 63;
  const int KG = a.K / kGroup;
  const uint16_t *row = a.s4 + static_cast<int64_t>(p) * KG;
  uint32_t mx = 0;
  for (int g = lane; g < KG; g += 64) mx = max(mx, static_cast<uint32_t>(row[g]) & 0x7FFFu);
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), sft, 64)));
  if (lane != 0) return;
  int c = 0;
  if (mx != 0) {
    const int be = static_cast<int>(mx >> 7);          // biased exponent (0: subnormal)
    c = max(-116, min(117, (be == 0 ? -126 : be - 127) - 10));
  }
  a.rsh[p] = __uint_as_float(static_cast<uint32_t>(127 + c) << 23);
}

// Per-row power-of-two scale 2^e of the f16 x_rot: from the bound
// max |x H| <= sqrt(block) max |x|, e puts the scaled row below 2^15.  One
// wavefront per row, its 16-byte chunks read with several loads in flight.
// The blocks from row_blocks on compute the INT4 row shifts (row_shift).
__global__ __launch_bounds__(kThreads) void rowscale_kernel(PrologueArgs a, int row_blocks) {
  if (static_cast<int>(blockIdx.x) >= row_blocks) {
    const int p = (blockIdx.x - row_blocks) * (kThreads / 64) + (threadIdx.x >> 6);
    if (p < a.n4) row_shift(a, p);
    return;
  }
  const int lane = threadIdx.x & 63, m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const u32x4 *row = reinterpret_cast<const u32x4 *>(a.x + static_cast<int64_t>(m) * a.K);
  const int nch = a.K / 8;
  float mx = 0.0f;
#pragma unroll 8
  for (int c = lane; c < nch; c += 64) {
    const u32x4 w = row[c];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xFFFF0000u))));
  }
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) mx = fmaxf(mx, __shfl_xor(mx, sft, 64));
  int e = 0;
  if (mx > 0.0f && mx <= 3.0e38f) e = max(-120, min(120, ilogbf(mx) + a.exp_bias));
  if (lane == 0) a.sc[m] = ldexpf(1.0f, e);
}

template <int VPL, int MT>
hipError_t launch_vpl(const PrologueArgs &a, int n_wg_blocks, hipStream_t s) {
  constexpr int B = 64 * VPL;
  const size_t lds = VPL >= 8 ? static_cast<size_t>(MT) * (B + 8) * 2 : static_cast<size_t>(MT) * (B + 4) * 4;
  if (lds > 65536) {
    static std::atomic<uint64_t> done{0};
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void *>(prologue_kernel<VPL, MT>), static_cast<int>(lds), done);
    if (e != hipSuccess) return e;
  }
  dim3 grid((a.M + MT - 1) / MT, n_wg_blocks);
  return launch_kernel(reinterpret_cast<const void *>(prologue_kernel<VPL, MT>), grid, dim3(kThreads), lds, s, a);
}

}  // namespace

hipError_t launch_fwht(const PrologueArgs &a, int block, hipStream_t s) {
  switch (block) {
    case 64: return launch_fwht_vpl<1>(a, s);
    case 128: return launch_fwht_vpl<2>(a, s);
    case 256: return launch_fwht_vpl<4>(a, s);
    case 512: return launch_fwht_vpl<8>(a, s);
    case 1024: return launch_fwht_vpl<16>(a, s);
    case 2048: return launch_fwht_vpl<32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prologue(const PrologueArgs &a, int block, int n_wg_blocks, int cus, hipStream_t s) {
  if (a.fuse_scale && (a.K != block || block < 256)) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  {
    // row scales of x (unless the rotation finds them) and the INT4 row shifts
    int row_blocks = a.fuse_scale ? 0 : (a.M + kThreads / 64 - 1) / (kThreads / 64);
    const int shift_blocks = (a.n4 + kThreads / 64 - 1) / (kThreads / 64);
    void *args[] = {const_cast<PrologueArgs *>(&a), &row_blocks};
    if (row_blocks + shift_blocks > 0) {
      e = hipLaunchKernel(reinterpret_cast<const void *>(rowscale_kernel), dim3(row_blocks + shift_blocks),
                          dim3(kThreads), args, 0, s);
      if (e != hipSuccess) return e;
    }
  }
  switch (block) {
    case 64: e = launch_vpl<1, 32>(a, n_wg_blocks, s); break;
    case 128: e = launch_vpl<2, 32>(a, n_wg_blocks, s); break;
    case 256: e = launch_vpl<4, 32>(a, n_wg_blocks, s); break;
    case 512: e = launch_vpl<8, 32>(a, n_wg_blocks, s); break;
    case 1024: e = launch_vpl<16, 16>(a, n_wg_blocks, s); break;
    case 2048: e = launch_vpl<32, 16>(a, n_wg_blocks, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || a.nsr == 0) return e;
  // t from the f16 tiles: K split so that the grid has about two workgroups
  // per compute unit, at most kTSplitMax ranges
  const int KG = a.K / kGroup, mtiles = (a.M + kPfTileM - 1) / kPfTileM;
  const int want = std::max(1, std::min(kTSplitMax, (2 * cus + mtiles - 1) / mtiles));
  const int spw = (KG + want - 1) / want;
  const int nsplit = (KG + spw - 1) / spw;
  {
    int spw_arg = spw;
    void *args[] = {const_cast<PrologueArgs *>(&a), &spw_arg};
    const void *fn = a.nsr_pad > 32 ? reinterpret_cast<const void *>(tgemm_kernel<2>)
                                    : reinterpret_cast<const void *>(tgemm_kernel<1>);
    e = hipLaunchKernel(fn, dim3(mtiles, nsplit), dim3(kThreads), args, 0, s);
    if (e != hipSuccess || nsplit == 1) return e;
  }
  const int64_t n4 = static_cast<int64_t>(a.M) * a.nsr_pad / 4;
  int ncol = nsplit;
  void *args[] = {const_cast<PrologueArgs *>(&a), &ncol};
  return hipLaunchKernel(reinterpret_cast<const void *>(treduce_kernel), dim3((n4 + kThreads - 1) / kThreads),
                         dim3(kThreads), args, 0, s);
}

}  // namespace dvssq
