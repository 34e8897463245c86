// Prefill path (large M) of y = (x H) W_hat^T + ((x H) V^T) U^T
// (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2, runtime
// equation).  A tiled GEMM on the f16 matrix cores: x_rot tiles (f16, scaled
// by a power of two per row, from the prologue) times weights dequantized in
// registers as exact f16 values -- INT4 rows as (n - 8) s_g 2^-c (same card,
// INT4 equation; 2^c one power of two per row from the prologue, applied to
// the accumulator afterwards), INT8 rows as the code q, whose fp32 row scale
// (Spark-X2.5-4B-Hadamard-GSQ model card, Tier A) is applied likewise.
// Both operands hold each run of 8 inputs in the order 0,2,4,6,1,3,5,7, which
// leaves the K-reduction unchanged.  The epilogue undoes the row scale, then
// adds the low-rank term as one bf16 MFMA slab of t (bf16) times the U rows.
#include <type_traits>

#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int BK = kGroup;              // inputs per step: one INT4 group
constexpr int kThreads = 256;
constexpr int MF = kPfTileM / 32;        // 32-token fragments of a wavefront
constexpr int NF = kPfTileN / 4 / 32;    // 32-row weight fragments of a wavefront
constexpr int kTileA = kPfTileM * BK;    // f16 per x_rot tile
// s_waitcnt immediates: vmcnt(n), the other counters free
constexpr int kVmcnt0 = 0x0F70;
constexpr int kVmcnt4 = 0x0F74;
constexpr int kVmcnt8 = 0x0F78;
// padded LDS row of the staged t (bf16): NS slabs of 16 plus 8, so that the
// 32 rows one matrix-core operand reads start on different banks
template <int NS>
constexpr int TS = NS * 16 + 8;

// One workgroup: kPfTileM tokens by kPfTileN weight rows of one tier, the four
// wavefronts side by side over the weight rows (128 tokens x 64 rows each).
// x_rot tiles go through LDS (double buffered, one contiguous 16 KB copy per
// step); each wavefront loads its own weight bytes straight into registers --
// lane (fr, fh) of fragment j takes row 32 j + fr and inputs 32 fh .. 32 fh + 31
// of the group, which are contiguous in the packed rows -- and dequantizes
// them there.  Loads run one step ahead of the matrix cores.
template <bool T8, int NS, bool SPLIT>
__device__ __forceinline__ void prefill_tile(const PrefillArgs &a, uint16_t *A0, uint16_t *A1, uint16_t *A2,
                                             uint16_t *ts, float *scs, int mtile, int tile0, int split) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, fh = lane >> 5;
  const int KGa = a.K / BK;                                   // steps of the whole K
  const int s0 = split * a.kspw;                              // this workgroup's K-range
  const int KG = min(KGa, s0 + a.kspw) - s0;                  // its steps
  const int rows = T8 ? a.n8 : a.n4;
  const int p0 = tile0 + 64 * wave;   // first weight row (inside the tier) of this wavefront
  const uint16_t *ag = a.xr + (static_cast<int64_t>(mtile) * KGa + s0) * kTileA;
  const int m0 = mtile * kPfTileM;

  // the epilogue's token-side operands, staged in LDS while the main loop runs:
  // t rows of the tile as bf16 (padded rows of TS) and the row scales.  With a
  // K split, the first range alone adds the low-rank term.
  const bool lowrank = !SPLIT || split == 0;
  if (!lowrank) {
    if (tid < kPfTileM) scs[tid] = m0 + tid < a.M ? a.sc[m0 + tid] : 0.0f;
  } else {
    const auto rt = make_rsrc(a.t, static_cast<uint32_t>(a.M) * (NS * 16) * 4);
    const int row = tid >> 1, half = tid & 1;
    const uint32_t base = static_cast<uint32_t>((m0 + row) * (NS * 16) + half * (NS * 8)) * 4;
    u32x4 tv[2 * NS];
#pragma unroll
    for (int c = 0; c < 2 * NS; ++c) tv[c] = buf_load16(rt, base + 16 * c);
    const auto rsc = make_rsrc(a.sc, static_cast<uint32_t>(a.M) * 4);
    const uint32_t sv = buf_load4(rsc, tid < kPfTileM ? static_cast<uint32_t>(m0 + tid) * 4 : kOutOfRange);
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 w = tv[2 * c + q];
        o[2 * q] = pack_bf16x2(__uint_as_float(w[0]), __uint_as_float(w[1]));
        o[2 * q + 1] = pack_bf16x2(__uint_as_float(w[2]), __uint_as_float(w[3]));
      }
      *reinterpret_cast<u32x4 *>(ts + row * TS<NS> + half * (NS * 8) + 8 * c) = o;
    }
    if (tid < kPfTileM) scs[tid] = __uint_as_float(sv);
  }

  // weight bytes of this workgroup's rows only, so that 32-bit offsets suffice
  const int64_t rb = T8 ? a.K : a.K / 2;   // packed bytes per row
  const int nrow = min(kPfTileN, rows - tile0);
  const auto rq = make_rsrc((T8 ? static_cast<const uint8_t *>(static_cast<const void *>(a.q8)) : a.q4) + tile0 * rb,
                            static_cast<uint32_t>(nrow * rb));
  const auto rs = make_rsrc(a.s4 + static_cast<int64_t>(tile0) * KGa, static_cast<uint32_t>(T8 ? 0 : nrow * KGa * 2));
  uint32_t oq[NF], os[NF];
  // INT4 rows: 2^c of the row (prologue); group scales enter the f16 weights as s4 2^-c
  float rsh[NF], rinv[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int rl = 64 * wave + 32 * j + fr;   // row inside the workgroup's tile
    const bool ok = rl < nrow;
    oq[j] = ok ? static_cast<uint32_t>(rl * rb + (T8 ? 32 : 16) * fh + (T8 ? 64 : 32) * s0) : kOutOfRange;
    os[j] = ok ? static_cast<uint32_t>((rl * KGa + s0) * 2) : kOutOfRange;
    rsh[j] = T8 || !ok ? 1.0f : a.rsh[tile0 + rl];
    rinv[j] = __uint_as_float((254u << 23) - __float_as_uint(rsh[j]));   // 2^-c
  }

  // x_rot tiles: a direct copy into LDS (each wavefront instruction fills 1 KB
  // of one tile, lane l at byte 16 l)
  const auto ra = make_rsrc(ag, static_cast<uint32_t>(KG) * kTileA * 2);
  auto load_a = [&](int g, uint16_t *dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void *)(dst + (kThreads * i + 64 * wave) * 8), 16, lane * 16,
          g * (kTileA * 2) + (kThreads * i + 64 * wave) * 16, 0, 0);
  };
  // raw weight bytes of NB steps in flight: INT4 rows (16 bytes + a group
  // scale per lane) two steps ahead, INT8 rows (32 bytes) one step ahead
  constexpr int NB = T8 ? 2 : 3;
  u32x4 Q[NB][NF][T8 ? 2 : 1];
  uint32_t S[NB][NF];
  auto load_b = [&](int g, auto set) {
    constexpr int b = decltype(set)::value;
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      if constexpr (T8) {
        Q[b][j][0] = buf_load16(rq, oq[j] + 64 * g);
        Q[b][j][1] = buf_load16(rq, oq[j] + 64 * g + 16);
      } else {
        Q[b][j][0] = buf_load16(rq, oq[j] + 32 * g);
        S[b][j] = buf_load2(rs, os[j] + 2 * g);
      }
    }
  };

  f32x16 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // One step of 64 inputs: x_rot tile g sits in LDS buffer cur, tile g + 2
  // is copied into buffer nx2 (three distinct LDS arrays, so that a copy into
  // one is never taken to alias reads of another).  Every step issues the
  // same eight loads (the last steps repeat the last group), so the wait at
  // the top of a step leaves exactly the next step's loads in flight.
  auto step = [&](int g, const uint16_t *cur, uint16_t *nx2, auto use, auto fill) {
    constexpr int bu = decltype(use)::value;
    // a bare barrier: a workgroup fence here would also wait for the copies
    // still in flight for the next steps; the asm statements keep the
    // compiler from moving memory accesses across it
    __builtin_amdgcn_s_waitcnt(T8 ? kVmcnt4 : kVmcnt8);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (T8) {
      load_b(min(g + 1, KG - 1), fill);
      load_a(min(g + 2, KG - 1), nx2);
    } else {
      load_a(min(g + 2, KG - 1), nx2);
      load_b(min(g + 2, KG - 1), fill);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto dequant = [&](int j, int ks) -> u32x4 {
      if constexpr (T8) {
        return int8_to_f16(Q[bu][j][ks >> 1][2 * (ks & 1)], Q[bu][j][ks >> 1][2 * (ks & 1) + 1]);
      } else {
        const float sc = bf16_to_f32(S[bu][j]) * rinv[j];
        return int4_to_f16(Q[bu][j][0][ks], pack_f16x2(sc, sc), pack_f16x2(-24.0f * sc, -24.0f * sc));
      }
    };
    // operands of 16-input step ks + 1 are read and dequantized while the
    // matrix cores work on step ks
    const uint16_t *as = cur + fh * 1024 + fr * 8;   // chunk 2 ks + fh, row 32 i + fr
    u32x4 af[2][MF], bf[2][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) af[0][i] = *reinterpret_cast<const u32x4 *>(as + i * 256);
#pragma unroll
    for (int j = 0; j < NF; ++j) bf[0][j] = dequant(j, 0);
    // let the scheduler interleave the operand reads with the matrix-core
    // instructions (it helps most where one wavefront runs per SIMD)
    __builtin_amdgcn_iglp_opt(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks & 1;
      if (ks < 3) {
#pragma unroll
        for (int i = 0; i < MF; ++i) af[c ^ 1][i] = *reinterpret_cast<const u32x4 *>(as + (ks + 1) * 2048 + i * 256);
#pragma unroll
        for (int j = 0; j < NF; ++j) bf[c ^ 1][j] = dequant(j, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = mfma32x32x16_f16(af[c][i], bf[c][j], acc[i][j]);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using INB1 = std::integral_constant<int, (NB > 2 ? 2 : 0)>;   // set 2 (INT4) or 0 (INT8)

  // pipeline fill in the order the steps issue their loads
  load_a(0, A0);
  load_b(0, I0{});
  if constexpr (T8) {
    load_a(min(1, KG - 1), A1);
  } else {
    load_a(min(1, KG - 1), A1);
    load_b(min(1, KG - 1), I1{});
  }
  // six steps per pass: buffers of A rotate by 3, sets of B by NB; the
  // passes run unconditionally (exact load counts at every wait), the last
  // fewer than six steps after them
  auto six = [&](int g, int n) {
    if constexpr (T8) {
      if (n > 0) step(g, A0, A2, I0{}, I1{});
      if (n > 1) step(g + 1, A1, A0, I1{}, I0{});
      if (n > 2) step(g + 2, A2, A1, I0{}, I1{});
      if (n > 3) step(g + 3, A0, A2, I1{}, I0{});
      if (n > 4) step(g + 4, A1, A0, I0{}, I1{});
      if (n > 5) step(g + 5, A2, A1, I1{}, I0{});
    } else {
      if (n > 0) step(g, A0, A2, I0{}, INB1{});
      if (n > 1) step(g + 1, A1, A0, I1{}, I0{});
      if (n > 2) step(g + 2, A2, A1, INB1{}, I1{});
      if (n > 3) step(g + 3, A0, A2, I0{}, INB1{});
      if (n > 4) step(g + 4, A1, A0, I1{}, I0{});
      if (n > 5) step(g + 5, A2, A1, INB1{}, I1{});
    }
  };
  int g = 0;
  for (; g + 6 <= KG; g += 6) six(g, 6);
  if (g < KG) six(g, KG - g);
  // the last steps' repeated copies into LDS are never read: let them land
  // before the workgroup can end
  __builtin_amdgcn_s_waitcnt(kVmcnt0);

  // ---- epilogue: row scale 2^e, INT8 row scale, low-rank slab, bf16 scatter
  // through idx -- or, with a K split, this range's result as fp32 at
  // [split][m][packed row] for psum_kernel.  Weight-side loads first, in one batch
  int pj[NF], col[NF];
  bool okj[NF];
  float s8[NF];
  u32x4 bu[NF][NS];   // U of row pj, slots 16 js + 8 fh .. + 7 of the low-rank vector
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int pl = p0 + 32 * j + fr;
    okj[j] = pl < rows;
    pj[j] = (T8 ? a.n4 : 0) + (okj[j] ? pl : 0);
    col[j] = a.idx[pj[j]];
    s8[j] = T8 ? a.s8[okj[j] ? pl : 0] : rsh[j];
  }
  const int seg_cols = a.N / a.n_seg;
  if (!lowrank) {
    // no low-rank term in this K-range
  } else if ((a.r & 7) == 0) {
    // slots of one segment are whole runs of 8: one 16-byte load each
    const auto ru = make_rsrc(a.U, static_cast<uint32_t>(a.N) * a.r * 2);
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int seg = col[j] / seg_cols;
#pragma unroll
      for (int js = 0; js < NS; ++js) {
        const int il = 16 * js + 8 * fh - seg * a.r;
        const bool in = okj[j] && il >= 0 && il < a.r;
        bu[j][js] = buf_load16(ru, in ? static_cast<uint32_t>(pj[j] * a.r + il) * 2 : kOutOfRange);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int seg = col[j] / seg_cols;
#pragma unroll
      for (int js = 0; js < NS; ++js)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t pair = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int il = 16 * js + 8 * fh + 2 * q + e - seg * a.r;
            uint32_t u = 0;
            if (okj[j] && il >= 0 && il < a.r) u = a.U[static_cast<int64_t>(pj[j]) * a.r + il];
            pair |= u << (16 * e);
          }
          bu[j][js][q] = pair;
        }
    }
  }
#pragma unroll
  for (int j = 0; j < NF; ++j) {
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 sc4 = *reinterpret_cast<const f32x4 *>(scs + 32 * i + 8 * k + 4 * fh);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][4 * k + v] *= sc4[v] * s8[j];
      }
    if (lowrank)
#pragma unroll
      for (int js = 0; js < NS; ++js)
#pragma unroll
        for (int i = 0; i < MF; ++i) {
          const u32x4 av = *reinterpret_cast<const u32x4 *>(ts + (32 * i + fr) * TS<NS> + 16 * js + 8 * fh);
          acc[i][j] = mfma32x32x16(av, bu[j][js], acc[i][j]);
        }
    if (!okj[j]) continue;
    if constexpr (SPLIT) {
      float *dst = a.part + static_cast<int64_t>(split) * a.M * a.N + pj[j];
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 32 * i + 8 * (v / 4) + 4 * fh + (v % 4);
          if (m < a.M) dst[static_cast<int64_t>(m) * a.N] = acc[i][j][v];
        }
    } else {
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + 32 * i + 8 * (v / 4) + 4 * fh + (v % 4);
          if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + col[j]] = f32_to_bf16(acc[i][j][v]);
        }
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __align__(16) uint16_t A0[kTileA];
  __shared__ __align__(16) uint16_t A1[kTileA];
  __shared__ __align__(16) uint16_t A2[kTileA];
  __shared__ __align__(16) uint16_t ts[kPfTileM * TS<4>];
  __shared__ __align__(16) float scs[kPfTileM];
  // consecutive workgroups share a weight tile (its bytes stay in L2); with a
  // K split, the ranges of one tile sit m_tiles workgroups apart
  const int mtile = blockIdx.x % a.m_tiles, rest = blockIdx.x / a.m_tiles;
  const int split = rest % a.ksplit, ntile = rest / a.ksplit;
  const bool t8 = ntile >= a.n4_tiles;
  const int tile0 = (t8 ? ntile - a.n4_tiles : ntile) * kPfTileN;
  if (a.ksplit > 1) {
    if (a.nsr_pad == 64) {
      if (t8) prefill_tile<true, 4, true>(a, A0, A1, A2, ts, scs, mtile, tile0, split);
      else prefill_tile<false, 4, true>(a, A0, A1, A2, ts, scs, mtile, tile0, split);
    } else {
      if (t8) prefill_tile<true, 2, true>(a, A0, A1, A2, ts, scs, mtile, tile0, split);
      else prefill_tile<false, 2, true>(a, A0, A1, A2, ts, scs, mtile, tile0, split);
    }
  } else if (a.nsr_pad == 64) {
    if (t8) prefill_tile<true, 4, false>(a, A0, A1, A2, ts, scs, mtile, tile0, 0);
    else prefill_tile<false, 4, false>(a, A0, A1, A2, ts, scs, mtile, tile0, 0);
  } else {
    if (t8) prefill_tile<true, 2, false>(a, A0, A1, A2, ts, scs, mtile, tile0, 0);
    else prefill_tile<false, 2, false>(a, A0, A1, A2, ts, scs, mtile, tile0, 0);
  }
}

// After a K split: y[m][idx[p]] = bf16(the ranges' results summed in range
// order; the first range carries the low-rank term).  Four consecutive packed
// rows of one token per thread.
__global__ __launch_bounds__(kThreads) void psum_kernel(PrefillArgs a) {
  const int nq = a.N / 4;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= static_cast<int64_t>(a.M) * nq) return;
  const int m = static_cast<int>(e / nq), p0 = static_cast<int>(e - static_cast<int64_t>(m) * nq) * 4;
  const int64_t plane4 = static_cast<int64_t>(a.M) * a.N / 4;
  const f32x4 *src = reinterpret_cast<const f32x4 *>(a.part + static_cast<int64_t>(m) * a.N + p0);
  f32x4 v[kPfSplitMax];
#pragma unroll
  for (int k = 0; k < kPfSplitMax; ++k) v[k] = k < a.ksplit ? src[k * plane4] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 col = *reinterpret_cast<const u32x4 *>(a.idx + p0);
  f32x4 acc = v[0];
#pragma unroll
  for (int k = 1; k < kPfSplitMax; ++k)
    if (k < a.ksplit) acc += v[k];
  uint16_t *yr = a.y + static_cast<int64_t>(m) * a.N;
#pragma unroll
  for (int q = 0; q < 4; ++q) yr[static_cast<int>(col[q])] = f32_to_bf16(acc[q]);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  const int grid = (a.n4_tiles + a.n8_tiles) * a.m_tiles * a.ksplit;
  const hipError_t e = launch_kernel(reinterpret_cast<const void *>(prefill_kernel), dim3(grid), dim3(kThreads), 0, s, a);
  if (e != hipSuccess || a.ksplit == 1) return e;
  const int64_t n = static_cast<int64_t>(a.M) * (a.N / 4);
  return launch_kernel(reinterpret_cast<const void *>(psum_kernel), dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, a);
}

}  // namespace dvssq
