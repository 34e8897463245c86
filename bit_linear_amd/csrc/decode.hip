// Decode path (M <= 32) of y = (x H) W_hat^T + ((x H) V^T) U^T in ONE kernel
// launch (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2,
// runtime equation; rotation: same card, Mathematical Foundations 1 and
// Spark-X2.5-4B-Hadamard-GSQ model card, Tier B equation; tiers: MiniCPM card
// INT4 equation and Spark card Tier A).  It serves the calls for which the
// small-M kernel (decode_small.hip) finds no plan: per-wavefront load counts,
// LDS for the activation planes (e.g. blocks of 2048 at M = 32) or 32-bit
// offsets out of its range.
//
// Roles inside the launch (workgroups of four wavefronts):
//  * producer workgroups (the lowest block indices, one per "unit" of
//    max(block, 256) inputs and per 8 activation rows) rotate the
//    activations with the fast Walsh-Hadamard transform, store x_rot as f16
//    scaled by a power of two 2^-e per (row, unit) so that it cannot overflow
//    f16, store the unit's partial t = x_rot V^T (fp32), and publish a 64-bit
//    generation flag.  These stores are device-scope (they bypass the
//    non-coherent per-XCD L2), and the flag is written only after they have
//    completed (s_waitcnt), so no cache-wide fence is needed.
//  * consumer workgroups own 16 packed rows; their four wavefronts split the
//    K-range.  Each wavefront issues ALL of its weight loads (at most 10 spans
//    of 128 inputs, 16-byte loads) before anything else, so nearly the whole
//    layer is in flight at once; then the workgroup waits for the flags, stages
//    the f16 x_rot of its K-range in LDS and runs 16x16x32 f16 MFMAs.  INT4
//    codes become exact f16 weights with one packed FMA per pair: a nibble
//    moved to bits 6-9 of a half and or-ed with 0x4C00 is the f16 value
//    16 + n, and fma(16 + n, s, -24 s) = (n - 8) s exactly (24 s and (n - 8) s
//    fit f16's 11 bits for any 8-bit-mantissa scale s).  INT8 codes become
//    exact f16 q (v_perm + xor + one packed add) and the fp32 row scale is
//    applied to the accumulator.  The accumulator of each unit is multiplied
//    back by 2^e at unit boundaries.  The four partial tiles are summed in LDS,
//    then the low-rank term t U^T is one bf16 MFMA per 32 columns of t.
//  * when a layer has too few rows to fill the GPU, K is also split over S
//    workgroups; each writes its fp32 partial with device-scope stores, and
//    the last of the S to arrive (per-group counter, cleared by the producers
//    of the same launch) sums the partials in a fixed order.
// Producers carry the lowest block indices, so they are dispatched before any
// consumer that waits on them; the wait is bounded.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;                   // packed rows per consumer group
constexpr int kProdRows = 8;                // activation rows per producer
constexpr int kVPrefetch = 8;               // V k-steps in flight per producer wave
constexpr long kSpinLimit = 1L << 22;       // bounded wait for a producer flag

__device__ __forceinline__ void st_dev(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// plain accesses when producer and consumer are separate launches
template <bool DEV, typename T>
__device__ __forceinline__ void st(T *p, T v) {
  if constexpr (DEV) st_dev(p, v);
  else *p = v;
}
template <bool DEV, typename T>
__device__ __forceinline__ T ld(const T *p) {
  if constexpr (DEV) return ld_dev(p);
  else return *p;
}
// wait until every store this thread issued has completed
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// --------------------------------------------------------------------------- producer

// Producer outputs x_rot (f16), scales and t.  kModeFused: device-scope
// stores, then the generation flag (consumers in the same launch);
// kModeSplit: plain stores (consumers in the next launch).
constexpr int kModeFused = 0, kModeSplit = 1;

// VPU: inputs per lane of one unit (unit = 64 * VPU).
template <int VPU, int MODE>
__device__ void produce(const DecodeArgs &a, int pidx, uint8_t *smem) {
  constexpr bool FUSED = MODE != kModeSplit;   // device-scope stores
  constexpr int P = 64 * VPU;
  constexpr int LDR = P + 8;                 // bf16 LDS row
  constexpr int RPW = kProdRows / kWaves;    // rows per wavefront
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = pidx % a.nunit, rg = pidx / a.nunit;
  const int m0 = rg * kProdRows;
  const int mrows = min(kProdRows, a.M - m0);
  const int k0 = u * P;
  const int nsteps = P / 16;
  const int n_it = a.nsr_pad / 32;
  uint16_t *xb = reinterpret_cast<uint16_t *>(smem);
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // 1. issue the activation loads and the first V fragments (clamped,
  // in-bounds addresses that feed no select, so they stay in flight)
  u32x2 xw[RPW][VPU / 4];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int ml = min(wave + kWaves * r, mrows - 1);
    const uint16_t *src = a.x + static_cast<int64_t>(m0 + ml) * a.K + k0 + lane * VPU;
#pragma unroll
    for (int j = 0; j < VPU / 4; ++j) xw[r][j] = *reinterpret_cast<const u32x2 *>(src + 4 * j);
  }
  const int arow = lane & 31, half = lane >> 5;
  const int my_steps = (nsteps - wave + kWaves - 1) / kWaves;
  u32x4 vb[kVPrefetch][2];
  auto vload = [&](int i, int slot) {
    const int s = min(wave + kWaves * min(i, my_steps - 1), nsteps - 1);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int row = min(32 * it + arow, a.nsr - 1);
      vb[slot][it] = *reinterpret_cast<const u32x4 *>(a.V + static_cast<int64_t>(row) * a.K + k0 + 16 * s + 8 * half);
    }
  };
#pragma unroll
  for (int i = 0; i < kVPrefetch; ++i) vload(i, i);

  if (a.S > 1) {  // clear this launch's split-K counters (each producer its share)
    const int n = a.g4 + a.g8;
    const int lo = static_cast<int>(static_cast<int64_t>(n) * pidx / a.nprod);
    const int hi = static_cast<int>(static_cast<int64_t>(n) * (pidx + 1) / a.nprod);
    for (int i = lo + tid; i < hi; i += kThreads) __hip_atomic_store(a.cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 2. rotate, scale, store
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int ml = wave + kWaves * r;
    uint16_t *row = xb + ml * LDR + lane * VPU;
    if (ml >= mrows) {
#pragma unroll
      for (int j = 0; j < VPU; j += 2) *reinterpret_cast<uint32_t *>(row + j) = 0u;
      continue;
    }
    float v[VPU];
#pragma unroll
    for (int j = 0; j < VPU / 4; ++j) {
      v[4 * j] = __uint_as_float(xw[r][j][0] << 16);
      v[4 * j + 1] = __uint_as_float(xw[r][j][0] & 0xFFFF0000u);
      v[4 * j + 2] = __uint_as_float(xw[r][j][1] << 16);
      v[4 * j + 3] = __uint_as_float(xw[r][j][1] & 0xFFFF0000u);
    }
    if (a.rotate) {
      // butterflies: strides 1 .. VPU/2 inside the lane, VPU .. block/2 across lanes
#pragma unroll
      for (int s = 1; s < VPU; s <<= 1)
#pragma unroll
        for (int j = 0; j < VPU; ++j)
          if (!(j & s)) {
            const float p = v[j], q = v[j + s];
            v[j] = p + q;
            v[j + s] = p - q;
          }
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        if (s * VPU >= a.block) break;
        const bool upper = (lane & s) != 0;
#pragma unroll
        for (int j = 0; j < VPU; ++j) {
          const float p = __shfl_xor(v[j], s, 64);
          v[j] = upper ? (p - v[j]) : (v[j] + p);
        }
      }
#pragma unroll
      for (int j = 0; j < VPU; ++j) v[j] *= a.hscale;
    }
    // power-of-two scale of this (row, unit): max |x_rot| * 2^-e lands in [2^14, 2^15)
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < VPU; ++j) mx = fmaxf(mx, fabsf(v[j]));
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));
    const int e = (mx > 0.0f && mx <= 3.0e38f) ? max(-120, min(120, ilogbf(mx) - 14)) : 0;
    const float down = ldexpf(1.0f, -e);
    const int m = m0 + ml;
    if (lane == 0) st<FUSED>(a.sc + u * kDecodeRows + m, ldexpf(1.0f, e));
    // unscaled bf16 copy for the t product
#pragma unroll
    for (int j = 0; j < VPU; j += 2) *reinterpret_cast<uint32_t *>(row + j) = pack_bf16x2(v[j], v[j + 1]);
    // scaled f16, each run of 8 inputs stored in the order 0,2,4,6,1,3,5,7
    uint16_t *dst = a.xq + static_cast<int64_t>(m) * a.K + k0;
    if constexpr (VPU >= 8) {
#pragma unroll
      for (int r8 = 0; r8 < VPU / 8; ++r8) {
        const float *w = v + 8 * r8;
        const uint64_t lo = pack_f16x2(w[0] * down, w[2] * down) |
                            (static_cast<uint64_t>(pack_f16x2(w[4] * down, w[6] * down)) << 32);
        const uint64_t hi = pack_f16x2(w[1] * down, w[3] * down) |
                            (static_cast<uint64_t>(pack_f16x2(w[5] * down, w[7] * down)) << 32);
        uint64_t *d64 = reinterpret_cast<uint64_t *>(dst + lane * VPU + 8 * r8);
        st<FUSED>(d64, lo);
        st<FUSED>(d64 + 1, hi);
      }
    } else {
      // VPU == 4: a run spans this lane (inputs 0-3 if even, 4-7 if odd) and its
      // xor-1 partner; the even lane stores pairs (0,2) (4,6), the odd lane (1,3) (5,7)
      const uint32_t pa = pack_f16x2(v[0] * down, v[2] * down);
      const uint32_t pb = pack_f16x2(v[1] * down, v[3] * down);
      const bool odd = lane & 1;
      const uint32_t recv = __shfl_xor(odd ? pa : pb, 1, 64);
      const uint32_t o0 = odd ? recv : pa;
      const uint32_t o1 = odd ? pb : recv;
      st<FUSED>(reinterpret_cast<uint64_t *>(dst + 8 * (lane >> 1) + 4 * (lane & 1)),
             static_cast<uint64_t>(o0) | (static_cast<uint64_t>(o1) << 32));
    }
  }
  __syncthreads();

  // 3. partial t of this unit on the matrix cores: rows m (x_rot, bf16) x rows i of V
  f32x16 acc[2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) acc[it][e2] = 0.0f;
  for (int i0 = 0; i0 < my_steps; i0 += kVPrefetch) {
#pragma unroll
    for (int jj = 0; jj < kVPrefetch; ++jj) {
      const int i = i0 + jj;
      const bool ok = i < my_steps;
      const int s = wave + kWaves * min(i, my_steps - 1);
      u32x4 av = *reinterpret_cast<const u32x4 *>(xb + (arow & (kProdRows - 1)) * LDR + 16 * s + 8 * half);
      av = (ok && arow < kProdRows) ? av : z4;
      acc[0] = mfma32x32x16(av, arow < a.nsr ? vb[jj][0] : z4, acc[0]);
      if (n_it > 1) acc[1] = mfma32x32x16(av, 32 + arow < a.nsr ? vb[jj][1] : z4, acc[1]);
      vload(i + kVPrefetch, jj);
    }
  }
  __syncthreads();
  float *red = reinterpret_cast<float *>(smem);  // [kWaves][2][32 m][32 i]
  {
    const int col = lane & 31;
    for (int it = 0; it < n_it; ++it)
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) {
        const int m = 8 * (v2 / 4) + 4 * half + (v2 % 4);
        red[((wave * 2 + it) * 32 + m) * 32 + col] = acc[it][v2];
      }
  }
  __syncthreads();
  for (int e2 = tid; e2 < mrows * a.nsr_pad; e2 += kThreads) {
    const int ml = e2 / a.nsr_pad, i = e2 % a.nsr_pad;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[((w * 2 + i / 32) * 32 + ml) * 32 + (i % 32)];
    const int64_t ti = (static_cast<int64_t>(u) * kDecodeRows + m0 + ml) * a.nsr_pad + i;
    st<FUSED>(a.tp + ti, s);
  }
  if constexpr (MODE == kModeFused) {
    drain_stores();
    __syncthreads();
    if (tid == 0) st_dev(a.flag + pidx, a.gen);
  }
}

// --------------------------------------------------------------------------- consumer

// MSUB: 16-token MFMA subtiles (1: M <= 16, 2: M <= 32); MAXS: most spans of
// 128 inputs one wavefront handles; T8: INT8 tier; FUSED: the producers run in
// the same launch (wait for their flags, device-scope loads).
template <int MSUB, int MAXS, bool T8, bool FUSED>
__device__ void consume(const DecodeArgs &a, int cidx, uint8_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int grp = cidx / a.S, split = cidx % a.S;
  const int rows = T8 ? a.n8 : a.n4;
  const int gbase = (T8 ? grp - a.g4 : grp) * kRows;    // first row of the group inside its tier
  const int pl = gbase + n;                              // this lane's weight row inside the tier
  const bool row_ok = pl < rows;
  const int plc = min(pl, rows - 1);
  const int p = (T8 ? a.n4 : 0) + pl;                    // packed row
  const int pc = (T8 ? a.n4 : 0) + plc;
  const int k0 = split * a.KW;
  const int nsp = (a.KW + 127) / 128;                    // spans of 128 inputs; the last may hold 64
  const int spw = (nsp + kWaves - 1) / kWaves;           // spans per wavefront (<= MAXS)
  const int js0 = wave * spw, js1 = min(nsp, js0 + spw);
  const int KG = a.K / kGroup;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // ---- 1. every weight load of this wavefront, issued first (clamped,
  // in-bounds addresses feeding no select: nothing waits for them yet)
  u32x4 cb[MAXS][2];
  uint32_t sb[MAXS];
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int j = min(js0 + i, nsp - 1);
    const int kk = min(128 * j + 32 * q, a.KW - 32);
    if constexpr (!T8) {
      cb[i][0] = *reinterpret_cast<const u32x4 *>(a.q4 + static_cast<int64_t>(plc) * (a.K / 2) + (k0 + kk) / 2);
      sb[i] = a.s4[static_cast<int64_t>(plc) * KG + (k0 + kk) / kGroup];
    } else {
      const int8_t *src = a.q8 + static_cast<int64_t>(plc) * a.K + k0 + kk;
      cb[i][0] = *reinterpret_cast<const u32x4 *>(src);
      cb[i][1] = *reinterpret_cast<const u32x4 *>(src + 16);
    }
  }
  // low-rank factors of the group's 16 rows: one contiguous range of U, fetched
  // now as aligned dwords (all threads) and parked in LDS after the main loop
  const int base = (T8 ? a.n4 : 0) + gbase;              // first packed row of the group
  const int64_t ue0 = static_cast<int64_t>(base) * a.r;  // its first U element
  const int64_t ud0 = ue0 / 2;
  const int64_t ud_last = (static_cast<int64_t>(a.N) * a.r + 1) / 2 - 1;
  const uint32_t *U32 = reinterpret_cast<const uint32_t *>(a.U);
  uint32_t uw[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) uw[j] = U32[std::min<int64_t>(ud0 + tid + kThreads * j, ud_last)];
  const int col = a.idx[pc];
  const int seg = col / (a.N / a.n_seg);
  const float s8 = T8 ? a.s8[plc] : 1.0f;

  // ---- 2. wait for every producer of this launch (one thread per flag)
  if constexpr (FUSED) {
    for (int i = tid; i < a.nprod; i += kThreads) {
      long spins = 0;
      while (ld_dev(a.flag + i) != a.gen && spins < kSpinLimit) {
        __builtin_amdgcn_s_sleep(1);
        ++spins;
      }
    }
    __syncthreads();
  }

  // ---- 3. stage x_rot (f16), unit scales and the t of units starting in range
  const int P = a.unit;
  const int LDX = a.KW + 8;
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
  const int u0 = k0 / P, u1 = (k0 + a.KW - 1) / P;          // units overlapping the range
  float *sf = reinterpret_cast<float *>(smem + static_cast<size_t>(a.M) * LDX * 2);
  float *ts = sf + (u1 - u0 + 1) * kDecodeRows;
  float *red = ts + a.M * a.nsr_pad;                        // [kWaves][MSUB][4][64]
  uint32_t *ush = reinterpret_cast<uint32_t *>(red + kWaves * MSUB * 4 * 64);  // [3 * kThreads]
  const int ut0 = (k0 + P - 1) / P, ut1 = (k0 + a.KW + P - 1) / P;  // units starting in range
  const bool has_t = ut0 < ut1;
  {
    // all staging loads of a thread are issued before any is used
    constexpr int XB = 4;
    const int per = a.KW / 4;
    const int nx = a.M * per;
    for (int e0 = tid; e0 < nx; e0 += XB * kThreads) {
      uint64_t v[XB];
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int e = min(e0 + b * kThreads, nx - 1);
        v[b] = ld<FUSED>(reinterpret_cast<const uint64_t *>(a.xq + static_cast<int64_t>(e / per) * a.K + k0 + (e % per) * 4));
      }
#pragma unroll
      for (int b = 0; b < XB; ++b) {
        const int e = e0 + b * kThreads;
        if (e < nx) *reinterpret_cast<uint64_t *>(xs + (e / per) * LDX + (e % per) * 4) = v[b];
      }
    }
    const int nsf = (u1 - u0 + 1) * a.M;
    for (int e = tid; e < nsf; e += kThreads)
      sf[(e / a.M) * kDecodeRows + e % a.M] = ld<FUSED>(a.sc + (u0 + e / a.M) * kDecodeRows + e % a.M);
    if (has_t)
      for (int e = tid; e < a.M * a.nsr_pad; e += kThreads) {
        const int m = e / a.nsr_pad, i = e % a.nsr_pad;
        const float *src = a.tp + static_cast<int64_t>(m) * a.nsr_pad + i;
        const int64_t ustride = static_cast<int64_t>(kDecodeRows) * a.nsr_pad;
        float s = 0.0f;
        for (int ub0 = ut0; ub0 < ut1; ub0 += 8) {   // 8 independent loads in flight, summed in order
          float v8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v8[j] = ld<FUSED>(src + min(ub0 + j, ut1 - 1) * ustride);
#pragma unroll
          for (int j = 0; j < 8; ++j) s += (ub0 + j < ut1) ? v8[j] : 0.0f;
        }
        ts[m * a.nsr_pad + i] = s;
      }
  }
  __syncthreads();

  // ---- 4. this wavefront's spans: straight-line code, masked past its range
  f32x4 C[MSUB], acc[MSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) C[ms][i] = acc[ms][i] = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int j = js0 + i;
    const bool span_ok = j < js1;
    const int jc = min(j, nsp - 1);
    const bool kq_ok = span_ok && (128 * jc + 32 * q < a.KW);
    const bool w_ok = kq_ok && row_ok;
    u32x4 bw[4];
    if constexpr (!T8) {
      const float s = w_ok ? bf16_to_f32(sb[i]) : 0.0f;   // zero scale -> zero weights
      const uint32_t s2 = pack_f16x2(s, s);
      const uint32_t c24 = pack_f16x2(-24.0f * s, -24.0f * s);
#pragma unroll
      for (int d = 0; d < 4; ++d) bw[d] = int4_to_f16(cb[i][0][d], s2, c24);
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x4 &c = cb[i][d >> 1];
        bw[d] = int8_to_f16(w_ok ? c[2 * (d & 1)] : 0u, w_ok ? c[2 * (d & 1) + 1] : 0u);
      }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms) {
        const int m = 16 * ms + n;
        const u32x4 xv = *reinterpret_cast<const u32x4 *>(xs + min(m, a.M - 1) * LDX +
                                                          min(128 * jc + 32 * q + 8 * d, a.KW - 8));
        C[ms] = mfma_f16((m < a.M && kq_ok) ? xv : z4, bw[d], C[ms]);
      }
    }
    const int kend = k0 + 128 * (jc + 1);
    const bool boundary = span_ok && ((kend % P == 0) || (j == js1 - 1));
    const int uu = min((k0 + 128 * jc) / P - u0, u1 - u0);
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int m = 16 * ms + 4 * q + r4;
        const float f = sf[uu * kDecodeRows + min(m, a.M - 1)];
        const float g = (boundary && m < a.M) ? f : 0.0f;
        acc[ms][r4] = fmaf(g, C[ms][r4], acc[ms][r4]);
        C[ms][r4] = boundary ? 0.0f : C[ms][r4];
      }
  }

  // ---- 5. sum the four wavefronts' tiles; wavefront 0 finishes
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) red[((wave * MSUB + ms) * 4 + r4) * 64 + lane] = acc[ms][r4];
#pragma unroll
  for (int j = 0; j < 3; ++j) ush[tid + kThreads * j] = uw[j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += red[((w * MSUB + ms) * 4 + r4) * 64 + lane];
      acc[ms][r4] = s * s8;
    }

  // ---- 6. low-rank term of the units that start in this range
  if (has_t) {
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(ush);
    const int uoff = static_cast<int>(ue0 - 2 * ud0);
    for (int st = 0; st < a.nsr_pad / 32; ++st) {
      u32x4 bv;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t pair = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ig = 32 * st + 8 * q + 2 * h + e;
          const int il = ig - seg * a.r;
          const bool ok = row_ok && ig < a.nsr && il >= 0 && il < a.r;
          const uint32_t uv = ok ? u16[n * a.r + il + uoff] : 0u;
          pair |= uv << (16 * e);
        }
        bv[h] = pair;
      }
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms) {
        const int m = 16 * ms + n;
        u32x4 av = z4;
        if (m < a.M) {
          const float *t = ts + m * a.nsr_pad + 32 * st + 8 * q;
#pragma unroll
          for (int h = 0; h < 4; ++h) av[h] = pack_bf16x2(t[2 * h], t[2 * h + 1]);
        }
        acc[ms] = mfma_bf16(av, bv, acc[ms]);
      }
    }
  }

  // ---- 7. output
  if (a.S == 1) {
    if (!row_ok) return;
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int m = 16 * ms + 4 * q + r4;
        if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + col] = f32_to_bf16(acc[ms][r4]);
      }
    return;
  }
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int m = 16 * ms + 4 * q + r4;
      if (m < a.M && row_ok) st_dev(a.part + (static_cast<int64_t>(split) * kDecodeRows + m) * a.N + p, acc[ms][r4]);
    }
  drain_stores();
  int old = 0;
  if (lane == 0) old = atomicAdd(a.cnt + grp, 1);
  old = __shfl(old, 0, 64);
  if (old != a.S - 1) return;
  const int nrows = min(kRows, rows - gbase);
  for (int e = lane; e < kRows * a.M; e += 64) {
    const int rr = e % kRows, m = e / kRows;
    if (rr >= nrows) continue;
    const int pp = base + rr;
    float s = 0.0f;
    for (int sp = 0; sp < a.S; ++sp) s += ld_dev(a.part + (static_cast<int64_t>(sp) * kDecodeRows + m) * a.N + pp);
    a.y[static_cast<int64_t>(m) * a.N + a.idx[pp]] = f32_to_bf16(s);
  }
}

template <int MODE>
__device__ __forceinline__ void produce_any(const DecodeArgs &a, int pidx, uint8_t *smem) {
  switch (a.unit) {
    case 256: produce<4, MODE>(a, pidx, smem); break;
    case 512: produce<8, MODE>(a, pidx, smem); break;
    case 1024: produce<16, MODE>(a, pidx, smem); break;
    default: produce<32, MODE>(a, pidx, smem); break;
  }
}

// FUSED: producers (block index < nprod) and consumers in one launch;
// otherwise consumers only, after decode_prologue_kernel.
template <int MSUB, int MAXS, bool FUSED>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  if (FUSED && b < a.nprod) {
    produce_any<kModeFused>(a, b, smem);
  } else {
    const int c = FUSED ? b - a.nprod : b;
    if (c / a.S < a.g4) consume<MSUB, MAXS, false, FUSED>(a, c, smem);
    else consume<MSUB, MAXS, true, FUSED>(a, c, smem);
  }
}

__global__ __launch_bounds__(kThreads) void decode_prologue_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  produce_any<kModeSplit>(a, blockIdx.x, smem);
}

hipError_t set_lds(const void *fn, size_t lds, std::atomic<uint64_t> &done) {
  if (lds <= 65536) return hipSuccess;
  return ensure_lds_limit(fn, 160 * 1024, done);
}

size_t prologue_lds_bytes(int unit) {
  return std::max<size_t>(static_cast<size_t>(kProdRows) * (unit + 8) * 2,
                          static_cast<size_t>(kWaves) * 2 * 32 * 32 * 4);
}

template <int MSUB, int MAXS>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
  const size_t lds = decode_lds_bytes(a.M, a.unit, a.KW, a.nsr_pad);
  const int groups = (a.g4 + a.g8) * a.S;
  if (a.fused) {
    static std::atomic<uint64_t> done{0};
    const hipError_t e = set_lds(reinterpret_cast<const void *>(decode_kernel<MSUB, MAXS, true>), lds, done);
    if (e != hipSuccess) return e;
    return launch_kernel(reinterpret_cast<const void *>(decode_kernel<MSUB, MAXS, true>), dim3(a.nprod + groups),
                         dim3(kThreads), lds, s, a);
  }
  hipError_t e = launch_kernel(reinterpret_cast<const void *>(decode_prologue_kernel), dim3(a.nprod), dim3(kThreads),
                               prologue_lds_bytes(a.unit), s, a);
  if (e != hipSuccess) return e;
  static std::atomic<uint64_t> done{0};
  e = set_lds(reinterpret_cast<const void *>(decode_kernel<MSUB, MAXS, false>), lds, done);
  if (e != hipSuccess) return e;
  return launch_kernel(reinterpret_cast<const void *>(decode_kernel<MSUB, MAXS, false>), dim3(groups), dim3(kThreads),
                       lds, s, a);
}

template <int MSUB>
hipError_t launch_m(const DecodeArgs &a, hipStream_t s) {
  const int spw = ((a.KW + 127) / 128 + kWaves - 1) / kWaves;
  if (spw <= 2) return launch_t<MSUB, 2>(a, s);
  if (spw <= 4) return launch_t<MSUB, 4>(a, s);
  if (spw <= 5) return launch_t<MSUB, 5>(a, s);
  if (spw <= 6) return launch_t<MSUB, 6>(a, s);
  if (spw <= 8) return launch_t<MSUB, 8>(a, s);
  return launch_t<MSUB, 10>(a, s);
}

}  // namespace

size_t decode_lds_bytes(int M, int unit, int KW, int nsr_pad) {
  const size_t prod = prologue_lds_bytes(unit);
  const size_t cons = static_cast<size_t>(M) * (KW + 8) * 2 + static_cast<size_t>(KW / unit + 2) * kDecodeRows * 4 +
                      static_cast<size_t>(M) * nsr_pad * 4 + static_cast<size_t>(kWaves) * 2 * 4 * 64 * 4 + 3 * kThreads * 4 + 16;
  return std::max(prod, cons);
}

int decode_max_spans() { return 10 * kWaves; }

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.unit != 256 && a.unit != 512 && a.unit != 1024 && a.unit != 2048) return hipErrorInvalidValue;
  return a.M <= 16 ? launch_m<1>(a, s) : launch_m<2>(a, s);
}

}  // namespace dvssq
