// Decode path (M <= 32) of y = (x H) W_hat^T + ((x H) V^T) U^T in ONE kernel
// launch (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2,
// runtime equation; rotation: same card, Mathematical Foundations 1 and
// Spark-X2.5-4B-Hadamard-GSQ model card, Tier B equation; tiers: MiniCPM card
// INT4 equation and Spark card Tier A).
//
// Roles inside the launch:
//  * producer workgroups (the lowest block indices, one per "unit" of
//    max(block, 256) inputs) rotate the activations with the fast
//    Walsh-Hadamard transform, store x_rot as f16 scaled by a power of two
//    2^-e per (row, unit) so that it cannot overflow f16, store the unit's
//    partial t = x_rot V^T (fp32), and publish a 64-bit generation flag.  All
//    these stores are device-scope (they bypass the non-coherent per-XCD L2),
//    and the flag is written only after they have completed (s_waitcnt), so no
//    cache-wide fence is needed.
//  * consumer workgroups (4 wavefronts, 16 packed rows each) first issue
//    their weight loads -- the HBM stream that dominates the call -- then wait
//    for the flags, stage the f16 x_rot of their K-range in LDS and run
//    16x16x32 f16 MFMAs.  INT4 codes become exact f16 weights with one packed
//    FMA per pair: a nibble moved to bits 6-9 of a half and or-ed with 0x4C00
//    is the f16 value 16 + n, and fma(16 + n, s, -24 s) = (n - 8) s exactly
//    (24 s and (n - 8) s fit f16's 11 bits for any 8-bit-mantissa scale s).
//    INT8 codes become exact f16 q (v_perm + xor + one packed
//    add) and the fp32 row scale is applied to the accumulator.  The
//    accumulator of each unit is multiplied back by 2^e at unit boundaries.
//    The low-rank term t U^T is one bf16 MFMA per 32 columns of t.
//  * when a layer has too few rows to fill the GPU, K is split over S
//    consumer groups; each writes its fp32 partial with device-scope stores,
//    and the last of the S to arrive (per-group counter, cleared by the
//    producers of the same launch) sums the partials in a fixed order.
// Producers carry the lowest block indices, so they are dispatched before any
// consumer that waits on them; the wait is bounded.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;
constexpr int kPrefetch = 8;           // spans (128 inputs) of codes in flight per lane
constexpr long kSpinLimit = 1L << 22;  // bounded wait for a producer flag

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
// wait until every store this thread issued has completed
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// --------------------------------------------------------------------------- producer

template <int VPU>  // inputs per lane of one unit (unit = 64 * VPU)
__device__ void produce(const DecodeArgs &a, int u, uint8_t *smem) {
  constexpr int P = 64 * VPU;
  constexpr int LDR = P + 8;  // bf16 LDS row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = u * P;
  uint16_t *xb = reinterpret_cast<uint16_t *>(smem);

  if (a.S > 1) {  // clear this launch's split-K counters (each producer its share)
    const int n = a.g4 + a.g8;
    const int lo = static_cast<int>(static_cast<int64_t>(n) * u / a.nunit);
    const int hi = static_cast<int>(static_cast<int64_t>(n) * (u + 1) / a.nunit);
    for (int i = lo + tid; i < hi; i += kThreads) __hip_atomic_store(a.cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  for (int m = wave; m < a.M; m += 4) {
    float v[VPU];
    const uint16_t *src = a.x + static_cast<int64_t>(m) * a.K + k0 + lane * VPU;
#pragma unroll
    for (int j = 0; j < VPU; j += 4) {
      const u32x2 w = *reinterpret_cast<const u32x2 *>(src + j);
      v[j] = __uint_as_float(w[0] << 16);
      v[j + 1] = __uint_as_float(w[0] & 0xFFFF0000u);
      v[j + 2] = __uint_as_float(w[1] << 16);
      v[j + 3] = __uint_as_float(w[1] & 0xFFFF0000u);
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
    if (lane == 0) st_dev(a.sc + u * kDecodeRows + m, ldexpf(1.0f, e));
    // unscaled bf16 copy for the t product
#pragma unroll
    for (int j = 0; j < VPU; j += 2)
      *reinterpret_cast<uint32_t *>(xb + m * LDR + lane * VPU + j) = pack_bf16x2(v[j], v[j + 1]);
    // scaled f16, each run of 8 inputs stored in the order 0,4,1,5,2,6,3,7
    uint16_t *dst = a.xq + static_cast<int64_t>(m) * a.K + k0;
    if constexpr (VPU >= 8) {
#pragma unroll
      for (int r8 = 0; r8 < VPU / 8; ++r8) {
        const float *w = v + 8 * r8;
        const uint64_t lo = pack_f16x2(w[0] * down, w[4] * down) |
                            (static_cast<uint64_t>(pack_f16x2(w[1] * down, w[5] * down)) << 32);
        const uint64_t hi = pack_f16x2(w[2] * down, w[6] * down) |
                            (static_cast<uint64_t>(pack_f16x2(w[3] * down, w[7] * down)) << 32);
        uint64_t *d64 = reinterpret_cast<uint64_t *>(dst + lane * VPU + 8 * r8);
        st_dev(d64, lo);
        st_dev(d64 + 1, hi);
      }
    } else {
      // VPU == 4: a run spans this lane (first or second half) and its xor-1 partner
      const uint32_t p0 = pack_f16x2(v[0] * down, v[1] * down);
      const uint32_t p1 = pack_f16x2(v[2] * down, v[3] * down);
      const bool odd = lane & 1;
      const uint32_t recv = __shfl_xor(odd ? p0 : p1, 1, 64);
      uint32_t o0, o1;
      if (!odd) {
        o0 = (p0 & 0xFFFFu) | (recv << 16);
        o1 = (p0 >> 16) | (recv & 0xFFFF0000u);
      } else {
        o0 = (recv & 0xFFFFu) | (p1 << 16);
        o1 = (recv >> 16) | (p1 & 0xFFFF0000u);
      }
      st_dev(reinterpret_cast<uint64_t *>(dst + 8 * (lane >> 1) + 4 * (lane & 1)),
             static_cast<uint64_t>(o0) | (static_cast<uint64_t>(o1) << 32));
    }
  }
  __syncthreads();

  // partial t of this unit on the matrix cores: rows m (x_rot, bf16) x rows i of V
  const int n_it = a.nsr_pad / 32;
  f32x16 acc[2];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int e2 = 0; e2 < 16; ++e2) acc[it][e2] = 0.0f;
  {
    const int arow = lane & 31, half = lane >> 5;
    for (int s = wave; s < P / 16; s += 4) {
      u32x4 av = {0u, 0u, 0u, 0u};
      if (arow < a.M) av = *reinterpret_cast<const u32x4 *>(xb + arow * LDR + 16 * s + 8 * half);
      for (int it = 0; it < n_it; ++it) {
        const int i = 32 * it + arow;
        u32x4 bv = {0u, 0u, 0u, 0u};
        if (i < a.nsr) bv = *reinterpret_cast<const u32x4 *>(a.V + static_cast<int64_t>(i) * a.K + k0 + 16 * s + 8 * half);
        if (it == 0) acc[0] = mfma32x32x16(av, bv, acc[0]);
        else acc[1] = mfma32x32x16(av, bv, acc[1]);
      }
    }
  }
  __syncthreads();
  float *red = reinterpret_cast<float *>(smem);  // [4 waves][2][32 m][32 i]
  {
    const int col = lane & 31, half = lane >> 5;
    for (int it = 0; it < n_it; ++it)
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) {
        const int m = 8 * (v2 / 4) + 4 * half + (v2 % 4);
        red[((wave * 2 + it) * 32 + m) * 32 + col] = acc[it][v2];
      }
  }
  __syncthreads();
  for (int e2 = tid; e2 < a.M * a.nsr_pad; e2 += kThreads) {
    const int m = e2 / a.nsr_pad, i = e2 % a.nsr_pad;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += red[((w * 2 + i / 32) * 32 + m) * 32 + (i % 32)];
    st_dev(a.tp + (static_cast<int64_t>(u) * kDecodeRows + m) * a.nsr_pad + i, s);
  }
  drain_stores();
  __syncthreads();
  if (tid == 0) st_dev(a.flag + u, a.gen);
}

// --------------------------------------------------------------------------- consumer

template <int MSUB>  // 16-token MFMA subtiles: 1 (M <= 16) or 2 (M <= 32)
__device__ void consume(const DecodeArgs &a, int cidx, uint8_t *smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int grp = cidx / a.S, split = cidx % a.S;
  const bool t8 = grp >= a.g4;
  const int rows = t8 ? a.n8 : a.n4;
  const int gbase = (t8 ? grp - a.g4 : grp) * 64;       // first row of the group inside its tier
  const int pl = gbase + wave * 16 + n;                  // this lane's weight row inside the tier
  const bool row_ok = pl < rows;
  const int p = (t8 ? a.n4 : 0) + pl;                    // packed row
  const int k0 = split * a.KW;
  const int nsp = (a.KW + 127) / 128;   // spans of 128 inputs; the last may hold 64
  const int KG = a.K / kGroup;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // ---- 1. weight stream first: kPrefetch spans in flight per lane
  u32x4 cb[kPrefetch][2];
  uint32_t sb[kPrefetch];
  auto issue = [&](int j, int slot) {
    const bool ok = row_ok && (128 * j + 32 * q < a.KW);
    if (!t8) {
      cb[slot][0] = ok ? *reinterpret_cast<const u32x4 *>(a.q4 + static_cast<int64_t>(pl) * (a.K / 2) +
                                                           (k0 + 128 * j) / 2 + 16 * q)
                       : z4;
      sb[slot] = ok ? a.s4[static_cast<int64_t>(pl) * KG + (k0 + 128 * j + 32 * q) / kGroup] : 0u;
    } else {
      const int8_t *src = a.q8 + static_cast<int64_t>(pl) * a.K + k0 + 128 * j + 32 * q;
      cb[slot][0] = ok ? *reinterpret_cast<const u32x4 *>(src) : z4;
      cb[slot][1] = ok ? *reinterpret_cast<const u32x4 *>(src + 16) : z4;
    }
  };
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j)
    if (j < nsp) issue(j, j);

  // ---- 2. wait for every producer of this launch
  if (tid == 0) {
    for (int u = 0; u < a.nunit; ++u) {
      long spins = 0;
      while (ld_dev(a.flag + u) != a.gen && spins < kSpinLimit) {
        __builtin_amdgcn_s_sleep(1);
        ++spins;
      }
    }
  }
  __syncthreads();

  // ---- 3. stage x_rot (f16), unit scales and the t of units starting in range
  const int P = a.unit;
  const int LDX = a.KW + 8;
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
  const int u0 = k0 / P, u1 = (k0 + a.KW - 1) / P;          // units overlapping the range
  float *sf = reinterpret_cast<float *>(smem + static_cast<size_t>(a.M) * LDX * 2);
  float *ts = sf + (u1 - u0 + 1) * kDecodeRows;
  const int ut0 = (k0 + P - 1) / P, ut1 = (k0 + a.KW + P - 1) / P;  // units starting in range
  const bool has_t = ut0 < ut1;
  {
    const int per = a.KW / 4;
    for (int e = tid; e < a.M * per; e += kThreads) {
      const int m = e / per, c4 = (e % per) * 4;
      const uint64_t v = ld_dev(reinterpret_cast<const uint64_t *>(a.xq + static_cast<int64_t>(m) * a.K + k0 + c4));
      *reinterpret_cast<uint64_t *>(xs + m * LDX + c4) = v;
    }
    for (int e = tid; e < (u1 - u0 + 1) * a.M; e += kThreads) {
      const int uu = e / a.M, m = e % a.M;
      sf[uu * kDecodeRows + m] = ld_dev(a.sc + (u0 + uu) * kDecodeRows + m);
    }
    if (has_t)
      for (int e = tid; e < a.M * a.nsr_pad; e += kThreads) {
        const int m = e / a.nsr_pad, i = e % a.nsr_pad;
        float s = 0.0f;
        for (int u = ut0; u < ut1; ++u) s += ld_dev(a.tp + (static_cast<int64_t>(u) * kDecodeRows + m) * a.nsr_pad + i);
        ts[m * a.nsr_pad + i] = s;
      }
  }
  __syncthreads();

  // ---- 4. main loop over spans of 128 inputs
  f32x4 C[MSUB], acc[MSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) C[ms][i] = acc[ms][i] = 0.0f;

  for (int j0 = 0; j0 < nsp; j0 += kPrefetch) {
#pragma unroll
    for (int jj = 0; jj < kPrefetch; ++jj) {
      const int j = j0 + jj;
      if (j >= nsp) break;
      const bool kq_ok = 128 * j + 32 * q < a.KW;
      u32x4 bw[4];
      if (!t8) {
        const float s = bf16_to_f32(sb[jj]);
        const uint32_t s2 = pack_f16x2(s, s);
        const uint32_t c24 = pack_f16x2(-24.0f * s, -24.0f * s);
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = int4_to_f16(cb[jj][0][d], s2, c24);
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) bw[d] = int8_to_f16(cb[jj][d >> 1][2 * (d & 1)], cb[jj][d >> 1][2 * (d & 1) + 1]);
      }
      if (j + kPrefetch < nsp) issue(j + kPrefetch, jj);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
          const int m = 16 * ms + n;
          const u32x4 av = (m < a.M && kq_ok) ? *reinterpret_cast<const u32x4 *>(xs + m * LDX + 128 * j + 32 * q + 8 * d) : z4;
          C[ms] = mfma_f16(av, bw[d], C[ms]);
        }
      }
      const int kend = k0 + 128 * (j + 1);
      if (kend % P == 0 || j == nsp - 1) {
        const int uu = (k0 + 128 * j) / P - u0;
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * ms + 4 * q + i;
            const float f = (m < a.M) ? sf[uu * kDecodeRows + m] : 0.0f;
            acc[ms][i] = fmaf(f, C[ms][i], acc[ms][i]);
            C[ms][i] = 0.0f;
          }
      }
    }
  }
  if (t8) {
    const float s8 = row_ok ? a.s8[pl] : 0.0f;
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[ms][i] *= s8;
  }

  // ---- 5. low-rank term of the units that start in this range
  if (has_t) {
    const int seg = row_ok ? a.idx[p] / (a.N / a.n_seg) : 0;
    for (int st = 0; st < a.nsr_pad / 32; ++st) {
      u32x4 bv;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t pair = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int ig = 32 * st + 8 * q + 2 * h + e;
          const int il = ig - seg * a.r;
          uint32_t uv = 0;
          if (row_ok && ig < a.nsr && il >= 0 && il < a.r) uv = a.U[static_cast<int64_t>(p) * a.r + il];
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

  // ---- 6. output
  if (a.S == 1) {
    if (!row_ok) return;
    const int col = a.idx[p];
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * ms + 4 * q + i;
        if (m < a.M) a.y[static_cast<int64_t>(m) * a.N + col] = f32_to_bf16(acc[ms][i]);
      }
    return;
  }
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * ms + 4 * q + i;
      if (m < a.M && row_ok) st_dev(a.part + (static_cast<int64_t>(split) * kDecodeRows + m) * a.N + p, acc[ms][i]);
    }
  drain_stores();
  __syncthreads();
  int *flagw = reinterpret_cast<int *>(smem);
  if (tid == 0) flagw[0] = atomicAdd(a.cnt + grp, 1);
  __syncthreads();
  if (flagw[0] != a.S - 1) return;
  const int base = (t8 ? a.n4 : 0) + gbase;
  const int nrows = min(64, rows - gbase);
  for (int e = tid; e < 64 * a.M; e += kThreads) {
    const int rr = e & 63, m = e >> 6;
    if (rr >= nrows) continue;
    const int pp = base + rr;
    float s = 0.0f;
    for (int sp = 0; sp < a.S; ++sp) s += ld_dev(a.part + (static_cast<int64_t>(sp) * kDecodeRows + m) * a.N + pp);
    a.y[static_cast<int64_t>(m) * a.N + a.idx[pp]] = f32_to_bf16(s);
  }
}

template <int VPU, int MSUB>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  if (static_cast<int>(blockIdx.x) < a.nunit) produce<VPU>(a, blockIdx.x, smem);
  else consume<MSUB>(a, blockIdx.x - a.nunit, smem);
}

template <int VPU, int MSUB>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
  constexpr int P = 64 * VPU;
  const size_t prod = std::max<size_t>(static_cast<size_t>(a.M) * (P + 8) * 2, 4 * 2 * 32 * 32 * 4);
  const int nu_local = a.KW / a.unit + 2;
  const size_t cons = static_cast<size_t>(a.M) * (a.KW + 8) * 2 + static_cast<size_t>(nu_local) * kDecodeRows * 4 +
                      static_cast<size_t>(a.M) * a.nsr_pad * 4 + 16;
  const size_t lds = std::max(prod, cons);
  if (lds > 65536) {
    static size_t set_to = 0;
    if (lds > set_to) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_kernel<VPU, MSUB>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      set_to = 160 * 1024;
    }
  }
  const int grid = a.nunit + (a.g4 + a.g8) * a.S;
  hipLaunchKernelGGL((decode_kernel<VPU, MSUB>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int VPU>
hipError_t launch_v(const DecodeArgs &a, hipStream_t s) {
  return a.M <= 16 ? launch_t<VPU, 1>(a, s) : launch_t<VPU, 2>(a, s);
}

}  // namespace

size_t decode_lds_bytes(int M, int unit, int KW, int nsr_pad) {
  const size_t prod = std::max<size_t>(static_cast<size_t>(M) * (unit + 8) * 2, 4 * 2 * 32 * 32 * 4);
  const size_t cons = static_cast<size_t>(M) * (KW + 8) * 2 + static_cast<size_t>(KW / unit + 2) * kDecodeRows * 4 +
                      static_cast<size_t>(M) * nsr_pad * 4 + 16;
  return std::max(prod, cons);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  switch (a.unit) {
    case 256: return launch_v<4>(a, s);
    case 512: return launch_v<8>(a, s);
    case 1024: return launch_v<16>(a, s);
    case 2048: return launch_v<32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dvssq
