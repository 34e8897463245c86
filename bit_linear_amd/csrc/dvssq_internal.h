// Internal declarations of the DV-SSQ HIP library (gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/dvssq.h"

namespace dvssq {

// ------------------------------------------------------------------ vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Launch of a kernel whose only parameter is an argument struct.  Returns the
// status of this launch itself (not a sticky error left by earlier calls).
template <typename Args>
inline hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, size_t lds, hipStream_t s, const Args &a) {
  void *args[] = {const_cast<Args *>(&a)};
  return hipLaunchKernel(fn, grid, block, args, lds, s);
}

// Launch of a kernel with plain parameters.
template <typename... T>
inline hipError_t launch_kernel_args(const void *fn, dim3 grid, dim3 block, size_t lds, hipStream_t s, T... v) {
  void *args[] = {static_cast<void *>(&v)...};
  return hipLaunchKernel(fn, grid, block, args, lds, s);
}

constexpr int kGroup = 64;      // INT4 group size
constexpr int kDecodeRows = 32; // M rows held by the decode workspace (MFMA tile height)

// ------------------------------------------------------------------ scalar helpers
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// two fp32 -> packed bf16x2 (nearest-even), low half = lo
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// The gated MLP block's intermediate h = gelu(gate) * up (Spark-X2.5-4B GGUF
// page, "The model": a GELU feed-forward block; ASHQ1 page, Architecture:
// ffn_gate, ffn_up, ffn_down): GELU is the exact v Phi(v) with
// Phi(v) = erfc(-v / sqrt 2) / 2 (relatively accurate in the negative tail,
// where 1 + erf(v / sqrt 2) would cancel), the product rounded once to bf16.
// Every kernel that forms h uses these two functions, so h has the same bits
// wherever it is formed.
__device__ __forceinline__ float gelu_exact(float v) { return 0.5f * v * erfcf(v * -0.70710678118654752f); }
// two bf16 gate values and the matching up values -> two bf16 h values
__device__ __forceinline__ uint32_t geglu_bf16x2(uint32_t g, uint32_t u) {
  const float lo = gelu_exact(__uint_as_float(g << 16)) * __uint_as_float(u << 16);
  const float hi = gelu_exact(__uint_as_float(g & 0xFFFF0000u)) * __uint_as_float(u & 0xFFFF0000u);
  return pack_bf16x2(lo, hi);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ buffer loads
// Buffer resources over one array (raw addressing, byte offsets).  A load at
// an offset at or past num_records returns zeros and makes no memory access.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ------------------------------------------------------------------ f16 operands
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pk_fma(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, a),
                                                                __builtin_bit_cast(f16x2, b),
                                                                __builtin_bit_cast(f16x2, c)));
}
__device__ __forceinline__ uint32_t pk_add(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) + __builtin_bit_cast(f16x2, b));
}
// One dword of packed INT4 codes (byte j: code k+j low, k+j+4 high) -> 8 exact
// f16 (n - 8) s in slots k+0,2,4,6,1,3,5,7.  Each nibble pair is moved to bits
// 6-9 of the two halves; or-ed with 0x4C00
// that is the f16 value 16 + n.  With s = m 2^E (m < 256, a bf16 value in
// [2^-17, 2^11)), s, -24 s = -3m 2^(E+3) and (n - 8) s are multiples of 2^-24
// with at most 10, 10 and 11 significant bits, so s and -24 s are exact f16
// and the fused fma(16 + n, s, -24 s) returns (n - 8) s exactly.
__device__ __forceinline__ u32x4 int4_to_f16(uint32_t w, uint32_t s2, uint32_t c24) {
  const uint32_t m = 0x03C003C0u, o = 0x4C004C00u;
  u32x4 r;
  r[0] = pk_fma(((w << 6) & m) | o, s2, c24);
  r[1] = pk_fma(((w << 2) & m) | o, s2, c24);
  r[2] = pk_fma(((w >> 2) & m) | o, s2, c24);
  r[3] = pk_fma(((w >> 6) & m) | o, s2, c24);
  return r;
}

// 8 INT8 codes (k+0..3 in lo, k+4..7 in hi) -> 8 exact f16 q, slots k+0,2,4,6,1,3,5,7
__device__ __forceinline__ u32x4 int8_to_f16(uint32_t lo, uint32_t hi) {
  const uint32_t m1152 = 0xE480E480u;  // f16 -1152 twice
  // byte pairs (k0,k2) (k4,k6) (k1,k3) (k5,k7); selector bytes 0-3 pick lo, 4-7 hi, 0x0C zero
  const uint32_t sel[4] = {0x0C020C00u, 0x0C060C04u, 0x0C030C01u, 0x0C070C05u};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pk_add(__builtin_amdgcn_perm(hi, lo, sel[i]) ^ 0x64806480u, m1152);
  return r;
}

// ------------------------------------------------------------------ launch set-up
// Allow a kernel more than 64 KB of dynamic LDS (up to `bytes`), once per
// device: the attribute belongs to the current device.  `done` holds one bit
// per device id already set up (ids >= 64 are set up on every call).
inline hipError_t ensure_lds_limit(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// ------------------------------------------------------------------ Hadamard blocks on the matrix cores
typedef int16_t s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16_bf16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}

// bf16 entry (a, b) of the 16x16 block-diagonal matrix with Sylvester blocks H_R
__device__ __forceinline__ uint32_t sylvester_bf16(int a, int b, int R) {
  if ((a ^ b) & ~(R - 1)) return 0u;   // different blocks (R a power of two)
  return (__popc(a & b & (R - 1)) & 1) ? 0xBF80u : 0x3F80u;
}

// bf16 entries (4q + j, n), j < 4, of H_16 (Sylvester, +-1) as two packed
// pairs.  The sign is the parity of (4q + j) & n = parity(q & (n >> 2)) xor
// parity(j & (n & 3)); the second term, as a 4-bit mask over j, is 0x0, 0xA,
// 0xC, 0x6 for n & 3 = 0 .. 3.
__device__ __forceinline__ u32x2 sylvester_h16(int n, int q) {
  uint32_t t = (0x6CA0u >> (4 * (n & 3))) & 0xFu;
  t ^= (__popc(q & (n >> 2)) & 1) ? 0xFu : 0u;
  u32x2 h;
  h[0] = 0x3F803F80u | ((t & 1u) << 15) | ((t & 2u) << 30);
  h[1] = 0x3F803F80u | ((t & 4u) << 13) | ((t & 8u) << 28);
  return h;
}

// Rotation of C blocks of 256 inputs (or one block of b < 256 inputs, C = 1)
// of one row by one wavefront: lane (n, q) = (lane % 16, lane / 16) holds, for
// every 256-block c, the inputs 256 c + 16 n + 4 q + j, j < 4 (xw: bf16 pairs),
// and gets x H at the same positions, scaled by hscale = 1/sqrt(block).  A
// Sylvester block of 256 is H_16 (x) H_16, so a block viewed as a 16x16 matrix X
// becomes Hs X H_16 (Hs = H_16, or I (x) H_{b/16} for b < 256): one bf16 MFMA for
// X H_16 (exact products, fp32 sums) and two for the second factor on that fp32
// result split into bf16 high and low parts; blocks of 512 .. 2048 combine
// their 256-blocks with butterflies in registers.
template <int C>
__device__ __forceinline__ void rotate_blocks(const u32x2 (&xw)[C], float (&y)[C][4], int block, float hscale) {
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const u32x2 h1 = sylvester_h16(n, q);
  u32x2 h2 = h1;
  if (block < 256) {
    const int Rb = block / 16;
    h2[0] = sylvester_bf16(4 * q, n, Rb) | (sylvester_bf16(4 * q + 1, n, Rb) << 16);
    h2[1] = sylvester_bf16(4 * q + 2, n, Rb) | (sylvester_bf16(4 * q + 3, n, Rb) << 16);
  }
  const f32x4 zf = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const f32x4 F = mfma16_bf16(xw[c], h1, zf);  // X H_16, lane: rows 4q+j, column n
    u32x2 hi, lo;
    hi[0] = pack_bf16x2(F[0], F[1]);
    hi[1] = pack_bf16x2(F[2], F[3]);
    lo[0] = pack_bf16x2(F[0] - __uint_as_float(hi[0] << 16), F[1] - __uint_as_float(hi[0] & 0xFFFF0000u));
    lo[1] = pack_bf16x2(F[2] - __uint_as_float(hi[1] << 16), F[3] - __uint_as_float(hi[1] & 0xFFFF0000u));
    f32x4 D = mfma16_bf16(hi, h2, zf);             // (Hs X H_16)^T, high part ...
    D = mfma16_bf16(lo, h2, D);                    // ... plus low part
#pragma unroll
    for (int j = 0; j < 4; ++j) y[c][j] = D[j];
  }
#pragma unroll
  for (int sft = 1; sft < C; sft <<= 1)
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (!(c & sft))
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = y[c][j], p1 = y[c + sft][j];
          y[c][j] = p0 + p1;
          y[c + sft][j] = p0 - p1;
        }
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) y[c][j] *= hscale;
}

// ------------------------------------------------------------------ decode helpers
// device-scope (agent) relaxed stores and loads: visible to every workgroup
__device__ __forceinline__ void st_dev(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ld_dev16(const void *p) {
  const uint64_t *q = static_cast<const uint64_t *>(p);
  const uint64_t lo = ld_dev(q), hi = ld_dev(q + 1);
  u32x4 r;
  r[0] = static_cast<uint32_t>(lo);
  r[1] = static_cast<uint32_t>(lo >> 32);
  r[2] = static_cast<uint32_t>(hi);
  r[3] = static_cast<uint32_t>(hi >> 32);
  return r;
}
// Arrival on a tagged counter {stamp : 32, count : 32} that needs no
// initialization; returns the count after this arrival.  The first arriver of
// a call (the word still holds another stamp) installs {stamp, 1} by
// compare-and-swap; every later arriver adds 1 with one fetch-add, so
// arrivals that come together do not retry against each other.
__device__ inline uint32_t arrive_tagged(uint64_t *cnt, uint32_t stamp) {
  uint64_t old = ld_dev(cnt);
  for (;;) {
    if (static_cast<uint32_t>(old >> 32) == stamp)
      return static_cast<uint32_t>(__hip_atomic_fetch_add(cnt, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) +
             1u;
    if (__hip_atomic_compare_exchange_strong(cnt, &old, (static_cast<uint64_t>(stamp) << 32) | 1u, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      return 1u;
    // old now holds the word another arriver wrote: its stamp is this call's
  }
}
// wait until every store this thread issued has completed
__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// cross-lane steps on the DPP network (rows of 16 lanes): xor 1, xor 2 inside
// a quad, mirror inside 8 and inside 16 lanes
#define DVSSQ_DPP(v, ctrl) __builtin_amdgcn_update_dpp(0, (v), (ctrl), 0xF, 0xF, false)
__device__ __forceinline__ float wave_max(float v) {
  int b = __float_as_int(v);
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(DVSSQ_DPP(b, 0xB1))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(DVSSQ_DPP(b, 0x4E))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(DVSSQ_DPP(b, 0x141))));
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(DVSSQ_DPP(b, 0x140))));
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float m1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float m2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float m3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}
__device__ __forceinline__ int quad_sum(int v) {
  v += DVSSQ_DPP(v, 0xB1);
  v += DVSSQ_DPP(v, 0x4E);
  return v;
}
// four bytes (the low byte of each value) in one dword, v0 lowest
__device__ __forceinline__ uint32_t pack_bytes(int v0, int v1, int v2, int v3) {
  const uint32_t lo = __builtin_amdgcn_perm(static_cast<uint32_t>(v1), static_cast<uint32_t>(v0), 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm(static_cast<uint32_t>(v3), static_cast<uint32_t>(v2), 0x0C0C0400u);
  return lo | (hi << 16);
}

// 15-bit quantization of one rotated (row, unit) item held by a wavefront:
// max |X| in [2^13, 2^14] with X = rint(x_rot 2^-e); X = 256 x1 + x2 with x2
// the signed low byte.  Returns e; p1 / p2 get the lane's four x1 / x2 bytes of
// each 256-block and gsum 8 x the sum of X over the lane's group of 64 inputs
// (the same in the 16 lanes of that group).
template <int C>
__device__ __forceinline__ int quantize_item(const float (&y)[C][4], uint32_t (&p1)[C], uint32_t (&p2)[C],
                                             int (&gsum)[C]) {
  float mx = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(y[c][j]));
  mx = wave_max(mx);
  const int e = (mx > 0.0f && mx <= 3.0e38f) ? max(-100, min(114, ilogbf(mx) - 13)) : 0;
  const float down = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    int X[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) X[j] = __float2int_rn(y[c][j] * down);
    p1[c] = pack_bytes((X[0] + 128) >> 8, (X[1] + 128) >> 8, (X[2] + 128) >> 8, (X[3] + 128) >> 8);
    p2[c] = pack_bytes(X[0], X[1], X[2], X[3]);
    int g = quad_sum(X[0] + X[1] + X[2] + X[3]);
    g += __shfl_xor(g, 16, 64);
    g += __shfl_xor(g, 32, 64);
    gsum[c] = 8 * g;
  }
  return e;
}

// Rotation of one (row, unit) item by one wavefront (rotate_blocks), or the
// plain bf16 values when x already holds x H.
template <int C>
__device__ __forceinline__ void rotate_x_item(int rotate, int block, float hscale, const u32x2 (&xw)[C],
                                              float (&y)[C][4]) {
  if (!rotate) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      y[c][0] = __uint_as_float(xw[c][0] << 16);
      y[c][1] = __uint_as_float(xw[c][0] & 0xFFFF0000u);
      y[c][2] = __uint_as_float(xw[c][1] << 16);
      y[c][3] = __uint_as_float(xw[c][1] & 0xFFFF0000u);
    }
    return;
  }
  rotate_blocks<C>(xw, y, block, hscale);
}

// ------------------------------------------------------------------ register FWHT
// Fast Walsh-Hadamard transform of one block of 64 VPL values held by a
// wavefront, VPL consecutive values per lane (Sylvester order, unnormalized):
// log2(VPL) butterfly stages in registers, then the six stages across lanes.
// value of lane l ^ S (S = 1 .. 32): DPP quad permutes for 1 and 2, row shifts
// for 4 and 8 (lanes with bit S clear read S lanes up, the others S lanes
// down), and the permlane swaps of 16-lane rows / 32-lane halves for 16 and 32
template <int S>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  const int x = __float_as_int(v);
  if constexpr (S == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  } else if constexpr (S == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  } else if constexpr (S == 4 || S == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x100 + S, 0xF, 0xF, false);
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x110 + S, 0xF, 0xF, false);
    return __int_as_float((lane & S) ? dn : up);
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  }
}

// one butterfly stage across lanes: lanes with bit S clear keep v + p, the
// others p - v (p = the partner's value)
template <int S, int VPL>
__device__ __forceinline__ void lane_stage(float (&v)[VPL], int lane) {
  const float sg = (lane & S) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) v[j] = fmaf(sg, v[j], xor_lane<S>(v[j], lane));
}

template <int VPL>
__device__ __forceinline__ void fwht_wave(float (&v)[VPL], int lane) {
#pragma unroll
  for (int s = 1; s < VPL; s <<= 1)
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (!(j & s)) {
        const float a = v[j], b = v[j + s];
        v[j] = a + b;
        v[j + s] = a - b;
      }
  lane_stage<1>(v, lane);
  lane_stage<2>(v, lane);
  lane_stage<4>(v, lane);
  lane_stage<8>(v, lane);
  lane_stage<16>(v, lane);
  lane_stage<32>(v, lane);
}

// ------------------------------------------------------------------ prefill tiles
// The prefill GEMM takes kPfTileM tokens by kPfTileN weight rows per workgroup
// and one INT4 group (64 inputs) per step.  Its x_rot operand is stored as
// tiles of kPfTileM rows by 64 inputs (16 KB), tile (m / 128, k / 64) at
// ((m / 128) (K / 64) + k / 64) 8192 f16, rows past M left unwritten.  Inside
// a tile, run r = (k % 64) / 8 of 8 inputs fills chunk 2 (r % 4) + r / 4 of
// 128 rows x 8 f16: one matrix-core step of 16 inputs per lane half reads two
// whole chunks, and one step of the GEMM copies one contiguous tile.
constexpr int kPfTileM = 128;
constexpr int kPfTileN = 256;
__host__ __device__ inline int64_t xr_tile_offset(int m, int k, int K) {
  const int r = (k & 63) >> 3;
  return ((static_cast<int64_t>(m >> 7) * (K >> 6) + (k >> 6)) * 8 + 2 * (r & 3) + (r >> 2)) * 1024 + (m & 127) * 8;
}
inline int64_t pf_rows(int M) { return (static_cast<int64_t>(M) + kPfTileM - 1) / kPfTileM * kPfTileM; }

// ------------------------------------------------------------------ workspace
// Byte offsets inside the caller's workspace.  Decode and prefill regions
// overlap (one call at a time per workspace).
constexpr int kMaxSplit = 16;   // largest decode split-K factor
constexpr int kTSplitMax = 16;  // largest number of K-ranges of the prefill's t product

// The first kStatusBytes of every workspace are its status area: the int32 at
// offset 0 is set to DVSSQ_STATUS_WAIT_TIMEOUT by a kernel whose bounded wait
// gave up (sticky: the library never clears it).
constexpr int64_t kStatusBytes = 256;

struct WsLayout {
  // decode
  int64_t d_xq;    // int8 planes [2][32][K]: x_rot quantized to X = 256 x1 + x2 per (row, unit)
  int64_t d_tp;    // fp32 [nunit][32][nsr_pad]: partial t = x_rot V^T of each unit
  int64_t d_flag;  // u64 [nunit * 2]: generation stamp written by each producer
  int64_t d_x8g;   // int32 [K/64][32]: 8 x (sum of the quantized x of a group)
  int64_t d_escg;  // fp32 [nunit][32]: 2^e of each (unit, row)
  int64_t d_cntw;  // u64 [groups]: tagged split-K arrival counters
  int64_t d_part;  // fp32 [S][32][N]: split-K partial outputs (last: a call uses S <= kMaxSplit planes)
  int64_t d_end;
  // prefill
  int64_t p_xr;    // f16 x_rot tiles of [M_max rounded up to 128][K], scaled by 2^-e per row
  int64_t p_sc;    // fp32 [M_max] 2^e per row
  int64_t p_rsh;   // fp32 [n_int4] 2^c per INT4 row: its group scales are used as s4 2^-c
  int64_t p_t;     // fp32 [M_max][nsr_pad] t = x_rot V^T
  int64_t p_tpart; // fp32 [kTSplitMax][M_max][nsr_pad] partial t of each K-range
  int64_t p_part;  // fp32 [ksplit][M][N] partial sums of a split GEMM (pf_part_bytes)
  int64_t p_end;
  int64_t total;
};

inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }
inline int nsr_pad_of(int n_seg, int r) { return (n_seg * r + 31) / 32 * 32; }
inline int decode_unit(int block) { return block > 256 ? block : 256; }
inline int decode_groups(int n) { return (n + 15) / 16; }   // 16 packed rows per consumer group
inline int decode_producers(int nunit, int M) { return nunit * ((M + 15) / 16); }

// Prefill K split: a GEMM of fewer tiles than kPfSplitTiles (half the compute
// units of an MI355X) runs each tile as up to kPfSplitMax workgroups over
// K-ranges of at least kPfSplitMinSteps steps, aiming at one workgroup per
// compute unit (from one per compute unit on, a split no longer paid for its
// partial sums: measured).  Returns the number of ranges (1: no split); *spw =
// steps per range.
constexpr int kPfSplitTiles = 128, kPfSplitMax = 4, kPfSplitMinSteps = 2;
inline int pf_ksplit(int tiles, int KG, int *spw) {
  int want = 1;
  if (tiles < kPfSplitTiles) {
    want = (2 * kPfSplitTiles) / tiles;
    want = want < kPfSplitMax ? want : kPfSplitMax;
    const int most = KG / kPfSplitMinSteps;
    want = want < most ? want : most;
    want = want > 1 ? want : 1;
  }
  const int w = (KG + want - 1) / want;
  if (spw) *spw = w;
  return (KG + w - 1) / w;
}

// fp32 partial sums of a split prefill GEMM, largest over 1 <= M <= M_max
inline int64_t pf_part_bytes(const dvssq_layout &L) {
  const int nt = (L.n_int4 + kPfTileN - 1) / kPfTileN + (L.n_int8 + kPfTileN - 1) / kPfTileN;
  const int mt_max = (L.M_max + kPfTileM - 1) / kPfTileM;
  int64_t best = 0;
  for (int mt = 1; mt <= mt_max && mt * nt < kPfSplitTiles; ++mt) {
    const int ns = pf_ksplit(mt * nt, L.K / kGroup, nullptr);
    if (ns < 2) continue;
    const int64_t rows = L.M_max < mt * kPfTileM ? L.M_max : mt * kPfTileM;
    const int64_t b = 4 * ns * rows * L.N;
    best = b > best ? b : best;
  }
  return best;
}

inline WsLayout ws_layout(const dvssq_layout &L) {
  WsLayout w{};
  const int64_t K = L.K, N = L.N;
  const int nsp = nsr_pad_of(L.n_seg, L.r);
  const int64_t nunit = K / decode_unit(L.block);
  int64_t cur = kStatusBytes;
  w.d_xq = cur;   cur = align256(cur + 2 * kDecodeRows * K);
  w.d_tp = cur;   cur = align256(cur + 4 * nunit * kDecodeRows * nsp);
  w.d_flag = cur; cur = align256(cur + 8 * decode_producers(nunit, kDecodeRows));
  w.d_x8g = cur;  cur = align256(cur + 4 * (K / kGroup) * kDecodeRows);
  w.d_escg = cur; cur = align256(cur + 4 * nunit * kDecodeRows);
  w.d_cntw = cur; cur = align256(cur + 8 * (decode_groups(L.n_int4) + decode_groups(L.n_int8)));
  w.d_part = cur; cur = align256(cur + 4 * int64_t(kMaxSplit) * kDecodeRows * N);
  w.d_end = cur;
  cur = kStatusBytes;
  w.p_xr = cur;   cur = align256(cur + 2 * pf_rows(L.M_max) * K);
  w.p_sc = cur;   cur = align256(cur + 4 * static_cast<int64_t>(L.M_max));
  w.p_rsh = cur;  cur = align256(cur + 4 * static_cast<int64_t>(L.n_int4));
  w.p_t = cur;    cur = align256(cur + 4 * static_cast<int64_t>(L.M_max) * nsp);
  w.p_tpart = cur; cur = align256(cur + 4 * kTSplitMax * static_cast<int64_t>(L.M_max) * nsp);
  w.p_part = cur; cur = align256(cur + pf_part_bytes(L));
  w.p_end = cur;
  w.total = w.d_end > w.p_end ? w.d_end : w.p_end;
  return w;
}

// ------------------------------------------------------------------ kernel arguments
struct PrologueArgs {
  const uint16_t *x;   // bf16 [M][K]
  uint16_t *xr;        // dvssq_fwht: bf16 [M][K]; prefill: f16 x_rot 2^-e in the GEMM tiles (xr_tile_offset)
  float *sc;           // prefill: fp32 [M] 2^e per row
  const uint16_t *V;   // bf16 [nsr][K] or null (no t)
  float *t;            // fp32 [M][nsr_pad] or null
  float *tpart;        // prefill: fp32 [ranges][M][nsr_pad] partial t of each K-range
  int M, K, nsr, nsr_pad;
  int blocks_per_wg;   // prefill: Hadamard blocks rotated by one workgroup
  int rotate;          // 0: x is already rotated (copy + t only)
  float hscale;        // 1/sqrt(block)
  int exp_bias;        // prefill: row exponent = ilogb(max |x|) + exp_bias (log2 sqrt(block) if rotating, + 1 - 15)
  int fuse_scale;      // prefill with K == block >= 256: the rotation kernel finds the row exponents itself
  const uint16_t *s4;  // prefill: bf16 [n4][K/64] INT4 group scales
  float *rsh;          // prefill: fp32 [n4] 2^c per INT4 row (from its largest group scale)
  int n4;              // prefill: INT4 rows
};

struct DecodeArgs {
  // packed layer
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const uint16_t *V;
  const int32_t *idx;
  const uint16_t *x;   // bf16 [M][K], or with gated the fused gate+up output [M][2K]
  uint16_t *hout;      // gated: bf16 [M][K], the intermediate h as the producers formed it (may be null)
  // workspace
  float *tp;           // fp32 [nunit][32][nsr_pad]
  uint64_t *flag;      // [nprod]
  float *part;         // fp32 [S][32][N]
  int8_t *xg1, *xg2;   // x_rot quantized to X = 256 x1 + x2, int8 planes [32][K]
  int *x8g;            // [K/64][32] 8 x sum of X over each group
  float *escg;         // [nunit][32] 2^e of each (unit, row)
  uint64_t *cntw;      // tagged arrival counters [g4 + g8]
  int *status;         // the workspace's status word
  uint16_t *y;         // bf16 [M][N]
  uint64_t gen;        // generation stamp of this call
  uint32_t tag;        // 32-bit tag of this call, never 0
  int N, K, r, n_seg, n4, n8, M, block, unit, nunit, nprod, nsr, nsr_pad, S, KW, g4, g8, rotate;
  int publish;         // 1: producers publish their flags (0 only under DVSSQ_TEST_NO_PUBLISH)
  int spin_limit;      // polls of a producer flag before the wait gives up
  int RT, MAXG;        // small-M path: 16-row tiles per workgroup, most groups per wavefront
  int KQ, GPW;         // small-M path: wavefronts per tile, groups per wavefront (even)
  int planes;          // small-M path: producers publish x_rot planes, consumers copy them (else rotate)
  int gated;           // 1: the input row m is h = geglu(x[m][0 .. K), x[m][K .. 2K)), formed as it loads
  int ngrp_w, nu_w;    // small-M path: groups of 64 and rotation units in one K-range (K / S)
  uint32_t magic_s;    // small-M path: ceil(2^32 / S), S > 1: x / S = umulhi(x, magic_s) for x < 2^16
  uint64_t lut_rt, lut_kq;  // small-M path: tile and K-slice of wavefront w in bits 4w .. 4w + 3
  uint64_t lut_m, lut_u;    // small-M path: token row and unit of the first item of wavefront w
  float hscale;        // 1/sqrt(block)
};

struct PrefillArgs {
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const int32_t *idx;
  const uint16_t *xr;  // f16 tiles (xr_tile_offset) scaled per row, runs of 8 in order 0,2,4,6,1,3,5,7
  const float *sc;     // fp32 [M] 2^e per row
  const float *t;      // fp32 [M][nsr_pad]
  uint16_t *y;         // bf16 [M][N]
  float *part;         // K split: fp32 [ksplit][M][N] partial sums per packed row
  const float *rsh;    // fp32 [n4] 2^c per INT4 row (group scales enter the f16 weights as s4 2^-c)
  int N, K, r, n_seg, n4, n8, M, nsr, nsr_pad;
  int n4_tiles, n8_tiles, m_tiles;
  int ksplit, kspw;    // K-ranges per tile (1: no split) and GEMM steps per range
};

struct GegluArgs {
  const uint16_t *ygu;  // bf16 [M][2I]: gate (columns 0 .. I-1) and up (I .. 2I-1)
  uint16_t *h;          // bf16 [M][I] = gelu(gate) * up
  int M, I;             // I a multiple of 8
};

struct DenseArgs {
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const uint16_t *V;
  const int32_t *idx;
  uint16_t *w;      // bf16 [N][K], original output order
  int N, K, r, n_seg, n4;
  float hscale;     // 1/sqrt(block)
};

// launchers (return hipError_t of the launch)
hipError_t launch_materialize(const DenseArgs &a, int block, hipStream_t s);
hipError_t launch_geglu(const GegluArgs &a, hipStream_t s);
hipError_t launch_fwht(const PrologueArgs &a, int block, hipStream_t s);
hipError_t launch_prologue(const PrologueArgs &a, int block, int n_wg_blocks, int cus, hipStream_t s);
// small-M decode (M <= 4): int8 matrix cores, 16-wavefront workgroups
struct SmallPlan {
  int RT;    // 16-row tiles per workgroup (1 .. 7)
  int S;     // split-K factor
  int MAXG;  // groups of 64 inputs loaded per wavefront (4, 8)
  int KQ;    // wavefronts per tile
  int GPW;   // groups of 64 per wavefront (even)
};
// false when no plan fits (the caller then takes the general decode path)
bool plan_decode_small(const dvssq_layout &L, int M, int cus, SmallPlan *plan);
int small_producers(int nunit, int M);   // t producers of the small-M kernel (one per unit and 16 rows)
hipError_t launch_decode_small(const DecodeArgs &a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_stream_read(const void *buf, int64_t bytes, void *sink, hipStream_t s);

// GPU quantizer: workspace byte offsets (per segment, reused) and the launch
struct QuantizeWs {
  int64_t R, Q, Z, Bt, G, J, sig, norm0, sgn, ord, S, salient, pos, bytes;
};
QuantizeWs quantize_ws_layout(const dvssq_layout &L, int l);
hipError_t launch_quantize(const dvssq_layout &L, const uint16_t *W, const double *omega, int l, int power_iters,
                           uint8_t *blob, uint8_t *ws, hipStream_t s);

// KV-BSS attention (attention.hip)
struct AttnArgs {
  const uint16_t *q, *k, *v;   // bf16 q [B][Mq][Hq][D], k and v [B][Nk][Hkv][D]
  uint16_t *o;                 // bf16 [B][Mq][Hq][D]
  int B, Mq, Nk, Hq, Hkv, D, window;
  int rep;                     // Hq / Hkv
  int rows;                    // Mq rep: (query, head) rows of one (sequence, KV head)
  int tiles;                   // workgroups per (sequence, KV head): ceil(rows / (16 attn_waves(D)))
  float scale, haze;
  // split-key form (rows <= 16, two launches): workspace regions and the call's stamp
  int nchunk;                  // key ranges of kAttnChunk keys per (sequence, KV head)
  float *logits;               // fp32 [B Hkv][16][Nk], -inf where not visible
  float *cmax;                 // fp32 [B Hkv][nchunk][16] row maxima of each range
  float *part;                 // fp32 [B Hkv][nchunk][16][D] sum of exp(s - m) v of each range
  float *partl;                // fp32 [B Hkv][nchunk][16] sum of exp(s - m) of each range
  uint64_t *cnt;               // arrival counters [B Hkv], zeroed by the first launch
};
hipError_t launch_kvbss_attention(const AttnArgs &a, hipStream_t s);
// wavefronts per attention workgroup (each takes 16 rows of the tile)
constexpr int attn_waves(int) { return 4; }
// split-key form: keys per range (one workgroup each), and when it is taken
constexpr int kAttnChunk = 512;
inline bool attn_split(int rows, int Nk) { return rows <= 16 && Nk > kAttnChunk; }
struct AttnWs {
  int64_t logits, cmax, part, partl, cnt, bytes;
};
inline AttnWs attn_ws_layout(int B, int Hkv, int Nk, int D) {
  AttnWs w{};
  const int64_t bg = static_cast<int64_t>(B) * Hkv, nchunk = (Nk + kAttnChunk - 1) / kAttnChunk;
  int64_t cur = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = cur;
    cur = (cur + bytes + 255) / 256 * 256;
    return o;
  };
  w.logits = take(bg * 16 * Nk * 4);
  w.cmax = take(bg * nchunk * 16 * 4);
  w.part = take(bg * nchunk * 16 * D * 4);
  w.partl = take(bg * nchunk * 16 * 4);
  w.cnt = take(bg * 8);
  w.bytes = cur;
  return w;
}

// few-token decode (1 <= M <= kGemvMaxM): 32-row tiles on the int8 32x32x32 matrix cores
constexpr int kGemvMaxM = 4;
struct GemvArgs {
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const uint16_t *V;
  const int32_t *idx;
  const uint16_t *x;   // bf16 [M][K], or with gated the fused gate+up output [M][2K]
  uint16_t *y;         // bf16 [M][N]
  uint16_t *hout;      // gated: bf16 [M][K], the intermediate h as the producers formed it (may be null)
  uint64_t *tp;        // stamped partial t {fp32 bits, stamp << 32} [nunit][8][nsr_pad]
  float *part;         // split-K: fp32 [S][M][N] results per packed row
  uint64_t *cnt;       // tagged arrival counters [32-row tiles]
  int *status;         // the workspace's status word
  uint32_t stamp;      // nonzero 32-bit stamp of this call
  int N, K, r, n_seg, n4, n8, M, block, unit, nunit, nsr, nsr_pad;
  int S, KW, nu_w;     // K-ranges, inputs and rotation units per range
  int W, GPW;          // wavefronts per workgroup, most groups of 64 of a wavefront (even)
  uint64_t lut_units;  // rotation units of the range per compute wavefront, 4 bits each (in wavefront order)
  int t4, t8;          // 32-row tiles of each tier
  int nprod;           // producer workgroups (one per rotation unit)
  int lead4;           // INT4 consumers placed before the INT8 consumers and the producers (< 0: producers first)
  int rotate, publish, spin_limit;
  int gated;           // 1: the input row m is h = geglu(x[m][0 .. K), x[m][K .. 2K)), formed as it loads
  float hscale;        // 1/sqrt(block)
};
struct GemvPlan {
  int S, W, GPW, local_rot;
  uint64_t lut_units;   // rotation units of each compute wavefront, 4 bits each
};
bool plan_gemv(const dvssq_layout &L, int M, int cus, bool gated, GemvPlan *plan);
hipError_t launch_gemv(const GemvArgs &a, hipStream_t s);

// Decode call after its argument checks (check_call): the single-launch kernel
// or the prefill route, with the workspace regions of W.  *ws_need (if not
// null) receives the bytes of ws the call touches; with dry_run nothing is
// launched.
// gated: x is the fused gate+up output [M][2K] of the block's first layer and
// the input row m is h = geglu(x[m][0 .. K), x[m][K .. 2K)), formed by the
// kernels as they load it (h also written to hout when not null); only the
// single-launch kernels take it (decode_takes_gated)
int decode_dispatch(const dvssq_layout &L, const WsLayout &W, const void *blob, const void *x, void *y, int32_t M,
                    void *ws, uint32_t flags, hipStream_t s, int64_t *ws_need, bool dry_run, bool gated = false,
                    uint16_t *hout = nullptr);
// argument checks of dvssq_linear_decode except the workspace pointer
int decode_check_args(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M, uint32_t flags);

}  // namespace dvssq
