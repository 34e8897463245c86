// Internal declarations of the DV-SSQ HIP library (gfx950).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kGroup = 64;      // INT4 group size
constexpr int kDecodeRows = 32; // M rows held by the decode workspace (MFMA tile height)
constexpr int kChunk = 256;     // decode split-K chunk (inputs), 4 groups

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

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ workspace
// Byte offsets inside the caller's workspace.  Decode and prefill regions
// overlap (one call at a time per workspace).
struct WsLayout {
  // decode
  int64_t d_xr;    // bf16 [32][K], rotated x, each 8-input run stored in the order 0,4,1,5,2,6,3,7
  int64_t d_xs;    // fp32 [K/64][32] group sums of the bf16 rotated x
  int64_t d_tp;    // fp32 [K/block][32][nsr_pad] per-block partial t = x_rot V^T
  int64_t d_part;  // fp32 [nchunk][32][N] split-K partial outputs
  int64_t d_cnt;   // int32 [n_tiles] arrivals per 32-row tile
  int64_t d_end;
  // prefill
  int64_t p_xr;    // bf16 [M_max][K] rotated x, natural order
  int64_t p_t;     // fp32 [M_max][nsr_pad] t = x_rot V^T
  int64_t p_end;
  int64_t total;
};

inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }
inline int nsr_pad_of(int n_seg, int r) { return (n_seg * r + 15) / 16 * 16; }
inline int decode_tiles(int n4, int n8) { return (n4 + 31) / 32 + (n8 + 31) / 32; }

inline WsLayout ws_layout(const dvssq_layout &L) {
  WsLayout w{};
  const int64_t K = L.K, N = L.N;
  const int nsp = nsr_pad_of(L.n_seg, L.r);
  const int64_t nchunk = (K + kChunk - 1) / kChunk;
  int64_t cur = 0;
  w.d_xr = cur;   cur = align256(cur + 2 * kDecodeRows * K);
  w.d_xs = cur;   cur = align256(cur + 4 * (K / kGroup) * kDecodeRows);
  w.d_tp = cur;   cur = align256(cur + 4 * (K / L.block) * kDecodeRows * nsp);
  w.d_part = cur; cur = align256(cur + 4 * nchunk * kDecodeRows * N);
  w.d_cnt = cur;  cur = align256(cur + 4 * decode_tiles(L.n_int4, L.n_int8));
  w.d_end = cur;
  cur = 0;
  w.p_xr = cur;   cur = align256(cur + 2 * static_cast<int64_t>(L.M_max) * K);
  w.p_t = cur;    cur = align256(cur + 4 * static_cast<int64_t>(L.M_max) * nsp);
  w.p_end = cur;
  w.total = w.d_end > w.p_end ? w.d_end : w.p_end;
  return w;
}

// ------------------------------------------------------------------ kernel arguments
struct PrologueArgs {
  const uint16_t *x;   // bf16 [M][K]
  uint16_t *xr;        // bf16 [rows][K] output (permuted or natural order)
  float *xs;           // fp32 [K/64][32] group sums (decode) or null
  const uint16_t *V;   // bf16 [nsr][K] or null (no t)
  float *tp;           // fp32 [n_out][tp_rows][nsr_pad]: partial or full t
  int *cnt_zero;       // int32 counters to clear (decode) or null
  int n_cnt;
  int M, K, nsr, nsr_pad;
  int tp_rows;         // row stride count of tp (32 for decode, M_max for prefill)
  int blocks_per_wg;   // Hadamard blocks handled (and t-accumulated) by one workgroup
  int permuted;        // 1: decode order of each 8-input run
  int rotate;          // 0: x is already rotated (copy + sums + t only)
  float scale;         // 1/sqrt(block)
};

struct DecodeArgs {
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const int32_t *idx;
  const uint16_t *xr;  // bf16 [32][K] permuted
  const float *xs;     // fp32 [K/64][32]
  const float *tp;     // fp32 [K/block][32][nsr_pad]
  float *part;         // fp32 [nchunk][32][N]
  int *cnt;            // int32 [n_tiles]
  uint16_t *y;         // bf16 [M][N]
  int N, K, r, n_seg, n4, n8, M, block, nsr, nsr_pad, nchunk, n4_tiles, n8_tiles;
};

struct PrefillArgs {
  const uint8_t *q4;
  const uint16_t *s4;
  const int8_t *q8;
  const float *s8;
  const uint16_t *U;
  const int32_t *idx;
  const uint16_t *xr;  // bf16 [M][K] natural
  const float *t;      // fp32 [M][nsr_pad]
  uint16_t *y;         // bf16 [M][N]
  int N, K, r, n_seg, n4, n8, M, nsr, nsr_pad;
  int n4_tiles, n8_tiles, m_tiles;
};

// launchers (return hipError_t of the launch)
hipError_t launch_prologue(const PrologueArgs &a, int block, int m_rows_per_wg, int n_wg_blocks,
                           hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

}  // namespace dvssq
