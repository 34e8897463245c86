// Small-M decode path (1 <= M <= 32) of y = (x H) W_hat^T + ((x H) V^T) U^T in
// one kernel launch (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical
// Foundations 2, runtime equation; rotation: same card, Mathematical
// Foundations 1, and Spark-X2.5-4B-Hadamard-GSQ model card, Tier B equation;
// tiers: MiniCPM card INT4 equation and Spark card Tier A).
//
// t producers (the lowest block indices, one per rotation unit of max(block,
// 256) inputs and 16 rows) rotate their unit of x and store the partial
// t = x_rot V^T with device-scope stores, then publish a 64-bit generation
// flag.  For M > 4 they also publish the quantized planes below, which the
// consumers then copy instead of rotating every (row, unit) themselves.
//
// Consumers are 16-wavefront workgroups (about one per compute unit): RT tiles
// of 16 packed rows, each served by KQ wavefronts that split the K-range, plus
// at least one spare wavefront that waits for the t producers and copies t to
// LDS.  A wavefront's memory counter completes in order, so every load whose
// result is needed before the main loop is issued before the weight loads:
// each compute wavefront first loads the activations of one (row, unit) item,
// then all of its weight loads, then rotates and quantizes its item into LDS
// while the weights stream in.  Each (row, unit) becomes a 15-bit integer
// X = 256 x1 + x2 with a power-of-two scale 2^e, stored as two int8 planes with
// 8 x (the sum of X over every group of 64 inputs), and multiplied with the
// codes on the int8 matrix cores (16x16x64), which sum exactly in int32:
//   INT4 group g:  sum_k (n_k - 8) X_k = sum_k n_k X_k - 8 sum_k X_k, the
//                  nibbles n_k in [0, 15] being valid int8 operands; the
//                  group's bf16 scale is applied in fp32;
//   INT8 rows:     sum_k q_k X_k, the row scale applied at the end.
// The unit scale 2^e multiplies each unit's partial sum.  Rotation: a
// Sylvester block of 256 is H_16 (x) H_16, so a 256-input block viewed as a
// 16x16 matrix X becomes Hs X H_16 (Hs = H_16, or I (x) H_{b/16} for b < 256):
// one bf16 MFMA for X H_16 (exact products, fp32 sums) and two for the second
// factor on that fp32 result split into bf16 high and low parts; units of
// 512 .. 2048 inputs combine their 256-blocks with butterflies in registers.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 1024;          // 16 wavefronts per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;               // packed rows per MFMA tile
constexpr int kProdRows = 16;           // activation rows per producer (one per wavefront)
constexpr int kTab = 32;                // token rows of the per-row LDS tables (M <= 32)
constexpr int kRed = 8;                 // partial-tile rows per lane in LDS (two token tiles of 4)
constexpr int kMaxRT = 7;               // largest number of 16-row tiles per workgroup
constexpr int kUVec = kMaxRT * kTile * 64 * 2 / 16 / 64;  // 16-byte U loads per spare lane (r <= 64)
constexpr int kRowVec = (kMaxRT * kTile + 63) / 64;         // column / INT8-scale loads per spare lane
constexpr int kLoadBatch = 16;          // device-scope loads issued together before their first use


// Groups of 64 inputs per wavefront when KQ wavefronts split ngrp groups: an
// even number, so that every wavefront's first group is even and its group
// scales load as aligned pairs.
__host__ __device__ inline int groups_per_wave(int ngrp, int KQ) { return ((ngrp + KQ - 1) / KQ + 1) & ~1; }

__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}
// Rotation of one (row, unit) item by one wavefront (rotate_blocks), or the
// plain bf16 values when x already holds x H.
template <int C>
__device__ __forceinline__ void rotate_item(const DecodeArgs &a, const u32x2 (&xw)[C], float (&y)[C][4]) {
  if (!a.rotate) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      y[c][0] = __uint_as_float(xw[c][0] << 16);
      y[c][1] = __uint_as_float(xw[c][0] & 0xFFFF0000u);
      y[c][2] = __uint_as_float(xw[c][1] << 16);
      y[c][3] = __uint_as_float(xw[c][1] & 0xFFFF0000u);
    }
    return;
  }
  rotate_blocks<C>(xw, y, a.block, a.hscale);
}

// --------------------------------------------------------------------------- producer

// Partial t of one rotation unit (C blocks of 256) for up to 8 activation rows.
// GT: gated input (h = geglu(gate, up) formed from the block's gate+up output).
template <int C, bool GT>
__device__ void produce(const DecodeArgs &a, int pidx, uint8_t *smem) {
  constexpr int P = 256 * C;
  constexpr int LDB = P + 8;             // bf16 x_rot row in LDS
  constexpr int KS = P / 32;             // k-steps of the t product
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int u = pidx % a.nunit, rg = pidx / a.nunit;
  const int m0 = rg * kProdRows, mrows = min(kProdRows, a.M - m0);
  const int k0 = u * P;
  const int nsp = a.nsr_pad, ni = nsp / 16;
  uint16_t *xb = reinterpret_cast<uint16_t *>(smem);                   // [8][LDB]
  float *tred = reinterpret_cast<float *>(smem + kProdRows * LDB * 2);  // [kWaves][4][64]
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  // t split: wavefront w takes 16 columns (it) of t and one chunk (kc) of the k-steps
  const int nkc = kWaves / ni;
  const int it = wave % ni, kc = wave / ni;
  const bool t_wave = kc < nkc;
  const int ksp = (KS + nkc - 1) / nkc;
  u32x4 vb[8];
  auto vload = [&](int j, int slot) {
    const int ks = min(kc * ksp + j, KS - 1);
    const int row = min(it * 16 + n, a.nsr - 1);
    vb[slot] = *reinterpret_cast<const u32x4 *>(a.V + static_cast<int64_t>(row) * a.K + k0 + 32 * ks + 8 * q);
  };
  const bool r_wave = wave < mrows;
  const int m = m0 + min(wave, mrows - 1);
  const int64_t xrow = GT ? 2 * static_cast<int64_t>(a.K) : a.K;   // inputs per row of x
  u32x2 xw[C], xu[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
    xw[c] = *reinterpret_cast<const u32x2 *>(a.x + m * xrow + k0 + 256 * c + 16 * n + 4 * q);
  if constexpr (GT)
#pragma unroll
    for (int c = 0; c < C; ++c)
      xu[c] = *reinterpret_cast<const u32x2 *>(a.x + m * xrow + a.K + k0 + 256 * c + 16 * n + 4 * q);
  if (t_wave)
#pragma unroll
    for (int j = 0; j < 8; ++j) vload(j, j);

  // 1. rotate one row per wavefront; bf16 copy for the t product; with
  // a.planes, also the row's 15-bit planes, group sums and unit scale for the
  // consumers (device-scope stores, drained before the flag)
  if (r_wave) {
    if constexpr (GT)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        xw[c][0] = geglu_bf16x2(xw[c][0], xu[c][0]);
        xw[c][1] = geglu_bf16x2(xw[c][1], xu[c][1]);
        if (a.hout) *reinterpret_cast<u32x2 *>(a.hout + static_cast<int64_t>(m) * a.K + k0 + 256 * c + 16 * n + 4 * q) = xw[c];
      }
    float y[C][4];
    rotate_item<C>(a, xw, y);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      u32x2 w;
      w[0] = pack_bf16x2(y[c][0], y[c][1]);
      w[1] = pack_bf16x2(y[c][2], y[c][3]);
      *reinterpret_cast<u32x2 *>(xb + wave * LDB + 256 * c + 16 * n + 4 * q) = w;
    }
    if (a.planes) {
      uint32_t p1[C], p2[C];
      int gsum[C];
      const int e = quantize_item<C>(y, p1, p2, gsum);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int64_t kk = static_cast<int64_t>(m) * a.K + k0 + 256 * c + 16 * n + 4 * q;
        st_dev(reinterpret_cast<uint32_t *>(a.xg1 + kk), p1[c]);
        st_dev(reinterpret_cast<uint32_t *>(a.xg2 + kk), p2[c]);
        if ((lane & 0x33) == 0) st_dev(a.x8g + ((k0 + 256 * c + 16 * n) / kGroup) * kDecodeRows + m, gsum[c]);
      }
      if (lane == 0) st_dev(a.escg + u * kDecodeRows + m, __uint_as_float(static_cast<uint32_t>(127 + e) << 23));
    }
  } else if (wave < kProdRows) {
    for (int j = lane; j < P / 2; j += 64) *reinterpret_cast<uint32_t *>(xb + wave * LDB + 2 * j) = 0u;
  }
  __syncthreads();

  // 2. partial t of this unit: t[m][i] = sum_k x_rot[m][k] V[i][k] (bf16 MFMA)
  f32x4 tacc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (t_wave) {
    for (int j0 = 0; j0 < ksp; j0 += 8) {
      if (j0 > 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) vload(j0 + j, j);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ks = kc * ksp + j0 + j;
        const bool ok = j0 + j < ksp && ks < KS && n < kProdRows;
        u32x4 av = *reinterpret_cast<const u32x4 *>(xb + (n & (kProdRows - 1)) * LDB + 32 * min(ks, KS - 1) + 8 * q);
        av = ok ? av : z4;
        tacc = mfma_bf16(av, vb[j], tacc);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) tred[(wave * 4 + r) * 64 + lane] = tacc[r];
  __syncthreads();
  // tacc of wavefront (kc, it): row m = 4 (lane / 16) + r, column it * 16 + lane % 16
  for (int e = tid; e < mrows * nsp; e += kThreads) {
    const int ml = e / nsp, i = e % nsp;
    const int lw = 16 * (ml / 4) + (i % 16), r = ml % 4;
    float s = 0.0f;
    for (int c = 0; c < nkc; ++c) s += tred[((c * ni + i / 16) * 4 + r) * 64 + lw];
    st_dev(a.tp + (static_cast<int64_t>(u) * kDecodeRows + m0 + ml) * nsp + i, s);
  }
  drain_stores();
  __syncthreads();
  if (tid == 0 && a.publish) st_dev(a.flag + pidx, a.gen);
}

// --------------------------------------------------------------------------- consumer

// t of the K-range into LDS: element e = m nsp + i (lanes t0, t0 + nt, ...)
// is the sum of the partial t of units u0 .. u0 + nu - 1, in unit order; the
// loads of a batch are all issued before the first is used, so their
// latencies overlap.
__device__ void sum_t(const DecodeArgs &a, int t0, int nt, int u0, int nu, float *ts) {
  const int nsp = a.nsr_pad;
  const int64_t ustride = static_cast<int64_t>(kDecodeRows) * nsp;
  for (int e = t0; e < a.M * nsp; e += nt) {
    const int m = e / nsp, i = e - m * nsp;
    const float *src = a.tp + (static_cast<int64_t>(u0) * kDecodeRows + m) * nsp + i;
    float s = 0.0f;
    for (int u = 0; u < nu; u += kLoadBatch) {
      float v[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) v[j] = u + j < nu ? ld_dev(src + (u + j) * ustride) : 0.0f;
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) s += v[j];
    }
    ts[e] = i < a.nsr ? s : 0.0f;
  }
}

// Copy of the producers' planes (rows 0 .. M-1, inputs k0 .. k0 + KW - 1),
// 8 x group sums and unit scales into LDS by the lanes t0, t0 + nt, ... of the
// workgroup; 16-byte chunks, read with device-scope loads.  Chunk c of row m
// goes to chunk index c Mp + m of the LDS planes (Mp rows per chunk column).
template <bool T8>
__device__ void copy_planes(const DecodeArgs &a, int t0, int nt, int k0, int KW, int ngrp, int u0, int nu, int Mp,
                            int8_t *xs1, int8_t *xs2, int *x8, float *esc) {
  constexpr int kBatch = 4;
  const int M = a.M;
  const int cpr = KW / 16;                               // chunks per row
  const int nch = M * cpr;
  const float inv = 1.0f / static_cast<float>(cpr);
  for (int e0 = t0; e0 < nch; e0 += kBatch * nt) {
    u32x4 v1[kBatch], v2[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = min(e0 + j * nt, nch - 1);
      const int m = static_cast<int>((static_cast<float>(e) + 0.5f) * inv), c = e - m * cpr;
      const int64_t g = static_cast<int64_t>(m) * a.K + k0 + 16 * c;
      v1[j] = ld_dev16(a.xg1 + g);
      v2[j] = ld_dev16(a.xg2 + g);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = e0 + j * nt;
      if (e < nch) {
        const int m = static_cast<int>((static_cast<float>(e) + 0.5f) * inv), c = e - m * cpr;
        *reinterpret_cast<u32x4 *>(xs1 + (c * Mp + m) * 16) = v1[j];
        *reinterpret_cast<u32x4 *>(xs2 + (c * Mp + m) * 16) = v2[j];
      }
    }
  }
  if constexpr (!T8)
    for (int e = t0; e < ngrp * M; e += nt) {
      const int g = e / M, m = e - g * M;
      x8[g * kTab + m] = ld_dev(a.x8g + (k0 / kGroup + g) * kDecodeRows + m);
    }
  for (int e = t0; e < nu * M; e += nt) {
    const int u = e / M, m = e - u * M;
    esc[u * kTab + m] = ld_dev(a.escg + (u0 + u) * kDecodeRows + m);
  }
}

// Spare wavefronts of a consumer workgroup: load the U rows, output columns
// and INT8 row scales of the workgroup's rows (wbase .. wbase + wrows - 1),
// then wait for the t producers of the K-range and sum their partial t.  Each
// result goes to LDS between the workgroup's two barriers, (A) and (B), which
// the compute wavefronts pass at the same points of their own path.
template <bool T8>
__device__ void spare(const DecodeArgs &a, int sw, int nsw, int wbase, int wrows, int u0, int nu, u32x4 *ush,
                      int *cols, float *s8s, float *ts, int *tout) {
  const int lane = threadIdx.x & 63;
  const int M = a.M, nsp = a.nsr_pad;
  u32x4 uv[kUVec];
  uint32_t rv[kRowVec], sv[kRowVec];
  const auto ru = make_rsrc(a.U, static_cast<uint32_t>(a.N) * a.r * 2);
  const uint32_t ub = static_cast<uint32_t>(wbase) * a.r * 2, ubytes = static_cast<uint32_t>(wrows) * a.r * 2;
#pragma unroll
  for (int j = 0; j < kUVec; ++j) {
    const uint32_t o = static_cast<uint32_t>(sw * 64 + lane + nsw * 64 * j) * 16;
    uv[j] = buf_load16(ru, o < ubytes ? ub + o : kOutOfRange);
  }
  const auto ri = make_rsrc(a.idx, static_cast<uint32_t>(a.N) * 4);
  const auto rs8 = make_rsrc(a.s8, static_cast<uint32_t>(a.n8) * 4);
#pragma unroll
  for (int j = 0; j < kRowVec; ++j) {
    const int e = sw * 64 + lane + nsw * 64 * j;
    const bool ok = e < wrows;
    rv[j] = buf_load4(ri, ok ? static_cast<uint32_t>(wbase + e) * 4 : kOutOfRange);
    sv[j] = T8 ? buf_load4(rs8, ok ? static_cast<uint32_t>(wbase + e - a.n4) * 4 : kOutOfRange) : 0u;
  }
  // Every spare wavefront waits for every flag it depends on, each wait
  // bounded by a.spin_limit polls; the first spare wavefront records in LDS
  // whether any of its waits gave up (read by all after barrier B).
  auto wait_flags = [&]() {
    const int nrg = (M + kProdRows - 1) / kProdRows;
    bool late = false;
    for (int i = lane; i < nu * nrg; i += 64) {
      const int rg = i / nu, uu = i - rg * nu;
      int spins = 0;
      while (ld_dev(a.flag + rg * a.nunit + u0 + uu) != a.gen) {
        if (++spins > a.spin_limit) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    const bool any_late = __builtin_amdgcn_ballot_w64(late) != 0;
    if (sw == 0 && lane == 0) *tout = any_late ? 1 : 0;
    __builtin_amdgcn_wave_barrier();
  };
  if (a.planes) {
    wait_flags();
    __syncthreads();   // (P)
  }
  __syncthreads();   // (A)
#pragma unroll
  for (int j = 0; j < kUVec; ++j)
    if (sw * 64 + lane + nsw * 64 * j < kUVec * 64) ush[sw * 64 + lane + nsw * 64 * j] = uv[j];
#pragma unroll
  for (int j = 0; j < kRowVec; ++j) {
    const int e = sw * 64 + lane + nsw * 64 * j;
    if (e < kMaxRT * kTile) {
      cols[e] = static_cast<int>(rv[j]);
      s8s[e] = T8 ? __uint_as_float(sv[j]) : 1.0f;
    }
  }
  if (!a.planes) wait_flags();
  if (!a.planes) sum_t(a, sw * 64 + lane, nsw * 64, u0, nu, ts);
  __syncthreads();   // (B)
}

// MT: largest M (1 or 4); C: 256-blocks per rotation unit; MAXG: groups of 64
// inputs loaded per wavefront; T8: INT8 tier.  a.RT tiles of 16 rows per
// workgroup, a.KQ wavefronts per tile splitting the K-range in runs of a.GPW
// groups (an even number); the wavefronts from RT * KQ on are spare.  Values
// that are the same across a wavefront are kept in scalar registers: the
// vector ALU, shared by the four wavefronts of each SIMD, is the scarce unit.
template <int MT, int C, int MAXG, bool T8, bool GT>
__device__ void consume(const DecodeArgs &a, int cidx, uint8_t *smem) {
  constexpr int R = MT == 1 ? 1 : 4;    // accumulator rows per lane and token tile
  constexpr int NT = MT > 16 ? 2 : 1;   // token tiles of 16
  // lane (n, q) holds, in row r of token tile t, token 16 t + tq + r (MT > 1) or token 0 (MT = 1)
  constexpr int P = 256 * C;
  constexpr int gpu = P / kGroup;       // groups per rotation unit
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int tq = MT == 1 ? 0 : 4 * q;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // per-wavefront and per-workgroup indices from host-made tables, without divisions
  const int RT = a.RT, KQ = a.KQ, NCW = RT * KQ;
  const int rt = static_cast<int>((a.lut_rt >> (4 * wave)) & 15u), kq = static_cast<int>((a.lut_kq >> (4 * wave)) & 15u);
  const int grp = a.S == 1 ? cidx : static_cast<int>(__umulhi(static_cast<uint32_t>(cidx), a.magic_s));
  const int split = cidx - grp * a.S;
  const int rows = T8 ? a.n8 : a.n4;
  const int ntiles = static_cast<int>((static_cast<uint32_t>(rows) + kTile - 1) >> 4);
  const int tile0 = (T8 ? grp - a.g4 : grp) * RT;       // first tile of the workgroup inside the tier
  const int wbase = (T8 ? a.n4 : 0) + min(tile0, ntiles - 1) * kTile;   // first packed row of the workgroup
  const int M = a.M, KW = a.KW;
  const int k0 = split * KW;
  const int ngrp = a.ngrp_w;                            // groups of 64 in the K-range
  const int nu = a.nu_w, u0 = split * nu;               // rotation units in the K-range, first one
  const int nsp = a.nsr_pad;
  const int nitem = M * nu;                             // (row, unit) items to rotate

  // LDS: int8 planes, 8 x group sums, unit scales, partial tiles, U rows, columns, INT8 scales, t
  // planes: 16-byte chunk c (inputs 16 c .. 16 c + 15 of the K-range) of token
  // m at chunk index c MT + m, so that the 16 tokens of an operand read sit in
  // 16 consecutive chunks
  int8_t *xs1 = reinterpret_cast<int8_t *>(smem);
  int8_t *xs2 = xs1 + MT * KW;
  int *x8 = reinterpret_cast<int *>(xs2 + MT * KW);                  // [ngrp][4]
  float *esc = reinterpret_cast<float *>(x8 + ngrp * kTab);          // [nu][4]
  float *red = esc + nu * kTab;                                      // [kWaves][kRed][64]
  u32x4 *ush = reinterpret_cast<u32x4 *>(red + kWaves * kRed * 64);  // U rows wbase .. wbase + 16 RT - 1
  int *cols = reinterpret_cast<int *>(ush + kUVec * 64);           // [16 RT] output columns
  float *s8s = reinterpret_cast<float *>(cols + kMaxRT * kTile);   // [16 RT] INT8 row scales
  float *ts = s8s + kMaxRT * kTile;                                // [M][nsp]
  int *tout = reinterpret_cast<int *>(ts + M * nsp);               // 1: a wait for the producers gave up

  if (wave >= NCW) {
    const int wrows = min(RT * kTile, (T8 ? a.n4 + a.n8 : a.n4) - wbase);
    spare<T8>(a, wave - NCW, kWaves - NCW, wbase, wrows, u0, nu, ush, cols, s8s, ts, tout);
    return;
  }
  const int tile = tile0 + rt;
  const bool tile_ok = tile < ntiles;
  const int gbase = min(tile, ntiles - 1) * kTile;
  const int base = (T8 ? a.n4 : 0) + gbase;             // first packed row of the tile
  const int pl = gbase + n;                             // this lane's row inside the tier
  const bool row_ok = tile_ok && pl < rows;
  const int plc = min(pl, rows - 1);
  const int gpw = a.GPW;
  const int g0 = kq * gpw, g1 = min(ngrp, g0 + gpw);
  const int gs = max(0, min(g0, ngrp - MAXG));          // first loaded group (MAXG <= ngrp), even
  const int KG = static_cast<int>(static_cast<uint32_t>(a.K) >> 6);
  // groups gs + i with i in [g0 - gs, g1 - gs) are this wavefront's
  const uint32_t vmask = ((1u << max(0, g1 - gs)) - 1u) & ~((1u << max(0, g0 - gs)) - 1u);

  // ---- 1. activations of this wavefront's first item, before anything else.
  // Loads go through buffer resources: a lane with nothing to load gets an
  // offset past the end, which reads zeros without touching memory, so the
  // loads are issued unconditionally and each wait covers only what it needs.
  const uint32_t xrow = GT ? 2u * a.K : static_cast<uint32_t>(a.K);   // inputs per row of x
  const auto rx = make_rsrc(a.x, static_cast<uint32_t>(M) * xrow * 2);
  // gated: the gate values at x[m][k], the up values at x[m][K + k]
  const uint32_t uoff = static_cast<uint32_t>(a.K) * 2;
  u32x2 xw[C], xu[C];
  {
    const int m = static_cast<int>((a.lut_m >> (4 * wave)) & 15u), u = static_cast<int>((a.lut_u >> (4 * wave)) & 15u);
    const uint32_t off = !a.planes && wave < nitem ? (static_cast<uint32_t>(m) * xrow + k0 + u * P + 16 * n + 4 * q) * 2
                                      : kOutOfRange;
#pragma unroll
    for (int c = 0; c < C; ++c) xw[c] = buf_load8(rx, off + 512 * c);
    if constexpr (GT)
#pragma unroll
      for (int c = 0; c < C; ++c) xu[c] = buf_load8(rx, off == kOutOfRange ? kOutOfRange : off + uoff + 512 * c);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. weight loads of this wavefront: groups gs .. gs + MAXG - 1, those
  // outside g0 .. g1 - 1 replaced by zeros (their scale pairs too: g0 and g1
  // are even, so a pair of groups is either wholly inside or wholly outside)
  u32x2 c4[T8 ? 1 : MAXG];
  uint32_t sb[T8 ? 1 : MAXG / 2];                      // bf16 group scales, two per dword
  u32x4 c8[T8 ? MAXG : 1];
  if constexpr (!T8) {
    const auto r4 = make_rsrc(a.q4, static_cast<uint32_t>(a.n4) * (a.K / 2));
    const auto rs = make_rsrc(a.s4, static_cast<uint32_t>(a.n4) * KG * 2);
    const uint32_t o4 = row_ok ? static_cast<uint32_t>(plc) * (static_cast<uint32_t>(a.K) >> 1) +
                                     ((static_cast<uint32_t>(k0) + 64u * gs) >> 1) + 8u * q
                               : kOutOfRange;
    const uint32_t os = row_ok ? (static_cast<uint32_t>(plc) * KG + (static_cast<uint32_t>(k0) >> 6) + gs) * 2 : kOutOfRange;
#pragma unroll
    for (int i = 0; i < MAXG; ++i) c4[i] = buf_load8(r4, (vmask >> i) & 1u ? o4 + 32 * i : kOutOfRange);
#pragma unroll
    for (int i = 0; i < MAXG / 2; ++i) sb[i] = buf_load4(rs, (vmask >> (2 * i)) & 1u ? os + 4 * i : kOutOfRange);
  } else {
    const auto r8 = make_rsrc(a.q8, static_cast<uint32_t>(a.n8) * a.K);
    const uint32_t o8 = row_ok ? static_cast<uint32_t>(plc) * a.K + k0 + 64 * gs + 16 * q : kOutOfRange;
#pragma unroll
    for (int i = 0; i < MAXG; ++i) c8[i] = buf_load16(r8, (vmask >> i) & 1u ? o8 + 64 * i : kOutOfRange);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. items -> quantized int8 planes in LDS.  The first item is handled
  // outside any loop, so its wait covers only the activation loads issued
  // before the weights; later items (M > 1) are loaded here.
  auto quantize = [&](int m, int u, u32x2(&xv)[C], const u32x2(&uv)[C]) {
    if constexpr (GT)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        xv[c][0] = geglu_bf16x2(xv[c][0], uv[c][0]);
        xv[c][1] = geglu_bf16x2(xv[c][1], uv[c][1]);
      }
    float y[C][4];
    rotate_item<C>(a, xv, y);
    uint32_t p1[C], p2[C];
    int gsum[C];
    const int e = quantize_item<C>(y, p1, p2, gsum);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int kk = u * P + 256 * c + 16 * n + 4 * q;
      *reinterpret_cast<uint32_t *>(xs1 + ((kk >> 4) * MT + m) * 16 + (kk & 15)) = p1[c];
      *reinterpret_cast<uint32_t *>(xs2 + ((kk >> 4) * MT + m) * 16 + (kk & 15)) = p2[c];
      if (!T8 && (lane & 0x33) == 0) x8[(kk / kGroup) * kTab + m] = gsum[c];
    }
    if (lane == 0) esc[u * kTab + m] = __uint_as_float(static_cast<uint32_t>(127 + e) << 23);
  };
  if (a.planes) {
    // the producers quantized every (row, unit): once the spare wavefronts
    // have seen their flags (barrier P), copy this K-range's planes, group
    // sums and unit scales into LDS
    __syncthreads();   // (P)
    copy_planes<T8>(a, wave * 64 + lane, NCW * 64, k0, KW, ngrp, u0, nu, MT, xs1, xs2, x8, esc);
    sum_t(a, wave * 64 + lane, NCW * 64, u0, nu, ts);
  } else {
    if (wave < nitem)
      quantize(static_cast<int>((a.lut_m >> (4 * wave)) & 15u), static_cast<int>((a.lut_u >> (4 * wave)) & 15u), xw,
               xu);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = wave + NCW; it < nitem; it += NCW) {
      const int m = it % M, u = it / M;
      u32x2 xv[C], uv[C];
      const uint32_t off = (static_cast<uint32_t>(m) * xrow + k0 + u * P + 16 * n + 4 * q) * 2;
#pragma unroll
      for (int c = 0; c < C; ++c) xv[c] = buf_load8(rx, off + 512 * c);
      if constexpr (GT)
#pragma unroll
        for (int c = 0; c < C; ++c) uv[c] = buf_load8(rx, off + uoff + 512 * c);
      quantize(m, u, xv, uv);
    }
  }
  __syncthreads();   // (A) planes, group sums and unit scales are in LDS

  // ---- 4. main loop: two int8 MFMAs per group and token tile (the second one
  // starts from -8 x the group sum of X, the INT4 offset), straight-line; the
  // MFMAs of group i+1 are issued before the scalar work of group i.  Each
  // group adds D = 256 D1 + D2 times its scale (bf16 group scale x unit scale;
  // for INT8 rows the unit scale alone, the row scale comes at the end).
  float acc[NT][R];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[t][r] = 0.0f;
  {
    const int8_t *pa1[NT], *pa2[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int mA = MT == 1 ? 0 : min(16 * t + n, M - 1);
      pa1[t] = xs1 + (q * MT + mA) * 16;
      pa2[t] = xs2 + (q * MT + mA) * 16;
    }
    auto bop = [&](int i) -> u32x4 {
      u32x4 b;
      if constexpr (!T8) {
        const uint32_t w0 = c4[i][0], w1 = c4[i][1];
        b[0] = w0 & 0x0F0F0F0Fu;
        b[1] = (w0 >> 4) & 0x0F0F0F0Fu;
        b[2] = w1 & 0x0F0F0F0Fu;
        b[3] = (w1 >> 4) & 0x0F0F0F0Fu;
      } else {
        b = c8[i];
      }
      return b;
    };
    auto cinit = [&](int g, int t) -> i32x4 {   // -8 x the group sums of X (INT4), 0 (INT8)
      i32x4 c = {0, 0, 0, 0};
      if constexpr (!T8) {
        const i32x4 xg = *reinterpret_cast<const i32x4 *>(x8 + g * kTab + 16 * t + tq);
#pragma unroll
        for (int r = 0; r < R; ++r) c[r] = -xg[r];
      }
      return c;
    };
    const i32x4 zi = {0, 0, 0, 0};
    i32x4 d1[NT], d2[NT];
    {
      const u32x4 b = bop(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        d1[t] = mfma_i8(*reinterpret_cast<const u32x4 *>(pa1[t] + 64 * MT * gs), b, zi);
        d2[t] = mfma_i8(*reinterpret_cast<const u32x4 *>(pa2[t] + 64 * MT * gs), b, cinit(gs, t));
      }
    }
#pragma unroll
    for (int i = 0; i < MAXG; ++i) {
      const int g = gs + i;
      i32x4 e1[NT], e2[NT];
      if (i + 1 < MAXG) {
        const u32x4 b = bop(i + 1 < MAXG ? i + 1 : i);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          e1[t] = mfma_i8(*reinterpret_cast<const u32x4 *>(pa1[t] + 64 * MT * (g + 1)), b, zi);
          e2[t] = mfma_i8(*reinterpret_cast<const u32x4 *>(pa2[t] + 64 * MT * (g + 1)), b, cinit(g + 1, t));
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) e1[t] = e2[t] = zi;
      }
      // groups outside g0 .. g1 - 1 have zero codes; INT4 ones also a zero scale
      float sg = 1.0f;
      if constexpr (!T8) {
        const uint32_t sw = sb[i / 2];
        sg = __uint_as_float((i & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4 ev = *reinterpret_cast<const f32x4 *>(esc + (g / gpu) * kTab + 16 * t + tq);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float cs = T8 ? ev[r] : sg * ev[r];
          acc[t][r] = fmaf(cs, static_cast<float>((d1[t][r] << 8) + d2[t][r]), acc[t][r]);
        }
        d1[t] = e1[t];
        d2[t] = e2[t];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- 5. partial tiles -> LDS
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) red[(wave * kRed + t * R + r) * 64 + lane] = acc[t][r];
  __syncthreads();   // (B) partial tiles, U rows, columns, INT8 scales and t are in LDS
  if (kq != 0) return;

  // ---- 6. first wavefront of each tile: sum the K-slices, add the low-rank term
  const int col = cols[rt * kTile + n];
  float cacc[NT][R];
  {
    const float s8 = s8s[rt * kTile + n];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float s = 0.0f;
        for (int w = 0; w < KQ; ++w) s += red[((rt * KQ + w) * kRed + t * R + r) * 64 + lane];
        cacc[t][r] = s * s8;
      }
  }
  {
    const int seg = (a.n_seg == 2 && plc >= rows / 2) ? 1 : 0;   // segments in packed order
    const uint16_t *u16 = reinterpret_cast<const uint16_t *>(ush) + (rt * kTile + n) * a.r;
    const float *tseg = ts + seg * a.r;
    if constexpr (MT <= 4) {
      // lane (n, q) takes the rank indices q, q + 4, ... of row n; the four
      // lanes of a row then add up their shares
      float lr[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) lr[m] = 0.0f;
      for (int i = q; i < a.r; i += 4) {
        const float uv = bf16_to_f32(u16[i]);
#pragma unroll
        for (int m = 0; m < MT; ++m) lr[m] = fmaf(m < M ? tseg[m * nsp + i] : 0.0f, uv, lr[m]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        lr[m] += __shfl_xor(lr[m], 16, 64);
        lr[m] += __shfl_xor(lr[m], 32, 64);
      }
      // token m sits in row m of the lanes with q = 0
#pragma unroll
      for (int r = 0; r < R; ++r) cacc[0][r] += (q == 0 && r < MT) ? lr[r < MT ? r : 0] : 0.0f;
    } else {
      // each lane adds the low-rank term of its own tokens
      for (int i = 0; i < a.r; ++i) {
        const float uv = bf16_to_f32(u16[i]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int m = 16 * t + tq + r;
            cacc[t][r] = fmaf(m < M ? tseg[m * nsp + i] : 0.0f, uv, cacc[t][r]);
          }
      }
    }
  }

  // ---- 7. output: direct, or split-K partials summed by the last arriver.
  // If a wait for the producers gave up, t and the planes may be stale: every
  // output of this workgroup becomes NaN (a split-K sum with a NaN partial is
  // NaN) and the workspace's status word records the timeout.
  if (*tout) {
    if (lane == 0) st_dev(a.status, DVSSQ_STATUS_WAIT_TIMEOUT);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) cacc[t][r] = __builtin_nanf("");
  }
  const bool out_lane = row_ok && (MT != 1 || q == 0);
  if (a.S == 1) {
    if (!out_lane) return;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int m = 16 * t + tq + r;
        if (m < M) a.y[static_cast<int64_t>(m) * a.N + col] = f32_to_bf16(cacc[t][r]);
      }
    return;
  }
  if (!tile_ok) return;
  const int p = base + n;
  if (out_lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int m = 16 * t + tq + r;
        if (m < M) st_dev(a.part + (static_cast<int64_t>(split) * kDecodeRows + m) * a.N + p, cacc[t][r]);
      }
  }
  drain_stores();
  int last = 0;
  if (lane == 0) {
    uint64_t *cnt = a.cntw + (T8 ? (a.n4 + kTile - 1) / kTile : 0) + tile;
    last = arrive_tagged(cnt, a.tag) == static_cast<uint32_t>(a.S);
  }
  last = __shfl(last, 0, 64);
  if (!last) return;
  const int nrows = min(kTile, rows - gbase);
  for (int e = lane; e < kTile * M; e += 64) {
    const int rr = e % kTile, m = e / kTile;
    if (rr >= nrows) continue;
    const int pp = base + rr;
    const float *src = a.part + static_cast<int64_t>(m) * a.N + pp;
    const int64_t sstride = static_cast<int64_t>(kDecodeRows) * a.N;
    float s = 0.0f;
    for (int sp = 0; sp < a.S; sp += kLoadBatch) {   // partials summed in split order
      float v[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) v[j] = sp + j < a.S ? ld_dev(src + (sp + j) * sstride) : 0.0f;
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) s += v[j];
    }
    a.y[static_cast<int64_t>(m) * a.N + a.idx[pp]] = f32_to_bf16(s);
  }
}

template <int MT, int C, int MAXG, bool GT>
__global__ __launch_bounds__(kThreads) void decode_small_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  if (b < a.nprod) {
    produce<C, GT>(a, b, smem);
    return;
  }
  const int c = b - a.nprod;   // consumer index = group * S + split
  if (c < a.g4 * a.S) consume<MT, C, MAXG, false, GT>(a, c, smem);
  else consume<MT, C, MAXG, true, GT>(a, c, smem);
}

size_t producer_lds(int unit) {
  return static_cast<size_t>(kProdRows) * (unit + 8) * 2 + static_cast<size_t>(kWaves) * 4 * 64 * 4;
}

size_t consumer_lds(int M, int unit, int KW, int nsr_pad) {
  const size_t nu = KW / unit, ngrp = KW / kGroup;
  const size_t mt = M <= 1 ? 1 : M <= 4 ? 4 : M <= 16 ? 16 : 32;   // token rows of the plane layout
  return static_cast<size_t>(2) * mt * KW + ngrp * kTab * 4 + nu * kTab * 4 + static_cast<size_t>(kWaves) * kRed * 64 * 4 +
         static_cast<size_t>(kUVec) * 64 * 16 + 2 * kMaxRT * kTile * 4 +
         static_cast<size_t>(M) * nsr_pad * 4 + 16;
}

size_t small_lds(int M, int unit, int KW, int nsr_pad) {
  return std::max(producer_lds(unit), consumer_lds(M, unit, KW, nsr_pad));
}

template <int MT, int C, int MAXG, bool GT>
hipError_t launch_gt(const DecodeArgs &a, hipStream_t s) {
  const size_t lds = small_lds(a.M, a.unit, a.KW, a.nsr_pad);
  if (lds > 65536) {
    static std::atomic<uint64_t> done{0};
    const hipError_t e =
        ensure_lds_limit(reinterpret_cast<const void *>(decode_small_kernel<MT, C, MAXG, GT>), 160 * 1024, done);
    if (e != hipSuccess) return e;
  }
  const int grid = a.nprod + (a.g4 + a.g8) * a.S;
  return launch_kernel(reinterpret_cast<const void *>(decode_small_kernel<MT, C, MAXG, GT>), dim3(grid), dim3(kThreads),
                       lds, s, a);
}

template <int MT, int C, int MAXG>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
  return a.gated ? launch_gt<MT, C, MAXG, true>(a, s) : launch_gt<MT, C, MAXG, false>(a, s);
}

template <int MT, int C>
hipError_t launch_g(const DecodeArgs &a, hipStream_t s) {
  if (a.MAXG == 8) return launch_t<MT, C, 8>(a, s);
  return launch_t<MT, C, 4>(a, s);
}

template <int MT>
hipError_t launch_m(const DecodeArgs &a, hipStream_t s) {
  switch (a.unit) {
    case 256: return launch_g<MT, 1>(a, s);
    case 512: return launch_g<MT, 2>(a, s);
    case 1024: return launch_g<MT, 4>(a, s);
    default: return launch_g<MT, 8>(a, s);
  }
}

}  // namespace

// Workgroup shape and split for a GPU of `cus` compute units: RT tiles of 16
// rows per workgroup (15 / RT wavefronts per tile split K), S equal parts of
// K, each a whole number of rotation units, with at most 8 groups of 64 per
// wavefront (the register file holds 16 wavefronts of at most 128 registers)
// and the LDS within 160 KB.  Every workgroup, a t producer included, holds a
// whole compute unit.  The plan minimises an estimated cost fitted to
// measured runs (every feasible plan timed on spark_up, spark_down, gate+up
// and the MiniCPM layers at M = 1 .. 32): the rounds of workgroups, each
// weighted by the activation planes a workgroup copies per byte of its weights
// (M > 4), plus 0.4 + 0.05 S for a split (it adds a reduction) and 4 x the
// bytes of its fp32 partials per byte of the packed layer, minus 0.2 x the
// share of compute units kept busy; ties go to more workgroups.
bool plan_decode_small(const dvssq_layout &L, int M, int cus, SmallPlan *plan) {
  if (M < 1 || M > 32) return false;
  // byte offsets of the buffer loads stay below 2^31
  const int64_t big = std::max<int64_t>(static_cast<int64_t>(L.n_int4) * L.K / 2,
                                        std::max<int64_t>(static_cast<int64_t>(L.n_int8) * L.K,
                                                          static_cast<int64_t>(L.N) * L.r * 2));
  if (big >= (int64_t{1} << 31) || static_cast<int64_t>(M) * L.K * 2 >= (int64_t{1} << 31)) return false;
  const int unit = L.block > 256 ? L.block : 256;
  if (L.K % unit) return false;
  const int nunit = L.K / unit;
  const int nsp = (L.n_seg * L.r + 31) / 32 * 32;
  const int t4 = (L.n_int4 + kTile - 1) / kTile, t8 = (L.n_int8 + kTile - 1) / kTile;
  const int nprod = small_producers(nunit, M);
  const int gmax = 8;
  double best = -1e30;
  int best_wgs = 0;
  bool found = false;
  for (int RT : {1, 2, 3, 4, 5, 7}) {
    const int KQ = (kWaves - 1) / RT;
    for (int S = 1; S <= kMaxSplit && S <= nunit; ++S) {
      if (nunit % S) continue;
      const int KW = L.K / S, ngrp = KW / kGroup;
      const int gpw = groups_per_wave(ngrp, KQ);
      if (gpw > gmax) continue;
      const int maxg = gpw <= 4 ? 4 : 8;
      if (maxg > ngrp) continue;
      if (small_lds(M, unit, KW, nsp) > 160 * 1024) continue;
      // every workgroup, the t producers included, holds a whole compute unit
      const int wgs = ((t4 + RT - 1) / RT + (t8 + RT - 1) / RT) * S + nprod;
      const int rounds = (wgs + cus - 1) / cus;
      // activation planes a workgroup copies (M > 4) per byte of its weights
      const double planes = M >= 5 ? 2.0 * M / (RT * kTile * (0.5 + 2.0 / kGroup)) : 0.0;
      // split-K partials written and read back (fp32 [S][M][N]) per byte of the packed layer
      const double part = S > 1 ? 4.0 * S * M * static_cast<double>(L.N) / static_cast<double>(L.blob_bytes) : 0.0;
      const double util = static_cast<double>(wgs) / (static_cast<double>(cus) * rounds);
      const double cost =
          rounds * (1.0 + 0.3 * planes) + (S > 1 ? 0.4 + 0.05 * S : 0.0) + 4.0 * part - 0.2 * util;
      const double score = -cost;
      if (score > best + 1e-9 || (score > best - 1e-9 && wgs > best_wgs)) {
        best = score;
        best_wgs = wgs;
        plan->RT = RT;
        plan->S = S;
        plan->MAXG = maxg;
        plan->KQ = KQ;
        plan->GPW = gpw;
        found = true;
      }
    }
  }
  return found;
}

int small_producers(int nunit, int M) { return nunit * ((M + kProdRows - 1) / kProdRows); }

hipError_t launch_decode_small(const DecodeArgs &a, hipStream_t s) {
  if (a.unit != 256 && a.unit != 512 && a.unit != 1024 && a.unit != 2048) return hipErrorInvalidValue;
  return a.M <= 1 ? launch_m<1>(a, s) : a.M <= 4 ? launch_m<4>(a, s) : a.M <= 16 ? launch_m<16>(a, s) : launch_m<32>(a, s);
}

}  // namespace dvssq
