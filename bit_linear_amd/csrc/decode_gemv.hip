// Decode path for a few tokens (1 <= M <= 4) of
//     y = (x H) W_hat^T + ((x H) V^T) U^T
// in one kernel launch (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical
// Foundations 2, runtime equation; rotation: same card, Mathematical
// Foundations 1, and Spark-X2.5-4B-Hadamard-GSQ model card, Tier B equation;
// tiers: MiniCPM card INT4 equation and Spark card Tier A).
//
// Consumers: one workgroup of W wavefronts per (32 packed rows, K-range).
// Each wavefront streams its own groups of 64 inputs of the 32 rows with
// 16-byte loads, one INT4 group (32 bytes of a row) per pair of lanes (two
// 16-byte loads of a row per INT8 group), the operand layout of the int8
// matrix core v_mfma_i32_32x32x32_i8: lane (r, h) holds row r, bytes 16 h ..
// 16 h + 15 of the group.  A wavefront's groups are whole rotation units:
// before any weight load it copies the activations of its units straight
// into LDS (buffer loads to LDS); after them, it rotates and quantizes its
// (token, rotation unit) items while the weights stream in (two items at a
// time, so that their dependent chains interleave): each item of x_rot becomes a 15-bit integer
// X = 256 x1 + x2 with a power-of-two scale 2^e, stored as two int8 planes.
// Per group, four matrix-core instructions (the low and the high nibbles of
// the codes, times each plane) sum exactly in int32:
//   INT4 group g:  sum_k (n_k - 8) X_k = sum_k n_k X_k - 8 sum_k X_k, the
//                  nibbles n_k in [0, 15] being valid int8 operands; the
//                  group's bf16 scale and 2^e are applied in fp32;
//   INT8 rows:     sum_k q_k X_k, the row scale applied at the end.
// Nibble j of a byte (low or high) serves input 8 i + j or 8 i + j + 4 of a
// run of 8, so the planes keep, in each run of 32 inputs, first the inputs
// that low nibbles hold (0-3, 8-11, 16-19, 24-27), then the others.
//
// Producers (the lowest block indices, one per rotation unit) rotate their
// unit of x and compute its partial t = x_rot V^T (bf16 matrix cores, fp32
// sums), published as 64-bit words {fp32 value, 32-bit stamp of the call}:
// a consumer that reads a word sees the value and whether it belongs to this
// call in one load, with no separate flag.  Consumers read the partial t of
// their K-range's units once their main loop is done, sum them in unit order
// and add the low-rank term in fp32.  With a K split, the ranges' fp32
// results are summed in range order by the last workgroup of the row tile to
// arrive (tagged arrival counter).  Every wait is bounded: one that gives up
// poisons the workgroup's outputs with NaN and sets the workspace status word.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kRows = 32;         // packed rows per tile (matrix-core N dimension)
constexpr int kTokPad = 8;        // token slots of the per-token LDS tables and of t
constexpr int kLoadBatch = 16;    // device-scope loads issued together

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ i32x16 mfma32_i8(u32x4 a, u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}

// it / M for 0 <= it < 2048 and 1 <= M <= 32, with rM = ceil(2^16 / M)
// (a multiply instead of a division)
__device__ __forceinline__ int div_m(int it, uint32_t rM) { return static_cast<int>((static_cast<uint32_t>(it) * rM) >> 16); }

// s_waitcnt with vmcnt <= n (n < 64) and the other counters free
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 0xC07F;    // lgkmcnt(0), vmcnt and expcnt free

// a workgroup barrier that waits for nothing itself (the callers wait for
// exactly what they need first); the asm statements keep the compiler from
// moving memory accesses across it
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// position of input j (0 .. 31) of a run of 32 in the planes: the inputs of
// low nibbles first (j with bit 2 clear), then the others
__device__ __forceinline__ int plane_pos(int j) { return (j & 4) ? 16 + ((j >> 3) << 2) + (j & 3) : ((j >> 3) << 2) + (j & 3); }

// --------------------------------------------------------------------------- producer
// Partial t of rotation unit u for the M rows: t[m][i] = sum_{k in u} x_rot[m][k] V[i][k].
// The loads of x and of the first V k-steps go out together at the start.
template <int MT, int C, bool GT>
__device__ __forceinline__ void gemv_produce(const GemvArgs &a, int u, uint8_t *smem) {
  constexpr int P = 256 * C;
  constexpr int LDB = P + 8;            // bf16 x_rot row in LDS
  constexpr int KS = P / 32;            // k-steps of the t product
  constexpr int VJ = 2;                 // k-steps per wavefront per batch of V loads
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = static_cast<int>(blockDim.x >> 6);   // every wavefront of the block (>= 2)
  const int n = lane & 15, q = lane >> 4;
  const int M = MT == 1 ? 1 : a.M, k0 = u * P;   // MT = 1: one token
  const int nsp = a.nsr_pad, NI = nsp / 16;
  uint16_t *xb = reinterpret_cast<uint16_t *>(smem);                  // [16][LDB], rows >= M zero
  float *tred = reinterpret_cast<float *>(smem + 16 * LDB * 2);       // [W][NI][4][64]
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const auto rv = make_rsrc(a.V, static_cast<uint32_t>(a.nsr) * a.K * 2);
  const int xrow = GT ? 2 * a.K : a.K;            // inputs per row of x
  const auto rx = make_rsrc(a.x, static_cast<uint32_t>(M) * xrow * 2);

  // x rows wave, wave + W (M <= 4 <= 2 W) (gated: the gate and the up
  // values), then the first batch of V
  u32x2 xw[2][C], xu[2][C];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = wave + j * W;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      xw[j][c] = buf_load8(rx, m < M ? static_cast<uint32_t>(m * xrow + k0 + 256 * c + 16 * n + 4 * q) * 2 : kOutOfRange);
      xu[j][c] = u32x2{0u, 0u};
    }
  }
  if (GT)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = wave + j * W;
#pragma unroll
      for (int c = 0; c < C; ++c)
        xu[j][c] = buf_load8(rx, m < M ? static_cast<uint32_t>(m * xrow + a.K + k0 + 256 * c + 16 * n + 4 * q) * 2
                                       : kOutOfRange);
    }
  u32x4 vb[VJ][4];
  auto load_v = [&](int ks0) {
#pragma unroll
    for (int j = 0; j < VJ; ++j)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int ks = ks0 + j * W, i = it * 16 + n;
        const bool ok = ks < KS && it < NI && i < a.nsr;
        vb[j][it] = buf_load16(rv, ok ? static_cast<uint32_t>(i * a.K + k0 + 32 * ks + 8 * q) * 2 : kOutOfRange);
      }
  };
  load_v(wave);
  __builtin_amdgcn_sched_barrier(0);

  // zero the token rows the matrix cores read but no row of x fills
  for (int e = tid; e < (16 - M) * (LDB / 2); e += 64 * W)
    reinterpret_cast<uint32_t *>(xb + M * LDB)[e] = 0u;
  // x has landed (the V loads may still be in flight): rotate, bf16 into LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(VJ * 4));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = wave + j * W;
    if (m < M) {
      if (GT) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xw[j][c][0] = geglu_bf16x2(xw[j][c][0], xu[j][c][0]);
          xw[j][c][1] = geglu_bf16x2(xw[j][c][1], xu[j][c][1]);
          if (a.hout) *reinterpret_cast<u32x2 *>(a.hout + static_cast<int64_t>(m) * a.K + k0 + 256 * c + 16 * n + 4 * q) = xw[j][c];
        }
      }
      float y[C][4];
      rotate_x_item<C>(a.rotate, a.block, a.hscale, xw[j], y);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        u32x2 w;
        w[0] = pack_bf16x2(y[c][0], y[c][1]);
        w[1] = pack_bf16x2(y[c][2], y[c][3]);
        *reinterpret_cast<u32x2 *>(xb + m * LDB + 256 * c + 16 * n + 4 * q) = w;
      }
    }
  }
  __syncthreads();
  // t product on the bf16 matrix cores: wavefront w takes the k-steps w, w + W, ...
  f32x4 tacc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) tacc[it] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int ks0 = wave; ks0 < KS; ks0 += VJ * W) {
    if (ks0 != wave) load_v(ks0);
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const int ks = ks0 + j * W;
      u32x4 av = *reinterpret_cast<const u32x4 *>(xb + n * LDB + 32 * min(ks, KS - 1) + 8 * q);
      av = ks < KS ? av : z4;
#pragma unroll
      for (int it = 0; it < 4; ++it)
        if (it < NI) tacc[it] = mfma_bf16(av, vb[j][it], tacc[it]);
    }
  }
  // tacc[it] of lane (n, q): t[4 q + v][16 it + n]; sum the wavefronts in LDS
#pragma unroll
  for (int it = 0; it < 4; ++it)
    if (it < NI)
#pragma unroll
      for (int v = 0; v < 4; ++v) tred[((wave * NI + it) * 4 + v) * 64 + lane] = tacc[it][v];
  __syncthreads();
  for (int e = tid; e < M * nsp; e += 64 * W) {
    const int m = e / nsp, i = e - m * nsp;
    const int it = i >> 4, ln = (i & 15) + 16 * (m >> 2), v = m & 3;
    float s = 0.0f;
    for (int w = 0; w < W; ++w) s += tred[((w * NI + it) * 4 + v) * 64 + ln];
    const uint64_t word = (static_cast<uint64_t>(a.stamp) << 32) | __float_as_uint(s);
    if (a.publish) st_dev(a.tp + (static_cast<int64_t>(u) * kTokPad + m) * nsp + i, word);
  }
}

// --------------------------------------------------------------------------- consumer
// value of lane l ^ 16 / l ^ 32 (gfx950 permlane swaps)
__device__ __forceinline__ uint32_t xor16(uint32_t v, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32(uint32_t v, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (lane & 32) ? r[0] : r[1];
}

// 15-bit quantization of one rotated (token, unit) item held by a wavefront
// (lane (n, q) holds inputs 256 c + 16 n + 4 q + j): X = rint(y 2^-e) with
// max |X| in [2^13, 2^14), e from the exponent of max |y| (e clamped so that
// 2^-e and 2^e are normal).  X = 256 x1 + x2 with x2 the signed low byte:
// p1 / p2 get the lane's four x1 / x2 bytes of each 256-block, gsum 8 x the
// sum of X over the lane's group of 64 inputs (the same in its 16 lanes).
// Returns the fp32 bits of 2^e.  The wave-wide max and sums use DPP and the
// permlane swaps only.
template <int C>
__device__ __forceinline__ uint32_t quantize_fast(const float (&y)[C][4], uint32_t (&p1)[C], uint32_t (&p2)[C],
                                                  int (&gsum)[C], int lane) {
  float mx = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(y[c][j]));
  uint32_t b = __float_as_uint(mx);
  b = max(b, static_cast<uint32_t>(DVSSQ_DPP(static_cast<int>(b), 0xB1)));    // quad: xor 1
  b = max(b, static_cast<uint32_t>(DVSSQ_DPP(static_cast<int>(b), 0x4E)));    // quad: xor 2
  b = max(b, static_cast<uint32_t>(DVSSQ_DPP(static_cast<int>(b), 0x141)));   // mirror in 8
  b = max(b, static_cast<uint32_t>(DVSSQ_DPP(static_cast<int>(b), 0x140)));   // mirror in 16
  b = max(b, xor16(b, lane));
  b = max(b, xor32(b, lane));
  // max|y| = b (non-negative floats order as their bits); eb its biased exponent
  const int eb = min(254, max(14, static_cast<int>(b >> 23)));
  const float down = __uint_as_float(static_cast<uint32_t>(267 - eb) << 23);   // 2^(13 - ilogb)
#pragma unroll
  for (int c = 0; c < C; ++c) {
    int X[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) X[j] = static_cast<int>(__builtin_rintf(y[c][j] * down));
    int x1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x1[j] = (X[j] + 128) >> 8;
    const uint32_t s2lo = __builtin_amdgcn_perm(static_cast<uint32_t>(X[1]), static_cast<uint32_t>(X[0]), 0x0C0C0400u);
    const uint32_t s2hi = __builtin_amdgcn_perm(static_cast<uint32_t>(X[3]), static_cast<uint32_t>(X[2]), 0x0C0C0400u);
    const uint32_t s1lo = __builtin_amdgcn_perm(static_cast<uint32_t>(x1[1]), static_cast<uint32_t>(x1[0]), 0x0C0C0400u);
    const uint32_t s1hi = __builtin_amdgcn_perm(static_cast<uint32_t>(x1[3]), static_cast<uint32_t>(x1[2]), 0x0C0C0400u);
    p2[c] = s2lo | (s2hi << 16);
    p1[c] = s1lo | (s1hi << 16);
    int g = X[0] + X[1] + X[2] + X[3];
    g += DVSSQ_DPP(g, 0xB1);
    g += DVSSQ_DPP(g, 0x4E);
    g += static_cast<int>(xor16(static_cast<uint32_t>(g), lane));
    g += static_cast<int>(xor32(static_cast<uint32_t>(g), lane));
    gsum[c] = 8 * g;
  }
  return static_cast<uint32_t>(eb - 13) << 23;
}

// LDS of a consumer workgroup: x of the range (bf16 [M][KW], in 1 KB chunks;
// gated: the gate values, then the up values, each rounded up to 1 KB),
// the planes [2][MT][XP], 8 x group sums [KGw][8], unit scales [nu][8],
// partial results [W][NV][64], low-rank terms [NV][64], t [MT][nsp], output
// columns [32], INT8 scales [32], timeout word
template <int MT>
struct GemvLds {
  static constexpr int NV = MT == 1 ? 1 : 4;   // result values per lane that can hold a token (lanes h = 0)
  int XP, xbytes, xslab;   // xslab: bytes of one wavefront's slab of x
  uint16_t *xs;
  int8_t *pl1, *pl2;
  int *x8;
  float *esc, *red, *lrs, *ts;
  int *cols;
  float *s8s;
  int *tout;
  __device__ __forceinline__ GemvLds(const GemvArgs &a, uint8_t *smem) {
    const int KW = a.KW, KGw = KW >> 6;
    XP = KW + 16;
    const int gx = a.gated ? 2 : 1;    // gated: the gate values, then the up values
    xslab = gx * ((a.M * a.GPW * kGroup * 2 + 1023) & ~1023);
    xbytes = a.W * xslab;
    xs = reinterpret_cast<uint16_t *>(smem);
    pl1 = reinterpret_cast<int8_t *>(smem + xbytes);
    pl2 = pl1 + MT * XP;
    x8 = reinterpret_cast<int *>(pl2 + MT * XP);
    esc = reinterpret_cast<float *>(x8 + KGw * kTokPad);
    red = esc + a.nu_w * kTokPad;
    lrs = red + a.W * NV * 64;
    ts = lrs + NV * 64;
    cols = reinterpret_cast<int *>(ts + MT * a.nsr_pad);
    s8s = reinterpret_cast<float *>(cols + kRows);
    tout = reinterpret_cast<int *>(s8s + kRows);
  }
};

// Items (token m, unit u) of the K-range -> their 15-bit planes, 8 x group
// sums and unit scales in LDS.  NI independent items (1 or 2) go through each
// phase together, so that their dependent chains (matrix-core rotation,
// wave-wide max, group sums) interleave.
template <int C, bool T8, int NI>
__device__ __forceinline__ void put_items(const GemvArgs &a, int lane, int8_t *pl1, int8_t *pl2, int *x8, float *esc,
                                          int XP, const int *ms, const int *us, const u32x2 (*xw)[C]) {
  constexpr int P = 256 * C;
  const int n = lane & 15, q = lane >> 4;
  float y[NI][C][4];
#pragma unroll
  for (int i = 0; i < NI; ++i) rotate_x_item<C>(a.rotate, a.block, a.hscale, xw[i], y[i]);
  uint32_t p1[NI][C], p2[NI][C], eb[NI];
  int gsum[NI][C];
#pragma unroll
  for (int i = 0; i < NI; ++i) eb[i] = quantize_fast<C>(y[i], p1[i], p2[i], gsum[i], lane);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int m = ms[i], u = us[i];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int kk = u * P + 256 * c + 16 * n + 4 * q;   // first of the lane's 4 inputs (range-local)
      const int pos = T8 ? kk : (kk & ~31) + plane_pos(kk & 31);
      *reinterpret_cast<uint32_t *>(pl1 + m * XP + pos) = p1[i][c];
      *reinterpret_cast<uint32_t *>(pl2 + m * XP + pos) = p2[i][c];
      if (!T8 && (lane & 0x33) == 0) x8[(kk >> 6) * kTokPad + m] = gsum[i][c];
    }
    if (lane == 0) esc[u * kTokPad + m] = __uint_as_float(eb[i]);
  }
}

// x of item (m, u) from an LDS copy (gated: h = geglu(gate, up) formed here;
// the up values sit uofs inputs after the gate values)
template <int C, bool GT>
__device__ __forceinline__ void fetch_item(const uint16_t *src, int e, int uofs, u32x2 (&xw)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
    xw[c] = *reinterpret_cast<const u32x2 *>(src + e + 256 * c);
    if (GT) {
      const u32x2 uv = *reinterpret_cast<const u32x2 *>(src + uofs + e + 256 * c);
      xw[c][0] = geglu_bf16x2(xw[c][0], uv[0]);
      xw[c][1] = geglu_bf16x2(xw[c][1], uv[1]);
    }
  }
}

// Spare wavefront of a consumer workgroup (wavefront W): loads the tile's U
// rows, output columns and INT8 scales, waits for the producers' t of the
// range's units (stamped words, a bounded number of reloads), sums them in unit
// order and forms the low-rank term of each (row, token), in parallel with the
// compute wavefronts' main loop.
template <int MT>
__device__ __forceinline__ void gemv_spare(const GemvArgs &a, int cidx, uint8_t *smem) {
  constexpr int NV = GemvLds<MT>::NV;
  const GemvLds<MT> sm(a, smem);
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int tile = cidx / a.S, sp = cidx - tile * a.S;
  const bool T8 = tile >= a.t4;
  const int rows = T8 ? a.n8 : a.n4;
  const int row0 = (T8 ? tile - a.t4 : tile) * kRows;
  const int nrow = min(kRows, rows - row0);
  const int prow = row0 + min(r, nrow - 1), pk = (T8 ? a.n4 : 0) + prow;
  const int M = MT == 1 ? 1 : a.M, KGw = a.KW >> 6, nu = a.nu_w, u0 = sp * nu, nsp = a.nsr_pad;
  u32x4 uv[8];
  const auto ru = make_rsrc(a.U, static_cast<uint32_t>(a.N) * a.r * 2);
  const uint32_t ob = static_cast<uint32_t>(pk) * a.r * 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) uv[j] = buf_load16(ru, 8 * j < a.r ? ob + 16 * j : kOutOfRange);
  const uint32_t colv = a.idx[pk];
  const float s8v = T8 ? a.s8[prow] : 1.0f;
  if (lane == 0) *sm.tout = 0;
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  // t[m][i] = sum over the range's units of their partial t, in unit order.
  // Each lane loads the words of its (token, i) for a batch of units at once
  // and the batch is reloaded whole until every word carries this call's
  // stamp: these loads return only after the weight loads issued before them
  // on this compute unit, so each retry costs one such round trip, not one
  // per word.
  bool late = false;
  const int64_t ustr = static_cast<int64_t>(kTokPad) * nsp;
  const uint64_t fresh_word = static_cast<uint64_t>(a.stamp) << 32;
  for (int e0 = 0; e0 < M * nsp; e0 += 64) {
    const int e = e0 + lane;
    const int m = e / nsp, i = e - m * nsp;
    const bool act = e < M * nsp && i < a.nsr;
    const uint64_t *src = a.tp + (static_cast<int64_t>(u0) * kTokPad + m) * nsp + i;
    float s = 0.0f;
    for (int u = 0; u < nu; u += kLoadBatch) {
      uint64_t v[kLoadBatch];
      for (int spins = 0;; ++spins) {
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) v[j] = act && u + j < nu ? ld_dev(src + (u + j) * ustr) : fresh_word;
        bool fresh = true;
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) fresh = fresh && static_cast<uint32_t>(v[j] >> 32) == a.stamp;
        if (__builtin_amdgcn_ballot_w64(!fresh) == 0) break;
        if (spins >= a.spin_limit) {
          late = late || !fresh;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j)
        if (act && u + j < nu) s += __uint_as_float(static_cast<uint32_t>(v[j]));
    }
    if (e < M * nsp) sm.ts[e] = s;
  }
  if (__builtin_amdgcn_ballot_w64(late) != 0 && lane == 0) *sm.tout = 1;
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_wave_barrier();
  // low-rank term of tokens v < NV of row r (lanes h = 0): sum_i t[v][seg r + i] U[row][i]
  float lr[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) lr[v] = 0.0f;
  if (h == 0) {
    const int seg = (a.n_seg == 2 && prow >= rows / 2) ? 1 : 0;
    const float *tseg = sm.ts + seg * a.r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (8 * j < a.r) {
        float tv[NV][8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int v = 0; v < NV; ++v) tv[v][e] = (8 * j + e < a.r && v < M) ? tseg[v * nsp + 8 * j + e] : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t dw = uv[j][e >> 1];
          const float uf = (8 * j + e < a.r) ? __uint_as_float((e & 1) ? (dw & 0xFFFF0000u) : (dw << 16)) : 0.0f;
#pragma unroll
          for (int v = 0; v < NV; ++v) lr[v] = fmaf(tv[v][e], uf, lr[v]);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) sm.lrs[v * 64 + lane] = lr[v];
  if (h == 0) {
    sm.cols[r] = static_cast<int>(colv);
    sm.s8s[r] = s8v;
  }
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __syncthreads();  // (3) results
}

// MT: largest M (1 or 4); C: 256-blocks per rotation unit; G: most groups per
// compute wavefront (its load registers); T8: INT8 tier.  The compute
// wavefronts 0 .. W-1 of a consumer workgroup (wavefront W is gemv_spare).
template <int MT, int C, int G, bool T8, bool GT>
__device__ __forceinline__ void gemv_consume(const GemvArgs &a, int cidx, uint8_t *smem) {
  constexpr int P = 256 * C;
  constexpr int GPU = P / kGroup;       // groups per rotation unit
  constexpr int NV = GemvLds<MT>::NV;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(tid >> 6));
  const int W = a.W;
  const int r = lane & 31, h = lane >> 5;
  const int tile = cidx / a.S, sp = cidx - tile * a.S;
  const int rows = T8 ? a.n8 : a.n4;
  const int row0 = (T8 ? tile - a.t4 : tile) * kRows;    // first row of the tile inside the tier
  const int nrow = min(kRows, rows - row0);
  const int M = MT == 1 ? 1 : a.M, K = a.K, KW = a.KW, k0 = sp * KW;
  const uint32_t rM = (65536u + M - 1) / M;   // div_m
  const int KG = K >> 6, KGw = KW >> 6, gk0 = k0 >> 6;   // groups: whole K, this range, first of the range
  const int nu = a.nu_w, u0 = sp * nu;
  // this wavefront's rotation units of the range (lut_units: 4 bits per
  // wavefront, in wavefront order); its first group inside the range, its groups
  int ustart = 0;
  for (int j = 0; j < wave; ++j) ustart += static_cast<int>((a.lut_units >> (4 * j)) & 15u);
  const int ucnt = static_cast<int>((a.lut_units >> (4 * wave)) & 15u);
  const int gw0 = ustart * GPU;
  const int ng = max(0, min(ucnt * GPU, KGw - gw0));
  const int nsp = a.nsr_pad;
  const bool row_ok = r < nrow;
  const int prow = row0 + min(r, nrow - 1);                // row inside the tier
  const int pk = (T8 ? a.n4 : 0) + prow;                   // packed row

  const GemvLds<MT> sm(a, smem);
  const int XP = sm.XP, xbytes = sm.xbytes;
  uint16_t *xs = sm.xs;
  int8_t *pl1 = sm.pl1, *pl2 = sm.pl2;
  int *x8 = sm.x8;
  float *esc = sm.esc, *red = sm.red, *lrs = sm.lrs;
  int *cols = sm.cols;
  float *s8s = sm.s8s;
  int *tout = sm.tout;

  // ---- 1. activations first, straight into LDS: each wavefront copies the
  // rows of its own rotation units (its groups are whole units) into its own
  // slab [M][lnu P] (1 KB per wavefront instruction, lane l's 16 bytes at
  // byte 16 l; 16 | 2 lnu P, so a lane's bytes never straddle rows)
  const int lu0 = ustart, lnu = ng / GPU;
  const int n = lane & 15, q = lane >> 4;
  const int LW = lnu * P;                               // inputs of the slab's rows
  uint16_t *slab = xs + wave * (sm.xslab >> 1);         // this wavefront's slab
  int uofs = 0;                                         // gated: the up values, inputs after the gate values
  {
    const int span = 2 * LW, nch = (M * span + 1023) >> 10;
    uofs = GT ? nch * 512 : 0;
    const int xrow = GT ? 2 * K : K;
    const auto rx = make_rsrc(a.x, static_cast<uint32_t>(M) * xrow * 2);
    const int kbase = k0 + lu0 * P;
    uint8_t *dst = reinterpret_cast<uint8_t *>(slab);
    for (int h2 = 0; h2 < (GT ? 2 : 1); ++h2)
      for (int c = 0; c < nch; ++c) {
        const int f = c * 1024 + lane * 16;             // flattened byte
        const int m = f / span, kb = f - m * span;
        const uint32_t off = m < M ? static_cast<uint32_t>(m * 2 * xrow + 2 * (h2 * K + kbase) + kb) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void *)(dst + (h2 * nch + c) * 1024), 16, off, 0, 0, 0);
      }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. this wavefront's weight loads (the same count in every compute
  // wavefront: out-of-range offsets read zeros without touching memory)
  u32x4 wq[G][T8 ? 2 : 1];
  uint32_t sb[T8 ? 1 : G / 2];
  if constexpr (!T8) {
    const auto r4 = make_rsrc(a.q4, static_cast<uint32_t>(a.n4) * (K / 2));
    const auto rs = make_rsrc(a.s4, static_cast<uint32_t>(a.n4) * KG * 2);
    const uint32_t ob = static_cast<uint32_t>(prow) * (K / 2) + (gk0 + gw0) * 32 + 16 * h;
    const uint32_t os = (static_cast<uint32_t>(prow) * KG + gk0 + gw0) * 2;
#pragma unroll
    for (int i = 0; i < G; ++i) wq[i][0] = buf_load16(r4, row_ok && i < ng ? ob + 32 * i : kOutOfRange);
#pragma unroll
    for (int i = 0; i < G / 2; ++i) sb[i] = buf_load4(rs, row_ok && 2 * i < ng ? os + 4 * i : kOutOfRange);
  } else {
    const auto r8 = make_rsrc(a.q8, static_cast<uint32_t>(a.n8) * K);
    const uint32_t ob = static_cast<uint32_t>(prow) * K + (gk0 + gw0) * 64 + 32 * h;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      wq[i][0] = buf_load16(r8, row_ok && i < ng ? ob + 64 * i : kOutOfRange);
      wq[i][1] = buf_load16(r8, row_ok && i < ng ? ob + 64 * i + 16 : kOutOfRange);
    }
  }
  constexpr int kAfterX = T8 ? 2 * G : G + G / 2;   // loads issued after the activations
  __builtin_amdgcn_sched_barrier(0);
  // the activations of this wavefront have landed
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterX));

  // ---- 3. rotate and quantize this wavefront's own items (no other
  // wavefront reads them), two at a time
  const int nit = M * lnu;
  int it = 0;
  for (; it + 2 <= nit; it += 2) {
    int ms[2], us[2];
    u32x2 xw[2][C];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ul = div_m(it + i, rM);
      ms[i] = it + i - ul * M;
      us[i] = lu0 + ul;
      fetch_item<C, GT>(slab, ms[i] * LW + ul * P + 16 * n + 4 * q, uofs, xw[i]);
    }
    put_items<C, T8, 2>(a, lane, pl1, pl2, x8, esc, XP, ms, us, xw);
  }
  if (it < nit) {
    const int ul = div_m(it, rM);
    int ms[1] = {it - ul * M}, us[1] = {lu0 + ul};
    u32x2 xw[1][C];
    fetch_item<C, GT>(slab, ms[0] * LW + ul * P + 16 * n + 4 * q, uofs, xw[0]);
    put_items<C, T8, 1>(a, lane, pl1, pl2, x8, esc, XP, ms, us, xw);
  }
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_wave_barrier();

  // ---- 4. main loop: four int8 matrix-core instructions per group
  float acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
  {
    const int t = min(r, M - 1);                         // A operand: token t, half h
    const int8_t *a1 = pl1 + t * XP + 32 * h, *a2 = pl2 + t * XP + 32 * h;
    const i32x16 z16 = {};
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (i < ng) {
        const int g = gw0 + i;                           // group inside the range
        const u32x4 x1l = *reinterpret_cast<const u32x4 *>(a1 + 64 * g);
        const u32x4 x1h = *reinterpret_cast<const u32x4 *>(a1 + 64 * g + 16);
        const u32x4 x2l = *reinterpret_cast<const u32x4 *>(a2 + 64 * g);
        const u32x4 x2h = *reinterpret_cast<const u32x4 *>(a2 + 64 * g + 16);
        u32x4 bl, bh;
        i32x16 c2 = z16;
        if constexpr (!T8) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            bl[d] = wq[i][0][d] & 0x0F0F0F0Fu;
            bh[d] = (wq[i][0][d] >> 4) & 0x0F0F0F0Fu;
          }
          if constexpr (NV == 1) {
            c2[0] = -x8[g * kTokPad];
          } else {
            const i32x4 xg = *reinterpret_cast<const i32x4 *>(x8 + g * kTokPad);
#pragma unroll
            for (int v = 0; v < 4; ++v) c2[v] = -xg[v];
          }
        } else {
          bl = wq[i][0];
          bh = wq[i][1];
        }
        i32x16 d1 = mfma32_i8(x1l, bl, z16);
        i32x16 d2 = mfma32_i8(x2l, bl, c2);
        d1 = mfma32_i8(x1h, bh, d1);
        d2 = mfma32_i8(x2h, bh, d2);
        float sg = 1.0f;
        if constexpr (!T8) {
          const uint32_t sw = sb[i / 2];
          sg = __uint_as_float((i & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
        }
        if constexpr (NV == 1) {
          const float ev = esc[(g / GPU) * kTokPad];
          acc[0] = fmaf(sg * ev, static_cast<float>((d1[0] << 8) + d2[0]), acc[0]);
        } else {
          const f32x4 ev = *reinterpret_cast<const f32x4 *>(esc + (g / GPU) * kTokPad);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = fmaf(sg * ev[v], static_cast<float>((d1[v] << 8) + d2[v]), acc[v]);
        }
      }
    }
  }

  // ---- 5. the wavefronts' partial results -> LDS; wavefront 0 adds them,
  // the spare wavefront's low-rank term, and applies the INT8 row scale
#pragma unroll
  for (int v = 0; v < NV; ++v) red[(wave * NV + v) * 64 + lane] = acc[v];
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __syncthreads();  // (3)
  if (wave != 0) return;
  float cacc[NV];
  const float rs8 = s8s[r];
  const int col = cols[r];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    float s = red[v * 64 + lane];
    for (int w = 1; w < W; ++w) s += red[(w * NV + v) * 64 + lane];
    cacc[v] = fmaf(s, rs8, lrs[v * 64 + lane]);
  }
  if (*tout) {
    if (lane == 0) st_dev(a.status, DVSSQ_STATUS_WAIT_TIMEOUT);
#pragma unroll
    for (int v = 0; v < NV; ++v) cacc[v] = __builtin_nanf("");
  }

  // ---- 6. output (lanes h = 0 hold tokens v < NV of row r): direct, or this
  // range's fp32 result and the ordered sum by the last workgroup of the tile
  if (a.S == 1) {
    if (!row_ok || h != 0) return;
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (v < M) a.y[static_cast<int64_t>(v) * a.N + col] = f32_to_bf16(cacc[v]);
    return;
  }
  if (row_ok && h == 0)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      if (v < M) st_dev(a.part + (static_cast<int64_t>(sp) * M + v) * a.N + pk, cacc[v]);
  drain_stores();
  int last = 0;
  if (lane == 0) {
    uint64_t *cnt = a.cnt + tile;
    last = arrive_tagged(cnt, a.stamp) == static_cast<uint32_t>(a.S);
  }
  last = __shfl(last, 0, 64);
  if (!last || !row_ok || h != 0) return;
  // the ranges of tokens v < M of row r, summed in range order
  const int64_t sstride = static_cast<int64_t>(M) * a.N;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (v >= M) continue;
    const float *src = a.part + static_cast<int64_t>(v) * a.N + pk;
    float s = 0.0f;
    for (int s0 = 0; s0 < a.S; s0 += kLoadBatch) {
      float pv[kLoadBatch];
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) pv[j] = s0 + j < a.S ? ld_dev(src + (s0 + j) * sstride) : 0.0f;
#pragma unroll
      for (int j = 0; j < kLoadBatch; ++j) s += pv[j];
    }
    a.y[static_cast<int64_t>(v) * a.N + col] = f32_to_bf16(s);
  }
}

template <int MT, int C, int G, bool GT>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  // Block b runs on compute unit b mod (compute units) while every block of
  // the grid is resident at once, so with cus < G <= 2 cus blocks the first
  // G - cus positions share a unit with the last ones.  Roles by position
  // (lead4 >= 0): INT4 consumers 0 .. lead4 - 1 (they share with INT4
  // consumers at the end), then the INT8 consumers (twice an INT4 tile's
  // bytes) and the producers, each on a unit of its own, then the other INT4
  // consumers (lead4 = 0 for larger grids: INT8 and producers first).
  // lead4 < 0 (a grid of one round): producers, INT4, INT8.
  const int b = blockIdx.x;
  const int n8c = a.t8 * a.S, lead = a.lead4;
  int c;   // consumer index = tile * S + range
  if (lead < 0) {
    if (b < a.nprod) {
      gemv_produce<MT, C, GT>(a, b, smem);
      return;
    }
    c = b - a.nprod;
  } else if (b < lead) {
    c = b;
  } else if (b < lead + n8c) {
    c = a.t4 * a.S + (b - lead);
  } else if (b < lead + n8c + a.nprod) {
    gemv_produce<MT, C, GT>(a, b - lead - n8c, smem);
    return;
  } else {
    c = b - n8c - a.nprod;
  }
  if (static_cast<int>(threadIdx.x >> 6) == a.W) gemv_spare<MT>(a, c, smem);
  else if (c < a.t4 * a.S) gemv_consume<MT, C, G, false, GT>(a, c, smem);
  else gemv_consume<MT, C, G, true, GT>(a, c, smem);
}

size_t producer_lds(int unit, int W, int nsp) {
  return static_cast<size_t>(16) * (unit + 8) * 2 + static_cast<size_t>(W) * (nsp / 16) * 4 * 64 * 4;
}

size_t consumer_lds(int MT, int M, int KW, int nu, int W, int GPW, int nsp, bool gated) {
  const size_t NV = MT == 1 ? 1 : 4, gx = gated ? 2 : 1;
  const size_t xslab = gx * ((static_cast<size_t>(M) * GPW * kGroup * 2 + 1023) & ~size_t(1023));
  const size_t xbytes = W * xslab;
  return xbytes + 2 * static_cast<size_t>(MT) * (KW + 16) + static_cast<size_t>(KW / kGroup + nu) * kTokPad * 4 +
         (static_cast<size_t>(W) + 1) * NV * 64 * 4 + static_cast<size_t>(MT) * nsp * 4 + 2 * kRows * 4 + 16;
}

template <int MT, int C, int G, bool GT>
hipError_t launch_gt(const GemvArgs &a, size_t lds, hipStream_t s) {
  if (lds > 65536) {
    static std::atomic<uint64_t> done{0};
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(gemv_kernel<MT, C, G, GT>), 160 * 1024, done);
    if (e != hipSuccess) return e;
  }
  const int grid = a.nprod + (a.t4 + a.t8) * a.S;
  return launch_kernel(reinterpret_cast<const void *>(gemv_kernel<MT, C, G, GT>), dim3(grid), dim3(64 * (a.W + 1)),
                       lds, s, a);
}

// the gated input (h formed from the gate+up output as it loads) is its own
// instantiation, so that the plain kernel carries none of its code
template <int MT, int C, int G>
hipError_t launch_t(const GemvArgs &a, size_t lds, hipStream_t s) {
  return a.gated ? launch_gt<MT, C, G, true>(a, lds, s) : launch_gt<MT, C, G, false>(a, lds, s);
}

template <int MT, int C>
hipError_t launch_g(const GemvArgs &a, size_t lds, hipStream_t s) {
  if (a.GPW <= 4) return launch_t<MT, C, 4>(a, lds, s);
  if (a.GPW <= 8) return launch_t<MT, C, 8>(a, lds, s);
  return launch_t<MT, C, 12>(a, lds, s);
}

template <int MT>
hipError_t launch_m(const GemvArgs &a, size_t lds, hipStream_t s) {
  switch (a.unit) {
    case 256: return launch_g<MT, 1>(a, lds, s);
    case 512: return launch_g<MT, 2>(a, lds, s);
    case 1024: return launch_g<MT, 4>(a, lds, s);
    default: return launch_g<MT, 8>(a, lds, s);
  }
}

}  // namespace

// One more compute wavefront where the even split puts two of them on one
// SIMD: the wavefronts of a workgroup sit on the four SIMDs in turn
// (wavefront w on SIMD w mod 4, the spare one on SIMD W mod 4), and two
// compute wavefronts on one SIMD share its issue slots, so with W = 5 the
// pair on SIMD 0 finishes its rotation and main loop well after the others.
// With W + 1 wavefronts of at most upw units each, the units go one by one
// to the wavefront whose SIMD carries the fewest so far (the spare counted as
// half a unit); taken if the busiest SIMD then carries fewer units.
bool spread_units(int nu, int upw, GemvPlan *p) {
  const int W = p->W, W1 = W + 1;
  if (W1 + 1 > 8 || nu > W1 * upw) return false;   // 64 (W1 + 1) threads within the launch bound
  auto busiest = [](const double (&l)[4]) { return std::max(std::max(l[0], l[1]), std::max(l[2], l[3])); };
  double even[4] = {0.0, 0.0, 0.0, 0.0}, load[4] = {0.0, 0.0, 0.0, 0.0};
  even[W % 4] += 0.5;
  for (int w = 0; w < W; ++w) even[w % 4] += static_cast<double>((p->lut_units >> (4 * w)) & 15u);
  load[W1 % 4] += 0.5;
  int cnt[8] = {0};
  for (int u = 0; u < nu; ++u) {
    int best = -1;
    for (int w = 0; w < W1; ++w) {
      if (cnt[w] >= upw) continue;
      if (best < 0 || load[w % 4] < load[best % 4] - 1e-9) best = w;
    }
    ++cnt[best];
    load[best % 4] += 1.0;
  }
  if (busiest(load) >= busiest(even) - 1e-9) return false;
  uint64_t lut = 0;
  for (int w = 0; w < W1; ++w) lut |= static_cast<uint64_t>(cnt[w]) << (4 * w);
  p->W = W1;
  p->lut_units = lut;
  return true;
}

// Plan of the few-token decode: S equal K-ranges (each a whole number of
// rotation units), the smallest S that gives every compute unit a workgroup
// (or the largest feasible), and W compute wavefronts per workgroup (plus the
// spare one), each taking GPW (even, at most 12) of the range's groups, about
// 8 where W <= 7 allows.
bool plan_gemv(const dvssq_layout &L, int M, int cus, bool gated, GemvPlan *p) {
  if (M < 1 || M > kGemvMaxM) return false;
  const int unit = L.block > 256 ? L.block : 256;
  if (L.K % unit) return false;
  const int64_t big = std::max<int64_t>(static_cast<int64_t>(L.n_int4) * L.K / 2,
                                        std::max<int64_t>(static_cast<int64_t>(L.n_int8) * L.K,
                                                          static_cast<int64_t>(L.N) * L.r * 2));
  if (big >= (int64_t{1} << 31) || static_cast<int64_t>(M) * L.K * 4 >= (int64_t{1} << 31)) return false;
  const int nunit = L.K / unit, KG = L.K / kGroup;
  const int tiles = (L.n_int4 + kRows - 1) / kRows + (L.n_int8 + kRows - 1) / kRows;
  const int nsp = (L.n_seg * L.r + 31) / 32 * 32;
  const int MT = M <= 1 ? 1 : 4;
  bool found = false;
  for (int S = 1; S <= kMaxSplit && S <= nunit; ++S) {
    if (nunit % S) continue;
    const int KGr = KG / S, nu = nunit / S;
    int gpw = 8, W = (KGr + gpw - 1) / gpw;
    if (W > 7) {
      W = 7;
      gpw = ((KGr + W - 1) / W + 1) & ~1;
      if (gpw > 12) continue;
      W = (KGr + gpw - 1) / gpw;
    } else {
      gpw = ((KGr + W - 1) / W + 1) & ~1;
      // blocks of 256: whole units of 4 groups per wavefront (rotated by it)
      if (unit == 256 && gpw % 4) {
        gpw = (gpw + 3) & ~3;
        W = (KGr + gpw - 1) / gpw;
      }
    }
    const size_t lds =
        std::max(consumer_lds(MT, M, L.K / S, nu, W, gpw, nsp, gated), producer_lds(unit, W + 1, nsp));
    if (lds > 160 * 1024) continue;
    p->S = S;
    p->W = W;
    p->GPW = gpw;
    // each wavefront rotates its own units when its groups are whole units (at most two)
    const int gpu = unit / kGroup;
    p->local_rot = (gpw % gpu == 0 && gpw <= 2 * gpu) ? 1 : 0;
    p->lut_units = 0;
    for (int w = 0; w < W; ++w)   // gpw / gpu units each, the last wavefront the rest
      p->lut_units |= static_cast<uint64_t>(std::min(gpw / gpu, nu - w * (gpw / gpu))) << (4 * w);
    if (p->local_rot) {
      const GemvPlan even = *p;
      if (!spread_units(nu, gpw / gpu, p) ||
          std::max(consumer_lds(MT, M, L.K / S, nu, p->W, p->GPW, nsp, gated), producer_lds(unit, p->W + 1, nsp)) >
              160 * 1024)
        *p = even;
    }
    found = true;
    if (tiles * S >= cus) break;
  }
  // Taken where it measured faster than the 16-row kernel (decode_small): the
  // wavefronts rotate their own units (blocks of 256 or 512), and the K-range
  // is whole unless M = 1 (the split's ordered partial sums cost more than the
  // 16-row kernel's at M > 1).  Blocks of 1024 and 2048 leave one wavefront a
  // whole unit to rotate per token and stay on the 16-row kernel.
  return found && p->local_rot && (p->S == 1 || M == 1);
}

hipError_t launch_gemv(const GemvArgs &a, hipStream_t s) {
  if (a.unit != 256 && a.unit != 512 && a.unit != 1024 && a.unit != 2048) return hipErrorInvalidValue;
  const int MT = a.M <= 1 ? 1 : 4;
  const size_t lds = std::max(consumer_lds(MT, a.M, a.KW, a.nu_w, a.W, a.GPW, a.nsr_pad, a.gated != 0),
                              producer_lds(a.unit, a.W + 1, a.nsr_pad));
  return a.M <= 1 ? launch_m<1>(a, lds, s) : launch_m<4>(a, lds, s);
}

}  // namespace dvssq
