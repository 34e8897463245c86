// KV-BSS attention (Spark-X2.5-4B-Hadamard-GSQ model card, section 2, KV-BSS:
// focus factor scaling and attention haze truncation; Spark-X2.5-4B discussion
// 14, Mathematical Formulation 1-2 and the eager attention change) for causal
// grouped-query attention (Spark-X2.5-4B GGUF page, "The model": 16 query
// heads, 4 KV heads, head_dim 256, sliding window 512 on the sliding layers):
//   s_j = scale (q . k_j), m = max over the row's visible keys,
//   keys with s_j < m - haze dropped, o = sum exp(s_j - m) v_j / sum exp(s_j - m).
//
// The haze threshold depends on the row's final maximum, which a one-pass
// online softmax only knows at the end, after it has already summed keys
// that the threshold drops.  So each workgroup passes over its keys twice:
// the first pass forms the logits on the matrix cores and keeps their row
// maxima; the second forms them again and sums exp(s - m) v with m fixed,
// which needs no rescaling of the running sums.  The cost is one more
// Q K^T product per key block.
//
// Workgroup: W = 4 wavefronts, 64 rows of one (sequence, KV head): the rows
// are the (query, head) pairs of the KV head's query group, query-major, so
// every row of the tile reads the same K and V.  Wavefront w owns rows 16 w
// .. 16 w + 15.  Keys go in blocks of 32, K and V each staged row-major in LDS
// by buffer-to-LDS loads (no registers), double-buffered in four LDS arrays of
// their own (so the compiler can tell the block being read from the one being
// filled) so that the next block's loads run under the current block's
// matrix-core work.  Per block and wavefront (v_mfma_f32_16x16x32_bf16, lane
// l = (i = l % 16, g = l / 16)):
//   S^T = K Q^T: A = 16 keys x 32 dims of K (lane: key i, dims 8 g .. + 7),
//       B = the wavefront's q (lane: row i, dims 8 g .. + 7, in registers);
//       lane l gets S[row i][keys 4 g .. 4 g + 3] of the 16-key tile;
//   O += P V: A = P, built in registers from the two tiles' S^T values (slots
//       0-3: keys 4 g + e, slots 4-7: keys 16 + 4 g + e); B = V, whose
//       matching keys (4 consecutive per 64-bit read) come from LDS by the
//       transposing read ds_read_b64_tr_b16: within 16 lanes, lane 4 j + c
//       points at key row j, dims 4 c .. 4 c + 3, and lane i receives dim i
//       of the four rows.
// Every operand read of a block is issued before its first matrix-core
// instruction.  LDS rows are 2 D bytes; the 16-byte chunks of key row k sit
// XOR-swizzled by sw(k) (two bits of k per position), so that both the K
// reads (16 keys, one chunk) and the transposing V reads (4 keys, two
// chunks) hit distinct banks.  fp32 logits and sums; P rounded to bf16 for
// the matrix cores; output bf16.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kKeys = 32;            // keys per block
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct AttnLds {
  static constexpr int kBlock = kKeys * D * 2;    // bytes of one K or V block
};

// chunk swizzle of key row k: D / 8 chunks of 16 bytes per row
template <int D>
__device__ __forceinline__ int swz(int k) {
  if constexpr (D >= 128) return (2 * (k & 7)) ^ ((k >> 3) & 1);
  else return (2 * (k & 3)) ^ ((k >> 2) & 1);
}

// Buffer-to-LDS copies of key blocks: a lane's source offset inside a block
// is fixed (row, swizzled chunk), so it is computed once (StageMap); a block
// adds its scalar base (sequence, first key, KV head) as the buffer's scalar
// offset (below 2^31: the host limits K and V to 2^30 elements), and keys
// past the end of the sequence read zeros.  Each of the W wavefronts issues
// D / (16 W) copies of 1 KB (lane l's 16 bytes land at byte 16 l).
template <int D, int W>
struct StageMap {
  static constexpr int PER = D / (16 * W);
  static_assert(PER >= 1, "one 1 KB copy per wavefront at least");
  uint32_t voff[PER];   // byte offset of the lane's 16 bytes from the block's first key row
  int row[PER];         // the key row (inside the block) they come from
  __device__ __forceinline__ StageMap(const AttnArgs &a, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int o = 1024 * (wave * PER + t) + 16 * lane;
      row[t] = o / (2 * D);
      const int c = (o % (2 * D)) / 16;
      voff[t] = static_cast<uint32_t>((row[t] * a.Hkv * D + 8 * (c ^ swz<D>(row[t]))) * 2);
    }
  }
  __device__ __forceinline__ void stage(const AttnArgs &a, __amdgpu_buffer_rsrc_t rs, int b, int g, int kb,
                                        uint8_t *dst, int wave) const {
    const uint32_t base = static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Nk + kb) * a.Hkv + g) * D) * 2);
    const int lim = a.Nk - kb;                 // rows of the block inside the sequence
#pragma unroll
    for (int t = 0; t < PER; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(dst + 1024 * (wave * PER + t)),
                                               16, row[t] < lim ? voff[t] : kOutOfRange, static_cast<int>(base), 0, 0);
  }
};

// S^T tiles of the wavefront's 16 rows against the 32 keys of a K block:
// s[nt][v] = S[row l % 16][key 16 nt + 4 (l / 16) + v], unscaled.  Every
// operand read of the block is issued before the first matrix-core
// instruction, so the LDS latency is waited for once per block.
template <int D>
__device__ __forceinline__ void logits_t(const u32x4 (&qa)[D / 32], const uint8_t *kblk, int lane, f32x4 (&s)[2]) {
  const int i = lane & 15, gq = lane >> 4;
  u32x4 ka[2][D / 32];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int key = 16 * nt + i;
    const uint8_t *kr = kblk + key * 2 * D;
    const int w = gq ^ swz<D>(key);            // chunk 4 st + g sits at slot (4 st + g) ^ sw = w ^ 4 st
#pragma unroll
    for (int st = 0; st < D / 32; ++st) ka[nt][st] = *reinterpret_cast<const u32x4 *>(kr + 16 * (w ^ (4 * st)));
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < D / 32; ++st) acc = mfma_bf16(ka[nt][st], qa[st], acc);
    s[nt] = acc;
  }
}

constexpr int kVm0 = 0x0F70;    // s_waitcnt vmcnt(0), the other counters free
// s_waitcnt with vmcnt <= n (n < 64) and the other counters free
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Per-row state of a wavefront lane (row 16 w + l % 16 of the tile).
struct RowState {
  int pos, jlo;        // position, first visible key
  bool rok;            // the row exists
};

// Pass 1 on block t (keys kb .. kb + 31) held in kcur; the next block is
// staged into knxt meanwhile.  kcur and knxt are distinct LDS arrays, so the
// compiler sees that the reads of kcur do not wait for the copy into knxt.
template <int D, int W>
__device__ __forceinline__ void max_block(const AttnArgs &a, const StageMap<D, W> &sm, __amdgpu_buffer_rsrc_t rk, int b, int g, int kb,
                                          bool more, bool full, const uint8_t *kcur, uint8_t *knxt,
                                          const u32x4 (&qa)[D / 32], const RowState &rs, int wave, int lane, float &mx) {
  const int gq = lane >> 4;
  __builtin_amdgcn_s_waitcnt(kVm0);
  __syncthreads();                           // block t in LDS; block t - 1 no longer read
  if (more) sm.stage(a, rk, b, g, kb + kKeys, knxt, wave);
  f32x4 s[2];
  logits_t<D>(qa, kcur, lane, s);
  if (full) {                                // every key of the block visible to every row
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[nt][v] * a.scale);
  } else {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = kb + 16 * nt + 4 * gq + v;
        if (j <= rs.pos && j >= rs.jlo) mx = fmaxf(mx, s[nt][v] * a.scale);
      }
  }
}

// Pass 2 on block t: O += P V and l += sum P over the kept keys, with the
// next block's K and V staged into knxt / vnxt meanwhile.
template <int D, int W>
__device__ __forceinline__ void sum_block(const AttnArgs &a, const StageMap<D, W> &sm, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          int b, int g, int kb, bool more, bool full, const uint8_t *kcur, const uint8_t *vcur,
                                          uint8_t *knxt, uint8_t *vnxt, const u32x4 (&qa)[D / 32], const RowState &rs,
                                          float thr, float mb, int wave, int lane, f32x4 (&oacc)[D / 16], float &lsum) {
  const int i = lane & 15, gq = lane >> 4;
  const int vj = i >> 2, vc = i & 3;         // transposing reads: lane 4 j + c points at key row j, dims 4 c ..
  __builtin_amdgcn_s_waitcnt(kVm0);
  __syncthreads();
  if (more) {
    sm.stage(a, rk, b, g, kb + kKeys, knxt, wave);
    sm.stage(a, rv, b, g, kb + kKeys, vnxt, wave);
  }
  f32x4 s[2];
  logits_t<D>(qa, kcur, lane, s);
  // key rows of the two reads (keys 4 g + j and 16 + 4 g + j), this lane's
  // half chunk; chunk 2 dt + (c >> 1) of a row sits at slot (2 dt + (c >> 1)) ^ sw
  const int k0 = 4 * gq + vj, k1 = 16 + 4 * gq + vj;
  const uint8_t *v0 = vcur + k0 * 2 * D + 8 * (vc & 1), *v1 = vcur + k1 * 2 * D + 8 * (vc & 1);
  const int u0 = (vc >> 1) ^ swz<D>(k0), u1 = (vc >> 1) ^ swz<D>(k1);
  u32x4 vop[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(v0 + 16 * (u0 ^ (2 * dt))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(v1 + 16 * (u1 ^ (2 * dt))));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    vop[dt] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
  // thr is +inf on rows past the end, so they keep no key
  float p[2][4];
  if (full) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sv = s[nt][v] * a.scale;
        p[nt][v] = sv < thr ? 0.0f : __builtin_amdgcn_exp2f(sv * kLog2e - mb);   // argument in [-17.4, 0]
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = kb + 16 * nt + 4 * gq + v;
        const float sv = s[nt][v] * a.scale;
        const bool keep = j <= rs.pos && j >= rs.jlo && !(sv < thr);
        p[nt][v] = keep ? __builtin_amdgcn_exp2f(sv * kLog2e - mb) : 0.0f;
      }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) lsum += p[nt][v];
  u32x4 pa;
  pa[0] = pack_bf16x2(p[0][0], p[0][1]);
  pa[1] = pack_bf16x2(p[0][2], p[0][3]);
  pa[2] = pack_bf16x2(p[1][0], p[1][1]);
  pa[3] = pack_bf16x2(p[1][2], p[1][3]);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = mfma_bf16(pa, vop[dt], oacc[dt]);
}

template <int D, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void kvbss_attention_kernel(AttnArgs a) {
  constexpr int kRowsPerWg = 16 * W;
  // K and V blocks, two buffers each, as four arrays of their own
  __shared__ __align__(16) uint8_t k0buf[AttnLds<D>::kBlock], k1buf[AttnLds<D>::kBlock];
  __shared__ __align__(16) uint8_t v0buf[AttnLds<D>::kBlock], v1buf[AttnLds<D>::kBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, gq = lane >> 4;

  // Tiles of later queries see more keys.  Workgroup k takes (sequence, KV
  // head) k mod nseq, so that with nseq dividing the 8 XCDs (or a multiple of
  // them) each XCD's L2 serves one set of K and V; its tiles go heaviest first
  // over the first half of the grid and lightest first over the second, so
  // that the two workgroups a compute unit receives (the dispatcher places the
  // first half, then the second) carry about the same work together.
  const int nseq = a.B * a.Hkv, k = static_cast<int>(blockIdx.x);
  const int bg = k % nseq, q = k / nseq, hq = (a.tiles + 1) / 2;
  const int tile = q < hq ? a.tiles - 1 - q : q - hq;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int r0 = tile * kRowsPerWg;
  const int r1 = min(a.rows, r0 + kRowsPerWg) - 1;       // last row of the tile
  const int p0 = a.Nk - a.Mq;                             // position of query 0
  const int pmin = p0 + r0 / a.rep, pmax = p0 + r1 / a.rep;
  const int klo = a.window > 0 ? max(0, pmin - a.window + 1) : 0;
  const int kb0 = klo & ~(kKeys - 1);
  const int nblk = (pmax - kb0) / kKeys + 1;
  // blocks [tf0, tf1) are visible in full to every row of the tile
  const int tf0 = a.window > 0 ? (max(0, pmax - a.window + 1) - kb0 + kKeys - 1) / kKeys : 0;
  const int tf1 = (pmin + 1 - kb0) / kKeys;

  const uint32_t kvbytes = static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Nk * a.Hkv * D * 2);
  const auto rk = make_rsrc(a.k, kvbytes);
  const auto rv = make_rsrc(a.v, kvbytes);
  const auto rq = make_rsrc(a.q, static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Mq * a.Hq * D * 2));

  // this lane's row 16 wave + i: q (B operand of S^T), position, first visible key
  const int r = r0 + 16 * wave + i;
  const int ri = r / a.rep;
  RowState rs;
  rs.rok = r < a.rows;
  rs.pos = rs.rok ? p0 + ri : -1;
  rs.jlo = a.window > 0 ? rs.pos - a.window + 1 : 0;
  u32x4 qa[D / 32];
  {
    const int h = g * a.rep + (r - ri * a.rep);
    const uint32_t base = static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Mq + ri) * a.Hq + h) * D + 8 * gq) * 2);
#pragma unroll
    for (int st = 0; st < D / 32; ++st) qa[st] = buf_load16(rq, rs.rok ? base + 64 * st : kOutOfRange);
  }

  // ---- pass 1: the row maximum of the scaled logits over the visible keys
  float mx = -INFINITY;
  const StageMap<D, W> sm(a, wave, lane);
  sm.stage(a, rk, b, g, kb0, k0buf, wave);
  for (int t = 0; t < nblk; t += 2) {
    max_block<D, W>(a, sm, rk, b, g, kb0 + t * kKeys, t + 1 < nblk, t >= tf0 && t < tf1, k0buf, k1buf, qa, rs, wave, lane, mx);
    if (t + 1 < nblk)
      max_block<D, W>(a, sm, rk, b, g, kb0 + (t + 1) * kKeys, t + 2 < nblk, t + 1 >= tf0 && t + 1 < tf1, k1buf, k0buf, qa, rs, wave, lane, mx);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float thr = rs.rok ? mx - a.haze : INFINITY;    // keys below are dropped
  const float mb = rs.rok ? mx * kLog2e : 0.0f;

  // ---- pass 2: O = sum exp(s - m) v over the kept keys, l = sum exp(s - m)
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float lsum = 0.0f;
  __syncthreads();                           // pass 1's last block no longer read
  sm.stage(a, rk, b, g, kb0, k0buf, wave);
  sm.stage(a, rv, b, g, kb0, v0buf, wave);
  for (int t = 0; t < nblk; t += 2) {
    sum_block<D, W>(a, sm, rk, rv, b, g, kb0 + t * kKeys, t + 1 < nblk, t >= tf0 && t < tf1, k0buf, v0buf, k1buf, v1buf, qa, rs, thr, mb,
                    wave, lane, oacc, lsum);
    if (t + 1 < nblk)
      sum_block<D, W>(a, sm, rk, rv, b, g, kb0 + (t + 1) * kKeys, t + 2 < nblk, t + 1 >= tf0 && t + 1 < tf1, k1buf, v1buf, k0buf, v0buf, qa, rs, thr,
                      mb, wave, lane, oacc, lsum);
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // ---- output: lane (n = l % 16, g) holds rows 16 wave + 4 g + v, dims 16 dt + n
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = r0 + 16 * wave + 4 * gq + v;
    const float l = __shfl(lsum, 4 * gq + v, 64);       // lanes 0 .. 15 hold rows 0 .. 15
    if (rr >= a.rows) continue;
    const int ii = rr / a.rep, h = g * a.rep + (rr - ii * a.rep);
    uint16_t *orow = a.o + ((static_cast<int64_t>(b) * a.Mq + ii) * a.Hq + h) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) orow[16 * dt + i] = f32_to_bf16(oacc[dt][v] * inv);
  }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, hipStream_t s) {
  // static LDS only (the four block buffers); tiles of 16 W rows
  constexpr int W = attn_waves(D);
  const int grid = a.B * a.Hkv * a.tiles;
  return launch_kernel(reinterpret_cast<const void *>(kvbss_attention_kernel<D, W>), dim3(grid), dim3(64 * W), 0, s,
                       a);
}

// --------------------------------------------------------------------------
// Split-key form for a few rows (Mq (Hq / Hkv) <= 16, a decode step over a
// long context): the one-launch kernel would give each (sequence, KV head)
// one workgroup.  Here each (sequence, KV head, range of kAttnChunk keys) is a
// workgroup, in two launches, because the haze threshold of a row needs the
// maximum over all ranges before any range can sum:
//   1. kvbss_logits_kernel: the scaled logits of the range (-inf where not
//      visible) into the workspace, and the range's row maxima;
//   2. kvbss_vsum_kernel: the row maxima over all ranges, then the range's
//      sum of exp(s - m) v and of exp(s - m) over the kept keys, and the last
//      workgroup of the (sequence, KV head) to arrive (an arrival counter that
//      launch 1 zeroes) sums the ranges in range order and writes o.
// Rows: lane l's row is l % 16 = (query, head) pair r of the KV head's group.
// Each wavefront takes the 32-key blocks w, w + 4, ... of the range: K comes
// straight from global memory as the A operand of S^T = K Q^T; V goes to the
// wavefront's own LDS region by buffer-to-LDS loads and is read back by the
// transposing read, as in the one-launch kernel.

template <int D>
__global__ __launch_bounds__(256) void kvbss_logits_kernel(AttnArgs a) {
  __shared__ float red[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, gq = lane >> 4;
  const int bg = static_cast<int>(blockIdx.x) / a.nchunk, c = static_cast<int>(blockIdx.x) - bg * a.nchunk;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const bool rok = i < a.rows;
  const int ri = i / a.rep;
  const int pos = rok ? a.Nk - a.Mq + ri : -1;
  const int jlo = a.window > 0 ? pos - a.window + 1 : 0;
  const uint32_t kvbytes = static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Nk * a.Hkv * D * 2);
  const auto rk = make_rsrc(a.k, kvbytes);
  const auto rq = make_rsrc(a.q, static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Mq * a.Hq * D * 2));
  u32x4 qa[D / 32];
  {
    const int h = g * a.rep + (i - ri * a.rep);
    const uint32_t base = static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Mq + ri) * a.Hq + h) * D + 8 * gq) * 2);
#pragma unroll
    for (int st = 0; st < D / 32; ++st) qa[st] = buf_load16(rq, rok ? base + 64 * st : kOutOfRange);
  }
  float *lg = a.logits + (static_cast<int64_t>(bg) * 16 + i) * a.Nk;
  float mx = -INFINITY;
  for (int t = 0; t < kAttnChunk / 128; ++t) {
    const int kb = c * kAttnChunk + 32 * (wave + 4 * t);
    if (kb >= a.Nk) break;
    u32x4 ka[2][D / 32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = kb + 16 * nt + i;
      const uint32_t base =
          static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Nk + key) * a.Hkv + g) * D + 8 * gq) * 2);
#pragma unroll
      for (int st = 0; st < D / 32; ++st) ka[nt][st] = buf_load16(rk, key < a.Nk ? base + 64 * st : kOutOfRange);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < D / 32; ++st) acc = mfma_bf16(ka[nt][st], qa[st], acc);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = kb + 16 * nt + 4 * gq + v;
        const float sv = (rok && j <= pos && j >= jlo) ? acc[v] * a.scale : -INFINITY;
        mx = fmaxf(mx, sv);
        if (j < a.Nk) lg[j] = sv;
      }
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (gq == 0) red[wave][i] = mx;
  __syncthreads();
  if (threadIdx.x < 16)
    a.cmax[(static_cast<int64_t>(bg) * a.nchunk + c) * 16 + i] =
        fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i]));
  // the arrival counter of the second launch starts at zero (this launch
  // completes before that one starts on the stream)
  if (c == 0 && threadIdx.x == 0) a.cnt[bg] = 0;
}

// One block of pass 2 of the split form for a wavefront: P from the row's
// logits sl (keys 16 nt + 4 g + v of block kb), V from the wavefront's LDS
// region vcur by transposing reads.
template <int D>
__device__ __forceinline__ void vsum_block(const AttnArgs &a, const float (&sl)[2][4], int kb, bool rok, float thr,
                                           float mb, const uint8_t *vcur, int lane, f32x4 (&oacc)[D / 16],
                                           float &lsum) {
  const int i = lane & 15, gq = lane >> 4;
  const int vj = i >> 2, vc = i & 3;
  float p[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = kb + 16 * nt + 4 * gq + v;
      const float sv = j < a.Nk ? sl[nt][v] : -INFINITY;
      p[nt][v] = (rok && !(sv < thr) && sv > -INFINITY) ? __builtin_amdgcn_exp2f(sv * kLog2e - mb) : 0.0f;
      lsum += p[nt][v];
    }
  u32x4 pa;
  pa[0] = pack_bf16x2(p[0][0], p[0][1]);
  pa[1] = pack_bf16x2(p[0][2], p[0][3]);
  pa[2] = pack_bf16x2(p[1][0], p[1][1]);
  pa[3] = pack_bf16x2(p[1][2], p[1][3]);
  const int k0 = 4 * gq + vj, k1 = 16 + 4 * gq + vj;
  const uint8_t *v0 = vcur + k0 * 2 * D + 8 * (vc & 1), *v1 = vcur + k1 * 2 * D + 8 * (vc & 1);
  const int u0 = (vc >> 1) ^ swz<D>(k0), u1 = (vc >> 1) ^ swz<D>(k1);
  u32x4 vop[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(v0 + 16 * (u0 ^ (2 * dt))));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(v1 + 16 * (u1 ^ (2 * dt))));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    vop[dt] = u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = mfma_bf16(pa, vop[dt], oacc[dt]);
  __builtin_amdgcn_s_waitcnt(0xC07F);         // lgkmcnt(0): the reads are done before the region is refilled
  __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(256, 1) void kvbss_vsum_kernel(AttnArgs a) {
  constexpr int VB = kKeys * D * 2;           // bytes of one V block
  constexpr int NB = kAttnChunk / 128;        // blocks per wavefront
  constexpr int NL = D / 16;                  // 16-byte loads per lane for one block
  // one V block per wavefront; later the wavefronts' sums
  __shared__ __align__(16) uint8_t va[4 * VB];
  __shared__ float lred[4][16];
  __shared__ int last_sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, gq = lane >> 4;
  const int bg = static_cast<int>(blockIdx.x) / a.nchunk, c = static_cast<int>(blockIdx.x) - bg * a.nchunk;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const bool rok = i < a.rows;
  const uint32_t kvbytes = static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Nk * a.Hkv * D * 2);
  const auto rv = make_rsrc(a.v, kvbytes);

  // this wavefront's blocks w, w + 4, ... of the range and the row's logits of
  // each (keys 16 nt + 4 g + v; index clamped, past the end masked at use)
  const int kbw = c * kAttnChunk + 32 * wave;
  const int nb = min(NB, max(0, (a.Nk - kbw + 127) / 128));
  const float *lg = a.logits + (static_cast<int64_t>(bg) * 16 + i) * a.Nk;
  float sl[NB][2][4];
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) sl[t][nt][v] = lg[min(kbw + 128 * t + 16 * nt + 4 * gq + v, a.Nk - 1)];

  // V block t, load u of this lane: key row (64 u + lane) / (D / 8), 16-byte
  // chunk (64 u + lane) % (D / 8); stored at the row's swizzled slot
  auto load_v = [&](int t, u32x4 (&r)[NL]) {
    const int kb = kbw + 128 * t;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int f = 64 * u + lane, row = f / (D / 8), cch = f % (D / 8);
      const int j = kb + row;
      r[u] = buf_load16(rv, j < a.Nk ? static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Nk + j) * a.Hkv + g) * D +
                                                              8 * cch) * 2)
                                     : kOutOfRange);
    }
  };
  uint8_t *wv = va + wave * VB;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float lsum = 0.0f;
  u32x4 vr[NL];
  if (nb > 0) load_v(0, vr);
  // the rows' maxima over every range: the workgroup's threads share the
  // 16 x nchunk range maxima (independent loads), then an LDS reduction
  {
    float mt = -INFINITY;
    const float *cm = a.cmax + static_cast<int64_t>(bg) * a.nchunk * 16;
    const int tid = static_cast<int>(threadIdx.x), row = tid & 15;
#pragma unroll 4
    for (int cc = tid >> 4; cc < a.nchunk; cc += 16) mt = fmaxf(mt, cm[cc * 16 + row]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (gq == 0) lred[wave][i] = mt;
  }
  __syncthreads();
  const float m = fmaxf(fmaxf(lred[0][i], lred[1][i]), fmaxf(lred[2][i], lred[3][i]));
  const float thr = m - a.haze;
  const float mb = rok ? m * kLog2e : 0.0f;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (t >= nb) break;
    // block t from registers into the wavefront's region (the previous
    // block's reads have completed: lgkmcnt(0) at the end of vsum_block)
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int f = 64 * u + lane, row = f / (D / 8), cch = f % (D / 8);
      *reinterpret_cast<u32x4 *>(wv + row * 2 * D + 16 * (cch ^ swz<D>(row))) = vr[u];
    }
    if (t + 1 < nb) load_v(t + 1, vr);        // the next block streams in under this one's work
    __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the block is in LDS
    __builtin_amdgcn_wave_barrier();
    vsum_block<D>(a, sl[t], kbw + 128 * t, rok, thr, mb, wv, lane, oacc, lsum);
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // the wavefronts' sums through LDS (va reused: [4][16][D] fp32 = 4 V blocks)
  __syncthreads();
  float *osum = reinterpret_cast<float *>(va);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v) osum[(wave * 16 + 4 * gq + v) * D + 16 * dt + i] = oacc[dt][v];
  if (gq == 0) lred[wave][i] = lsum;
  __syncthreads();
  const int64_t pbase = (static_cast<int64_t>(bg) * a.nchunk + c) * 16;
  for (int e = threadIdx.x; e < a.rows * D; e += 256) {
    const int row = e / D, d = e - row * D;
    const float sum = osum[row * D + d] + osum[(16 + row) * D + d] + osum[(32 + row) * D + d] + osum[(48 + row) * D + d];
    st_dev(a.part + (pbase + row) * D + d, sum);
  }
  if (static_cast<int>(threadIdx.x) < a.rows)
    st_dev(a.partl + pbase + threadIdx.x,
           lred[0][threadIdx.x] + lred[1][threadIdx.x] + lred[2][threadIdx.x] + lred[3][threadIdx.x]);
  drain_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    last_sh = __hip_atomic_fetch_add(a.cnt + bg, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
              static_cast<uint64_t>(a.nchunk);
  __syncthreads();
  if (!last_sh) return;
  // the last range to arrive: o = sum over ranges (in range order) / l; a
  // thread takes 4 dims of one row (16-byte loads), the device-scope loads
  // issued in batches of kBatch ranges before their first use
  constexpr int kBatch = 32;
  const int64_t rbase = static_cast<int64_t>(bg) * a.nchunk * 16;
  if (static_cast<int>(threadIdx.x) < a.rows) {
    float l = 0.0f;
    for (int c0 = 0; c0 < a.nchunk; c0 += kBatch) {
      float pv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) pv[j] = c0 + j < a.nchunk ? ld_dev(a.partl + rbase + (c0 + j) * 16 + threadIdx.x) : 0.0f;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) l += pv[j];
    }
    lred[0][threadIdx.x] = l;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.rows * (D / 4); e += 256) {
    const int row = e / (D / 4), d = 4 * (e - row * (D / 4));
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = 0; c0 < a.nchunk; c0 += kBatch) {
      u32x4 pv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        pv[j] = c0 + j < a.nchunk ? ld_dev16(a.part + (rbase + (c0 + j) * 16 + row) * D + d) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += __uint_as_float(pv[j][q]);
    }
    const int qi = row / a.rep, h = g * a.rep + (row - qi * a.rep);
    uint16_t *orow = a.o + ((static_cast<int64_t>(b) * a.Mq + qi) * a.Hq + h) * D + d;
    const float inv = 1.0f / lred[0][row];
#pragma unroll
    for (int q = 0; q < 4; ++q) orow[q] = f32_to_bf16(sum[q] * inv);
  }
}

template <int D>
hipError_t launch_split(const AttnArgs &a, hipStream_t s) {
  const int grid = a.B * a.Hkv * a.nchunk;
  hipError_t e = launch_kernel(reinterpret_cast<const void *>(kvbss_logits_kernel<D>), dim3(grid), dim3(256), 0, s, a);
  if (e != hipSuccess) return e;
  return launch_kernel(reinterpret_cast<const void *>(kvbss_vsum_kernel<D>), dim3(grid), dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_kvbss_attention(const AttnArgs &a, hipStream_t s) {
  const bool split = attn_split(a.rows, a.Nk);
  switch (a.D) {
    case 64: return split ? launch_split<64>(a, s) : launch_d<64>(a, s);
    case 128: return split ? launch_split<128>(a, s) : launch_d<128>(a, s);
    case 256: return split ? launch_split<256>(a, s) : launch_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dvssq
