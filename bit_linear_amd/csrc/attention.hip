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
// Workgroup: 4 wavefronts, 64 rows of one (sequence, KV head): the rows are
// the (query, head) pairs of the KV head's query group, query-major, so every
// row of the tile reads the same K and V.  Wavefront w owns rows 16 w .. 16 w
// + 15: their q in registers (the A operand of v_mfma_f32_16x16x32_bf16: lane
// l holds row l % 16, dims 8 (l / 16) .. + 7 of each 32-dim step), the output
// accumulators D / 16 tiles of 16 x 16 in registers.  Per block of 64 keys:
// K [64][D] is staged in LDS row-major (the B operand reads 16 bytes of a key
// row), V transposed [D][64] (the B operand of P V reads 8 keys of one dim),
// and each wavefront's P [16][64] (bf16) goes through LDS to become the A
// operand of P V.  fp32 logits and sums; P rounded to bf16 for the matrix
// cores; output bf16.
#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 64;
constexpr int kKeys = 64;            // keys per block
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttnLds {
  static constexpr int KS = D + 8;          // K row stride (bf16)
  static constexpr int VS = kKeys + 8;      // transposed V row stride (bf16)
  static constexpr int PS = kKeys + 8;      // P row stride (bf16)
  static constexpr int bytes = (kKeys * KS + D * VS + 4 * 16 * PS) * 2;
};

// Stage K block [kb, kb + 64) of KV head g into LDS (zeros past the end of
// the sequence; those keys are never visible)
template <int D>
__device__ __forceinline__ void stage_k(const AttnArgs &a, __amdgpu_buffer_rsrc_t rk, int b, int g, int kb,
                                        uint16_t *ks) {
  constexpr int CH = D / 8;                 // 16-byte chunks of a key row
  for (int c = threadIdx.x; c < kKeys * CH; c += kThreads) {
    const int row = c / CH, col = c - row * CH;
    const int j = kb + row;
    const uint32_t off =
        j < a.Nk ? static_cast<uint32_t>(((static_cast<int64_t>(b) * a.Nk + j) * a.Hkv + g) * D + 8 * col) * 2
                 : kOutOfRange;
    *reinterpret_cast<u32x4 *>(ks + row * AttnLds<D>::KS + 8 * col) = buf_load16(rk, off);
  }
}

// Stage V block transposed: vt[d][key]; each thread takes a pair of keys and
// 8 dims and writes the 8 (key, key + 1) pairs as 32-bit words
template <int D>
__device__ __forceinline__ void stage_vt(const AttnArgs &a, __amdgpu_buffer_rsrc_t rv, int b, int g, int kb,
                                         uint16_t *vt) {
  constexpr int CH = D / 8;
  for (int c = threadIdx.x; c < (kKeys / 2) * CH; c += kThreads) {
    const int jp = c % (kKeys / 2), col = c / (kKeys / 2);
    const int j = kb + 2 * jp;
    const int64_t base = ((static_cast<int64_t>(b) * a.Nk + j) * a.Hkv + g) * D + 8 * col;
    const u32x4 v0 = buf_load16(rv, j < a.Nk ? static_cast<uint32_t>(base * 2) : kOutOfRange);
    const u32x4 v1 = buf_load16(rv, j + 1 < a.Nk ? static_cast<uint32_t>((base + static_cast<int64_t>(a.Hkv) * D) * 2)
                                                 : kOutOfRange);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dims 8 col + 2 e (low halves) and 8 col + 2 e + 1 (high halves)
      const uint32_t lo = (v0[e] & 0xFFFFu) | (v1[e] << 16);
      const uint32_t hi = (v0[e] >> 16) | (v1[e] & 0xFFFF0000u);
      *reinterpret_cast<uint32_t *>(vt + (8 * col + 2 * e) * AttnLds<D>::VS + 2 * jp) = lo;
      *reinterpret_cast<uint32_t *>(vt + (8 * col + 2 * e + 1) * AttnLds<D>::VS + 2 * jp) = hi;
    }
  }
}

// logits of the wavefront's 16 rows against the 64 keys in LDS: s[nt] is the
// 16 x 16 tile of keys 16 nt .. 16 nt + 15 (lane l: rows 4 (l / 16) + v, key
// 16 nt + l % 16), unscaled
template <int D>
__device__ __forceinline__ void logits(const u32x4 (&qa)[D / 32], const uint16_t *ks, int lane, f32x4 (&s)[4]) {
  const int n = lane & 15, qd = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *kr = ks + (16 * nt + n) * AttnLds<D>::KS + 8 * qd;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) acc = mfma_bf16(qa[st], *reinterpret_cast<const u32x4 *>(kr + 32 * st), acc);
    s[nt] = acc;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void kvbss_attention_kernel(AttnArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  using LD = AttnLds<D>;
  uint16_t *ks = reinterpret_cast<uint16_t *>(smem);
  uint16_t *vt = ks + kKeys * LD::KS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, qd = lane >> 4;
  uint16_t *ps = vt + D * LD::VS + wave * 16 * LD::PS;

  // heaviest tiles (latest queries, most keys) first
  const int per_seq = a.Hkv * a.tiles;
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x - b * per_seq;
  const int g = rem / a.tiles;
  const int tile = a.tiles - 1 - (rem - g * a.tiles);
  const int r0 = tile * kRowsPerWg;
  const int r1 = min(a.rows, r0 + kRowsPerWg) - 1;       // last row of the tile
  const int p0 = a.Nk - a.Mq;                             // position of query 0
  const int pmin = p0 + r0 / a.rep, pmax = p0 + r1 / a.rep;
  const int klo = a.window > 0 ? max(0, pmin - a.window + 1) : 0;
  const int kb0 = klo & ~(kKeys - 1);

  const auto rk = make_rsrc(a.k, static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Nk * a.Hkv * D * 2));
  const auto rv = make_rsrc(a.v, static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Nk * a.Hkv * D * 2));
  const auto rq = make_rsrc(a.q, static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.Mq * a.Hq * D * 2));

  // q of row 16 wave + n (A operand); rows past the end read zeros
  u32x4 qa[D / 32];
  {
    const int r = r0 + 16 * wave + n;
    const int i = r / a.rep, h = g * a.rep + (r - i * a.rep);
    const bool ok = r < a.rows;
    const uint32_t base = ok ? static_cast<uint32_t>((((static_cast<int64_t>(b) * a.Mq + i) * a.Hq + h) * D + 8 * qd) * 2)
                             : kOutOfRange;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) qa[st] = buf_load16(rq, ok ? base + 64 * st : kOutOfRange);
  }
  // this lane's accumulator rows 16 wave + 4 qd + v: position and first visible key
  int pos[4], jlo[4];
  bool rok[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = r0 + 16 * wave + 4 * qd + v;
    rok[v] = r < a.rows;
    pos[v] = rok[v] ? p0 + r / a.rep : -1;
    jlo[v] = a.window > 0 ? pos[v] - a.window + 1 : 0;
  }

  // ---- pass 1: row maxima of the scaled logits over the visible keys
  float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  for (int kb = kb0; kb <= pmax; kb += kKeys) {
    __syncthreads();
    stage_k<D>(a, rk, b, g, kb, ks);
    __syncthreads();
    f32x4 s[4];
    logits<D>(qa, ks, lane, s);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = kb + 16 * nt + n;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (j <= pos[v] && j >= jlo[v]) mx[v] = fmaxf(mx[v], s[nt][v] * a.scale);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], o, 64));
  float thr[4], mb[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    thr[v] = mx[v] - a.haze;            // keys below are dropped
    mb[v] = rok[v] ? mx[v] * kLog2e : 0.0f;
  }

  // ---- pass 2: o = sum exp(s - m) v over the kept keys, l = sum exp(s - m)
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = kb0; kb <= pmax; kb += kKeys) {
    __syncthreads();
    stage_k<D>(a, rk, b, g, kb, ks);
    stage_vt<D>(a, rv, b, g, kb, vt);
    __syncthreads();
    f32x4 s[4];
    logits<D>(qa, ks, lane, s);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = kb + 16 * nt + n;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sv = s[nt][v] * a.scale;
        const bool keep = rok[v] && j <= pos[v] && j >= jlo[v] && !(sv < thr[v]);
        const float p = keep ? exp2f(sv * kLog2e - mb[v]) : 0.0f;
        lsum[v] += p;
        ps[(4 * qd + v) * LD::PS + 16 * nt + n] = f32_to_bf16(p);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's P is in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int st = 0; st < kKeys / 32; ++st) {
      const u32x4 pa = *reinterpret_cast<const u32x4 *>(ps + n * LD::PS + 32 * st + 8 * qd);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const u32x4 vb = *reinterpret_cast<const u32x4 *>(vt + (16 * dt + n) * LD::VS + 32 * st + 8 * qd);
        oacc[dt] = mfma_bf16(pa, vb, oacc[dt]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) lsum[v] += __shfl_xor(lsum[v], o, 64);

  // ---- output rows 16 wave + 4 qd + v, dims 16 dt + n
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (!rok[v]) continue;
    const int r = r0 + 16 * wave + 4 * qd + v;
    const int i = r / a.rep, h = g * a.rep + (r - i * a.rep);
    uint16_t *orow = a.o + ((static_cast<int64_t>(b) * a.Mq + i) * a.Hq + h) * D;
    const float inv = 1.0f / lsum[v];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) orow[16 * dt + n] = f32_to_bf16(oacc[dt][v] * inv);
  }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, hipStream_t s) {
  const size_t lds = AttnLds<D>::bytes;
  if (lds > 65536) {
    static std::atomic<uint64_t> done{0};
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void *>(kvbss_attention_kernel<D>), 160 * 1024, done);
    if (e != hipSuccess) return e;
  }
  const int grid = a.B * a.Hkv * a.tiles;
  return launch_kernel(reinterpret_cast<const void *>(kvbss_attention_kernel<D>), dim3(grid), dim3(kThreads), lds, s,
                       a);
}

}  // namespace

hipError_t launch_kvbss_attention(const AttnArgs &a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    case 256: return launch_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dvssq
