// Host side of the C ABI declared in include/dvssq.h: argument validation,
// packed-layout arithmetic and kernel dispatch.  Every check runs before the
// first HIP call, so each error path is reachable without a GPU.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <chrono>

#include "dvssq_internal.h"

using namespace dvssq;

namespace {

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_shape(int32_t N, int32_t K, int32_t r, int32_t block, int32_t n_seg, int32_t M_max) {
  if (N <= 0 || K <= 0 || r < 1 || r > 64 || M_max < 1) return DVSSQ_EINVAL;
  if (n_seg != 1 && n_seg != 2) return DVSSQ_EINVAL;
  if (n_seg * r > 64) return DVSSQ_EINVAL;
  if (K % DVSSQ_GROUP != 0 || N % (8 * n_seg) != 0) return DVSSQ_EINVAL;
  if (block <= 0 || K % block != 0) return DVSSQ_EINVAL;
  if (!is_pow2(block) || block < 64 || block > 2048) return DVSSQ_EUNSUPPORTED;
  if (static_cast<int64_t>(N) * K > (int64_t(1) << 40)) return DVSSQ_EINVAL;
  return DVSSQ_OK;
}

// Re-derives the layout from its shape fields and compares: rejects a layout
// that did not come from dvssq_pack_info (or was edited).
int check_layout(const dvssq_layout *L) {
  if (L == nullptr) return DVSSQ_EINVAL;
  dvssq_layout ref;
  const int rc = dvssq_pack_info(L->N, L->K, L->r, L->block, L->n_seg, L->M_max, &ref);
  if (rc != DVSSQ_OK) return rc;
  if (memcmp(&ref, L, sizeof ref) != 0) return DVSSQ_EINVAL;
  return DVSSQ_OK;
}

int check_call(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M,
               void *ws, int32_t M_limit) {
  int rc = check_layout(L);
  if (rc != DVSSQ_OK) return rc;
  if (!blob || !x || !y || !ws) return DVSSQ_EINVAL;
  if (M < 1 || M > L->M_max) return DVSSQ_EINVAL;
  if (M > M_limit) return DVSSQ_EUNSUPPORTED;
  if (!aligned(blob, 256) || !aligned(ws, 256) || !aligned(x, 16) || !aligned(y, 16)) return DVSSQ_EINVAL;
  const size_t xb = static_cast<size_t>(M) * L->K * 2, yb = static_cast<size_t>(M) * L->N * 2;
  if (overlap(x, xb, y, yb) || overlap(y, yb, blob, L->blob_bytes) || overlap(y, yb, ws, L->ws_bytes) ||
      overlap(x, xb, ws, L->ws_bytes))
    return DVSSQ_EINVAL;
  return DVSSQ_OK;
}

struct Blob {
  const uint8_t *b;
  const dvssq_layout *L;
  const int32_t *idx() const { return reinterpret_cast<const int32_t *>(b + L->off_idx); }
  const uint8_t *q4() const { return b + L->off_q4; }
  const uint16_t *s4() const { return reinterpret_cast<const uint16_t *>(b + L->off_s4); }
  const int8_t *q8() const { return reinterpret_cast<const int8_t *>(b + L->off_q8); }
  const float *s8() const { return reinterpret_cast<const float *>(b + L->off_s8); }
  const uint16_t *U() const { return reinterpret_cast<const uint16_t *>(b + L->off_U); }
  const uint16_t *V() const { return reinterpret_cast<const uint16_t *>(b + L->off_V); }
};

// Generation stamps for the decode kernel's producer flags: a process-wide
// counter started from a clock- and address-derived 64-bit value, so a stamp
// left in a workspace by an earlier call or process is never mistaken for the
// current one.
uint64_t next_generation() {
  static std::atomic<uint64_t> counter{[] {
    uint64_t z = static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
    z ^= reinterpret_cast<uintptr_t>(&counter) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }()};
  uint64_t g;
  do g = counter.fetch_add(1, std::memory_order_relaxed); while (g == 0);
  return g;
}

// Split-K factor of the decode kernel: S equal parts of K, each a multiple of
// 128 inputs (so no 128-input span crosses a rotation unit) and at most
// decode_max_spans() spans, whose on-chip staging fits in LDS.  The smallest
// such S that gives >= 512 consumer workgroups within 80 KB of LDS (two
// workgroups per compute unit); failing that, the largest such S (LDS use
// falls as S grows).  0 when no S fits.
// Largest M decoded by the small-M kernel (int8 matrix cores, 16-wavefront
// consumer workgroups).
constexpr int kSmallMaxM = 32;
constexpr int kPlanesMinM = 5;   // from this M on, producers quantize x_rot once for all consumers

// Largest M decoded in one launch (producers and consumers together); larger
// M uses a separate rotation launch first.
constexpr int kDecodeFusedMaxM = 32;

int decode_split(int K, int groups, int M, int unit, int nsr_pad) {
  const int nspan = K / 128;
  int best = 0;
  for (int S = 1; S <= kMaxSplit && S <= nspan; ++S) {
    if (nspan % S || nspan / S > decode_max_spans()) continue;
    const size_t lds = decode_lds_bytes(M, unit, K / S, nsr_pad);
    if (lds > 160 * 1024) continue;
    if (lds <= 80 * 1024 && static_cast<int64_t>(groups) * S >= 512) return S;
    best = S;
  }
  return best;
}

float inv_sqrt_block(int block) {
  // 1/sqrt(b) rounded once to fp32: b = 2^e
  int e = 0;
  while ((1 << e) < block) ++e;
  double v = 1.0;
  for (int i = 0; i < e / 2; ++i) v *= 0.5;
  if (e % 2) v *= 0.70710678118654752440;
  return static_cast<float>(v);
}

}  // namespace

extern "C" {

int dvssq_pack_info(int32_t N, int32_t K, int32_t r, int32_t block, int32_t n_seg, int32_t M_max,
                    dvssq_layout *out) {
  if (out == nullptr) return DVSSQ_EINVAL;
  const int rc = check_shape(N, K, r, block, n_seg, M_max);
  if (rc != DVSSQ_OK) return rc;
  dvssq_layout L;
  memset(&L, 0, sizeof L);
  L.N = N;
  L.K = K;
  L.r = r;
  L.block = block;
  L.group = DVSSQ_GROUP;
  L.n_seg = n_seg;
  L.n_int8 = N / n_seg / 8 * n_seg;
  L.n_int4 = N - L.n_int8;
  L.M_max = M_max;
  const int64_t n4 = L.n_int4, n8 = L.n_int8;
  const int64_t sz[7] = {4LL * N,
                         n4 * (K / 2),
                         n4 * (K / DVSSQ_GROUP) * 2,
                         n8 * K,
                         n8 * 4,
                         2LL * N * r,
                         2LL * n_seg * r * K};
  int64_t *offs[7] = {&L.off_idx, &L.off_q4, &L.off_s4, &L.off_q8, &L.off_s8, &L.off_U, &L.off_V};
  int64_t cur = 0, algo = 0;
  for (int i = 0; i < 7; ++i) {
    *offs[i] = cur;
    cur = align256(cur + sz[i]);
    algo += sz[i];
  }
  L.blob_bytes = cur;
  L.algo_bytes = algo;
  L.ws_bytes = ws_layout(L).total;
  *out = L;
  return DVSSQ_OK;
}

int dvssq_fwht(const void *x, void *xrot, int32_t M, int32_t K, int32_t block, void *stream) {
  if (!x || !xrot || M < 0 || K <= 0) return DVSSQ_EINVAL;
  if (block <= 0 || K % block != 0) return DVSSQ_EINVAL;
  if (!is_pow2(block) || block < 64 || block > 2048) return DVSSQ_EUNSUPPORTED;
  if (!aligned(x, 16) || !aligned(xrot, 16)) return DVSSQ_EINVAL;
  if (x != xrot && overlap(x, static_cast<size_t>(M) * K * 2, xrot, static_cast<size_t>(M) * K * 2))
    return DVSSQ_EINVAL;
  if (M == 0) return DVSSQ_OK;
  PrologueArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.xr = static_cast<uint16_t *>(xrot);
  a.M = M;
  a.K = K;
  a.blocks_per_wg = 1;
  a.rotate = 1;
  a.hscale = inv_sqrt_block(block);
  const hipError_t e = launch_fwht(a, block, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

// Compute units of the current device, queried once per device (256 on MI355X).
static int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// the decode's shape conditions beyond the argument checks: K a whole number
// of rotation units, and a plan that fits
static int decode_supported(const dvssq_layout &L, int32_t M) {
  if (L.K % decode_unit(L.block) != 0) return DVSSQ_EUNSUPPORTED;
  SmallPlan sp{};
  if (M <= kSmallMaxM && plan_decode_small(L, M, compute_units(), &sp)) return sp.S > 0 ? DVSSQ_OK : DVSSQ_EUNSUPPORTED;
  const int S = decode_split(L.K, decode_groups(L.n_int4) + decode_groups(L.n_int8), M, decode_unit(L.block),
                             nsr_pad_of(L.n_seg, L.r));
  return S > 0 ? DVSSQ_OK : DVSSQ_EUNSUPPORTED;
}

int dvssq_linear_decode(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M,
                        void *ws, uint32_t flags, void *stream) {
  int rc = check_call(L, blob, x, y, M, ws, DVSSQ_DECODE_MAX_M);
  if (rc != DVSSQ_OK) return rc;
  if (flags & ~DVSSQ_X_ROTATED) return DVSSQ_EINVAL;
  if (L->K % decode_unit(L->block) != 0) return DVSSQ_EUNSUPPORTED;
  const int g4 = decode_groups(L->n_int4), g8 = decode_groups(L->n_int8);
  const int unit = decode_unit(L->block), nsp = nsr_pad_of(L->n_seg, L->r);
  SmallPlan sp{};
  const bool small = M <= kSmallMaxM && plan_decode_small(*L, M, compute_units(), &sp);
  const int S = small ? sp.S : decode_split(L->K, g4 + g8, M, unit, nsp);
  if (S == 0) return DVSSQ_EUNSUPPORTED;
  const WsLayout W = ws_layout(*L);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  const Blob B{static_cast<const uint8_t *>(blob), L};
  DecodeArgs d{};
  d.q4 = B.q4();
  d.s4 = B.s4();
  d.q8 = B.q8();
  d.s8 = B.s8();
  d.U = B.U();
  d.V = B.V();
  d.idx = B.idx();
  d.x = static_cast<const uint16_t *>(x);
  d.xq = reinterpret_cast<uint16_t *>(wsb + W.d_xq);
  d.sc = reinterpret_cast<float *>(wsb + W.d_sc);
  d.tp = reinterpret_cast<float *>(wsb + W.d_tp);
  d.flag = reinterpret_cast<uint64_t *>(wsb + W.d_flag);
  d.cnt = reinterpret_cast<int *>(wsb + W.d_cnt);
  d.part = reinterpret_cast<float *>(wsb + W.d_part);
  d.xg1 = reinterpret_cast<int8_t *>(wsb + W.d_xq);
  d.xg2 = d.xg1 + static_cast<int64_t>(kDecodeRows) * L->K;
  d.x8g = reinterpret_cast<int *>(wsb + W.d_x8g);
  d.escg = reinterpret_cast<float *>(wsb + W.d_escg);
  d.cntw = reinterpret_cast<uint64_t *>(wsb + W.d_cntw);
  d.y = static_cast<uint16_t *>(y);
  d.gen = next_generation();
  d.tag = static_cast<uint32_t>(d.gen ^ (d.gen >> 32));
  if (d.tag == 0) d.tag = 1;
  d.N = L->N;
  d.K = L->K;
  d.r = L->r;
  d.n_seg = L->n_seg;
  d.n4 = L->n_int4;
  d.n8 = L->n_int8;
  d.M = M;
  d.block = L->block;
  d.unit = decode_unit(L->block);
  d.nunit = L->K / d.unit;
  d.nprod = small ? small_producers(d.nunit, M) : decode_producers(d.nunit, M);
  d.nsr = L->n_seg * L->r;
  d.nsr_pad = nsr_pad_of(L->n_seg, L->r);
  d.g4 = small ? (g4 + sp.RT - 1) / sp.RT : g4;
  d.g8 = small ? (g8 + sp.RT - 1) / sp.RT : g8;
  d.S = S;
  d.RT = small ? sp.RT : 0;
  d.MAXG = small ? sp.MAXG : 0;
  d.KQ = small ? sp.KQ : 0;
  d.GPW = small ? sp.GPW : 0;
  d.planes = small && M >= kPlanesMinM;
  d.KW = L->K / d.S;
  if (small) {
    d.ngrp_w = d.KW / kGroup;
    d.nu_w = d.KW / d.unit;
    d.magic_s = d.S > 1 ? static_cast<uint32_t>(((uint64_t{1} << 32) + d.S - 1) / d.S) : 0u;
    d.lut_rt = d.lut_kq = d.lut_m = d.lut_u = 0;
    for (int w = 0; w < 16; ++w) {
      const uint64_t rt = static_cast<uint64_t>(std::min(w / sp.KQ, 15)), kq = static_cast<uint64_t>(w % sp.KQ);
      d.lut_rt |= rt << (4 * w);
      d.lut_kq |= kq << (4 * w);
      d.lut_m |= static_cast<uint64_t>(w % M) << (4 * w);
      d.lut_u |= static_cast<uint64_t>(w / M) << (4 * w);
    }
  }
  d.rotate = (flags & DVSSQ_X_ROTATED) ? 0 : 1;
  d.fused = M <= kDecodeFusedMaxM ? 1 : 0;
  d.hscale = inv_sqrt_block(L->block);
  const hipError_t e = small ? launch_decode_small(d, static_cast<hipStream_t>(stream))
                               : launch_decode(d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

// the prefill's own limits (32-bit offsets in the GEMM)
static int prefill_supported(const dvssq_layout &L, int32_t M) {
  if (L.K > (1 << 22) || M > (1 << 22) || static_cast<int64_t>(L.N) * L.r > (1 << 29)) return DVSSQ_EUNSUPPORTED;
  return DVSSQ_OK;
}

int dvssq_linear_prefill(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M,
                         void *ws, uint32_t flags, void *stream) {
  int rc = check_call(L, blob, x, y, M, ws, L ? L->M_max : 0);
  if (rc != DVSSQ_OK) return rc;
  if (flags & ~DVSSQ_X_ROTATED) return DVSSQ_EINVAL;
  // the GEMM addresses one workgroup's weight rows, t and U with 32-bit byte offsets
  if ((rc = prefill_supported(*L, M)) != DVSSQ_OK) return rc;
  const WsLayout W = ws_layout(*L);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  const Blob B{static_cast<const uint8_t *>(blob), L};
  const int nsp = nsr_pad_of(L->n_seg, L->r);
  hipStream_t s = static_cast<hipStream_t>(stream);

  PrologueArgs p{};
  p.x = static_cast<const uint16_t *>(x);
  p.xr = reinterpret_cast<uint16_t *>(wsb + W.p_xr);
  p.sc = reinterpret_cast<float *>(wsb + W.p_sc);
  p.V = B.V();
  p.t = reinterpret_cast<float *>(wsb + W.p_t);
  p.M = M;
  p.K = L->K;
  p.nsr = L->n_seg * L->r;
  p.nsr_pad = nsp;
  // one workgroup column per Hadamard block (the row scale comes from the whole
  // row in every column); their partial t are summed by a small kernel after
  p.tpart = reinterpret_cast<float *>(wsb + W.p_tpart);
  p.blocks_per_wg = 1;
  p.rotate = (flags & DVSSQ_X_ROTATED) ? 0 : 1;
  p.hscale = inv_sqrt_block(L->block);
  p.exp_bias = (p.rotate ? (__builtin_ctz(static_cast<unsigned>(L->block)) + 1) / 2 : 0) + 1 - 15;
  // a single Hadamard block of 256 or more: its rotation kernel sees whole rows
  p.fuse_scale = (L->K == L->block && L->block >= 256) ? 1 : 0;
  hipError_t e = launch_prologue(p, L->block, L->K / L->block, compute_units(), s);
  if (e != hipSuccess) return DVSSQ_EHIP;

  PrefillArgs f{};
  f.q4 = B.q4();
  f.s4 = B.s4();
  f.q8 = B.q8();
  f.s8 = B.s8();
  f.U = B.U();
  f.idx = B.idx();
  f.xr = p.xr;
  f.sc = p.sc;
  f.t = p.t;
  f.y = static_cast<uint16_t *>(y);
  f.N = L->N;
  f.K = L->K;
  f.r = L->r;
  f.n_seg = L->n_seg;
  f.n4 = L->n_int4;
  f.n8 = L->n_int8;
  f.M = M;
  f.nsr = p.nsr;
  f.nsr_pad = nsp;
  f.n4_tiles = (L->n_int4 + kPfTileN - 1) / kPfTileN;
  f.n8_tiles = (L->n_int8 + kPfTileN - 1) / kPfTileN;
  f.m_tiles = (M + kPfTileM - 1) / kPfTileM;
  f.ksplit = pf_ksplit(f.m_tiles * (f.n4_tiles + f.n8_tiles), L->K / kGroup, &f.kspw);
  f.part = reinterpret_cast<float *>(wsb + W.p_part);
  e = launch_prefill(f, s);
  return e == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

// ------------------------------------------------------------------ dense materialization
int dvssq_materialize(const dvssq_layout *L, const void *blob, void *w, void *stream) {
  const int rc = check_layout(L);
  if (rc != DVSSQ_OK) return rc;
  if (!blob || !w) return DVSSQ_EINVAL;
  if (!aligned(blob, 256) || !aligned(w, 16)) return DVSSQ_EINVAL;
  if (overlap(w, static_cast<size_t>(L->N) * L->K * 2, blob, L->blob_bytes)) return DVSSQ_EINVAL;
  const Blob B{static_cast<const uint8_t *>(blob), L};
  DenseArgs a{};
  a.q4 = B.q4();
  a.s4 = B.s4();
  a.q8 = B.q8();
  a.s8 = B.s8();
  a.U = B.U();
  a.V = B.V();
  a.idx = B.idx();
  a.w = static_cast<uint16_t *>(w);
  a.N = L->N;
  a.K = L->K;
  a.r = L->r;
  a.n_seg = L->n_seg;
  a.n4 = L->n_int4;
  a.hscale = inv_sqrt_block(L->block);
  return launch_materialize(a, L->block, static_cast<hipStream_t>(stream)) == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

// ------------------------------------------------------------------ gated MLP block
// workspace: [0, base) shared by the two projections (one after the other on
// the stream), then the fused gate+up output and the intermediate h, for up
// to min(gu.M_max, down.M_max) rows
struct MlpWs {
  int32_t M_cap;
  int64_t ygu, h, total;
};

static MlpWs mlp_ws(const dvssq_layout &gu, const dvssq_layout &down) {
  MlpWs w{};
  w.M_cap = std::min(gu.M_max, down.M_max);
  w.ygu = align256(std::max(gu.ws_bytes, down.ws_bytes));
  w.h = align256(w.ygu + 2 * static_cast<int64_t>(w.M_cap) * gu.N);
  w.total = align256(w.h + 2 * static_cast<int64_t>(w.M_cap) * down.K);
  return w;
}

static int check_mlp(const dvssq_layout *gu, const dvssq_layout *down) {
  if (gu == nullptr || down == nullptr) return DVSSQ_EINVAL;
  int rc = check_layout(gu);
  if (rc != DVSSQ_OK) return rc;
  rc = check_layout(down);
  if (rc != DVSSQ_OK) return rc;
  if (gu->n_seg != 2 || down->n_seg != 1 || gu->N != 2 * down->K || down->N != gu->K) return DVSSQ_EINVAL;
  return DVSSQ_OK;
}

int dvssq_mlp_ws_bytes(const dvssq_layout *gu, const dvssq_layout *down, int64_t *bytes) {
  if (bytes == nullptr) return DVSSQ_EINVAL;
  const int rc = check_mlp(gu, down);
  if (rc != DVSSQ_OK) return rc;
  *bytes = mlp_ws(*gu, *down).total;
  return DVSSQ_OK;
}

// argument checks shared by the decode and prefill forms of the block
static int check_mlp_call(const dvssq_layout *gu, const void *gu_blob, const dvssq_layout *down,
                          const void *down_blob, const void *x, void *y, int32_t M, void *ws, uint32_t flags) {
  const int rc = check_mlp(gu, down);
  if (rc != DVSSQ_OK) return rc;
  if (!gu_blob || !down_blob || !x || !y || !ws) return DVSSQ_EINVAL;
  if (flags & ~DVSSQ_X_ROTATED) return DVSSQ_EINVAL;
  if (M < 1 || M > gu->M_max || M > down->M_max) return DVSSQ_EINVAL;
  if (!aligned(ws, 256) || !aligned(y, 16) || !aligned(x, 16) || !aligned(gu_blob, 256) || !aligned(down_blob, 256))
    return DVSSQ_EINVAL;
  const MlpWs W = mlp_ws(*gu, *down);
  const size_t yb = static_cast<size_t>(M) * down->N * 2, xb = static_cast<size_t>(M) * gu->K * 2;
  if (overlap(y, yb, ws, W.total) || overlap(x, xb, ws, W.total) || overlap(x, xb, y, yb) ||
      overlap(y, yb, gu_blob, gu->blob_bytes) || overlap(y, yb, down_blob, down->blob_bytes))
    return DVSSQ_EINVAL;
  return DVSSQ_OK;
}

int dvssq_mlp_decode(const dvssq_layout *gu, const void *gu_blob, const dvssq_layout *down, const void *down_blob,
                     const void *x, void *y, int32_t M, void *ws, uint32_t flags, void *stream) {
  int rc = check_mlp_call(gu, gu_blob, down, down_blob, x, y, M, ws, flags);
  if (rc != DVSSQ_OK) return rc;
  if (M > DVSSQ_DECODE_MAX_M) return DVSSQ_EUNSUPPORTED;
  if ((rc = decode_supported(*gu, M)) != DVSSQ_OK || (rc = decode_supported(*down, M)) != DVSSQ_OK) return rc;
  const MlpWs W = mlp_ws(*gu, *down);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  void *ygu = wsb + W.ygu;
  void *h = wsb + W.h;
  // every check of the two projection calls has passed above (same M, buffers
  // disjoint by construction): after the first launch only a launch error can occur
  rc = dvssq_linear_decode(gu, gu_blob, x, ygu, M, ws, flags, stream);
  if (rc != DVSSQ_OK) return rc;
  GegluArgs g{static_cast<const uint16_t *>(ygu), static_cast<uint16_t *>(h), M, down->K};
  if (launch_geglu(g, static_cast<hipStream_t>(stream)) != hipSuccess) return DVSSQ_EHIP;
  return dvssq_linear_decode(down, down_blob, h, y, M, ws, 0, stream);
}

int dvssq_mlp_prefill(const dvssq_layout *gu, const void *gu_blob, const dvssq_layout *down, const void *down_blob,
                      const void *x, void *y, int32_t M, void *ws, uint32_t flags, void *stream) {
  int rc = check_mlp_call(gu, gu_blob, down, down_blob, x, y, M, ws, flags);
  if (rc != DVSSQ_OK) return rc;
  if ((rc = prefill_supported(*gu, M)) != DVSSQ_OK || (rc = prefill_supported(*down, M)) != DVSSQ_OK) return rc;
  const MlpWs W = mlp_ws(*gu, *down);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  void *ygu = wsb + W.ygu;
  void *h = wsb + W.h;
  rc = dvssq_linear_prefill(gu, gu_blob, x, ygu, M, ws, flags, stream);
  if (rc != DVSSQ_OK) return rc;
  GegluArgs g{static_cast<const uint16_t *>(ygu), static_cast<uint16_t *>(h), M, down->K};
  if (launch_geglu(g, static_cast<hipStream_t>(stream)) != hipSuccess) return DVSSQ_EHIP;
  return dvssq_linear_prefill(down, down_blob, h, y, M, ws, 0, stream);
}

const char *dvssq_status_str(int status) {
  switch (status) {
    case DVSSQ_OK: return "ok";
    case DVSSQ_EINVAL: return "invalid argument";
    case DVSSQ_EUNSUPPORTED: return "unsupported configuration";
    case DVSSQ_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
