// Host side of the C ABI declared in include/dvssq.h: argument validation,
// packed-layout arithmetic and kernel dispatch.  Every check runs before the
// first HIP call, so each error path is reachable without a GPU.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <cmath>

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

// Largest M decoded by the single-launch kernel (int8 matrix cores,
// 16-wavefront consumer workgroups).
constexpr int kSmallMaxM = 32;
constexpr int kPlanesMinM = 5;   // from this M on, producers quantize x_rot once for all consumers
// Polls of a producer flag before a consumer's wait gives up: about 0.1 s at
// the sleep of one poll; under DVSSQ_TEST_NO_PUBLISH a few polls only.
constexpr int kSpinLimit = 1 << 22;
constexpr int kTestSpinLimit = 64;

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

// The single-launch decode kernel takes the call when K is a whole number of
// rotation units of max(block, 256) inputs and one of its plans fits;
// otherwise the call runs the prefill path.
static bool decode_single_launch(const dvssq_layout &L, int32_t M, SmallPlan *sp) {
  if (L.K % decode_unit(L.block) != 0) return false;
  return M <= kSmallMaxM && plan_decode_small(L, M, compute_units(), sp) && sp->S > 0;
}

// the decode kernels take a gated input (the block's h formed in their loads):
// the single-launch kernels, with the gate+up rows addressable in 32 bits
static bool decode_takes_gated(const dvssq_layout &L, int32_t M) {
  SmallPlan sp{};
  return static_cast<int64_t>(M) * L.K * 4 < (int64_t{1} << 31) && decode_single_launch(L, M, &sp);
}

static int prefill_supported(const dvssq_layout &L, int32_t M);
static int prefill_launch(const dvssq_layout *L, const WsLayout &W, const void *blob, const void *x, void *y,
                          int32_t M, void *ws, uint32_t flags, hipStream_t s);

}  // extern "C"

namespace dvssq {

int decode_check_args(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M, uint32_t flags) {
  int rc = check_layout(L);
  if (rc != DVSSQ_OK) return rc;
  if (!blob || !x || !y) return DVSSQ_EINVAL;
  if (M < 1 || M > L->M_max) return DVSSQ_EINVAL;
  if (M > DVSSQ_DECODE_MAX_M) return DVSSQ_EUNSUPPORTED;
  if (!aligned(blob, 256) || !aligned(x, 16) || !aligned(y, 16)) return DVSSQ_EINVAL;
  const size_t xb = static_cast<size_t>(M) * L->K * 2, yb = static_cast<size_t>(M) * L->N * 2;
  if (overlap(x, xb, y, yb) || overlap(y, yb, blob, L->blob_bytes)) return DVSSQ_EINVAL;
  if (flags & ~(DVSSQ_X_ROTATED | DVSSQ_TEST_NO_PUBLISH)) return DVSSQ_EINVAL;
  SmallPlan sp{};
  if (!decode_single_launch(*L, M, &sp)) return prefill_supported(*L, M);
  return DVSSQ_OK;
}

// the few-token kernel (gemv_kernel), after the checks: one launch
static int gemv_launch(const dvssq_layout &L, const WsLayout &W, const GemvPlan &gp, const void *blob, const void *x,
                       void *y, int32_t M, void *ws, uint32_t flags, hipStream_t s, bool gated, uint16_t *hout) {
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  const Blob B{static_cast<const uint8_t *>(blob), &L};
  GemvArgs g{};
  g.q4 = B.q4();
  g.s4 = B.s4();
  g.q8 = B.q8();
  g.s8 = B.s8();
  g.U = B.U();
  g.V = B.V();
  g.idx = B.idx();
  g.x = static_cast<const uint16_t *>(x);
  g.gated = gated ? 1 : 0;
  g.hout = hout;
  g.y = static_cast<uint16_t *>(y);
  g.tp = reinterpret_cast<uint64_t *>(wsb + W.d_tp);
  g.part = reinterpret_cast<float *>(wsb + W.d_part);
  g.cnt = reinterpret_cast<uint64_t *>(wsb + W.d_cntw);
  g.status = reinterpret_cast<int *>(wsb);
  const uint64_t gen = next_generation();
  g.stamp = static_cast<uint32_t>(gen ^ (gen >> 32));
  if (g.stamp == 0) g.stamp = 1;
  g.N = L.N;
  g.K = L.K;
  g.r = L.r;
  g.n_seg = L.n_seg;
  g.n4 = L.n_int4;
  g.n8 = L.n_int8;
  g.M = M;
  g.block = L.block;
  g.unit = decode_unit(L.block);
  g.nunit = L.K / g.unit;
  g.nsr = L.n_seg * L.r;
  g.nsr_pad = nsr_pad_of(L.n_seg, L.r);
  g.S = gp.S;
  g.KW = L.K / gp.S;
  g.nu_w = g.nunit / gp.S;
  g.W = gp.W;
  g.GPW = gp.GPW;
  g.lut_units = gp.lut_units;
  g.t4 = (L.n_int4 + 31) / 32;
  g.t8 = (L.n_int8 + 31) / 32;
  g.nprod = g.nunit;
  {
    // with up to two blocks per compute unit, those beyond one per unit share
    // units with the first ones: let those be INT4 consumers on both sides;
    // larger grids: the INT8 consumers and the producers first, so that none
    // of them waits for a later round
    const int grid = g.nprod + (g.t4 + g.t8) * g.S, cus = compute_units();
    g.lead4 = grid <= cus ? -1 : grid > 2 * cus ? 0 : std::min(grid - cus, g.t4 * g.S);
  }
  g.rotate = (flags & DVSSQ_X_ROTATED) ? 0 : 1;
  g.publish = (flags & DVSSQ_TEST_NO_PUBLISH) ? 0 : 1;
  g.spin_limit = (flags & DVSSQ_TEST_NO_PUBLISH) ? kTestSpinLimit : kSpinLimit;
  g.hscale = inv_sqrt_block(L.block);
  return launch_gemv(g, s) == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

int decode_dispatch(const dvssq_layout &Lr, const WsLayout &W, const void *blob, const void *x, void *y, int32_t M,
                    void *ws, uint32_t flags, hipStream_t s, int64_t *ws_need, bool dry_run, bool gated,
                    uint16_t *hout) {
  const dvssq_layout *L = &Lr;
  GemvPlan gp{};
  if (M <= kGemvMaxM && L->K % decode_unit(L->block) == 0 && plan_gemv(*L, M, compute_units(), gated, &gp)) {
    if (ws_need) *ws_need = gp.S > 1 ? W.d_part + 4 * int64_t(gp.S) * M * L->N : W.d_part;
    if (dry_run) return DVSSQ_OK;
    return gemv_launch(*L, W, gp, blob, x, y, M, ws, flags, s, gated, hout);
  }
  SmallPlan sp{};
  if (!decode_single_launch(*L, M, &sp)) {
    if (gated) return DVSSQ_EUNSUPPORTED;   // the callers form h first (decode_takes_gated)
    if (ws_need) *ws_need = W.p_end;
    if (dry_run) return DVSSQ_OK;
    return prefill_launch(L, W, blob, x, y, M, ws, flags & DVSSQ_X_ROTATED, s);
  }
  if (ws_need) *ws_need = sp.S > 1 ? W.d_part + 4 * int64_t(sp.S) * kDecodeRows * L->N : W.d_part;
  if (dry_run) return DVSSQ_OK;
  const int g4 = decode_groups(L->n_int4), g8 = decode_groups(L->n_int8);
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
  d.gated = gated ? 1 : 0;
  d.hout = hout;
  d.tp = reinterpret_cast<float *>(wsb + W.d_tp);
  d.flag = reinterpret_cast<uint64_t *>(wsb + W.d_flag);
  d.part = reinterpret_cast<float *>(wsb + W.d_part);
  d.xg1 = reinterpret_cast<int8_t *>(wsb + W.d_xq);
  d.xg2 = d.xg1 + static_cast<int64_t>(kDecodeRows) * L->K;
  d.x8g = reinterpret_cast<int *>(wsb + W.d_x8g);
  d.escg = reinterpret_cast<float *>(wsb + W.d_escg);
  d.cntw = reinterpret_cast<uint64_t *>(wsb + W.d_cntw);
  d.status = reinterpret_cast<int *>(wsb);
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
  d.nprod = small_producers(d.nunit, M);
  d.nsr = L->n_seg * L->r;
  d.nsr_pad = nsr_pad_of(L->n_seg, L->r);
  d.g4 = (g4 + sp.RT - 1) / sp.RT;
  d.g8 = (g8 + sp.RT - 1) / sp.RT;
  d.S = sp.S;
  d.RT = sp.RT;
  d.MAXG = sp.MAXG;
  d.KQ = sp.KQ;
  d.GPW = sp.GPW;
  d.planes = M >= kPlanesMinM;
  d.KW = L->K / d.S;
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
  d.rotate = (flags & DVSSQ_X_ROTATED) ? 0 : 1;
  d.publish = (flags & DVSSQ_TEST_NO_PUBLISH) ? 0 : 1;
  d.spin_limit = (flags & DVSSQ_TEST_NO_PUBLISH) ? kTestSpinLimit : kSpinLimit;
  d.hscale = inv_sqrt_block(L->block);
  const hipError_t e = launch_decode_small(d, s);
  return e == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

}  // namespace dvssq

extern "C" {

int dvssq_linear_decode(const dvssq_layout *L, const void *blob, const void *x, void *y, int32_t M,
                        void *ws, uint32_t flags, void *stream) {
  int rc = check_call(L, blob, x, y, M, ws, DVSSQ_DECODE_MAX_M);
  if (rc != DVSSQ_OK) return rc;
  if ((rc = decode_check_args(L, blob, x, y, M, flags)) != DVSSQ_OK) return rc;
  return decode_dispatch(*L, ws_layout(*L), blob, x, y, M, ws, flags, static_cast<hipStream_t>(stream), nullptr,
                         false);
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
  return prefill_launch(L, ws_layout(*L), blob, x, y, M, ws, flags, static_cast<hipStream_t>(stream));
}

// The prefill's launches, after every argument check has passed, with the
// workspace regions of W.
static int prefill_launch(const dvssq_layout *L, const WsLayout &W, const void *blob, const void *x, void *y,
                          int32_t M, void *ws, uint32_t flags, hipStream_t s) {
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  const Blob B{static_cast<const uint8_t *>(blob), L};
  const int nsp = nsr_pad_of(L->n_seg, L->r);

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
  p.s4 = B.s4();
  p.rsh = reinterpret_cast<float *>(wsb + W.p_rsh);
  p.n4 = L->n_int4;
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
  f.rsh = p.rsh;
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

// ------------------------------------------------------------------ GPU quantizer
namespace {
constexpr int kQzMaxPowerIters = 16;
// rotation row of the quantizer in LDS: K fp64 + K int32 codes + a reduction
size_t quantize_row_lds(int K) { return static_cast<size_t>(K) * 12 + 256 * 8; }
int check_quantize(const dvssq_layout *L, int32_t l) {
  const int rc = check_layout(L);
  if (rc != DVSSQ_OK) return rc;
  const int64_t Ns = L->N / L->n_seg;
  if (l < L->r || l > std::min<int64_t>(Ns, L->K)) return DVSSQ_EINVAL;
  if (quantize_row_lds(L->K) > 160 * 1024) return DVSSQ_EUNSUPPORTED;
  return DVSSQ_OK;
}
}  // namespace

int64_t dvssq_quantize_ws_bytes(const dvssq_layout *L, int32_t l) {
  if (check_quantize(L, l) != DVSSQ_OK) return -1;
  return quantize_ws_layout(*L, l).bytes;
}

int dvssq_quantize(const dvssq_layout *L, const void *W, const double *omega, int32_t l, int32_t power_iters,
                   void *blob, void *ws, void *stream) {
  const int rc = check_quantize(L, l);
  if (rc != DVSSQ_OK) return rc;
  if (!W || !omega || !blob || !ws) return DVSSQ_EINVAL;
  if (power_iters < 0 || power_iters > kQzMaxPowerIters) return DVSSQ_EINVAL;
  if (!aligned(W, 16) || !aligned(omega, 8) || !aligned(blob, 256) || !aligned(ws, 256)) return DVSSQ_EINVAL;
  const size_t wb = static_cast<size_t>(L->N) * L->K * 2, ob = static_cast<size_t>(L->n_seg) * L->K * l * 8;
  const size_t sb = static_cast<size_t>(quantize_ws_layout(*L, l).bytes);
  if (overlap(W, wb, blob, L->blob_bytes) || overlap(W, wb, ws, sb) || overlap(omega, ob, blob, L->blob_bytes) ||
      overlap(omega, ob, ws, sb) || overlap(blob, L->blob_bytes, ws, sb))
    return DVSSQ_EINVAL;
  return launch_quantize(*L, static_cast<const uint16_t *>(W), omega, l, power_iters, static_cast<uint8_t *>(blob),
                         static_cast<uint8_t *>(ws), static_cast<hipStream_t>(stream)) == hipSuccess
             ? DVSSQ_OK
             : DVSSQ_EHIP;
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

int dvssq_mlp_ws_offsets(const dvssq_layout *gu, const dvssq_layout *down, int64_t *off_ygu, int64_t *off_h) {
  if (off_ygu == nullptr || off_h == nullptr) return DVSSQ_EINVAL;
  const int rc = check_mlp(gu, down);
  if (rc != DVSSQ_OK) return rc;
  const MlpWs w = mlp_ws(*gu, *down);
  *off_ygu = w.ygu;
  *off_h = w.h;
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
  // a projection that the single-launch kernel cannot take runs the prefill path
  SmallPlan sp{};
  if (!decode_single_launch(*gu, M, &sp) && (rc = prefill_supported(*gu, M)) != DVSSQ_OK) return rc;
  if (!decode_single_launch(*down, M, &sp) && (rc = prefill_supported(*down, M)) != DVSSQ_OK) return rc;
  const MlpWs W = mlp_ws(*gu, *down);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  void *ygu = wsb + W.ygu;
  void *h = wsb + W.h;
  // every check of the two projection calls has passed above (same M, buffers
  // disjoint by construction): after the first launch only a launch error can occur
  rc = dvssq_linear_decode(gu, gu_blob, x, ygu, M, ws, flags, stream);
  if (rc != DVSSQ_OK) return rc;
  // the down projection's single-launch kernels form h = gelu(gate) * up as
  // they load their input (h also lands in the workspace); the prefill
  // fallback takes h from the separate kernel
  if (decode_takes_gated(*down, M))
    return decode_dispatch(*down, ws_layout(*down), down_blob, ygu, y, M, ws, 0, static_cast<hipStream_t>(stream),
                           nullptr, false, true, static_cast<uint16_t *>(h));
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

int dvssq_stream_read(const void *buf, int64_t bytes, void *sink, void *stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return DVSSQ_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return DVSSQ_EINVAL;
  return launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)) == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

// the attention call's shape checks (shared with its workspace query)
static int check_attn_shape(const dvssq_attn_shape *sh) {
  if (!sh) return DVSSQ_EINVAL;
  const dvssq_attn_shape S = *sh;
  if (S.B < 1 || S.Mq < 1 || S.Nk < S.Mq || S.Hq < 1 || S.Hkv < 1 || S.Hq % S.Hkv != 0 || S.window < 0)
    return DVSSQ_EINVAL;
  if (!std::isfinite(S.scale) || std::isnan(S.haze) || S.haze < 0.0f) return DVSSQ_EINVAL;
  if (S.D != 64 && S.D != 128 && S.D != 256) return DVSSQ_EUNSUPPORTED;
  const int64_t kvn = static_cast<int64_t>(S.B) * S.Nk * S.Hkv * S.D, qn = static_cast<int64_t>(S.B) * S.Mq * S.Hq * S.D;
  if (kvn >= (int64_t{1} << 30) || qn >= (int64_t{1} << 30)) return DVSSQ_EUNSUPPORTED;
  const int64_t rows = static_cast<int64_t>(S.Mq) * (S.Hq / S.Hkv);
  const int64_t tiles = (rows + 16 * attn_waves(S.D) - 1) / (16 * attn_waves(S.D));
  if (static_cast<int64_t>(S.B) * S.Hkv * tiles >= (int64_t{1} << 31)) return DVSSQ_EUNSUPPORTED;
  return DVSSQ_OK;
}

static int64_t attn_ws_need(const dvssq_attn_shape &S) {
  const int rows = S.Mq * (S.Hq / S.Hkv);
  return attn_split(rows, S.Nk) ? attn_ws_layout(S.B, S.Hkv, S.Nk, S.D).bytes : 0;
}

int dvssq_kvbss_attention_ws_bytes(const dvssq_attn_shape *sh, int64_t *bytes) {
  if (!bytes) return DVSSQ_EINVAL;
  const int rc = check_attn_shape(sh);
  if (rc != DVSSQ_OK) return rc;
  *bytes = attn_ws_need(*sh);
  return DVSSQ_OK;
}

int dvssq_kvbss_attention(const dvssq_attn_shape *sh, const void *q, const void *k, const void *v, void *o, void *ws,
                          void *stream) {
  int rc = check_attn_shape(sh);
  if (rc != DVSSQ_OK) return rc;
  if (!q || !k || !v || !o) return DVSSQ_EINVAL;
  const dvssq_attn_shape S = *sh;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DVSSQ_EINVAL;
  const int64_t kvn = static_cast<int64_t>(S.B) * S.Nk * S.Hkv * S.D, qn = static_cast<int64_t>(S.B) * S.Mq * S.Hq * S.D;
  if (overlap(o, 2 * qn, q, 2 * qn) || overlap(o, 2 * qn, k, 2 * kvn) || overlap(o, 2 * qn, v, 2 * kvn))
    return DVSSQ_EINVAL;
  const int64_t need = attn_ws_need(S);
  if (need > 0) {
    if (!ws || !aligned(ws, 256)) return DVSSQ_EINVAL;
    if (overlap(ws, need, q, 2 * qn) || overlap(ws, need, k, 2 * kvn) || overlap(ws, need, v, 2 * kvn) ||
        overlap(ws, need, o, 2 * qn))
      return DVSSQ_EINVAL;
  }
  AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.o = static_cast<uint16_t *>(o);
  a.B = S.B;
  a.Mq = S.Mq;
  a.Nk = S.Nk;
  a.Hq = S.Hq;
  a.Hkv = S.Hkv;
  a.D = S.D;
  a.window = S.window;
  a.rep = S.Hq / S.Hkv;
  a.rows = S.Mq * a.rep;
  a.tiles = (a.rows + 16 * attn_waves(a.D) - 1) / (16 * attn_waves(a.D));
  a.scale = S.scale;
  a.haze = S.haze;
  if (need > 0) {
    const AttnWs w = attn_ws_layout(S.B, S.Hkv, S.Nk, S.D);
    uint8_t *wsb = static_cast<uint8_t *>(ws);
    a.nchunk = (S.Nk + kAttnChunk - 1) / kAttnChunk;
    a.logits = reinterpret_cast<float *>(wsb + w.logits);
    a.cmax = reinterpret_cast<float *>(wsb + w.cmax);
    a.part = reinterpret_cast<float *>(wsb + w.part);
    a.partl = reinterpret_cast<float *>(wsb + w.partl);
    a.cnt = reinterpret_cast<uint64_t *>(wsb + w.cnt);
  }
  return launch_kvbss_attention(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DVSSQ_OK : DVSSQ_EHIP;
}

const char *dvssq_status_str(int status) {
  switch (status) {
    case DVSSQ_OK: return "ok";
    case DVSSQ_EINVAL: return "invalid argument";
    case DVSSQ_EUNSUPPORTED: return "unsupported configuration";
    case DVSSQ_EHIP: return "HIP launch error";
    case DVSSQ_STATUS_WAIT_TIMEOUT: return "a bounded wait gave up (outputs poisoned with NaN)";
    default: return "unknown status";
  }
}

}  // extern "C"
