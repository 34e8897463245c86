// GPU quantizer: a bf16 weight W [N][K] -> the packed DV-SSQ layer, in the
// cards' order (Spark-X2.5-4B-Hadamard-GSQ model card, Architectural Pillars
// 1: Tier A salience and INT8 rows, Tier B rotation and INT4 groups, Tier C
// low-rank residual; MiniCPM5-2B-Hadamard-GSQ model card, Mathematical
// Foundations 1 and 2), per segment of N / n_seg rows:
//   1. salience of each row, the sum of its squared weights (ascending k, in
//      fp64), ranked descending with ties to the lower row; the top 1/8 of
//      the segment's rows form the INT8 tier;
//   2. rotation W H: per row, the Walsh-Hadamard butterflies of each block in
//      fp64, then the 1/sqrt(block) factor;
//   3. INT8 rows: s = fp32(max|w| / 127), q = clip(rint(w / s), -128, 127);
//   4. INT4 rows: per group of 64, s = bf16(max|w| / 7), q = clip(rint(w / s),
//      -8, 7) against the stored scale;
//   5. residual R = W H - W_hat and its rank-r factors by randomized subspace
//      iteration from a given Gaussian sketch (power_iters rounds of
//      orthonormalized R^T Q and R Z), a one-sided Jacobi SVD of the small
//      projection, A = U_r sqrt(S_r), B = sqrt(S_r) V_r^T, stored in bf16.
// Steps 1-4 repeat the same fp64 operations in the same order per value (no
// contraction into fused multiply-adds anywhere in this file), so codes,
// scales, the tier split and the packed order match a plain fp64 CPU
// implementation of these steps bit for bit; the factors of step 5 match it up
// to the order of fp64 sums.
#include "dvssq_internal.h"

#pragma clang fp contract(off)

namespace dvssq {

namespace {

constexpr int kQzThreads = 256;

// fp64 -> bf16, nearest with ties to even, straight from fp64 (no fp32 step):
// in the normal range the fp64 pattern is rounded to 8 significant bits by
// integer arithmetic (a carry moves into the exponent, and past the fp32
// range the conversion gives inf); below 2^-126 the value is rounded to a
// multiple of 2^-133, the bf16 subnormal spacing
__device__ inline uint16_t bf16_rne_from_double(double v) {
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = signbit(v) ? 0x8000 : 0;
  const double a = fabs(v);
  float f;
  if (a < 0x1p-126) {
    f = static_cast<float>(rint(a * 0x1p133) * 0x1p-133);
  } else {
    constexpr int kDrop = 52 - 7;     // explicit fraction bits of fp64 minus those of bf16
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(a));
    u += ((uint64_t{1} << (kDrop - 1)) - 1) + ((u >> kDrop) & 1);
    u &= ~((uint64_t{1} << kDrop) - 1);
    f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
  }
  return static_cast<uint16_t>(sign | (__float_as_uint(f) >> 16));
}

__device__ inline double bf16_to_double(uint16_t h) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(h) << 16));
}

// workgroup reductions over kQzThreads threads (LDS scratch of kQzThreads doubles)
__device__ inline double block_sum(double v, double *red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kQzThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = red[t] + red[t + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
// three sums at once (red: 3 x kQzThreads doubles)
__device__ inline void block_sum3(double &a, double &b, double &c, double *red) {
  const int t = threadIdx.x;
  red[t] = a;
  red[kQzThreads + t] = b;
  red[2 * kQzThreads + t] = c;
  __syncthreads();
  for (int s = kQzThreads / 2; s > 0; s >>= 1) {
    if (t < s) {
      red[t] = red[t] + red[t + s];
      red[kQzThreads + t] = red[kQzThreads + t] + red[kQzThreads + t + s];
      red[2 * kQzThreads + t] = red[2 * kQzThreads + t] + red[2 * kQzThreads + t + s];
    }
    __syncthreads();
  }
  a = red[0];
  b = red[kQzThreads];
  c = red[2 * kQzThreads];
  __syncthreads();
}
__device__ inline double block_max(double v, double *red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kQzThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = fmax(red[t], red[t + s]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// ---- 1. salience: one thread per row, the squares summed in ascending k
__global__ __launch_bounds__(kQzThreads) void qz_salience_kernel(const uint16_t *W, int64_t rows, int K, double *S) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kQzThreads + threadIdx.x;
  if (n >= rows) return;
  const uint16_t *w = W + n * K;
  double s = 0.0;
  for (int k = 0; k < K; k += 8) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(w + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_to_double(static_cast<uint16_t>(v[j] & 0xFFFFu));
      const double b = bf16_to_double(static_cast<uint16_t>(v[j] >> 16));
      s = s + a * a;
      s = s + b * b;
    }
  }
  S[n] = s;
}

// rank of row n: rows with a larger salience, or an equal one and a lower
// index; salient when the rank is below n8 (a stable descending sort's top n8)
__global__ __launch_bounds__(kQzThreads) void qz_rank_kernel(const double *S, int rows, int n8, int *salient) {
  __shared__ double tile[kQzThreads];
  const int n = blockIdx.x * kQzThreads + threadIdx.x;
  const double sn = n < rows ? S[n] : 0.0;
  int rank = 0;
  for (int m0 = 0; m0 < rows; m0 += kQzThreads) {
    __syncthreads();
    tile[threadIdx.x] = m0 + static_cast<int>(threadIdx.x) < rows ? S[m0 + threadIdx.x] : 0.0;
    __syncthreads();
    const int cnt = min(kQzThreads, rows - m0);
    for (int i = 0; i < cnt; ++i) {
      const double sm = tile[i];
      rank += (sm > sn || (sm == sn && m0 + i < n)) ? 1 : 0;
    }
  }
  if (n < rows) salient[n] = rank < n8 ? 1 : 0;
}

// packed position of row n of segment s: INT4 rows of the segment, then INT8
// rows, each in ascending row order; idx[pos] = the row's output index
__global__ __launch_bounds__(kQzThreads) void qz_pos_kernel(const int *salient, int rows, int seg, int n4s, int n8s,
                                                            int N4, int *pos, int32_t *idx) {
  __shared__ int tile[kQzThreads];
  const int n = blockIdx.x * kQzThreads + threadIdx.x;
  const int mine = n < rows ? salient[n] : 0;
  int before = 0;
  for (int m0 = 0; m0 < rows; m0 += kQzThreads) {
    __syncthreads();
    tile[threadIdx.x] = m0 + static_cast<int>(threadIdx.x) < rows ? salient[m0 + threadIdx.x] : -1;
    __syncthreads();
    const int cnt = min(kQzThreads, rows - m0);
    for (int i = 0; i < cnt; ++i) before += (m0 + i < n && tile[i] == mine) ? 1 : 0;
  }
  if (n >= rows) return;
  const int p = mine ? N4 + seg * n8s + before : seg * n4s + before;
  pos[n] = p;
  idx[p] = seg * rows + n;
}

struct RowArgs {
  const uint16_t *W;   // the segment's rows [rows][K]
  const int *salient, *pos;
  uint8_t *q4;
  uint16_t *s4;
  int8_t *q8;
  float *s8;
  double *R;           // residual [rows][K]
  int K, block, N4;
};

// ---- 2-4. one workgroup per row: rotate in LDS (fp64), quantize into the
// blob at the row's packed position, write the residual
__global__ __launch_bounds__(kQzThreads) void qz_rows_kernel(RowArgs a) {
  extern __shared__ __align__(16) uint8_t qsm[];
  const int K = a.K, b = a.block, t = threadIdx.x;
  const int64_t n = blockIdx.x;
  double *w = reinterpret_cast<double *>(qsm);       // [K]
  double *red = w + K;                               // [kQzThreads]
  int *qs = reinterpret_cast<int *>(red + kQzThreads);   // [K] INT4 codes
  for (int k = t; k < K; k += kQzThreads) w[k] = bf16_to_double(a.W[n * K + k]);
  __syncthreads();
  // butterflies of every block, len = 1, 2, ..., b/2: pair (j, j + len)
  for (int len = 1; len < b; len <<= 1) {
    for (int p = t; p < K / 2; p += kQzThreads) {
      const int blk = p / (b / 2), o = p - blk * (b / 2);
      const int j = blk * b + (o / len) * 2 * len + (o % len);
      const double x0 = w[j], x1 = w[j + len];
      w[j] = x0 + x1;
      w[j + len] = x0 - x1;
    }
    __syncthreads();
  }
  const double sc = 1.0 / sqrt(static_cast<double>(b));
  for (int k = t; k < K; k += kQzThreads) w[k] = w[k] * sc;
  __syncthreads();
  const int p = a.pos[n];
  double *rr = a.R + n * K;
  if (a.salient[n]) {
    // INT8 row: s = fp32(max|w| / 127), q = clip(rint(w / s), -128, 127)
    double amax = 0.0;
    for (int k = t; k < K; k += kQzThreads) amax = fmax(amax, fabs(w[k]));
    amax = block_max(amax, red);
    const float s = static_cast<float>(amax / 127.0);
    const double sd = static_cast<double>(s);
    const int64_t j = p - a.N4;
    if (t == 0) a.s8[j] = s;
    for (int k = t; k < K; k += kQzThreads) {
      double q = 0.0;
      if (s != 0.0f) q = fmin(127.0, fmax(-128.0, rint(w[k] / sd)));
      a.q8[j * K + k] = static_cast<int8_t>(q);
      rr[k] = w[k] - q * sd;
    }
  } else {
    // INT4 row: per group of 64, s = bf16(max|w| / 7), q = clip(rint(w / s), -8, 7)
    const int lane = t & 63, wave = t >> 6, KG = K / kGroup;
    for (int g = wave; g < KG; g += kQzThreads / 64) {
      const double v = w[g * kGroup + lane];
      double m = fabs(v);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
      const uint16_t sb = bf16_rne_from_double(m / 7.0);
      const double s = bf16_to_double(sb);
      if (lane == 0) a.s4[static_cast<int64_t>(p) * KG + g] = sb;
      double q = 0.0;
      if (s != 0.0) q = fmin(7.0, fmax(-8.0, rint(v / s)));
      qs[g * kGroup + lane] = static_cast<int>(q);
      rr[g * kGroup + lane] = v - q * s;
    }
    __syncthreads();
    // byte 4 i + j of a run of 8 codes: code 8 i + j (low nibble), 8 i + j + 4 (high)
    for (int e = t; e < K / 2; e += kQzThreads) {
      const int i = e >> 2, j = e & 3;
      const int lo = (qs[8 * i + j] + 8) & 0xF, hi = (qs[8 * i + j + 4] + 8) & 0xF;
      a.q4[static_cast<int64_t>(p) * (K / 2) + e] = static_cast<uint8_t>(lo | (hi << 4));
    }
  }
}

// ---- 5. randomized SVD of the residual (fp64)

// C [n][l] = A [n][k] B [k][l]; one thread per output, sum over ascending k
__global__ __launch_bounds__(kQzThreads) void qz_gemm_nn_kernel(const double *A, const double *B, double *C, int64_t n,
                                                                int k, int l) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kQzThreads + threadIdx.x;
  if (e >= n * l) return;
  const int64_t i = e / l;
  const int j = static_cast<int>(e - i * l);
  const double *a = A + i * k;
  double s = 0.0;
  for (int kk = 0; kk < k; ++kk) s = fma(a[kk], B[static_cast<int64_t>(kk) * l + j], s);
  C[e] = s;
}

// C [k][l] = A^T B with A [n][k], B [n][l]; one thread per output, sum over
// ascending n
__global__ __launch_bounds__(kQzThreads) void qz_gemm_tn_kernel(const double *A, const double *B, double *C, int64_t n,
                                                                int k, int l) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kQzThreads + threadIdx.x;
  if (e >= static_cast<int64_t>(k) * l) return;
  const int kk = static_cast<int>(e / l), j = static_cast<int>(e - static_cast<int64_t>(kk) * l);
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s = fma(A[i * k + kk], B[i * l + j], s);
  C[e] = s;
}

// Orthonormalize the l columns of Y [n][l] by modified Gram-Schmidt applied
// twice (one workgroup); a column whose norm falls to 1e-13 of its initial
// norm (or to zero) becomes zero
__global__ __launch_bounds__(kQzThreads) void qz_orth_kernel(double *Y, int64_t n, int l, double *norm0) {
  __shared__ double red[kQzThreads];
  const int t = threadIdx.x;
  for (int j = 0; j < l; ++j) {
    double s = 0.0;
    for (int64_t i = t; i < n; i += kQzThreads) s = fma(Y[i * l + j], Y[i * l + j], s);
    s = block_sum(s, red);
    if (t == 0) norm0[j] = sqrt(s);
  }
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass)
    for (int j = 0; j < l; ++j) {
      for (int p = 0; p < j; ++p) {
        double d = 0.0;
        for (int64_t i = t; i < n; i += kQzThreads) d = fma(Y[i * l + p], Y[i * l + j], d);
        d = block_sum(d, red);
        for (int64_t i = t; i < n; i += kQzThreads) Y[i * l + j] = Y[i * l + j] - d * Y[i * l + p];
        __syncthreads();
      }
      double s = 0.0;
      for (int64_t i = t; i < n; i += kQzThreads) s = fma(Y[i * l + j], Y[i * l + j], s);
      s = sqrt(block_sum(s, red));
      const bool dead = !(s > 1e-13 * norm0[j]) || s == 0.0;
      for (int64_t i = t; i < n; i += kQzThreads) Y[i * l + j] = dead ? 0.0 : Y[i * l + j] / s;
      __syncthreads();
    }
}

struct JacobiArgs {
  const double *Bt;    // [k][l] row-major
  double *G;           // working copy, column-major [l][k]
  double *J;           // [l][l] column-major (column j = right vector j)
  double *sig;         // [l]
  int *ord;            // [l]
  int k, l, max_sweeps;
  double tol;
};

// One-sided (Hestenes) Jacobi SVD of Bt [k][l] (k >= l) in one workgroup:
// cyclic pairs (p, q), p < q, rotated while |g_p . g_q| > tol sqrt(|g_p|^2
// |g_q|^2); then the column norms, their stable descending order, and for
// each column the sign that makes the largest-magnitude entry of its right
// vector positive (applied to both columns in place)
__global__ __launch_bounds__(kQzThreads) void qz_jacobi_kernel(JacobiArgs a) {
  __shared__ double red[3 * kQzThreads];
  __shared__ int rotated;
  const int t = threadIdx.x, k = a.k, l = a.l;
  for (int64_t e = t; e < static_cast<int64_t>(k) * l; e += kQzThreads) {
    const int i = static_cast<int>(e / l), j = static_cast<int>(e % l);
    a.G[static_cast<int64_t>(j) * k + i] = a.Bt[e];
  }
  for (int e = t; e < l * l; e += kQzThreads) a.J[e] = (e % l == e / l) ? 1.0 : 0.0;
  __syncthreads();
  for (int sweep = 0; sweep < a.max_sweeps; ++sweep) {
    if (t == 0) rotated = 0;
    __syncthreads();
    for (int p = 0; p < l - 1; ++p)
      for (int q = p + 1; q < l; ++q) {
        double *gp = a.G + static_cast<int64_t>(p) * k, *gq = a.G + static_cast<int64_t>(q) * k;
        double al = 0.0, be = 0.0, ga = 0.0;
        for (int i = t; i < k; i += kQzThreads) {
          al = fma(gp[i], gp[i], al);
          be = fma(gq[i], gq[i], be);
          ga = fma(gp[i], gq[i], ga);
        }
        block_sum3(al, be, ga, red);
        if (al == 0.0 || be == 0.0) continue;
        if (fabs(ga) <= a.tol * sqrt(al * be)) continue;
        if (t == 0) rotated = 1;
        const double zeta = (be - al) / (2.0 * ga);
        const double tt = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + tt * tt), s = c * tt;
        for (int i = t; i < k; i += kQzThreads) {
          const double x = gp[i], y = gq[i];
          gp[i] = c * x - s * y;
          gq[i] = s * x + c * y;
        }
        double *jp = a.J + p * l, *jq = a.J + q * l;
        for (int i = t; i < l; i += kQzThreads) {
          const double x = jp[i], y = jq[i];
          jp[i] = c * x - s * y;
          jq[i] = s * x + c * y;
        }
        __syncthreads();
      }
    __syncthreads();
    const int any = rotated;
    __syncthreads();
    if (!any) break;
  }
  // column norms
  for (int j = 0; j < l; ++j) {
    double s = 0.0;
    for (int i = t; i < k; i += kQzThreads) s = fma(a.G[static_cast<int64_t>(j) * k + i], a.G[static_cast<int64_t>(j) * k + i], s);
    s = block_sum(s, red);
    if (t == 0) a.sig[j] = sqrt(s);
  }
  __syncthreads();
  if (t == 0) {
    // stable descending order of the norms
    for (int j = 0; j < l; ++j) a.ord[j] = j;
    for (int i = 1; i < l; ++i)
      for (int j = i; j > 0 && a.sig[a.ord[j - 1]] < a.sig[a.ord[j]]; --j) {
        const int x = a.ord[j];
        a.ord[j] = a.ord[j - 1];
        a.ord[j - 1] = x;
      }
  }
  __syncthreads();
  // sign of each column from its right vector's largest-magnitude entry
  for (int j = 0; j < l; ++j) {
    if (t == 0) {
      int arg = 0;
      for (int i = 1; i < l; ++i)
        if (fabs(a.J[j * l + i]) > fabs(a.J[j * l + arg])) arg = i;
      red[0] = a.J[j * l + arg] < 0 ? -1.0 : 1.0;
    }
    __syncthreads();
    const double sg = red[0];
    const double inv = a.sig[j] > 0 ? 1.0 / a.sig[j] : 0.0;
    for (int i = t; i < k; i += kQzThreads)
      a.G[static_cast<int64_t>(j) * k + i] = a.sig[j] > 0 ? sg * a.G[static_cast<int64_t>(j) * k + i] * inv : 0.0;
    for (int i = t; i < l; i += kQzThreads) a.J[j * l + i] = sg * a.J[j * l + i];
    __syncthreads();
  }
}

struct FinishArgs {
  const double *Q;     // [n][l]
  const double *G;     // left vectors of Bt = right vectors of R, column-major [l][k], unit norm
  const double *J;     // [l][l] column-major
  const double *sig;   // [l]
  const int *ord;      // [l]
  const int *pos;      // packed row of each segment row
  uint16_t *U;         // blob: [N][r]
  uint16_t *V;         // blob: [n_seg r][K]
  double *sgn;         // [r] scratch
  int64_t n;
  int k, l, r, seg;
};

// the rank-r factors: for j < r (in descending singular value order), the
// sign making the largest-magnitude entry of the right vector positive,
// B[j] = sg sqrt(S_j) Ub[:, j], A[:, j] = sg sqrt(S_j) Q Vb[:, j]; bf16 into
// the blob (U at the rows' packed positions, V at rows seg r + j)
__global__ __launch_bounds__(kQzThreads) void qz_sign_kernel(FinishArgs a) {
  const int j = threadIdx.x;
  if (j >= a.r) return;
  const int c = a.ord[j];
  const double *u = a.G + static_cast<int64_t>(c) * a.k;
  int arg = 0;
  for (int i = 1; i < a.k; ++i)
    if (fabs(u[i]) > fabs(u[arg])) arg = i;
  a.sgn[j] = u[arg] < 0 ? -1.0 : 1.0;
}

__global__ __launch_bounds__(kQzThreads) void qz_factors_kernel(FinishArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kQzThreads + threadIdx.x;
  const int64_t nA = a.n * a.r, nB = static_cast<int64_t>(a.r) * a.k;
  if (e < nA) {
    const int64_t i = e / a.r;
    const int j = static_cast<int>(e - i * a.r);
    const int c = a.ord[j];
    double u = 0.0;
    for (int p = 0; p < a.l; ++p) u = fma(a.Q[i * a.l + p], a.J[c * a.l + p], u);
    const double v = a.sgn[j] * u * sqrt(a.sig[c]);
    a.U[static_cast<int64_t>(a.pos[i]) * a.r + j] = bf16_rne_from_double(v);
  } else if (e < nA + nB) {
    const int64_t f = e - nA;
    const int j = static_cast<int>(f / a.k), i = static_cast<int>(f - static_cast<int64_t>(j) * a.k);
    const int c = a.ord[j];
    const double v = a.sgn[j] * a.G[static_cast<int64_t>(c) * a.k + i] * sqrt(a.sig[c]);
    a.V[(static_cast<int64_t>(a.seg) * a.r + j) * a.k + i] = bf16_rne_from_double(v);
  }
}

__global__ __launch_bounds__(kQzThreads) void qz_zero_kernel(uint32_t *p, int64_t words) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * kQzThreads + threadIdx.x; e < words;
       e += static_cast<int64_t>(gridDim.x) * kQzThreads)
    p[e] = 0u;
}

int64_t blocks_for(int64_t n) { return (n + kQzThreads - 1) / kQzThreads; }

}  // namespace

// Workspace of the quantizer, per segment (reused): R [Ns][K], Q [Ns][l],
// Z and Bt [K][l], the Jacobi copy [l][K], J [l][l], norms, order, salience,
// flags, positions, signs
QuantizeWs quantize_ws_layout(const dvssq_layout &L, int l) {
  QuantizeWs w{};
  const int64_t Ns = L.N / L.n_seg, K = L.K;
  int64_t cur = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = cur;
    cur = (cur + bytes + 255) / 256 * 256;
    return o;
  };
  w.R = take(8 * Ns * K);
  w.Q = take(8 * Ns * l);
  w.Z = take(8 * K * l);
  w.Bt = take(8 * K * l);
  w.G = take(8 * K * l);
  w.J = take(8 * static_cast<int64_t>(l) * l);
  w.sig = take(8 * l);
  w.norm0 = take(8 * l);
  w.sgn = take(8 * 64);
  w.ord = take(4 * l);
  w.S = take(8 * Ns);
  w.salient = take(4 * Ns);
  w.pos = take(4 * Ns);
  w.bytes = cur;
  return w;
}

hipError_t launch_quantize(const dvssq_layout &L, const uint16_t *W, const double *omega, int l, int power_iters,
                           uint8_t *blob, uint8_t *ws, hipStream_t s) {
  const QuantizeWs w = quantize_ws_layout(L, l);
  const int Ns = L.N / L.n_seg, K = L.K, r = L.r;
  const int n8s = Ns / 8, n4s = Ns - n8s;
  double *R = reinterpret_cast<double *>(ws + w.R), *Q = reinterpret_cast<double *>(ws + w.Q);
  double *Z = reinterpret_cast<double *>(ws + w.Z), *Bt = reinterpret_cast<double *>(ws + w.Bt);
  double *G = reinterpret_cast<double *>(ws + w.G), *J = reinterpret_cast<double *>(ws + w.J);
  double *sig = reinterpret_cast<double *>(ws + w.sig), *norm0 = reinterpret_cast<double *>(ws + w.norm0);
  double *sgn = reinterpret_cast<double *>(ws + w.sgn), *S = reinterpret_cast<double *>(ws + w.S);
  int *ord = reinterpret_cast<int *>(ws + w.ord), *sal = reinterpret_cast<int *>(ws + w.salient);
  int *pos = reinterpret_cast<int *>(ws + w.pos);
  hipError_t e;
#define QZ_LAUNCH(kern, grid, lds, ...)                                                                    \
  do {                                                                                                     \
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kQzThreads), lds, s, __VA_ARGS__);  \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                   \
  } while (0)
  QZ_LAUNCH(qz_zero_kernel, 1024, 0, reinterpret_cast<uint32_t *>(blob), L.blob_bytes / 4);
  RowArgs ra{};
  ra.q4 = blob + L.off_q4;
  ra.s4 = reinterpret_cast<uint16_t *>(blob + L.off_s4);
  ra.q8 = reinterpret_cast<int8_t *>(blob + L.off_q8);
  ra.s8 = reinterpret_cast<float *>(blob + L.off_s8);
  ra.R = R;
  ra.salient = sal;
  ra.pos = pos;
  ra.K = K;
  ra.block = L.block;
  ra.N4 = static_cast<int>(L.n_int4);
  const size_t row_lds = static_cast<size_t>(K) * 8 + kQzThreads * 8 + static_cast<size_t>(K) * 4;
  if (row_lds > 65536) {
    static std::atomic<uint64_t> done{0};
    if ((e = ensure_lds_limit(reinterpret_cast<const void *>(qz_rows_kernel), 160 * 1024, done)) != hipSuccess)
      return e;
  }
  for (int seg = 0; seg < L.n_seg; ++seg) {
    const uint16_t *Ws = W + static_cast<int64_t>(seg) * Ns * K;
    QZ_LAUNCH(qz_salience_kernel, blocks_for(Ns), 0, Ws, static_cast<int64_t>(Ns), K, S);
    QZ_LAUNCH(qz_rank_kernel, blocks_for(Ns), 0, S, Ns, n8s, sal);
    QZ_LAUNCH(qz_pos_kernel, blocks_for(Ns), 0, sal, Ns, seg, n4s, n8s, static_cast<int>(L.n_int4), pos,
              reinterpret_cast<int32_t *>(blob + L.off_idx));
    ra.W = Ws;
    QZ_LAUNCH(qz_rows_kernel, Ns, row_lds, ra);
    // randomized subspace iteration on R from the segment's sketch
    const double *om = omega + static_cast<int64_t>(seg) * K * l;
    QZ_LAUNCH(qz_gemm_nn_kernel, blocks_for(static_cast<int64_t>(Ns) * l), 0, R, om, Q, static_cast<int64_t>(Ns), K, l);
    QZ_LAUNCH(qz_orth_kernel, 1, 0, Q, static_cast<int64_t>(Ns), l, norm0);
    for (int it = 0; it < power_iters; ++it) {
      QZ_LAUNCH(qz_gemm_tn_kernel, blocks_for(static_cast<int64_t>(K) * l), 0, R, Q, Z, static_cast<int64_t>(Ns), K, l);
      QZ_LAUNCH(qz_orth_kernel, 1, 0, Z, static_cast<int64_t>(K), l, norm0);
      QZ_LAUNCH(qz_gemm_nn_kernel, blocks_for(static_cast<int64_t>(Ns) * l), 0, R, Z, Q, static_cast<int64_t>(Ns), K, l);
      QZ_LAUNCH(qz_orth_kernel, 1, 0, Q, static_cast<int64_t>(Ns), l, norm0);
    }
    QZ_LAUNCH(qz_gemm_tn_kernel, blocks_for(static_cast<int64_t>(K) * l), 0, R, Q, Bt, static_cast<int64_t>(Ns), K, l);
    JacobiArgs ja{Bt, G, J, sig, ord, K, l, 80, 1e-15};
    QZ_LAUNCH(qz_jacobi_kernel, 1, 0, ja);
    FinishArgs fa{};
    fa.Q = Q;
    fa.G = G;
    fa.J = J;
    fa.sig = sig;
    fa.ord = ord;
    fa.pos = pos;
    fa.U = reinterpret_cast<uint16_t *>(blob + L.off_U);
    fa.V = reinterpret_cast<uint16_t *>(blob + L.off_V);
    fa.sgn = sgn;
    fa.n = Ns;
    fa.k = K;
    fa.l = l;
    fa.r = r;
    fa.seg = seg;
    QZ_LAUNCH(qz_sign_kernel, 1, 0, fa);
    QZ_LAUNCH(qz_factors_kernel, blocks_for(static_cast<int64_t>(Ns) * r + static_cast<int64_t>(r) * K), 0, fa);
  }
#undef QZ_LAUNCH
  return hipSuccess;
}

}  // namespace dvssq
