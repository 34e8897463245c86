/*
 * dvssq.h - C ABI of the DV-SSQ quantized linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 2,
 * runtime equation; Spark-X2.5-4B-Hadamard-GSQ model card, Architectural
 * Pillars 1) computes, for activations x [M][K]:
 *
 *     y = (x H) W_hat^T + ((x H) V^T) U^T
 *
 * H    block-diagonal normalized Sylvester Walsh-Hadamard matrix, blocks of
 *      `block` inputs (Spark card, Tier B equation: H_K = diag(H_256, ...);
 *      MiniCPM card, Mathematical Foundations 1: H_2048 for d = 2048).
 * W_hat the rotated weight in two tiers: INT4 codes in groups of 64 inputs with
 *      one bf16 scale per group (MiniCPM card, Mathematical Foundations 2, INT4
 *      equation), and INT8 codes with one fp32 scale per row for the 1/8 most
 *      salient rows (Spark card, Tier A).
 * U, V bf16 rank-r factors of the quantization residual, U = A = U_r sqrt(S_r),
 *      V = B = sqrt(S_r) V_r^T (MiniCPM card, Mathematical Foundations 2).
 *
 * The library only consumes packed layers; it never quantizes.  All device
 * memory (blob, x, y, workspace) belongs to the caller.  The library never
 * allocates, frees or synchronizes: every call validates its arguments on the
 * host, then enqueues kernels on the caller's HIP stream and returns.  It keeps
 * no state and may be called concurrently on different streams with different
 * workspaces.
 *
 * Packed blob (one device allocation of layout.blob_bytes; every sub-buffer at
 * a 256-byte aligned offset given by dvssq_pack_info).  Packed row order: the
 * INT4 tier rows first, then the INT8 tier rows; inside a tier, segment 0's rows
 * then segment 1's (n_seg = 2 is a fused gate+up layer, two projections of N/2
 * rows that read the same x), each in ascending original output index.
 *   idx  int32 [N]            packed row p -> original output column idx[p];
 *                             its segment is idx[p] / (N / n_seg)
 *   q4   uint8 [n_int4][K/2]  each run of 8 inputs k = 8i .. 8i+7 of a row
 *                             fills the 4 bytes 4i .. 4i+3: byte 4i+j holds the
 *                             code of input 8i+j in its low nibble and that of
 *                             input 8i+j+4 in its high nibble; nibble = q + 8
 *                             with q in [-8, 7]
 *   s4   bf16  [n_int4][K/64] scale of inputs 64g .. 64g+63
 *   q8   int8  [n_int8][K]    two's complement q in [-128, 127]
 *   s8   fp32  [n_int8]       per-row scale
 *   U    bf16  [N][r]         low-rank factor row of each packed row
 *   V    bf16  [n_seg*r][K]   segment s in rows s*r .. s*r+r-1 (rotated domain)
 * Dequantized rotated weight of packed row p: (nibble - 8) * s4 for INT4 rows,
 * q8 * s8 for INT8 rows.
 *
 * Return codes: DVSSQ_OK (0) or a negative DVSSQ_E* value; nothing aborts, no
 * exception crosses the boundary, and all argument checks happen before any HIP
 * call.
 */
#ifndef DVSSQ_H
#define DVSSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbols; the entry points below are its
   only exports. */
#pragma GCC visibility push(default)

#define DVSSQ_OK 0
#define DVSSQ_EINVAL (-1)       /* null pointer, bad shape, misalignment, M out of range */
#define DVSSQ_EUNSUPPORTED (-2) /* a valid request with no kernel (e.g. block not a power of two in [64, 2048]) */
#define DVSSQ_EHIP (-3)         /* a HIP launch reported an error */

#define DVSSQ_GROUP 64          /* INT4 group size G */
#define DVSSQ_DECODE_MAX_M 32   /* largest M accepted by dvssq_linear_decode */

/* flags */
#define DVSSQ_X_ROTATED 1u      /* x already holds x.H (bf16): skip the rotation */

typedef struct dvssq_layout {
  int32_t N;        /* output features (all segments) */
  int32_t K;        /* input features */
  int32_t r;        /* rank of the residual factors, 1..64 */
  int32_t block;    /* Hadamard block size b */
  int32_t group;    /* 64 */
  int32_t n_seg;    /* 1, or 2 for a fused gate+up layer */
  int32_t n_int8;   /* INT8-tier rows = N/8 (N/(8 n_seg) per segment) */
  int32_t n_int4;   /* INT4-tier rows = N - n_int8 */
  int32_t M_max;    /* largest M the workspace below is sized for */
  int32_t reserved;
  int64_t off_idx, off_q4, off_s4, off_q8, off_s8, off_U, off_V; /* byte offsets in the blob */
  int64_t blob_bytes;  /* size of the blob allocation, padding included */
  int64_t algo_bytes;  /* sum of the unpadded sub-buffers (the layer's own bytes) */
  int64_t ws_bytes;    /* device workspace needed by decode and prefill for M <= M_max */
} dvssq_layout;

/*
 * Describe the packed layout of a layer.  Host-only, pure; no HIP call.
 * Requires N % (8 n_seg) == 0, K % 64 == 0, K % block == 0, 1 <= r <= 64,
 * n_seg in {1, 2}, M_max >= 1.  block must be a power of two in [64, 2048]
 * (DVSSQ_EUNSUPPORTED otherwise).  out must not be null.
 */
int dvssq_pack_info(int32_t N, int32_t K, int32_t r, int32_t block, int32_t n_seg,
                    int32_t M_max, dvssq_layout *out);

/*
 * Rotate activations: xrot[m][bb*block + j] = sum_i x[m][bb*block + i] H_block[i][j],
 * H_block[i][j] = (-1)^popcount(i & j) / sqrt(block)  (Sylvester order;
 * MiniCPM card, Mathematical Foundations 1, X' = X H).
 * x, xrot: device bf16 [M][K] row-major, 16-byte aligned; xrot == x is allowed
 * (in place).  Butterflies in fp32, one bf16 rounding (nearest-even) at the end.
 * M >= 0 (M == 0 is a no-op), K % block == 0, block a power of two in [64, 2048].
 * stream: a hipStream_t (NULL = default stream).
 */
int dvssq_fwht(const void *x, void *xrot, int32_t M, int32_t K, int32_t block, void *stream);

/*
 * Decode forward (memory-bound GEMV path), 1 <= M <= min(32, L->M_max), one
 * kernel launch.  Needs K to be a multiple of max(block, 256)
 * (DVSSQ_EUNSUPPORTED otherwise).
 * L: from dvssq_pack_info.  blob: device, L->blob_bytes, 256-byte aligned.
 * x: device bf16 [M][K] (x.H when flags has DVSSQ_X_ROTATED).  y: device bf16
 * [M][N] in original column order; y must not overlap x, blob or ws.
 * ws: device workspace of L->ws_bytes, 256-byte aligned, contents need no
 * initialization; one ws must not be used by two calls in flight at once.
 * Each (row, max(block, 256) inputs) of the rotated activations is held as a
 * 15-bit integer with a power-of-two scale and multiplied exactly against the
 * integer codes (int32 products, fp32 group sums); where that kernel's plan does
 * not fit (per-wavefront load count, LDS, 32-bit offsets) a second kernel holds
 * it in f16 with the same scales against exact f16 weights, which needs the
 * INT4 scales s4 to lie in [2^-14, 63].  No overflow for finite fp32 values.
 * x and y must be 16-byte aligned.  Accumulation is fp32; y is rounded once to
 * bf16 (nearest-even).
 */
int dvssq_linear_decode(const dvssq_layout *L, const void *blob, const void *x, void *y,
                        int32_t M, void *ws, uint32_t flags, void *stream);

/*
 * Prefill forward (MFMA GEMM path), 1 <= M <= L->M_max: three to six kernel
 * launches (per-row scales, unless K == block >= 256, where the rotation finds
 * them; rotation; t and, when t is split over K-ranges, their ordered sum; the
 * GEMM and, when a GEMM of few tiles is split over K-ranges, the ordered sum of
 * their results).  Needs K <= 2^22,
 * M <= 2^22 and N r <= 2^29 (DVSSQ_EUNSUPPORTED otherwise).  Same arguments and ownership rules as
 * dvssq_linear_decode.  The rotated activations are held in f16 with one
 * power-of-two scale per row, the weights as exact f16 values (same s4 range
 * as decode), t = (x H) V^T in bf16 for the low-rank product; accumulation is
 * fp32.
 */
int dvssq_linear_prefill(const dvssq_layout *L, const void *blob, const void *x, void *y,
                         int32_t M, void *ws, uint32_t flags, void *stream);

/*
 * Dense materialization of a packed layer (MiniCPM5-2B-Hadamard-GSQ model card,
 * usage section: the quantized MLP weights materialized as plain BF16):
 *     w[idx[p]][k] = bf16( sum_j (W_hat[p] + U[p] V_seg(p))[j] H[j][k] ),
 * the layer's weight in the original input domain (H symmetric, H^T = H), so
 * that x w^T is the layer's forward up to the bf16 rounding of w.
 * w: device bf16 [N][K] row-major, original output order, 16-byte aligned,
 * disjoint from the blob; every row is written.  fp32 arithmetic, one bf16
 * rounding (nearest-even).  One kernel launch on `stream`.
 */
int dvssq_materialize(const dvssq_layout *L, const void *blob, void *w, void *stream);

/*
 * Workspace size of dvssq_mlp_decode / dvssq_mlp_prefill for the pair (gu,
 * down) and up to min(gu->M_max, down->M_max) rows, into *bytes.  Host-only.
 * DVSSQ_EINVAL if the pair does not form a gated MLP block (see
 * dvssq_mlp_decode) or bytes is null.
 */
int dvssq_mlp_ws_bytes(const dvssq_layout *gu, const dvssq_layout *down, int64_t *bytes);

/*
 * Gated MLP block, decode form (Spark-X2.5-4B GGUF page, "The model": a GELU
 * feed-forward block; ASHQ1 page, Architecture: ffn_gate, ffn_up, ffn_down):
 *
 *     y = down( gelu(gate(x)) * up(x) )
 *
 * gate and up are the two segments of the fused layer gu (segment 0 = gate,
 * output columns 0 .. I-1; segment 1 = up, I .. 2I-1), down is a one-segment
 * layer.  Requires gu->n_seg == 2, down->n_seg == 1, gu->N == 2 down->K (= 2I),
 * down->N == gu->K (DVSSQ_EINVAL otherwise), 1 <= M <= min(gu->M_max,
 * down->M_max), M <= 32, and both layers accepted by dvssq_linear_decode;
 * gu_blob and down_blob 256-byte aligned.
 * GELU is the exact v Phi(v) = v (1 + erf(v / sqrt 2)) / 2 in fp32; the tensors
 * between the projections are bf16 as in a BF16 model: the fused layer's output
 * is bf16 (as from dvssq_linear_decode), gelu(gate) * up is rounded once to bf16
 * and is the down projection's input.  Three kernel launches on `stream`: the
 * fused decode, the GELU product, the down decode.
 * x: device bf16 [M][gu->K] (x.H when flags has DVSSQ_X_ROTATED; the flag
 * concerns x only).  y: device bf16 [M][down->N]; x and y 16-byte aligned and
 * disjoint from each other, from the blobs and from ws.  ws: device,
 * dvssq_mlp_ws_bytes bytes, 256-byte aligned, no initialization needed, one
 * call in flight per ws; it holds the fused output and the intermediate.
 * Same ownership and error rules as dvssq_linear_decode.
 */
int dvssq_mlp_decode(const dvssq_layout *gu, const void *gu_blob, const dvssq_layout *down,
                     const void *down_blob, const void *x, void *y, int32_t M, void *ws,
                     uint32_t flags, void *stream);

/*
 * Gated MLP block, prefill form: the same block and arguments as
 * dvssq_mlp_decode, with both projections on the prefill path
 * (dvssq_linear_prefill) and 1 <= M <= min(gu->M_max, down->M_max) (no limit
 * of 32); the limits of dvssq_linear_prefill apply to both layers.
 */
int dvssq_mlp_prefill(const dvssq_layout *gu, const void *gu_blob, const dvssq_layout *down,
                      const void *down_blob, const void *x, void *y, int32_t M, void *ws,
                      uint32_t flags, void *stream);

/* Static text for a return code. */
const char *dvssq_status_str(int status);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* DVSSQ_H */
