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
 * Beside the layer's forward, the library quantizes a bf16 weight into a
 * packed layer on the GPU (dvssq_quantize) and runs the cards' KV-BSS
 * attention (dvssq_kvbss_attention).  All device
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
/* Test only, dvssq_linear_decode: the producers of t do not publish that they
   are done, so every consumer's bounded wait for them gives up after a few
   polls; the kernel then poisons its outputs and sets the status word (below).
   Lets a test force the timeout path without making any kernel hang. */
#define DVSSQ_TEST_NO_PUBLISH 0x80000000u

/* Workspace status word: the int32 at byte offset 0 of every workspace.  A
   kernel whose bounded wait for another workgroup gave up writes NaN (bf16
   0x7FC0) into every output element it owns and stores
   DVSSQ_STATUS_WAIT_TIMEOUT there.  The library never clears it; a caller that
   wants to read it zeroes it once after allocating the workspace.  Bytes
   1 .. DVSSQ_WS_STATUS_BYTES-1 are reserved. */
#define DVSSQ_WS_STATUS_BYTES 256
#define DVSSQ_STATUS_WAIT_TIMEOUT 1

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
 * Decode forward (memory-bound GEMV path), 1 <= M <= min(32, L->M_max)
 * (DVSSQ_EUNSUPPORTED above 32), normally one kernel launch.
 * L: from dvssq_pack_info.  blob: device, L->blob_bytes, 256-byte aligned.
 * x: device bf16 [M][K] (x.H when flags has DVSSQ_X_ROTATED).  y: device bf16
 * [M][N] in original column order; y must not overlap x, blob or ws.
 * ws: device workspace of L->ws_bytes, 256-byte aligned, contents need no
 * initialization (see the status word above); one ws must not be used by two
 * calls in flight at once.
 * Each (row, max(block, 256) inputs) of the rotated activations is held as a
 * 15-bit integer with a power-of-two scale and multiplied exactly against the
 * integer codes (int32 products), each group's scale applied in fp32, for any
 * finite scales.  Where K is not a multiple of max(block, 256) or no plan of
 * the single-launch kernel fits (LDS, per-wavefront load count, 32-bit
 * offsets: large M with blocks of 1024 or 2048), the call runs the prefill
 * path instead (dvssq_linear_prefill, same arguments).
 * x and y must be 16-byte aligned.  Accumulation is fp32; y is rounded once to
 * bf16 (nearest-even).  flags: DVSSQ_X_ROTATED, DVSSQ_TEST_NO_PUBLISH.
 */
int dvssq_linear_decode(const dvssq_layout *L, const void *blob, const void *x, void *y,
                        int32_t M, void *ws, uint32_t flags, void *stream);

/*
 * Decode forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same computation, kernels and arguments as
 * dvssq_linear_decode, except that the workspace is a scratch array of
 * DVSSQ_NOALLOC_SCRATCH_BYTES that the library holds in device memory on each
 * GPU it runs on, from the first call on that GPU until the process ends; the
 * call itself allocates nothing.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or other
 * threads) race and must not be made.  Nothing in the array needs to start at
 * zero.  DVSSQ_EUNSUPPORTED when the call needs more scratch than the array
 * holds (large N with a split-K plan at large M; decode shapes that take the
 * prefill route with very large K); DVSSQ_EHIP when the array's device address
 * cannot be obtained.  A wait that gives up poisons the outputs with NaN as in
 * dvssq_linear_decode (the status word is not visible to the caller here).
 */
#define DVSSQ_NOALLOC_SCRATCH_BYTES (32ll << 20)
int dvssq_linear_decode_noalloc(const dvssq_layout *L, const void *blob, const void *x, void *y,
                                int32_t M, uint32_t flags, void *stream);

/*
 * Prefill forward (MFMA GEMM path), 1 <= M <= L->M_max: three to six kernel
 * launches (per-row scales, unless K == block >= 256, where the rotation finds
 * them; rotation; t and, when t is split over K-ranges, their ordered sum; the
 * GEMM and, when a GEMM of few tiles is split over K-ranges, the ordered sum of
 * their results).  Needs K <= 2^22,
 * M <= 2^22 and N r <= 2^29 (DVSSQ_EUNSUPPORTED otherwise).  Same arguments and ownership rules as
 * dvssq_linear_decode.  The rotated activations are held in f16 with one
 * power-of-two scale per row, the weights as exact f16 values: INT8 codes as
 * they are (the row scale applied in fp32), INT4 codes as (n - 8) s4 2^-c with
 * one power of two 2^c per row taken from the row's largest group scale and
 * applied in fp32, which is exact for every group scale within 2^-27 of the
 * row's largest (a smaller one enters with an error below 2^-35 of the row's
 * largest weight).  t = (x H) V^T is rounded to bf16 for the low-rank
 * product; accumulation is fp32.  flags: DVSSQ_X_ROTATED.
 */
int dvssq_linear_prefill(const dvssq_layout *L, const void *blob, const void *x, void *y,
                         int32_t M, void *ws, uint32_t flags, void *stream);

/*
 * Dense materialization of a packed layer (Spark-X2.5-4B-Hadamard-GSQ model
 * card, Quickstart & Inference Guide: materialize_weights() turns the quantized
 * MLP weights into plain BF16):
 *     w[idx[p]][k] = bf16( sum_j (W_hat[p] + U[p] V_seg(p))[j] H[j][k] ),
 * the layer's weight in the original input domain (H symmetric, H^T = H), so
 * that x w^T is the layer's forward up to the bf16 rounding of w.
 * w: device bf16 [N][K] row-major, original output order, 16-byte aligned,
 * disjoint from the blob; every row is written.  fp32 arithmetic, one bf16
 * rounding (nearest-even).  One kernel launch on `stream`.
 */
int dvssq_materialize(const dvssq_layout *L, const void *blob, void *w, void *stream);

/*
 * GPU quantizer: the packed layer of a bf16 weight W, per segment of N/n_seg
 * rows (Spark-X2.5-4B-Hadamard-GSQ model card, Architectural Pillars 1: Tier A
 * salience and INT8 rows, Tier B rotation and INT4 groups, Tier C low-rank
 * residual; MiniCPM5-2B-Hadamard-GSQ model card, Mathematical Foundations 1
 * and 2):
 *   salience = sum of squares of a row (fp64, ascending k), the top 1/8 of
 *   the segment's rows (stable descending order) form the INT8 tier; rotation
 *   W H per row (fp64 butterflies, then 1/sqrt(block)); INT8 rows
 *   s = fp32(max|w|/127), q = clip(rint(w/s), -128, 127); INT4 groups of 64
 *   s = bf16(max|w|/7), q = clip(rint(w/s), -8, 7) against the stored scale;
 *   residual R = W H - W_hat; rank-r factors by randomized subspace iteration
 *   from the sketch (power_iters rounds), a one-sided Jacobi SVD of the
 *   projection, U = A = U_r sqrt(S_r), V rows = sqrt(S_r) V_r^T, bf16.
 * L: from dvssq_pack_info (N, K, r, block, n_seg).  W: device bf16 [N][K],
 * 16-byte aligned.  omega: device fp64 [n_seg][K][l], the Gaussian sketch of
 * each segment, r <= l <= min(N/n_seg, K).  power_iters: 0 .. 16.
 * blob: device, L->blob_bytes, 256-byte aligned; every byte is written (the
 * padding between sub-buffers zero).  ws: device workspace of
 * dvssq_quantize_ws_bytes(L, l) bytes, 256-byte aligned, no initialization.
 * W, omega, blob and ws must not overlap.  Codes, scales, idx and the tier
 * split are those of the same fp64 steps done in this order on a CPU, bit for
 * bit; U and V agree with them up to the order of fp64 sums (within a bf16
 * unit almost everywhere).  DVSSQ_EUNSUPPORTED for K > 13482 (one row in
 * LDS).  Kernels are launched on `stream`; the call does not synchronize.
 */
int64_t dvssq_quantize_ws_bytes(const dvssq_layout *L, int32_t l);
int dvssq_quantize(const dvssq_layout *L, const void *W, const double *omega, int32_t l, int32_t power_iters,
                   void *blob, void *ws, void *stream);

/*
 * Workspace size of dvssq_mlp_decode / dvssq_mlp_prefill for the pair (gu,
 * down) and up to min(gu->M_max, down->M_max) rows, into *bytes.  Host-only.
 * DVSSQ_EINVAL if the pair does not form a gated MLP block (see
 * dvssq_mlp_decode) or bytes is null.
 */
int dvssq_mlp_ws_bytes(const dvssq_layout *gu, const dvssq_layout *down, int64_t *bytes);

/*
 * Where dvssq_mlp_decode / dvssq_mlp_prefill leave the block's intermediates
 * in their workspace: after a call on M rows, bytes off_ygu .. hold the fused
 * layer's output, bf16 [M][gu->N] (gate then up), and bytes off_h .. hold
 * gelu(gate) * up, bf16 [M][down->K], the down projection's input.  Host-only;
 * same pairing rules and errors as dvssq_mlp_ws_bytes; off_ygu and off_h must
 * not be null.
 */
int dvssq_mlp_ws_offsets(const dvssq_layout *gu, const dvssq_layout *down, int64_t *off_ygu, int64_t *off_h);

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
 * and is the down projection's input.  Two kernel launches on `stream` when
 * the down projection takes the single-launch decode kernels: the fused
 * decode, then the down decode, which forms gelu(gate) * up where it loads
 * its input (and also writes it to the workspace); otherwise three: the fused
 * decode, the GELU product, the down projection.
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

/*
 * Measurement aid, not part of the layer: one kernel that reads `bytes` bytes
 * of the device buffer buf (16-byte aligned, bytes a multiple of 16) with a
 * plain streaming pattern (contiguous 16 KB per 256-thread workgroup, 16-byte
 * loads) and computes nothing, the achievable-bandwidth reference for a decode
 * call that reads a layer of the same size.  sink: device, 4 bytes, written
 * only for a contrived buffer content (keeps the loads alive).  1 <= bytes <=
 * 2^40.  One kernel launch on `stream`.
 */
int dvssq_stream_read(const void *buf, int64_t bytes, void *sink, void *stream);

/*
 * KV-BSS attention (Spark-X2.5-4B-Hadamard-GSQ model card, section 2, KV-BSS:
 * focus factor scaling and attention haze truncation; Spark-X2.5-4B discussion
 * 14, Mathematical Formulation 1-2 and its eager attention change), causal
 * grouped-query attention as in the Spark model (Spark-X2.5-4B GGUF page, "The
 * model": 16 query heads, 4 KV heads, head_dim 256, sliding window 512 on the
 * sliding layers).  For query i of sequence b and query head h:
 *     position p = Nk - Mq + i (the queries are the last Mq of the Nk tokens),
 *     visible keys j <= p (and j > p - window when window > 0),
 *     KV head h / (Hq / Hkv),
 *     s_j = scale * (q . k_j)          (scale = tau_focus / sqrt(D), tau_focus = 1.10),
 *     m = max of s_j over the visible keys,
 *     o = sum exp(s_j - m) v_j / sum exp(s_j - m) over the visible keys with
 *         s_j >= m - haze (haze = 12.0 on the pages; INFINITY keeps every key).
 * q and o: device bf16 [B][Mq][Hq][D]; k and v: device bf16 [B][Nk][Hkv][D];
 * all 16-byte aligned; o disjoint from q, k and v.  D is 64, 128 or 256
 * (DVSSQ_EUNSUPPORTED otherwise); 1 <= Mq <= Nk; Hq a multiple of Hkv; window
 * >= 0; scale finite; haze >= 0 (not NaN); B Nk Hkv D and B Mq Hq D below 2^30
 * (DVSSQ_EUNSUPPORTED above).  Logits and sums in fp32 (the logits from bf16
 * products on the matrix cores), exp(s - m) rounded to bf16 for the product
 * with v, output rounded to bf16.  ws: device workspace of
 * dvssq_kvbss_attention_ws_bytes bytes, 256-byte aligned, disjoint from q, k,
 * v and o, no initialization needed, one call in flight per ws; may be null
 * when that size is 0 (the shape runs one kernel launch).  A shape with
 * Mq (Hq / Hkv) <= 16 query rows per KV head and more than 512 keys (a decode
 * step over a long context) runs in two launches over ranges of 512 keys,
 * with the ranges summed in a fixed order; every other shape in one launch.
 * Kernels are launched on `stream`; the call does not synchronize.
 */
typedef struct dvssq_attn_shape {
  int32_t B, Mq, Nk, Hq, Hkv, D;
  int32_t window;       /* 0: full causal attention */
  float scale;          /* logit multiplier */
  float haze;           /* keys below the row maximum minus haze are dropped */
} dvssq_attn_shape;

/* Workspace bytes of dvssq_kvbss_attention for the shape (0 when it needs
 * none), into *bytes.  Host-only; the same shape checks and errors. */
int dvssq_kvbss_attention_ws_bytes(const dvssq_attn_shape *shape, int64_t *bytes);

int dvssq_kvbss_attention(const dvssq_attn_shape *shape, const void *q, const void *k, const void *v, void *o,
                          void *ws, void *stream);

/* Static text for a return code. */
const char *dvssq_status_str(int status);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* DVSSQ_H */
