/*
 * sparq24 — online 2:4 prune-and-compress, dense quantizers and the energy
 * reductions that compare them, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow Xiuyi Qin, "Is 2:4 Sparsity Still Worth It?
 * Semi-Structured Sparsity versus Quantization in LLM Inference"
 * (arXiv 2610.28947) as summarised on the paper-daily.com English page,
 * cited below as [PD §n] (n = the section number on that page).
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every call
 * ---------------------------------------------------------------------------
 * Operand.  A sparq24_tensor describes B x R vectors of length K along the
 *   GEMM reduction axis ("rows"); the hardware forms its groups of four along
 *   that axis [PD §1].  Element (b, r, k) lives at
 *   data + b*batch_stride + r*row_stride + k*k_stride   (strides in elements).
 *   Two layouts are accepted:
 *     K-contiguous: k_stride == 1 (e.g. X [tokens, hidden], W [out, in],
 *                   Q/K [heads*seq, head_dim], P [heads*q, keys]);
 *     transposed:   row_stride == 1 and k_stride >= R (e.g. V [heads, seq,
 *                   head_dim] pruned along seq: B = heads, R = head_dim,
 *                   K = seq, k_stride = head_dim), R <= 4194240 (65535
 *                   tiles of 64 rows, else SPARQ24_ERR_UNSUPPORTED).
 *                   sparq24_prune_compress reads it directly (16-bit
 *                   magnitude with R % 64 == 0 and K % 256 == 0: 8 x 8
 *                   blocks transposed in registers; otherwise an LDS-tiled
 *                   transpose); the
 *                   other calls (except sparq24_col_l2norm, which rejects it
 *                   with SPARQ24_ERR_UNSUPPORTED) first stage it as dense
 *                   K-contiguous rows in their workspace, which then needs
 *                   B*R*K elements more.
 *   K must be a multiple of 8 (two groups fill one metadata byte).
 * Outputs.  Always dense and K-contiguous, row-major over (b, r):
 *   kept values / kept codes [B][R][K/2], metadata [B][R][K/8],
 *   per-row scales [B][R], dense codes [B][R][K] (or [B][R][K/2] packed).
 * Memory.  Every array pointer is DEVICE memory owned by the caller, which
 *   must keep it alive until the stream work completes.  Inputs and outputs
 *   must not overlap.  The library allocates nothing and keeps no state
 *   between calls apart from device properties it caches on first use (the
 *   compute-unit count per device, each kernel's resident workgroups per CU);
 *   calls are safe from several host threads.
 * Alignment.  data, outputs and workspace must be 16-byte aligned, and
 *   batch_stride/row_stride (K-contiguous) or k_stride/batch_stride
 *   (transposed) times the element size must be multiples of 16 bytes
 *   whenever that dimension has more than one entry.
 * Streams.  Work is enqueued on `stream` (NULL = the default stream) and the
 *   call returns without synchronising.  A fault during execution surfaces at
 *   the caller's next synchronisation.
 * Workspace.  Calls taking (ws, ws_bytes): ws == NULL with ws_bytes != NULL
 *   is a size query: the call stores the bytes it needs in *ws_bytes,
 *   returns SPARQ24_OK and enqueues nothing.  Any other combination runs the
 *   call: if it needs workspace, ws must be non-NULL and *ws_bytes at least
 *   the queried size (else SPARQ24_ERR_WORKSPACE); if it needs none, ws and
 *   ws_bytes may both be NULL.  Workspace contents need no initialisation.
 * Errors.  Arguments are checked on the host before anything is enqueued;
 *   on any error nothing is enqueued.  No call aborts or throws.
 * Rounding.  Every fp32 step named below is one IEEE-754 single-precision
 *   operation (round to nearest even, subnormals kept).
 */
#ifndef SPARQ24_H
#define SPARQ24_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARQ24_OK = 0,
  SPARQ24_ERR_INVALID = 1,     /* null pointer, negative size, unknown enum value */
  SPARQ24_ERR_UNSUPPORTED = 2, /* dtype / format / bits / layout not offered by this call */
  SPARQ24_ERR_SHAPE = 3,       /* K % 8 (K % 32 for MXFP4, K % 16 for NVFP4), K too large, bad block size */
  SPARQ24_ERR_ALIGN = 4,       /* 16-byte alignment of a pointer or stride */
  SPARQ24_ERR_WORKSPACE = 5,   /* *ws_bytes smaller than required, or ws_bytes == NULL */
  SPARQ24_ERR_DEVICE = 6,      /* no usable HIP device */
  SPARQ24_ERR_LAUNCH = 7       /* the HIP runtime rejected a kernel launch */
} sparq24_status;

typedef enum { SPARQ24_F32 = 0, SPARQ24_BF16 = 1, SPARQ24_F16 = 2 } sparq24_dtype;

typedef struct {
  const void* data;
  int32_t dtype; /* sparq24_dtype */
  int64_t batch, rows, k;
  int64_t batch_stride, row_stride, k_stride; /* in elements */
} sparq24_tensor;

/* Pruning score [PD §2, the 2:4 side's pruners]: magnitude |x|, or Wanda
 * |w| * n_k with n_k the L2 norm of input channel k (an fp32 array of K
 * entries supplied by the caller, e.g. from sparq24_col_l2norm).  The Wanda
 * product is formed exactly (in fp64). */
typedef enum { SPARQ24_SCORE_MAGNITUDE = 0, SPARQ24_SCORE_WANDA = 1 } sparq24_score;

/* Quantization formats [PD §2-§3]:
 *  NONE  keep the storage type (the 2:4 side at 16 bits);
 *  INT   symmetric b-bit round-to-nearest-even, one scale per row,
 *        qmax = 2^(b-1)-1, s = fp32(amax/qmax), code = clamp(rne(fp32(x *
 *        fp32(qmax/amax))), -qmax, qmax); codes int8 for b <= 8, int16 above;
 *  FP8   OCP e4m3 of fp32(x * fp32(448/amax)), RNE, saturating at 448, sign
 *        copied; one fp32 scale s = fp32(amax/448) per row; uint8 codes;
 *  MXFP4 E2M1 codes with one E8M0 scale per 32 elements, 2^e with
 *        e = floor(log2 amax_blk) - 2 clamped to [-127,127];
 *  NVFP4 E2M1 codes with one e4m3 scale per 16 elements plus an fp32 tensor
 *        scale s_t = fp32(T/2688), T the tensor's absolute maximum; block
 *        code = e4m3(fp32(amax_blk * fp32(448/T))), elements are E2M1 of
 *        fp32(x * fp32(1/fp32(bval*s_t))).
 * E2M1 is RNE and saturating at 6 with the sign copied; two codes per byte,
 * element 2j in the low nibble.  A row (INT/FP8) or tensor (NVFP4) whose
 * absolute maximum is below 2^-64 gets scale 0 and zero codes. */
typedef enum {
  SPARQ24_Q_NONE = 0,
  SPARQ24_Q_INT = 1,
  SPARQ24_Q_FP8_E4M3 = 2,
  SPARQ24_Q_MXFP4 = 3,
  SPARQ24_Q_NVFP4 = 4
} sparq24_qfmt;

typedef struct {
  int32_t fmt;                 /* sparq24_qfmt */
  int32_t bits;                /* INT: 2..16; ignored otherwise */
  const float* tensor_amax_in; /* NVFP4: device pointer to T, or NULL to compute T */
} sparq24_qspec;

/* Largest K accepted by the calls that need a whole row at once
 * (prune_quantize, quantize INT/FP8, error_energy, predict_R). */
#define SPARQ24_MAX_ROW_K 32768
/* Largest number of quantizer pairs of one sparq24_predict_R call. */
#define SPARQ24_MAX_PAIRS 16

/* Online 2:4 prune-and-compress [PD §3, the fused online kernel; PD intro:
 * two of every four kept along the reduction axis].
 * In every aligned group of four along K, keep the two elements with the
 * largest score (ties keep the lower position).  values [B][R][K/2] receives
 * the kept elements in the input's storage type, in position order;
 * meta [B][R][K/8] receives per group the nibble (i0 | i1 << 2), group 2j in
 * the low nibble of byte j.  col_norm: NULL for magnitude, [K] fp32 for
 * Wanda.  Reads the operand once and writes each output once. */
sparq24_status sparq24_prune_compress(const sparq24_tensor* x, int32_t score,
                                      const float* col_norm, void* values,
                                      uint8_t* meta, hipStream_t stream);

/* Dense online quantization [PD §2: the quantized side pays its online
 * quantization; PD §3: INT8 with one scale per row, FP8, MXFP4, NVFP4].
 * INT/FP8: codes [B][R][K], scales fp32 [B][R].
 * MXFP4:   codes uint8 [B][R][K/2], scales uint8 E8M0 [B][R][K/32].
 * NVFP4:   codes uint8 [B][R][K/2], scales uint8 e4m3 [B][R][K/16], and
 *          tensor_scale_out (device, 1 fp32) receives s_t.
 * Workspace: NVFP4 without tensor_amax_in needs a few KB; others need none. */
sparq24_status sparq24_quantize(const sparq24_tensor* x, const sparq24_qspec* q,
                                void* codes, void* scales, float* tensor_scale_out,
                                void* ws, size_t* ws_bytes, hipStream_t stream);

/* Fused online prune + compress + quantize of the kept values [PD §4: the
 * 2:4 side quantizes its kept values to 2m bits; PD §5: 2:4 stacked on FP8;
 * PD §3: MXFP4 and NVFP4].  Same selection and metadata as
 * sparq24_prune_compress; the kept values of each row, in compressed order,
 * are quantized as a row of K/2 values:
 *   INT/FP8: codes [B][R][K/2] (int8, int16 above 8 bits, or e4m3 bytes) and
 *            scales fp32 [B][R], one per row from the absolute maximum of
 *            that row's kept values.
 *   MXFP4:   codes uint8 [B][R][K/4] (two E2M1 per byte, low nibble first),
 *            scales E8M0 [B][R][K/64] (one per 32 kept values); K % 64 == 0.
 *   NVFP4:   codes uint8 [B][R][K/4], scales e4m3 [B][R][K/32] (one per 16
 *            kept values), tensor_scale_out (device, 1 fp32) receives s_t;
 *            T is the largest |kept value| of the operand, or
 *            *q->tensor_amax_in.  K % 32 == 0.
 * tensor_scale_out is only read for NVFP4 (NULL otherwise).  Workspace:
 * NVFP4 without tensor_amax_in needs a few KB, a transposed operand its
 * staging copy, others none (pass ws = ws_bytes = NULL).  One read of the
 * operand (plus one for the NVFP4 tensor maximum), one write per output. */
sparq24_status sparq24_prune_quantize(const sparq24_tensor* x, int32_t score,
                                      const float* col_norm, const sparq24_qspec* q,
                                      void* codes, uint8_t* meta, void* scales,
                                      float* tensor_scale_out, void* ws, size_t* ws_bytes,
                                      hipStream_t stream);

/* Error energies of both sides [PD §4].
 * For each block of rows_per_block consecutive rows (flattened over (b, r);
 * 0 = the whole operand; the last block may be shorter), out[blk][4] fp64 =
 *   { sum x^2, sum of dropped x^2, sum over kept elements of (x - xhat)^2
 *     under kept_q, sum over all elements of (x - xhat)^2 under dense_q }.
 * kept_q: NONE, INT, FP8, MXFP4 (K % 64) or NVFP4 (K % 32; T over the kept
 * values of the whole operand), blocked over the compressed row as in
 * sparq24_prune_quantize.  dense_q: INT, FP8, MXFP4 or NVFP4 (NVFP4's T is
 * over the whole operand).  Sums are accumulated in fp64 in a fixed order,
 * so repeated calls give identical bits. */
sparq24_status sparq24_error_energy(const sparq24_tensor* x, int32_t score,
                                    const float* col_norm, const sparq24_qspec* kept_q,
                                    const sparq24_qspec* dense_q, int64_t rows_per_block,
                                    double* out, void* ws, size_t* ws_bytes,
                                    hipStream_t stream);

/* Predicted R [PD §4]: for every block and pair p (kept_q[p] vs dense_q[p]),
 * out[blk][p][5] fp64 = { E_prune, E_qkept, E_2:4, E_dense, R } with
 * E_prune = dropped energy / total, E_qkept = kept error / total,
 * E_2:4 = E_prune + E_qkept (disjoint elements, so the energies add),
 * E_dense = dense error / total and R = sqrt(E_2:4 / E_dense); IEEE fp64
 * division (0/0 = NaN, x/0 = inf).  1 <= npairs <= SPARQ24_MAX_PAIRS.
 * Equal quantizers appearing in several pairs are evaluated once. */
sparq24_status sparq24_predict_R(const sparq24_tensor* x, int32_t score,
                                 const float* col_norm, const sparq24_qspec* kept_q,
                                 const sparq24_qspec* dense_q, int32_t npairs,
                                 int64_t rows_per_block, double* out, void* ws,
                                 size_t* ws_bytes, hipStream_t stream);

/* sparq24_predict_R without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs and errors as
 * sparq24_predict_R, except that the workspace is a static device array of
 * SPARQ24_NOALLOC_SCRATCH_BYTES inside the library: each GPU it runs on holds
 * one copy until the process ends, and the call allocates nothing.  A call
 * whose workspace would exceed that size (as sparq24_predict_R's size query
 * reports it) returns SPARQ24_ERR_WORKSPACE and enqueues nothing.  Every call
 * on one GPU uses that GPU's array, so calls that overlap on one GPU (from
 * several host threads or on several streams) race; serialise them.  The
 * array's contents need no initialisation (each call writes before it reads). */
#define SPARQ24_NOALLOC_SCRATCH_BYTES (8u << 20)
sparq24_status sparq24_predict_R_noalloc(const sparq24_tensor* x, int32_t score,
                                         const float* col_norm, const sparq24_qspec* kept_q,
                                         const sparq24_qspec* dense_q, int32_t npairs,
                                         int64_t rows_per_block, double* out, hipStream_t stream);

/* Pairwise 4:8 prune-and-compress [PD §6: Blackwell's sparse FP4 splits each
 * group of eight into four adjacent pairs and keeps two].  In every aligned
 * group of eight along K the two pairs (2p, 2p+1) with the largest energy
 * fp64(a^2 + b^2) are kept, ties to the lower pair.  values [B][R][K/2]
 * receives the kept pairs in pair order; meta [B][R][K/16] receives per group
 * the nibble (p0 | p1 << 2), group 2j in the low nibble of byte j.
 * K % 16 == 0; K-contiguous operands only. */
sparq24_status sparq24_prune_compress_pairs48(const sparq24_tensor* x, void* values,
                                              uint8_t* meta, hipStream_t stream);

/* Pairwise 4:8 prune + quantize of the kept values [PD §6: with NVFP4 this is
 * Blackwell's sparse FP4 operand].  Selection and meta [B][R][K/16] as
 * sparq24_prune_compress_pairs48; codes, scales, tensor_scale_out, formats,
 * workspace and shape rules as sparq24_prune_quantize (kept values blocked
 * over the compressed row; the INT/FP8 row scale and the NVFP4 tensor
 * maximum come from the kept values, which need not hold the row's largest
 * element).  K % 16 == 0. */
sparq24_status sparq24_prune_quantize_pairs48(const sparq24_tensor* x, const sparq24_qspec* q,
                                              void* codes, uint8_t* meta, void* scales,
                                              float* tensor_scale_out, void* ws,
                                              size_t* ws_bytes, hipStream_t stream);

/* Predicted R of pairwise 4:8 against dense quantizers [PD §4, §6]: same
 * outputs and workspace protocol as sparq24_predict_R, with the pairwise 4:8
 * selection above in place of element-wise 2:4.  K % 16 == 0. */
sparq24_status sparq24_predict_R_pairs48(const sparq24_tensor* x, const sparq24_qspec* kept_q,
                                         const sparq24_qspec* dense_q, int32_t npairs,
                                         int64_t rows_per_block, double* out, void* ws,
                                         size_t* ws_bytes, hipStream_t stream);

/* Sparsity pattern selector of the rotated calls below. */
typedef enum {
  SPARQ24_PATTERN_24 = 0,      /* element-wise 2:4 */
  SPARQ24_PATTERN_PAIRS48 = 1, /* pairwise 4:8 */
  SPARQ24_PATTERN_DENSE = 2    /* no pruning (operator error only) */
} sparq24_pattern;

/* Block Hadamard rotation along K [PD §4: before low-bit quantization the
 * operand is multiplied by a rescaled +-1 orthogonal Hadamard matrix, which
 * spreads outliers over many elements].  Every aligned block of `block`
 * elements (a power of two, 8..4096, dividing K; so a whole row of up to
 * 4096 elements) becomes y = H x / sqrt(block)
 * with H the Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)).
 * Precision: the sums S = H x are fp64 butterflies, exact (so independent of
 * their order) whenever a block's values span at most 53 - log2(block) bits
 * from the largest magnitude's leading bit to the lowest set bit of any
 * element; a zero sum is +0; fp64(S * c), c the fp64 1/sqrt(block), is
 * rounded to fp32 and then to the storage type (round-to-nearest-even).
 * out [B][R][K] in x's storage type, K-contiguous.  Workspace: a transposed
 * operand's staging copy, else none.  Errors: block not a power of two in
 * range -> INVALID; K % block -> SHAPE; block > 512 with K > 8192 ->
 * UNSUPPORTED (such blocks are rotated by a whole 256-lane workgroup per
 * row, each lane holding at most four 8-element units of the row in
 * registers, so a row may span at most 256 * 4 * 8 = 8192 elements). */
sparq24_status sparq24_hadamard(const sparq24_tensor* x, int32_t block, void* out, void* ws,
                                size_t* ws_bytes, hipStream_t stream);

/* sparq24_quantize of the rotated operand, the rotation fused into the load
 * (one read of x): identical outputs to sparq24_hadamard followed by
 * sparq24_quantize.  block as sparq24_hadamard (0 is INVALID). */
sparq24_status sparq24_quantize_rot(const sparq24_tensor* x, int32_t block,
                                    const sparq24_qspec* q, void* codes, void* scales,
                                    float* tensor_scale_out, void* ws, size_t* ws_bytes,
                                    hipStream_t stream);

/* Magnitude prune (pattern 2:4 or pairwise 4:8) + quantization of the kept
 * values of the rotated operand, fused: identical outputs to sparq24_hadamard
 * followed by sparq24_prune_quantize (2:4, magnitude) or
 * sparq24_prune_quantize_pairs48. */
sparq24_status sparq24_prune_quantize_rot(const sparq24_tensor* x, int32_t block, int32_t pattern,
                                          const sparq24_qspec* q, void* codes, uint8_t* meta,
                                          void* scales, float* tensor_scale_out, void* ws,
                                          size_t* ws_bytes, hipStream_t stream);

/* Predicted R of the rotated operand ("Is 2:4 Sparsity Still Worth It?",
 * paper-daily.com English summary, §4: the pages report that a Hadamard
 * rotation raises R by about a factor of two on attention Q, K and on
 * linear-layer inputs), magnitude selection with the given pattern:
 * identical outputs to sparq24_hadamard followed by sparq24_predict_R (2:4)
 * or sparq24_predict_R_pairs48, up to the energy tolerance. */
sparq24_status sparq24_predict_R_rot(const sparq24_tensor* x, int32_t block, int32_t pattern,
                                     const sparq24_qspec* kept_q, const sparq24_qspec* dense_q,
                                     int32_t npairs, int64_t rows_per_block, double* out,
                                     void* ws, size_t* ws_bytes, hipStream_t stream);

/* One side of an operator-level comparison: the operand A as a GEMM would
 * consume it.  pattern: SPARQ24_PATTERN_DENSE (q: INT, FP8, MXFP4 or NVFP4
 * over all values, as sparq24_quantize), SPARQ24_PATTERN_24 or
 * SPARQ24_PATTERN_PAIRS48 (magnitude selection; q over the kept values as
 * sparq24_prune_quantize, or NONE to keep them in bf16). */
typedef struct {
  int32_t pattern;
  sparq24_qspec q;
} sparq24_side;

/* Operator-level output error [PD §2: accuracy is the relative error of the
 * operator output against a full-precision reference; PD §4: the energy
 * criterion predicts it].  For Y = A B^T with A [M][K] (the operand under
 * test) and B [N][K] (the unmodified second operand), both bf16 and
 * K-contiguous (batches folded into rows), out[m][0] = sum_n Y[m][n]^2 and
 * out[m][1 + s] = sum_n ((Ahat_s - A) B^T)[m][n]^2 for every side s, fp64
 * [M][1 + nsides].  The relative error energy of side s is the column sum
 * of 1 + s over the column sum of 0; the measured R of two sides is the
 * square root of the ratio of their error energies.
 * Arithmetic: Ahat - A per element is one fp32 FMA (code * scale - x), split
 * into bf16 hi + lo (within 2^-17 relative); products are bf16 MFMAs with
 * fp32 accumulation; per-row energies are fp32 over 128 output columns, then
 * summed in fp64.  K % 64 == 0; 1 <= nsides <= SPARQ24_MAX_PAIRS.
 * Workspace: M * 2K bf16 for one side's residual, (1 + nsides) * M * N/128
 * fp32 partials, NVFP4 partial maxima. */
sparq24_status sparq24_operator_error(const sparq24_tensor* a, const sparq24_tensor* b,
                                      const sparq24_side* sides, int32_t nsides, double* out,
                                      void* ws, size_t* ws_bytes, hipStream_t stream);

/* GEMM on the compressed 2:4 operand [PD §3: the 2:4 side multiplies the
 * pruned, compressed operand with a sparse GEMM]: c [M][N] fp32 (row-major)
 * = A B^T, A given as the output of sparq24_prune_compress (bf16 kept values
 * [M][K/2], metadata [M][K/8]), B a dense bf16 [N][K] K-contiguous operand.
 * gfx950's v_smfmac_f32_16x16x64_bf16 reads the layout as is: per lane 8
 * kept values of 16 logical k and their 16 metadata bits.  Products are
 * exact, sums fp32.  K % 64 == 0; pointers 16-byte aligned. */
sparq24_status sparq24_sparse_gemm(const void* values, const uint8_t* meta, int64_t m, int64_t k,
                                   const sparq24_tensor* b, float* c, hipStream_t stream);

/* The same GEMM tile on a dense bf16 A [M][K] (the comparison the pages
 * draw between a sparse GEMM and its dense rival): c [M][N] fp32 = A B^T. */
sparq24_status sparq24_dense_gemm(const sparq24_tensor* a, const sparq24_tensor* b, float* c,
                                  hipStream_t stream);

/* The dense FP8 rival's GEMM [PD §2: 2:4 with 16-bit values against dense
 * FP8 at equal nominal throughput]: c [M][N] fp32 = (scale_a[m] * scale_b[n])
 * * sum_k a[m][k] b[n][k] with a [M][K] and b [N][K] the e4m3 codes and
 * per-row scales of sparq24_quantize (FP8).  gfx950's
 * v_mfma_f32_16x16x128_f8f6f4; e4m3 products are exact in fp32, sums fp32,
 * then two fp32 scale multiplies.  K % 128 == 0. */
sparq24_status sparq24_fp8_gemm(const uint8_t* a, const float* scale_a, int64_t m,
                                const uint8_t* b, const float* scale_b, int64_t n, int64_t k,
                                float* c, hipStream_t stream);

/* Wanda's input-channel norms [PD §2]: norms[k] = fp32(sqrt(sum over all
 * (b, r) of x[b][r][k]^2)), the sum in fp64 (fixed order), the square root in
 * fp64, then rounded once.  x is an activation [tokens, channels] given with
 * rows = tokens and k = channels (K-contiguous).  Workspace: a few hundred KB. */
sparq24_status sparq24_col_l2norm(const sparq24_tensor* x, float* norms, void* ws,
                                  size_t* ws_bytes, hipStream_t stream);

/* Plain device copy of `bytes` bytes (16-byte aligned, bytes % 16 == 0): the
 * read-once/write-once bandwidth baseline the prune kernels are compared to. */
sparq24_status sparq24_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Storage bits per original element [PD §2: values, position indices and
 * scales are all charged].  Host-only arithmetic; no device needed.
 * sparse24 = 0: dense q; = 1: 2:4 with kept values in q (2 position bits per
 * kept value); = 2: pairwise 4:8 (2 bits per kept pair).  Sparse block
 * scales cover kept values, so they cost half as much per original element.
 * row_len: elements sharing one per-row scale (INT/FP8), 0 to leave scales
 * out.  value_bits:
 * width for SPARQ24_Q_NONE.  tensor_elems: NVFP4 tensor size, 0 to leave its
 * scale out.  Returns a negative value for an invalid spec. */
double sparq24_bits_per_element(const sparq24_qspec* q, int32_t sparse24, int64_t row_len,
                                int32_t value_bits, int64_t tensor_elems);

/* Static text for a status code. */
const char* sparq24_status_string(sparq24_status s);

/* Library version as "major.minor.patch". */
const char* sparq24_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARQ24_H */
