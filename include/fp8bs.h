/*
 * fp8bs.h -- C ABI of the block-scaled FP8 linear-layer library for AMD MI355X (gfx950).
 *
 * The operations are the FP8 linear-layer path described in two public pages:
 *  [P1] "Infraestructura de Entrenamiento FP8: Precisión Numérica de Nueva Generación"
 *       (introl.com blog): section "El panorama de la precisión numérica" (E4M3: 4 exponent /
 *       3 mantissa bits, range +-448; E5M2: 5 / 2 bits, wider range, used for gradients),
 *       section "Transformer Engine: la base de software" (delayed scaling with margin 0, an
 *       amax history of 16 reduced with "max", HYBRID = E4M3 forward / E5M2 backward),
 *       section "Estrategias de escalado y estabilidad" (per-tensor, block and delayed scaling).
 *  [P3] "NVIDIA NeMo RL logra una aceleración del 48% con entrenamiento de precisión FP8 de
 *       extremo a extremo" (hotbookzone.com): section "El avance técnico" (E4M3 block
 *       quantization, 128x128 tiles for weights and 1x128 blocks for activations; linear layers
 *       run FP8 math, the rest stays BF16), section "Ganancias de rendimiento en el mundo real"
 *       (quantization-kernel overhead; per-step scale recalibration; MoE), section "Por qué
 *       esto es importante para la economía de la IA" (power-of-2 scale factors).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller (for example PyTorch tensors).
 *    The library never allocates, frees or synchronizes; work is enqueued on `stream`
 *    (a hipStream_t; NULL means the default stream) and completes asynchronously.
 *  - Matrices are row-major; `ld*` arguments are row pitches in ELEMENTS.
 *  - Codes are one byte per element in the OCP E4M3 (bias 7, no infinities, NaN = S.1111.111,
 *    max 448) or E5M2 (bias 15, IEEE-like, max 57344) layout.
 *  - Every scale array holds DEQUANTIZATION factors: value = decode(code) * scale_inv.
 *    Scale layouts:
 *      1x128 blocks of a [R, C] matrix ....... float[ceil(C/128)][R]  (column block major)
 *      128x128 tiles of a [R, C] matrix ...... float[ceil(R/128)][ceil(C/128)]
 *      per tensor ............................. float[1]
 *      microscaling (32-element row blocks) ... E8M0 bytes [ceil(C/128)][R][4] (byte i of a word:
 *                                               columns 128 c + 32 i .. + 31; 2^(byte - 127))
 *  - Quantization: for each block, amax = max |x|; s = fl32(FMAX / amax) (IEEE division);
 *    amax == 0 or non-finite -> s = 1; s == +inf -> FLT_MAX; power-of-2 mode rounds s down to
 *    2^floor(log2 s); each code = round-to-nearest-even of fl32(x * s), saturating at +-FMAX
 *    (infinities included), NaN -> 0x7F with the input's sign; scale_inv = fl32(1 / s).
 *    Edge blocks are clipped to the tensor.
 *  - Return value: FP8BS_OK (0) or a negative status.  Arguments are validated on the host
 *    before anything is enqueued; on error nothing is launched.  A fault inside a kernel
 *    surfaces at the caller's next synchronization, as for any HIP launch.
 *  - Entry points are reentrant: the library keeps no state between calls.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- enums and status codes */
typedef enum { FP8BS_E4M3 = 0, FP8BS_E5M2 = 1 } fp8bs_format;

typedef enum {
  FP8BS_BLOCK_1x128 = 0,   /* one row by 128 consecutive columns of the stored matrix */
  FP8BS_BLOCK_128x128 = 1, /* 128x128 tile of the stored matrix */
  FP8BS_PER_TENSOR = 2     /* one scale for the whole tensor */
} fp8bs_granularity;

typedef enum { FP8BS_SCALE_FP32 = 0, FP8BS_SCALE_POW2 = 1 } fp8bs_scale_mode;

typedef enum {
  FP8BS_FPROP = 0, /* C[M,N] = A[M,K] . B[N,K]^T   (A = X, B = W: forward)              */
  FP8BS_DGRAD = 1, /* C[M,N] = A[M,K] . B[K,N]     (A = dY, B = W, K = out-features)     */
  FP8BS_WGRAD = 2  /* C[M,N] = A[K,M]^T . B[K,N]   (A = dY, B = X, K = tokens; C = dW)    */
} fp8bs_layout;

/* Output-tile configuration of the GEMM kernels (the *_tiled entry points).  FP8BS_TILE_AUTO
 * is the library's choice from the problem shape, which the untiled entry points always make;
 * the others force one configuration (for tuning and for testing every configuration). */
typedef enum {
  FP8BS_TILE_AUTO = 0,
  FP8BS_TILE_256x128_W4 = 1, /* 256 x 128 output tile, 4 waves, 3 LDS stages */
  FP8BS_TILE_256x128_W8 = 2, /* 256 x 128, 8 waves, 3 stages */
  FP8BS_TILE_256x256_W8 = 3, /* 256 x 256, 8 waves, 2 stages */
  FP8BS_TILE_128x128_W4 = 4  /* 128 x 128, 4 waves, 3 stages */
} fp8bs_tile;

enum {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL = -1,        /* a required pointer is NULL */
  FP8BS_ERR_SHAPE = -2,       /* negative size, pitch smaller than the row, size overflow */
  FP8BS_ERR_ALIGN = -3,       /* pointer or pitch misaligned for the vectorized kernel */
  FP8BS_ERR_UNSUPPORTED = -4, /* valid but unsupported combination (e.g. 1x128 on an MN-major operand) */
  FP8BS_ERR_LAUNCH = -5,      /* the HIP launch itself failed */
  FP8BS_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  FP8BS_ERR_ARG = -7          /* an enum or scalar argument out of range */
};

/* Human-readable text for a status code (static storage; never NULL). */
const char* fp8bs_status_string(int status);

/* ---------------------------------------------------------------- quantization */

/*
 * Blockwise quantization of a bf16 matrix x[rows, cols] (pitch ld_x elements) into codes
 * q_out[rows, cols] (pitch ld_q bytes) and per-block dequantization factors scale_inv_out.
 * [P3] "El avance técnico": 1x128 blocks (activations) and 128x128 tiles (weights), E4M3;
 * [P3] "Por qué esto es importante ...": power-of-2 mode; [P1] "El panorama ...": formats.
 *   fmt:  FP8BS_E4M3 or FP8BS_E5M2.
 *   gran: FP8BS_BLOCK_1x128 (scale_inv_out is float[ceil(cols/128)][rows]) or
 *         FP8BS_BLOCK_128x128 (scale_inv_out is float[ceil(rows/128)][ceil(cols/128)]).
 *   mode: FP8BS_SCALE_FP32 or FP8BS_SCALE_POW2.
 * rows == 0 or cols == 0 is a no-op.  Requirements: ld_x >= cols, ld_q >= cols.  Any pitch and
 * alignment is accepted; 16-byte aligned rows (ld_x % 8 == 0, ld_q % 16 == 0, aligned bases)
 * take the vectorized path.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH.
 */
int fp8_quantize_blockwise(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                           int fmt, int gran, int mode, void* q_out, int64_t ld_q,
                           float* scale_inv_out, void* stream);

/* Microscaling (MXFP8) quantization -- "Infraestructura de Entrenamiento FP8: Precisión Numérica
 * de Nueva Generación", sections "Estrategias de escalado y estabilidad" (block scaling, MXFP8)
 * and "Blackwell MXFP8 y NVFP4: mirando hacia adelante" (hardware-accelerated block scaling).
 * The pages state neither the block size nor the scale format; here a block is 32 consecutive
 * elements of a row and its scale an E8M0 byte.  Per block: the power-of-2 rule of
 * fp8_quantize_blockwise in FP8BS_SCALE_POW2 mode (s = the largest power of two with
 * amax * s <= FMAX; 1 for all-zero or non-finite blocks), codes = the saturating RNE encode of
 * x * s (NaN inputs give NaN codes), and the stored byte is the E8M0 code of the dequantization
 * factor 1/s, i.e. its binary exponent + 127 (2^(byte - 127) = 1/s; never 255).
 *   x_bf16          [rows][ld_x] bf16, device; ld_x >= cols
 *   q_out           [rows][ld_q] codes, device; ld_q >= cols
 *   scale_e8m0_out  [ceil(cols / 128)][rows][4] bytes, device, 4-byte aligned: byte i of word
 *                   (c, r) is the factor of row r, columns 128 c + 32 i .. + 31 (the column
 *                   block-major order of the 1x128 scales); chunks past cols hold 127 (2^0)
 * rows == 0 or cols == 0: no-op.  Caller-owned memory, nothing allocated; asynchronous on stream.
 * Errors: FP8BS_ERR_ARG (fmt), FP8BS_ERR_SHAPE, FP8BS_ERR_NULL, FP8BS_ERR_ALIGN,
 * FP8BS_ERR_LAUNCH. */
int fp8_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                    void* q_out, int64_t ld_q, void* scale_e8m0_out, void* stream);

/*
 * Blockwise quantization of several bf16 matrices in one launch: tensor i is quantized exactly as
 * fp8_quantize_blockwise(x_bf16[i], rows[i], cols[i], ld_x[i], fmt, gran[i], mode, q_out[i],
 * ld_q[i], scale_inv_out[i]) would quantize it (same codes, same scale layout).  [P3] "Ganancias
 * de rendimiento en el mundo real": the scales of every layer's weights are recalibrated each
 * step, and the quantization kernels' overhead counts; one grid for all of a step's weights
 * avoids a launch ramp and tail per tensor.
 *   count: 0 .. 16 tensors; the per-tensor arguments are HOST arrays of count entries (the
 *          pointers in them are device pointers); gran[i] is FP8BS_BLOCK_1x128 or
 *          FP8BS_BLOCK_128x128; fmt and mode apply to every tensor.
 * Empty tensors are skipped.  Every tensor is validated as in fp8_quantize_blockwise before
 * anything is launched; the first error found is returned.  Errors: FP8BS_ERR_NULL,
 * FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN, FP8BS_ERR_ARG (also count outside 0 .. 16),
 * FP8BS_ERR_LAUNCH.
 */
int fp8_quantize_blockwise_batched(int count, const void* const* x_bf16, const int64_t* rows,
                                   const int64_t* cols, const int64_t* ld_x, const int* gran,
                                   int fmt, int mode, void* const* q_out, const int64_t* ld_q,
                                   float* const* scale_inv_out, void* stream);

/*
 * Columnwise quantization with transposed output: blocks of 128 consecutive rows of one column
 * of x[rows, cols] (pitch ld_x elements), codes written transposed to qt_out[cols, rows] (pitch
 * ld_qt bytes): qt_out[c][r] = enc(x[r][c] * s(r / 128, c)).  [P3] "El avance técnico": one
 * scale per 128 consecutive activation elements along the contracted dimension -- for the
 * weight gradient dW = dY^T . X that dimension is the token (row) dimension of dY and X.
 * Scale rule, rounding, saturation, NaN/Inf handling and power-of-2 mode are those of
 * fp8_quantize_blockwise (the result equals fp8_quantize_blockwise of x^T with 1x128 blocks).
 *   scale_inv_out: float[ceil(rows/128)][cols] -- the 1x128 scale layout of the transposed
 *                  matrix, as the GEMM reads it for a K-major operand with 1x128 blocks.
 * rows == 0 or cols == 0 is a no-op.  Requirements: ld_x >= cols, ld_qt >= rows.  16-byte
 * aligned input and output rows (ld_x % 8 == 0, ld_qt % 16 == 0, aligned bases) take the
 * vectorized path.  Caller-owned device buffers; nothing is allocated.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN (scale_inv_out not 4-byte
 * aligned), FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH.
 */
int fp8_quantize_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                              int fmt, int mode, void* qt_out, int64_t ld_qt,
                              float* scale_inv_out, void* stream);

/* fp8_quantize_blockwise with FP8BS_BLOCK_1x128 and fp8_quantize_columnwise_t in one pass over x
 * (one read of the bf16 tensor for both, e.g. the output gradient dY of a layer: its 1x128
 * codes feed the data-gradient GEMM, its transposed 128x1 codes the weight-gradient GEMM) --
 * the sections of those two functions.  Results are bit for bit those of the two calls:
 *   q_out [rows][ld_q], scale_inv_out float[ceil(cols/128)][rows]       (fp8_quantize_blockwise)
 *   qt_out [cols][ld_qt], scale_inv_t_out float[ceil(rows/128)][cols]   (fp8_quantize_columnwise_t)
 * with the same fmt and mode for both.  Requirements: ld_x >= cols, ld_q >= cols, ld_qt >= rows.
 * rows == 0 or cols == 0 is a no-op.  Caller-owned device buffers; nothing is allocated.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN (a scale array not 4-byte aligned),
 * FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH. */
int fp8_quantize_1x128_and_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols,
                                        int64_t ld_x, int fmt, int mode, void* q_out, int64_t ld_q,
                                        float* scale_inv_out, void* qt_out, int64_t ld_qt,
                                        float* scale_inv_t_out, void* stream);

/* Microscaling (MXFP8) quantization along columns, codes written transposed -- the sections of
 * fp8_quantize_mx.  A block is 32 consecutive rows of one column of x[rows][cols], i.e. a
 * 32-element row block of x^T, quantized exactly as fp8_quantize_mx quantizes x^T (power-of-2
 * rule, saturating RNE codes, NaN codes for NaN inputs, E8M0 byte of 1/s).  It gives the
 * microscaling GEMM the operands of the products that contract over the rows of x: the weight
 * gradient dW = dY^T . X (x = dY and x = X, blocks along tokens) and the data gradient
 * dX = dY . W (x = W, blocks along its output features), both run by fp8_gemm_mx.
 *   x_bf16          [rows][ld_x] bf16, device; ld_x >= cols
 *   qt_out          [cols][ld_qt] codes of x^T, device; ld_qt >= rows
 *   scale_e8m0_out  [ceil(rows / 128)][cols][4] bytes, device, 4-byte aligned: the layout
 *                   fp8_quantize_mx writes for x^T (byte i of word (b, c): rows 128 b + 32 i ..
 *                   + 31 of column c); blocks past the last row hold 127 (2^0)
 * rows == 0 or cols == 0: no-op.  Caller-owned memory, nothing allocated; asynchronous on stream.
 * Errors: FP8BS_ERR_ARG (fmt), FP8BS_ERR_SHAPE, FP8BS_ERR_NULL, FP8BS_ERR_ALIGN,
 * FP8BS_ERR_LAUNCH. */
int fp8_quantize_mx_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                 int fmt, void* qt_out, int64_t ld_qt, void* scale_e8m0_out,
                                 void* stream);

/* fp8_quantize_mx and fp8_quantize_mx_columnwise_t in one pass over x (one read of, e.g., the
 * output gradient dY for both microscaling backward products) -- the sections of those two
 * functions; results bit for bit those of the two calls:
 *   q_out [rows][ld_q], scale_e8m0_out [ceil(cols/128)][rows][4]           (fp8_quantize_mx)
 *   qt_out [cols][ld_qt], scale_e8m0_t_out [ceil(rows/128)][cols][4]       (..._columnwise_t)
 * Requirements: ld_x >= cols, ld_q >= cols, ld_qt >= rows; scale arrays 4-byte aligned.
 * rows == 0 or cols == 0 is a no-op.  Caller-owned device buffers; nothing is allocated.
 * Errors: FP8BS_ERR_ARG (fmt), FP8BS_ERR_SHAPE, FP8BS_ERR_NULL, FP8BS_ERR_ALIGN,
 * FP8BS_ERR_LAUNCH. */
int fp8_quantize_mx_and_columnwise_t(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld_x,
                                     int fmt, void* q_out, int64_t ld_q, void* scale_e8m0_out,
                                     void* qt_out, int64_t ld_qt, void* scale_e8m0_t_out,
                                     void* stream);

/*
 * One step of per-tensor delayed scaling on a contiguous bf16 tensor x[numel].
 * [P1] "Transformer Engine: la base de software": the scale used in a step comes from the
 * largest magnitudes recorded in earlier steps (history of hist_len, reduced with "max",
 * margin), so no reduction over the current tensor sits in front of the cast.
 * State (caller-owned device memory, read and updated in place):
 *   amax_history: float[hist_len], newest first; start it at zeros.
 *   scale:        float[1], the scale the NEXT call will use; start it at 1.0f.
 * Per call: q_out[i] = encode(fl32(x[i] * scale)); *scale_inv_used = fl32(1 / scale);
 *   then amax = max |x| (NaN if any element is NaN) is pushed at history[0] (older entries
 *   shift by one), and if r = max(history) is positive and finite,
 *   scale = fl32(fl32(FMAX / r) / 2^margin) (FLT_MAX if that overflows; rounded down to a
 *   power of two in FP8BS_SCALE_POW2 mode); otherwise scale is kept.
 * workspace: device memory of at least fp8_quantize_delayed_workspace_size() bytes, 16-byte
 *   aligned, owned by the caller, no initialization needed; calls that share a workspace
 *   must be ordered on one stream.
 * Limits: 1 <= hist_len <= 1024, 0 <= margin <= 64.  numel == 0 still advances the state
 *   (amax = 0).  Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ARG,
 *   FP8BS_ERR_WORKSPACE, FP8BS_ERR_LAUNCH.
 */
int fp8_quantize_delayed(const void* x_bf16, int64_t numel, int fmt, int mode, int margin,
                         int hist_len, float* amax_history, float* scale, void* q_out,
                         float* scale_inv_used, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of workspace fp8_quantize_delayed needs (a constant). */
size_t fp8_quantize_delayed_workspace_size(void);

/*
 * fp8_quantize_delayed without the workspace argument, for callers that cannot allocate device
 * memory (code captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the per-workgroup amax partials go to a scratch array the library holds in each
 * device's memory for the life of the process (8 KiB: one 4-byte word for each of the at most
 * 2048 workgroups of the cast, whatever numel is, so no tensor is too large for it).  Nothing
 * is allocated or freed by the call; the array's device address is looked up once per device,
 * on the first call there.  Arguments, results and errors as fp8_quantize_delayed (no
 * FP8BS_ERR_WORKSPACE in practice; FP8BS_ERR_LAUNCH also if the scratch array cannot be
 * located).  Every call on one device shares that device's array: calls that overlap on one
 * GPU (different streams, or host threads, without ordering) race and must not be issued;
 * calls ordered on one stream are safe.  Each call writes every partial it reads, so no
 * clearing is needed between calls.
 */
int fp8_quantize_delayed_noalloc(const void* x_bf16, int64_t numel, int fmt, int mode, int margin,
                                 int hist_len, float* amax_history, float* scale, void* q_out,
                                 float* scale_inv_used, void* stream);

/*
 * Saturating round-to-nearest-even cast of fp32 values to FP8 codes, no scaling
 * (q_out[i] = encode(x[i])).  The precision-conversion step of [P1] "Transformer Engine: la
 * base de software", exposed on its own.  Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE,
 * FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH.
 */
int fp8_cast_fp32(const float* x, int64_t n, int fmt, void* q_out, void* stream);

/* ---------------------------------------------------------------- GEMM */

/*
 * Block-scaled FP8 x FP8 GEMM with fp32 accumulation and bf16 output.
 * [P3] "El avance técnico": linear layers run FP8 math with 128x128 weight / 1x128 activation
 * scales; the output stays BF16.  For each 128-wide block kb of the contraction, the fp32
 * partial sum of code products is multiplied by scale_a(m, kb) * scale_b(n, kb) and added to
 * the fp32 accumulator; C = bf16_rne(accumulator).
 *   layout: FP8BS_FPROP  A[M,K] pitch lda,  B[N,K] pitch ldb, C = A . B^T
 *           FP8BS_DGRAD  A[M,K] pitch lda,  B[K,N] pitch ldb, C = A . B
 *           FP8BS_WGRAD  A[K,M] pitch lda,  B[K,N] pitch ldb, C = A^T . B
 *   fa, fb: operand formats (any mix of E4M3 / E5M2, e.g. E5M2 gradients).
 *   ga, gb: granularity of each operand's scales, laid out as described at the top of this
 *           file on the operand's STORED matrix.  Supported: a K-major operand ([.,K] stored)
 *           takes 1x128, 128x128 or per-tensor; an MN-major operand ([K,.] stored) takes
 *           128x128 or per-tensor.  Other combinations return FP8BS_ERR_UNSUPPORTED.
 *           1x128 on both operands of FPROP is the blockwise weight gradient: with A = dY^T and
 *           B = X^T as written by fp8_quantize_columnwise_t (K = tokens), C = dW = dY^T . X.
 *   C_bf16: [M,N] pitch ldc (elements).
 * M, N or K == 0: C is left untouched when M or N is 0; with K == 0, C is set to zeros.
 * Requirements: 16-byte aligned A and B with lda % 16 == 0 and ldb % 16 == 0, 4-byte aligned C
 * with ldc % 2 == 0 (FP8BS_ERR_ALIGN otherwise); pitches at least the row widths.  Size limits
 * (FP8BS_ERR_SHAPE): lda, ldb < 2^23; M, N < 2^31 - 256; each scale array below 4 GiB.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN, FP8BS_ERR_UNSUPPORTED,
 * FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH.
 */
int fp8_gemm_blockscaled(int layout, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, int fa, int ga, const float* scale_inv_a,
                         const void* B, int64_t ldb, int fb, int gb, const float* scale_inv_b,
                         void* C_bf16, int64_t ldc, void* stream);

/*
 * Grouped (mixture-of-experts) block-scaled FP8 GEMM.  [P3] "Ganancias de rendimiento en el
 * mundo real": the FP8 recipe applied to an MoE model's expert layers.
 * Rows [group_offsets[g], group_offsets[g+1]) of A (tokens sorted by expert) are multiplied
 * by expert g's weight: C[r, :] = A[r, :] . B[g]^T for those rows.
 *   num_groups:    0 .. 1024 (FP8BS_ERR_ARG beyond).
 *   group_offsets: DEVICE int64[num_groups + 1], non-decreasing, offsets[0] = 0,
 *                  offsets[num_groups] = total_M (empty groups allowed).  Other offsets are
 *                  read as e[g] = min(max(offsets[0..g], 0), total_M): each is clamped to
 *                  [0, total_M] and raised to the largest offset before it, and group g covers
 *                  rows [e[g], e[g+1]).  So groups never overlap, a decreasing offset leaves
 *                  the groups it would reopen empty, rows outside [e[0], e[num_groups]) are
 *                  not written, and no access goes out of range.
 *   A:  [total_M, K] codes (format fa), pitch lda; scale_inv_a: 1x128 blocks,
 *       float[ceil(K/128)][total_M].
 *   B:  [num_groups][N][K] codes (format fb), rows of pitch ldb, groups of stride N * ldb;
 *       scale_inv_b: float[num_groups][ceil(N/128)][ceil(K/128)].
 *   C:  [total_M, N] bf16, pitch ldc.
 * Alignment and size limits as for fp8_gemm_blockscaled (total_M for M; scale_inv_a and one
 * group's scale_inv_b below 4 GiB).  Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE,
 * FP8BS_ERR_ALIGN, FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH.
 */
int fp8_grouped_gemm(int32_t num_groups, const int64_t* group_offsets, int64_t total_M,
                     int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                     const float* scale_inv_a, const void* B, int64_t ldb, int fb,
                     const float* scale_inv_b, void* C_bf16, int64_t ldc, void* stream);

/* Block-scaled FP8 fprop GEMM with the output quantized in the epilogue.  [P3] "Ganancias de
 * rendimiento en el mundo real" (the cost of separate quantization kernels) and "El avance
 * técnico" (1x128 activation blocks, E4M3).
 * Computes C = A . B^T (A[M,K], B[N,K], both E4M3) as fp8_gemm_blockscaled with layout
 * FP8BS_FPROP does, and in the same kernel quantizes the bf16-rounded output in 1x128 blocks
 * along N: Cq[M,N] (E4M3 codes, pitch ldcq bytes) and cq_scale_inv float[ceil(N/128)][M] are
 * exactly what fp8_quantize_blockwise(C_bf16, FP8BS_E4M3, FP8BS_BLOCK_1x128, mode_out) would
 * write -- the next layer's activation operand.
 *   ga, gb:      as fp8_gemm_blockscaled for FPROP, except 1x128 on B (FP8BS_ERR_UNSUPPORTED).
 *   pow2_inputs: 0 -- fp32 scales (fold); 1 -- the scales are powers of two and are applied by
 *                the MFMA (the precondition of fp8_gemm_blockscaled_pow2).
 *   C_bf16:      may be NULL (only the quantized output is written); else [M,N] pitch ldc.
 *   mode_out:    FP8BS_SCALE_FP32 or FP8BS_SCALE_POW2 for the output's scales.
 * Requirements: those of fp8_gemm_blockscaled; ldcq >= N; 4-byte aligned cq_scale_inv.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN, FP8BS_ERR_UNSUPPORTED,
 * FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH. */
int fp8_gemm_blockscaled_qout(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                              int ga, const float* scale_inv_a, const void* B, int64_t ldb,
                              int gb, const float* scale_inv_b, int pow2_inputs, void* C_bf16,
                              int64_t ldc, int mode_out, void* Cq, int64_t ldcq,
                              float* cq_scale_inv, void* stream);

/* Microscaling (MXFP8) GEMM, fprop layout -- the sections of fp8_quantize_mx.  C[M][N] (bf16,
 * round to nearest even) = sum over k of A[m][k] * 2^(sa(m, k/32) - 127) * B[n][k] *
 * 2^(sb(n, k/32) - 127): A[M][lda] and B[N][ldb] are FP8 codes of formats fa / fb (K-major,
 * the fp8_gemm_blockscaled fprop operands), sa [ceil(K/128)][M][4] and sb [ceil(K/128)][N][4]
 * their E8M0 scale bytes in the layout fp8_quantize_mx writes.  The matrix cores apply the
 * scales (the scaled MFMA, one byte per lane and 32-wide k chunk) and accumulate in fp32.  A
 * scale byte of 255 (E8M0 NaN) makes the products of its block NaN; bytes of chunks past K are
 * ignored.
 *   lda, ldb: multiples of 16, >= K, < 2^23; A, B 16-byte aligned
 *   sa, sb: 4-byte aligned, each below 4 GiB
 *   C_bf16: [M][ldc], ldc >= N, 4-byte aligned, even ldc
 * M == 0 or N == 0: no-op; K == 0: C = 0.  Errors: FP8BS_ERR_ARG (formats), FP8BS_ERR_SHAPE,
 * FP8BS_ERR_NULL, FP8BS_ERR_ALIGN, FP8BS_ERR_LAUNCH. */
int fp8_gemm_mx(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                const void* scale_e8m0_a, const void* B, int64_t ldb, int fb,
                const void* scale_e8m0_b, void* C_bf16, int64_t ldc, void* stream);

/* Grouped (mixture-of-experts) microscaling GEMM -- the passages of fp8_grouped_gemm (experts)
 * and fp8_quantize_mx (microscaling).  Groups, offsets, A, B, C, alignment and size limits as
 * fp8_grouped_gemm; the scales are E8M0 bytes, one per 32 K elements of every row, applied by
 * the matrix cores as in fp8_gemm_mx:
 *   scale_e8m0_a: [ceil(K/128)][total_M][4] bytes (fp8_quantize_mx of A)
 *   scale_e8m0_b: [num_groups][ceil(K/128)][N][4] bytes (fp8_quantize_mx of each expert's B,
 *                 one after the other)
 * both 4-byte aligned (FP8BS_ERR_ALIGN); scale_e8m0_a and one expert's scales below 4 GiB.
 * Errors: FP8BS_ERR_NULL, FP8BS_ERR_SHAPE, FP8BS_ERR_ALIGN, FP8BS_ERR_ARG, FP8BS_ERR_LAUNCH. */
int fp8_grouped_gemm_mx(int32_t num_groups, const int64_t* group_offsets, int64_t total_M,
                        int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                        const void* scale_e8m0_a, const void* B, int64_t ldb, int fb,
                        const void* scale_e8m0_b, void* C_bf16, int64_t ldc, void* stream);

/* Block-scaled FP8 GEMM with power-of-2 scales -- "NVIDIA NeMo RL logra una aceleración del 48%
 * ...", section "Por qué esto es importante para la economía de la IA" (the power-of-2 scale
 * option).  Same arguments, layouts, granularities, scale arrays, results and errors as
 * fp8_gemm_blockscaled; the difference is the precondition on the scales: every scale_inv value
 * read must be a power of two in [2^-127, 2^127] (what fp8_quantize_blockwise writes in
 * FP8BS_SCALE_POW2 mode).  Only the binary32 exponent field of each value is used: it is given
 * to the matrix core as an E8M0 block scale, so the products are scaled and accumulated inside
 * the MFMA with no per-block fold.  A scale that is not a power of two is taken as 2 raised to
 * its exponent (the result is then that of the rounded-down scale); no error is reported for it.
 * With per-tensor scales on both operands this call computes exactly what fp8_gemm_blockscaled
 * computes. */
int fp8_gemm_blockscaled_pow2(int layout, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, int fa, int ga, const float* scale_inv_a,
                              const void* B, int64_t ldb, int fb, int gb, const float* scale_inv_b,
                              void* C_bf16, int64_t ldc, void* stream);

/* Grouped (MoE) GEMM with power-of-2 scales: fp8_grouped_gemm's arguments, layouts and errors,
 * with the scale precondition and E8M0 use of fp8_gemm_blockscaled_pow2. */
int fp8_grouped_gemm_pow2(int32_t num_groups, const int64_t* group_offsets, int64_t total_M,
                          int64_t N, int64_t K, const void* A, int64_t lda, int fa,
                          const float* scale_inv_a, const void* B, int64_t ldb, int fb,
                          const float* scale_inv_b, void* C_bf16, int64_t ldc, void* stream);

/* The GEMM entry points with an explicit output-tile configuration `tile` (fp8bs_tile), for
 * tuning and for tests that cover every configuration; the results equal those of the
 * corresponding entry point up to fp32 summation order.  Same arguments and errors otherwise;
 * FP8BS_ERR_ARG also for a tile value out of range.
 *   fp8_gemm_blockscaled_tiled:      pow2 = 0 -> fp8_gemm_blockscaled, 1 -> ..._pow2.
 *   fp8_grouped_gemm_tiled:          pow2 = 0 -> fp8_grouped_gemm, 1 -> ..._pow2; tile must
 *                                    be AUTO, 256x128_W8, 256x256_W8 or 128x128_W4.
 *   fp8_gemm_blockscaled_qout_tiled: fp8_gemm_blockscaled_qout. */
int fp8_gemm_blockscaled_tiled(int tile, int pow2, int layout, int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda, int fa, int ga,
                               const float* scale_inv_a, const void* B, int64_t ldb, int fb,
                               int gb, const float* scale_inv_b, void* C_bf16, int64_t ldc,
                               void* stream);
int fp8_grouped_gemm_tiled(int tile, int pow2, int32_t num_groups, const int64_t* group_offsets,
                           int64_t total_M, int64_t N, int64_t K, const void* A, int64_t lda,
                           int fa, const float* scale_inv_a, const void* B, int64_t ldb, int fb,
                           const float* scale_inv_b, void* C_bf16, int64_t ldc, void* stream);
int fp8_gemm_blockscaled_qout_tiled(int tile, int64_t M, int64_t N, int64_t K, const void* A,
                                    int64_t lda, int ga, const float* scale_inv_a,
                                    const void* B, int64_t ldb, int gb,
                                    const float* scale_inv_b, int pow2_inputs, void* C_bf16,
                                    int64_t ldc, int mode_out, void* Cq, int64_t ldcq,
                                    float* cq_scale_inv, void* stream);

/* FP8 KV cache: write one token per sequence.  [P3] "Ganancias de rendimiento en el mundo real"
 * (FP8 extended to the KV cache); the cache format is the activation recipe of "El avance
 * técnico" applied to keys and values: each 128-element head vector is one 1x128 block, E4M3
 * (or E5M2) codes and an fp32 dequantization factor, by the rule of fp8_quantize_blockwise.
 *   Cache (caller-owned device memory, capacity T tokens per sequence):
 *     k_codes, v_codes:          uint8 [B][T][KVH][128] (16-byte aligned)
 *     k_scale_inv, v_scale_inv:  float [B][T][KVH]
 *   k_new_bf16, v_new_bf16: bf16 [B][KVH][128] (16-byte aligned), the new token's keys and
 *   values; positions: device int32 [B], the slot t of each sequence's token (a slot outside
 *   [0, T) leaves that sequence's cache unchanged).  Only the B written head-vector slots
 *   (codes and factors) are touched.  mode: FP8BS_SCALE_FP32 or FP8BS_SCALE_POW2.
 * B <= 65535.  Errors: FP8BS_ERR_ARG, FP8BS_ERR_SHAPE, FP8BS_ERR_NULL, FP8BS_ERR_ALIGN,
 * FP8BS_ERR_LAUNCH. */
int fp8_kv_cache_append(int64_t B, int64_t KVH, int64_t T, const void* k_new_bf16,
                        const void* v_new_bf16, const int32_t* positions, int fmt, int mode,
                        void* k_codes, float* k_scale_inv, void* v_codes, float* v_scale_inv,
                        void* stream);

/* Grouped-query decode attention over the FP8 KV cache of fp8_kv_cache_append.  [P3]
 * "Ganancias de rendimiento en el mundo real" (FP8 KV cache and attention).
 * For sequence b and query head h (KV head kv = h / (H / KVH)), with L_b = seq_lens[b]
 * clamped to [0, T] and the cache dequantized (code value x the head vector's factor):
 *   s_t = sm_scale * sum_d q[b][h][d] K[b][t][kv][d],  t < L_b
 *   out[b][h][:] = sum_t softmax(s)_t V[b][t][kv][:]     (zeros when L_b = 0)
 * computed to fp32 accuracy (matrix-core bf16 products of the exactly decoded cache with the bf16
 * queries and with the softmax weights split into bf16 hi + lo terms, fp32 sums, softmax online
 * in base 2), output rounded to bf16.
 *   q_bf16: [B][H][128] (16-byte aligned); seq_lens: device int32 [B]; out_bf16: [B][H][128].
 *   H / KVH must be 1, 2, 4 or 8, and (T + 32) * KVH * 128 < 2^32 (one sequence and KV head's
 *   rows are addressed with 32-bit offsets); else FP8BS_ERR_UNSUPPORTED.  Tokens at or past L_b are never read.  sm_scale must be
 *   finite.
 * Errors: FP8BS_ERR_ARG, FP8BS_ERR_SHAPE, FP8BS_ERR_NULL, FP8BS_ERR_ALIGN,
 * FP8BS_ERR_UNSUPPORTED, FP8BS_ERR_LAUNCH. */
int fp8_attention_decode(int64_t B, int64_t H, int64_t KVH, int64_t T, const void* q_bf16,
                         const void* k_codes, const float* k_scale_inv, const void* v_codes,
                         const float* v_scale_inv, const int32_t* seq_lens, float sm_scale,
                         int fmt, void* out_bf16, void* stream);

/* The same decode attention with each sequence split into chunks of `chunk` tokens (a positive
 * multiple of 32), one workgroup per (sequence, KV head, chunk), and the chunks' partial results
 * merged by a second kernel; the result is that of fp8_attention_decode up to fp32 rounding
 * order.  Spreading long sequences over more workgroups keeps the GPU busy when sequence
 * lengths differ.  [P3] "Ganancias de rendimiento en el mundo real".
 *   workspace: caller-owned device memory of at least
 *     fp8_attention_decode_workspace_size(B, H, KVH, T, chunk) bytes (4-byte aligned; may be
 *     null when T = 0), holding per (sequence, KV head, chunk, query head) the chunk's maximum
 *     logit, its sum of weights and its 128 weighted value sums (130 floats); its contents on
 *     entry do not matter.  Calls that share a workspace on different streams race.
 *   H / KVH must be 1, 2, 4 or 8, and (T + 32) * KVH * 128 < 2^32 (else FP8BS_ERR_UNSUPPORTED).
 *   Other arguments as above.
 * Errors: as fp8_attention_decode; FP8BS_ERR_SHAPE also for a chunk that is not a positive
 * multiple of 32 or a workspace smaller than required. */
int fp8_attention_decode_split(int64_t B, int64_t H, int64_t KVH, int64_t T, const void* q_bf16,
                               const void* k_codes, const float* k_scale_inv,
                               const void* v_codes, const float* v_scale_inv,
                               const int32_t* seq_lens, float sm_scale, int fmt, int64_t chunk,
                               void* workspace, size_t workspace_bytes, void* out_bf16,
                               void* stream);

/* Workspace bytes fp8_attention_decode_split needs: B * KVH * ceil(T / chunk) * (H / KVH) * 130 * 4;
 * 0 for non-positive sizes, H not a multiple of KVH, or a size that overflows. */
size_t fp8_attention_decode_workspace_size(int64_t B, int64_t H, int64_t KVH, int64_t T,
                                           int64_t chunk);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
