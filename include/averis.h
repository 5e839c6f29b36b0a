/*
 * averis.h -- C ABI of libaveris.so: the Averis mean-residual split before blockwise FP4
 * quantization, and the three quantized training GEMMs with the mean terms added back,
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "The Curse and Blessing of Mean Bias in FP4-Quantized LLM Training"
 * (arXiv 2603.10444).  Passages cited by page key:
 *   [rainbus]    explainer "均值偏置的诅咒与祝福：FP4量化大语言模型训练" (paper.rainbus.top)
 *   [paperlayer] source-linked summary of v2 (paperlayer.ai), sections 1-6 and appendices
 *   [chatpaper]  v1 abstract (chatpaper.ai)
 *
 * For activations X [l, m] (l = b*s tokens) and output gradients D [l, n] of a linear layer
 * with weight W [m, n] ([rainbus] 方法步骤详情):
 *   mu_X = (1/l) 1^T X,   X_R = X - 1 mu_X          (same for D)
 *   Y     = 1 (Q(mu_X) Q(W))   + Q(X_R) Q(W)
 *   dX    = 1 (Q(mu_D) Q(W)^T) + Q(D_R) Q(W)^T
 *   dW    = Q(X_R)^T Q(D_R)    + l Q(mu_X)^T Q(mu_D)   (cross terms vanish, dropped)
 * where Q is a blockwise FP4 (E2M1) quantizer applied independently to each operand, with
 * blocks along that operand's own GEMM reduction axis.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent), 16-byte aligned.
 *    Host pointers are named h_*.  The caller owns every buffer; the library never
 *    allocates, frees or keeps device memory between calls.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *    returns without waiting.  Inputs must stay valid until the stream reaches the work.
 *    Calls on different streams are independent; calls sharing a workspace must be ordered.
 *  - Workspaces (ws, ws_bytes >= the matching *_workspace_size query) are device scratch.  A
 *    split_quant workspace must be zero-filled before its first use: it holds per-column-strip
 *    arrival counters, and every call leaves them at zero again, so it can be reused as is by
 *    calls with the same cols (and E).  Zero it again before using it for other cols or E.
 *    The other workspaces need no initial contents.
 *  - Arguments are validated before anything is enqueued: on any error a non-zero status is
 *    returned, nothing is launched and no output is touched.  A failed launch returns
 *    AVERIS_E_HIP.  Faults inside kernels surface at the caller's next synchronisation.
 *  - Inputs must be finite.  Results for NaN/Inf inputs are unspecified; AVERIS_CHECK_FINITE
 *    makes split_quant report them (and scale underflow) in a device status word.
 *  - Results are deterministic: no floating-point atomics; every reduction has a fixed order.
 */
#ifndef AVERIS_H
#define AVERIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVERIS_ABI_VERSION 1

typedef enum {
  AVERIS_OK = 0,
  AVERIS_E_NULL = 1,      /* a required pointer is NULL */
  AVERIS_E_SHAPE = 2,     /* sizes inconsistent or outside the documented preconditions */
  AVERIS_E_ALIGN = 3,     /* pointer or leading dimension not 16-byte aligned */
  AVERIS_E_DTYPE = 4,     /* unknown element type */
  AVERIS_E_FORMAT = 5,    /* unknown FP4 format, or operands of different formats */
  AVERIS_E_FLAGS = 6,     /* unknown or contradictory flag bits */
  AVERIS_E_WORKSPACE = 7, /* workspace NULL or smaller than the *_workspace_size query */
  AVERIS_E_HIP = 8        /* a HIP runtime call or kernel launch failed */
} averis_status;

/* Block formats (readings of the pages' "blockwise FP4 quantization", [rainbus] 块量化):
 *  AVERIS_NVFP4: 16-element blocks, E4M3 block scale, plus an fp32 tensor decode scale
 *                s_dec = amax(operand) / (6 * 448).  Per block b with max magnitude a_b:
 *                e_b = E4M3(fl(fl(a_b / 6) / s_dec)); elements x -> E2M1(fl(x * fl(1 / fl(val(e_b) * s_dec)))).
 *                Decode: e2m1(code) * val(e_b) * s_dec.
 *  AVERIS_MXFP4: 32-element blocks, E8M0 scale 2^E with E = floor(log2 a_b) - 2 clamped to
 *                [-127, 127], stored as E + 127; elements x -> E2M1(x * 2^-E).  Decode:
 *                e2m1(code) * 2^E.  This is the format gfx950's scaled MFMA consumes natively.
 * E2M1 rounding is to nearest, ties to the even code, saturating at 6; the sign of a value
 * that rounds to zero is kept (code 0x8).  A block whose scale is zero (all-zero block, or
 * NVFP4 e_b == 0 or decode scale below 2^-126) has all-zero codes. */
typedef enum { AVERIS_NVFP4 = 1, AVERIS_MXFP4 = 2 } averis_format;

typedef enum { AVERIS_F32 = 0, AVERIS_BF16 = 1 } averis_dtype;

/* Flag bits. */
#define AVERIS_SPLIT       (1u << 0) /* subtract the column mean before quantizing (Averis);
                                        without it the quantizer is the vanilla one (and the
                                        one used for weights) */
#define AVERIS_HADAMARD16  (1u << 1) /* rotate every 16-block along K by H16/4 (Sylvester
                                        order) after the subtraction ([rainbus] Hadamard变换,
                                        技术新颖性: Averis and Hadamard compose) */
#define AVERIS_MEAN_GIVEN  (1u << 2) /* split_quant: `mean` is an input, not computed */
#define AVERIS_CHECK_FINITE (1u << 3) /* split_quant (dense and grouped): the call writes status
                                        bits into the first 4 bytes (uint32) of its workspace,
                                        readable once the stream reaches the work: 0 = nothing
                                        found, else an OR of AVERIS_STATUS_* */
#define AVERIS_STATUS_NONFINITE  (1u << 0) /* an input element is NaN or +-Inf */
#define AVERIS_STATUS_UNDERFLOW  (1u << 1) /* a nonzero block lost its range to scale underflow:
                                             NVFP4 block zeroed (E4M3 scale 0 or decode scale
                                             below 2^-126), MXFP4 block amax below 2^-125 (its
                                             exponent clamped at -127) */
#define AVERIS_ACCUMULATE  (1u << 4) /* bwd_dw: dW += result instead of dW = result */

/* A quantized operand [outer, k] with blocks along k (K-inner, row-major).
 *   codes:        device uint8 [outer][k_pad / 2]; element 2i in bits 3:0, 2i+1 in bits 7:4.
 *   scales:       device uint8, round_up(outer, 32) * (k_pad / g) bytes; g = 16 (E4M3 codes) or 32
 *                 (E8M0 codes).  Tiled for the GEMM: the scale of K-block b (elements b*g ..) of
 *                 row r is at byte ((r / 32) * (k_pad / 256) + b / S) * 32 * S + (r % 32) * S + b % S
 *                 with S = 256 / g, i.e. per 32-row group and 256-element K-step the 32 x S bytes
 *                 are contiguous.  Rows [outer, round_up(outer, 32)) hold zero scales.
 *   tensor_scale: device fp32 s_dec (NVFP4; one per group for grouped operands); NULL for MXFP4.
 *   k_pad:        storage length along k = k rounded up to a multiple of 256; elements in
 *                 [k, k_pad) hold code 0 and blocks past k scale byte 0.
 *   flags:        AVERIS_HADAMARD16 if the operand was rotated along k.
 * The caller fills every field before a call that writes the operand, and the library checks
 * outer/k/k_pad/fmt/flags against what the call expects. */
typedef struct averis_qtensor {
  uint8_t *codes;
  uint8_t *scales;
  float *tensor_scale;
  int64_t outer;
  int64_t k;
  int64_t k_pad;
  int32_t fmt;
  uint32_t flags;
} averis_qtensor;

int32_t averis_abi_version(void);
const char *averis_status_string(int32_t status);
/* SHA-1 (40 hex digits) of the sources the library was built from, fixed at build time, or
 * "unknown".  A loader compares it with its copy of the sources to refuse a stale library.
 * The returned string is static; the caller must not free it. */
const char *averis_source_digest(void);

/* -----------------------------------------------------------------------------------------
 * averis_split_quant -- column statistics, mean, subtraction, optional Hadamard, FP4 quant.
 * [rainbus] 方法步骤详情 (mu_X = (1/l) 1^T X, X_R = X - 1 mu_X, Q_b applied independently to
 * the mean and the residual); [paperlayer] §3 Method (the mean matrix is broadcast, never
 * materialized: X_R exists only as the quantized operands written here).
 *
 *  x      device [rows, cols] row-major, element type xdt, leading dimension ldx (elements).
 *         rows >= 0; cols > 0 and cols % 32 == 0 (for NVFP4 too: the row layout is quantized in
 *         32-element units); ldx >= cols, ldx * elem_size % 16 == 0.
 *  flags  AVERIS_SPLIT, AVERIS_HADAMARD16, AVERIS_MEAN_GIVEN (requires SPLIT),
 *         AVERIS_CHECK_FINITE (status bits in workspace word 0).
 *  mean   device fp32 [cols].  With SPLIT: written with mu (fp32 of the fixed-order fp64 sum
 *         divided by rows; rows == 0 gives 0), or read if MEAN_GIVEN.  Without SPLIT: unused
 *         (may be NULL).
 *  q_row  [outer = rows, k = cols] operand (the K = features layout used by fwd and dX), or NULL.
 *  q_col  [outer = cols, k = rows] operand (the K = tokens layout used by dW), or NULL.  Rows
 *         [rows, k_pad) are zero residuals.
 *  q_mean [outer = 1, k = cols] quantized mean (own tensor scale); required with SPLIT,
 *         must be NULL without it.
 * With NVFP4 each written operand gets the tensor scale of its own amax (after rotation).
 * At least one of q_row / q_col must be given.
 * ----------------------------------------------------------------------------------------- */
size_t averis_split_quant_workspace_size(int64_t rows, int64_t cols, int32_t fmt, uint32_t flags);

int32_t averis_split_quant(const void *x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                           int32_t fmt, uint32_t flags, float *mean,
                           const averis_qtensor *q_row, const averis_qtensor *q_col,
                           const averis_qtensor *q_mean, void *ws, size_t ws_bytes, void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_split_quant_batch -- averis_split_quant of up to AVERIS_BATCH_MAX independent tensors
 * in one statistics launch and one quantizing launch (two with NVFP4 + HADAMARD16), for tensors
 * that become ready together: a layer's weights at the start of a step, the q/k/v output
 * gradients that attention's backward returns at once, the gate/up gradients of the SwiGLU
 * backward.  Same method as averis_split_quant ([rainbus] 方法步骤详情), applied to each tensor
 * on its own: every output is bit-identical to that of averis_split_quant with the item's
 * arguments.
 *  n       1 .. AVERIS_BATCH_MAX items.
 *  items   host array; item i holds the x, rows, cols, ldx, mean, q_row, q_col, q_mean, ws and
 *          ws_bytes arguments of averis_split_quant (same meaning, layout and ownership).  Each
 *          item needs a workspace of its own (overlapping workspaces: AVERIS_E_WORKSPACE).
 *  xdt, fmt, flags  shared by every item; flags as averis_split_quant without
 *          AVERIS_CHECK_FINITE (AVERIS_E_FLAGS).
 * Every item is validated before anything is enqueued; the first invalid item's status is
 * returned and nothing is launched.
 * ----------------------------------------------------------------------------------------- */
#define AVERIS_BATCH_MAX 8
typedef struct averis_split_quant_item {
  const void *x;
  int64_t rows;
  int64_t cols;
  int64_t ldx;
  float *mean;
  const averis_qtensor *q_row;
  const averis_qtensor *q_col;
  const averis_qtensor *q_mean;
  void *ws;
  size_t ws_bytes;
} averis_split_quant_item;

int32_t averis_split_quant_batch(int32_t n, const averis_split_quant_item *items, int32_t xdt, int32_t fmt,
                                 uint32_t flags, void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_split_quant_sr -- averis_split_quant with stochastic rounding of every E2M1 code it
 * writes (residual layouts and quantized mean), for callers that round gradient operands
 * stochastically.  The pages round to nearest and do not use this; it is an option.
 *  seed   64-bit key of the counter-based Philox4x32-10 generator (Salmon et al., "Parallel
 *         random numbers: as easy as 1, 2, 3", SC 2011): key = (seed mod 2^32, seed / 2^32).
 *         Element k (along K) of outer index i of a layout (0 = q_row, 1 = q_col, 2 = q_mean)
 *         draws the 16-bit half k % 2 (low half first) of output word (k % 8) / 2 at counter
 *         (k / 8, i, layout, 0).  The same seed gives the same codes.
 * Rounding: the scaled magnitude a (the value times the block's reciprocal scale, as for round
 * to nearest) lies between neighbouring E2M1 magnitudes lo <= a < hi and becomes hi when
 * draw / 2^16 < (a - lo) / (hi - lo), else lo; a >= 6 gives 6; the sign is kept.  Block scales
 * and tensor scales are those of round to nearest.  Other arguments, preconditions and errors
 * as averis_split_quant.
 * ----------------------------------------------------------------------------------------- */
int32_t averis_split_quant_sr(const void *x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                              int32_t fmt, uint32_t flags, uint64_t seed, float *mean,
                              const averis_qtensor *q_row, const averis_qtensor *q_col,
                              const averis_qtensor *q_mean, void *ws, size_t ws_bytes, void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_split_quant_noalloc -- averis_split_quant without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It calls no allocating routine: its workspace is a
 * library-owned device array of averis_split_quant_noalloc_max_bytes() bytes (8 MiB), one per
 * GPU, held until the process ends.  Arguments, results and errors as averis_split_quant;
 * AVERIS_E_FLAGS for AVERIS_CHECK_FINITE (the status word would be in the hidden array);
 * AVERIS_E_WORKSPACE when averis_split_quant_workspace_size(rows, cols, ..) exceeds that size
 * (about rows * cols <= 2^28, e.g. 65536 x 4096), AVERIS_E_HIP if the array's device address
 * cannot be obtained.  The first call on a GPU clears the array (a kernel on `stream`).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU (other streams or
 * host threads without ordering) race and give undefined results.
 * ----------------------------------------------------------------------------------------- */
size_t averis_split_quant_noalloc_max_bytes(void);

int32_t averis_split_quant_noalloc(const void *x, int32_t xdt, int64_t rows, int64_t cols,
                                   int64_t ldx, int32_t fmt, uint32_t flags, float *mean,
                                   const averis_qtensor *q_row, const averis_qtensor *q_col,
                                   const averis_qtensor *q_mean, void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_linear_fwd -- Y = 1 (Q(mu_X) Q(W)) + Q(X_R) Q(W)   ([rainbus] 方法步骤详情, forward)
 *  xr    [outer = l, k = m]  (q_row of split_quant(X))
 *  mu_x  [outer = 1, k = m]  (q_mean of split_quant(X)), or NULL for the vanilla GEMM
 *  w     [outer = n, k = m]  (q_col of split_quant(W [m, n]) without SPLIT)
 *  y     device [l, n] row-major, element type ydt, leading dimension n <= ldy < 2^23; n % 8 == 0.
 * All operands share fmt and the HADAMARD16 bit.  The mean term Q(mu_X) Q(W) is one row added
 * to every output row: MXFP4 launches compute it inside the GEMM from the quantized mean (one
 * more scaled MFMA per wave and K-substep, on the weight fragments the tile already holds)
 * while k_pad <= 8192; NVFP4 and longer K compute it once per call as a GEMV and add it in the
 * epilogue.
 * ----------------------------------------------------------------------------------------- */
size_t averis_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t fmt);

int32_t averis_linear_fwd(const averis_qtensor *xr, const averis_qtensor *mu_x,
                          const averis_qtensor *w, void *y, int32_t ydt, int64_t ldy,
                          void *ws, size_t ws_bytes, void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_linear_bwd_dx -- dX = 1 (Q(mu_D) Q(W)^T) + Q(D_R) Q(W)^T   ([rainbus] 方法步骤详情)
 *  dr    [outer = l, k = n]  (q_row of split_quant(D))
 *  mu_d  [outer = 1, k = n]  or NULL (vanilla)
 *  w     [outer = m, k = n]  (q_row of split_quant(W [m, n]) without SPLIT)
 *  dx    device [l, m], element type dxdt, leading dimension m <= lddx < 2^23; m % 8 == 0.
 * ----------------------------------------------------------------------------------------- */
int32_t averis_linear_bwd_dx(const averis_qtensor *dr, const averis_qtensor *mu_d,
                             const averis_qtensor *w, void *dx, int32_t dxdt, int64_t lddx,
                             void *ws, size_t ws_bytes, void *stream);

/* -----------------------------------------------------------------------------------------
 * Producer-fused column statistics.  The split ([rainbus] 方法步骤详情: mu = (1/l) 1^T X over
 * all l token rows, before any element of X_R can be quantized) costs a pass over X for its
 * column statistics; [paperlayer] §3 Method describes the split as cheap elementwise work.
 * A GEMM that writes X (the forward GEMM whose output is the next linear's input, the
 * input-gradient GEMM whose output is the next D) can take the statistics of what it stores,
 * and split_quant then starts from them instead of reading X for them.
 *
 * averis_colstats: column partials of an output [rows, cols] over consecutive row blocks.
 *   sum       device fp32 [capacity]: sum[p * cols + c] = fp32 sum of column c over rows
 *             [p * part_rows, min((p + 1) * part_rows, rows)), of the values as stored
 *             (after rounding to the output type)
 *   min, max  device fp32 [capacity]: column minima and maxima of the same rows, or both NULL.
 *             Needed when the statistics feed an NVFP4 split without HADAMARD16, whose residual
 *             tensor scale comes from them.
 *   capacity  floats each given array holds; averis_colstats_capacity(rows, cols) suffices for
 *             every producer.
 *   rows, cols, parts, part_rows: written by the producer (parts = ceil(rows / part_rows)).
 * The arrays are caller-owned; a producer writes parts * cols floats of each.
 * ----------------------------------------------------------------------------------------- */
typedef struct averis_colstats {
  float *sum;
  float *min;
  float *max;
  int64_t capacity;
  int64_t rows, cols, parts, part_rows;
} averis_colstats;

int64_t averis_colstats_capacity(int64_t rows, int64_t cols);

/* averis_linear_fwd / averis_linear_bwd_dx that also write the column statistics of the output
 * into *stats (written by the same stream-ordered work).  Sums without minima and maxima are
 * taken in the GEMM epilogue by the single-split launches of the MXFP4 warp-specialized kernel
 * and of the NVFP4 two-stage kernel (64- or 128-row parts); other launches, and requests with
 * minima and maxima, take them in a pass over the stored output after the GEMM (512-row
 * parts).  Errors as the plain calls, and AVERIS_E_NULL (stats
 * or stats->sum NULL, or one of min / max NULL without the other), AVERIS_E_SHAPE (capacity
 * below averis_colstats_capacity of the output). */
int32_t averis_linear_fwd_stats(const averis_qtensor *xr, const averis_qtensor *mu_x,
                                const averis_qtensor *w, void *y, int32_t ydt, int64_t ldy,
                                averis_colstats *stats, void *ws, size_t ws_bytes, void *stream);

int32_t averis_linear_bwd_dx_stats(const averis_qtensor *dr, const averis_qtensor *mu_d,
                                   const averis_qtensor *w, void *dx, int32_t dxdt, int64_t lddx,
                                   averis_colstats *stats, void *ws, size_t ws_bytes, void *stream);

/* The producers of a transformer block's linear inputs, with the same column statistics: the
 * normalization writes the input of q/k/v and of gate/up, the activation the input of down.
 *   averis_rmsnorm_stats: y[r, c] = x[r, c] * rs_r * weight[c], rs_r = 1 / sqrt(s_r / cols + eps),
 *     s_r = sum_c x[r, c]^2 (RMSNorm, Zhang and Sennrich 2019).  fp32 arithmetic: s_r summed
 *     per lane over its columns in order, then across the 64 lanes of a wave; each product
 *     rounded; y rounded to dt.
 *   averis_swiglu_stats: y = silu(gate) * up, silu(g) = g / (1 + exp(-g)) (Shazeer 2020), fp32,
 *     each operation rounded, y rounded to dt.
 * x, gate, up: device [rows, cols] row-major of element type dt (ld elements, ld * size % 16
 * == 0); y: device [rows, cols] of type dt, leading dimension ldy; weight: device fp32 [cols];
 * cols % 32 == 0.  stats: NULL (no statistics) or as for averis_linear_fwd_stats (64-row
 * parts; min / max when both are set).  Errors: AVERIS_E_DTYPE, AVERIS_E_SHAPE (sizes, eps < 0,
 * capacity), AVERIS_E_NULL, AVERIS_E_ALIGN, AVERIS_E_HIP. */
int32_t averis_rmsnorm_stats(const void *x, int32_t dt, int64_t rows, int64_t cols, int64_t ldx,
                             const float *weight, float eps, void *y, int64_t ldy,
                             averis_colstats *stats, void *stream);

int32_t averis_swiglu_stats(const void *gate, const void *up, int32_t dt, int64_t rows, int64_t cols,
                            int64_t ld, void *y, int64_t ldy, averis_colstats *stats, void *stream);

/* averis_split_quant of x with SPLIT from the column statistics `stats` that x's producer wrote
 * (stats->rows == rows, stats->cols == cols): the mean is the fp64 sum of the partial sums in
 * part order divided by rows (as fp32, written to `mean`), and x is read once, by the
 * quantization.  flags: AVERIS_SPLIT required; AVERIS_HADAMARD16 and AVERIS_CHECK_FINITE as in
 * averis_split_quant; AVERIS_MEAN_GIVEN not allowed (AVERIS_E_FLAGS).  NVFP4 without
 * HADAMARD16 needs stats->min and stats->max (AVERIS_E_NULL).  Given the mean it writes, every
 * output equals averis_split_quant's with AVERIS_MEAN_GIVEN and that mean (the minima and
 * maxima are exact).  Other arguments, workspace and errors as averis_split_quant; dense only. */
int32_t averis_split_quant_stats(const void *x, int32_t xdt, int64_t rows, int64_t cols,
                                 int64_t ldx, int32_t fmt, uint32_t flags,
                                 const averis_colstats *stats, float *mean,
                                 const averis_qtensor *q_row, const averis_qtensor *q_col,
                                 const averis_qtensor *q_mean, void *ws, size_t ws_bytes,
                                 void *stream);

/* -----------------------------------------------------------------------------------------
 * averis_linear_bwd_dw -- dW = Q(X_R)^T Q(D_R) + l Q(mu_X)^T Q(mu_D)   ([rainbus] 方法步骤详情:
 * the cross terms vanish because the residuals have zero column means, so only two
 * quantized GEMMs are needed).
 *  xr_t  [outer = m, k = l]  (q_col of split_quant(X))
 *  dr_t  [outer = n, k = l]  (q_col of split_quant(D))
 *  mu_x, mu_d  quantized means, both or neither (NULL, NULL = vanilla: no rank-one term).
 *        If they carry HADAMARD16 the rotation is undone before the outer product.
 *  l     the unpadded token count (the rank-one factor); must equal xr_t->k.
 *  dw    device fp32 [m, n], leading dimension n <= lddw < 2^23; n % 8 == 0.  AVERIS_ACCUMULATE: dw += result.
 * The token axis is split across workgroups with fp32 partials reduced in a fixed order.
 * ----------------------------------------------------------------------------------------- */
size_t averis_linear_bwd_dw_workspace_size(int64_t m, int64_t n, int64_t l, int32_t fmt);

int32_t averis_linear_bwd_dw(const averis_qtensor *xr_t, const averis_qtensor *dr_t,
                             const averis_qtensor *mu_x, const averis_qtensor *mu_d, int64_t l,
                             float *dw, int64_t lddw, uint32_t flags, void *ws, size_t ws_bytes,
                             void *stream);

/* =========================================================================================
 * Grouped (MoE) variants.  [rainbus] 实验结果 and 结构化数据: the 7B-A1.5B mixture-of-experts
 * model is trained with Averis; the split is applied per expert on the expert's own token
 * slice, so every group gets its own mean, residual and (NVFP4) tensor scales, and the dW
 * rank-one factor is the group's own token count.
 *
 * Groups: E >= 1 groups of consecutive token rows, group e = rows [offsets[e], offsets[e+1]),
 * offsets[0] = 0, non-decreasing, L = offsets[E] rows in total (empty groups allowed).
 *   d_offsets  device int64 [E + 1], read by the kernels (16-byte aligned);
 *   h_offsets  host int64 [E + 1] with the same values, used to size the launch and to validate.
 * Grouped operand layouts (l_e = offsets[e+1] - offsets[e]):
 *   row layout (K = features): outer = sum_e round_up(l_e, 32), k = cols; group e's rows start
 *     at sum_{e'<e} round_up(l_e', 32), so scale groups never straddle groups; rows past l_e
 *     inside a group hold zero codes and scales.
 *   column layout (K = tokens): outer = cols, k = L, k_pad = sum_e round_up(l_e, 256); group e is
 *     a [cols, round_up(l_e, 256)] operand starting at token t_e = sum_{e'<e} round_up(l_e', 256):
 *     codes at byte cols * t_e / 2, tiled scales at byte cols * t_e / g.
 *   quantized means: outer = E, k = cols (row e = group e).
 *   tensor_scale (NVFP4): one fp32 per group.
 * Stacked weights W_e [m, n] (input [E * m, n], groups of m rows, m % 32 == 0) quantized with
 * SPLIT off give exactly the two weight operands: the row layout is E stacked [m, n] operands
 * (input-gradient B) and the column layout is E stacked [n, m] operands (forward B).
 * ========================================================================================= */
size_t averis_split_quant_grouped_workspace_size(int64_t rows, int64_t cols, int32_t E, int32_t fmt,
                                                 uint32_t flags);

/* Per group exactly averis_split_quant on its rows.  means: device fp32 [E][cols].  q_row,
 * q_col, q_mean as described above (q_mean required with SPLIT). */
int32_t averis_split_quant_grouped(const void *x, int32_t xdt, int64_t cols, int64_t ldx,
                                   const int64_t *d_offsets, const int64_t *h_offsets, int32_t E,
                                   int32_t fmt, uint32_t flags, float *means,
                                   const averis_qtensor *q_row, const averis_qtensor *q_col,
                                   const averis_qtensor *q_mean, void *ws, size_t ws_bytes,
                                   void *stream);

/* Workspace of the grouped forward / input-gradient GEMMs with N output columns per group. */
size_t averis_linear_grouped_workspace_size(int64_t N, int32_t E, int32_t fmt);

/* Per group e: Y[offsets[e] + r] = 1 (Q(mu_X,e) Q(W_e)) + Q(X_R,e) Q(W_e), one launch for all
 * groups.  xr: grouped row layout [sum round_up(l_e, 32), m]; mu_x: [E, m] or NULL; w: E stacked
 * [n, m] operands (outer = E * n, n % 32 == 0; the column layout of the stacked weights).
 * y: device [L, n], element type ydt, leading dimension n <= ldy < 2^23. */
int32_t averis_linear_fwd_grouped(const averis_qtensor *xr, const averis_qtensor *mu_x,
                                  const averis_qtensor *w, const int64_t *d_offsets,
                                  const int64_t *h_offsets, int32_t E, void *y, int32_t ydt,
                                  int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* Per group e: dX[offsets[e] + r] = 1 (Q(mu_D,e) Q(W_e)^T) + Q(D_R,e) Q(W_e)^T.  dr: grouped row
 * layout [sum round_up(l_e, 32), n]; mu_d [E, n] or NULL; w: E stacked [m, n] operands
 * (outer = E * m, m % 32 == 0; the row layout of the stacked weights); dx: [L, m]. */
int32_t averis_linear_bwd_dx_grouped(const averis_qtensor *dr, const averis_qtensor *mu_d,
                                     const averis_qtensor *w, const int64_t *d_offsets,
                                     const int64_t *h_offsets, int32_t E, void *dx, int32_t dxdt,
                                     int64_t lddx, void *ws, size_t ws_bytes, void *stream);

size_t averis_linear_bwd_dw_grouped_workspace_size(int64_t m, int64_t n, int32_t E, int32_t fmt);

/* Per group e: dW_e = Q(X_R,e)^T Q(D_R,e) + l_e Q(mu_X,e)^T Q(mu_D,e).  xr_t, dr_t: grouped
 * column layouts (outer m and n); mu_x [E, m], mu_d [E, n], both or neither; dw: device fp32
 * [E][m][lddw] (group stride m * lddw).  An empty group's dW is zero (or unchanged with
 * AVERIS_ACCUMULATE). */
int32_t averis_linear_bwd_dw_grouped(const averis_qtensor *xr_t, const averis_qtensor *dr_t,
                                     const averis_qtensor *mu_x, const averis_qtensor *mu_d,
                                     const int64_t *d_offsets, const int64_t *h_offsets, int32_t E,
                                     float *dw, int64_t lddw, uint32_t flags, void *ws,
                                     size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* AVERIS_H */
