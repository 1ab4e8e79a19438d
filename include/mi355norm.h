/*
 * mi355norm.h -- C ABI of the row-wise LayerNorm / RMSNorm library (forward,
 * fused residual add, FP8 output, and the backward)
 * for AMD Instinct MI355X (gfx950, CDNA4).  Library: libmi355norm.so.
 *
 * The operations (page titles as printed on the pages they come from):
 *
 *   LayerNorm forward, per row r of x[M, N]:
 *       mean_r = (1/N) * sum_i x[r,i]
 *       var_r  = (1/N) * sum_i (x[r,i] - mean_r)^2          (biased: divide by N)
 *       rstd_r = 1 / sqrt(var_r + eps)
 *       y[r,i] = (x[r,i] - mean_r) * rstd_r * gamma[i] + beta[i]
 *     -- "CUDA 算子工程：手写 FlashAttention v2 之路", ch. 7 "LayerNorm 与 RMSNorm",
 *        section 7.1 (definition) and 7.6 (fused kernel storing mean and rstd per
 *        row for the backward pass); "T3 讲解：LayerNorm / RMSNorm 的 forward",
 *        part ② (true-N divisor, biased variance, rstd stored, fp32 statistics)
 *        and part ⑥ (mean and rstd are fp32 whatever the I/O dtype).
 *
 *   RMSNorm forward, per row r:
 *       rstd_r = 1 / sqrt((1/N) * sum_i x[r,i]^2 + eps)
 *       y[r,i] = x[r,i] * rstd_r * gamma[i]
 *     -- "CUDA 算子工程" ch. 7, section 7.5; "CUDA算子优化(2)：RMSNorm", section 1;
 *        "T3 讲解" part ③.
 *
 *   Residual add + RMSNorm (the fused step named after vLLM's
 *   fused_add_rms_norm in "CUDA 算子工程" ch. 7, sections 7.9-7.10, and
 *   "T3 讲解" part ⑤), per row r:
 *       h[r,i] = x[r,i] + residual[r,i], rounded to the I/O dtype
 *                (stored: the updated residual stream)
 *       y[r,i] = RMSNorm(h)[r,i], taken of the stored h
 *     Read as exactly what a separate add followed by rms_fwd computes.
 *
 *   FP8 output (the norm fused with the quantisation of its output for the
 *   next GEMM, "CUDA 算子工程" ch. 7, section 7.9: vLLM's static FP8
 *   variants of rms_norm and fused_add_rms_norm), per element:
 *       code = E4M3(clamp(y / scale, -448, 448))
 *     y as above, computed in fp32; E4M3 = OCP FP8 E4M3 (1 sign, 4 exponent
 *     bits with bias 7, 3 fraction bits, no infinities, max 448, NaN =
 *     S.1111.111), round-to-nearest-even, one byte per element.
 *
 * The variance is computed by a stable method (two passes over register-
 * resident data for rows that fit one workgroup, Chan's parallel merge of
 * (n, mean, M2) partials for rows split across workgroups), never by
 * E[x^2] - E[x]^2 ("CUDA 算子工程" ch. 7, sections 7.3-7.4).
 *
 * Statistics and arithmetic are fp32 for every I/O dtype; y is rounded to
 * the I/O dtype with round-to-nearest-even.
 *
 * Conventions shared by ln_fwd and rms_fwd
 * ----------------------------------------
 *   x, y      device pointers to row-major, contiguous [M, N] arrays of `dtype`.
 *   gamma     device pointer to [N] of `dtype`, or NULL meaning gamma = 1.
 *   beta      device pointer to [N] of `dtype`, or NULL meaning beta = 0
 *             (LayerNorm only; must be NULL for rms_fwd).
 *   mean      device pointer to fp32 [M], or NULL: not written
 *             (LayerNorm only; must be NULL for rms_fwd).
 *   rstd      device pointer to fp32 [M], or NULL: not written.
 *   M         number of rows, >= 0.  M == 0 returns NORM_OK and launches nothing.
 *   N         row length, 1 <= N <= 2^24 (16,777,216).
 *   eps       finite and >= 0, added to the variance (or mean square) inside
 *             the square root.  eps == 0 on a constant row gives rstd = +inf
 *             and y = NaN, as IEEE arithmetic dictates.
 *   dtype     one of norm_dtype.
 *   stream    a hipStream_t, or NULL for the null stream of the current device.
 *
 *   Every pointer must be aligned to its element size.  16-byte aligned x, y,
 *   gamma, beta with N * sizeof(dtype) a multiple of 16 take the 128-bit
 *   vector path.  When only x is off a 16-byte boundary (a view into a wider
 *   buffer), the call still takes it, x being read in aligned 16-byte
 *   blocks realigned in registers (same tile, so the same results as on an
 *   aligned copy of x; rows split across workgroups then take the two
 *   kernels).  Anything else takes an element-wise path (slower, same
 *   accuracy).  Buffers must not overlap (y
 *   may not alias x: no in-place use).
 *
 * Ownership: the caller allocates and owns every buffer and keeps it alive
 * until the stream has passed the call.  The library keeps no pointer to
 * them after return.  Rows too long for one workgroup (N > 2^16 for 2-byte
 * and N > 2^15 for 4-byte types, with 16-byte alignment; N > 2^14 without)
 * are processed in batches of rows holding about 256 MiB of x, two kernel
 * launches per batch, and use a library-owned device workspace of at most a
 * few MiB (per row of a batch: 264 bytes plus 8 bytes per chunk of the row),
 * one per (device, stream), allocated on first need and replaced by a larger
 * one when a larger call needs it (no call waits for its stream); every
 * workspace is kept until the process exits.
 *
 * Graph capture: calls on the row path launch kernels only.  Calls that use
 * the workspace (long rows, and the backward below) may be captured into a
 * HIP graph once a call at least as large has run on the capturing stream
 * (the workspace then exists, and a capture records kernel launches only:
 * no allocation, synchronisation or memset).  A captured call keeps the
 * workspace it was captured with, which stays valid after later, larger
 * calls; its replays share it with the calls on the capturing stream and
 * with the other replays of graphs captured there, so none of those may
 * overlap in time (order them, e.g. replay on the capturing stream).  See
 * also norm_fwd_noalloc.
 *
 * Errors: arguments are validated on the host before any HIP call; a bad
 * argument returns its status and touches nothing.  A launch failure returns
 * NORM_ERR_HIP.  Execution is asynchronous on `stream`: faults surface at the
 * caller's next synchronisation.  The library never changes the current
 * device.  All functions are thread-safe.
 */
#ifndef MI355NORM_H
#define MI355NORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { NORM_F32 = 0, NORM_F16 = 1, NORM_BF16 = 2 } norm_dtype;

typedef enum {
    NORM_OK = 0,
    NORM_ERR_NULL_ARG = 1,   /* x or y (or residual, residual_out) NULL, M > 0  */
    NORM_ERR_BAD_SHAPE = 2,  /* M < 0, N < 1, N > 2^24, or M * N overflows       */
    NORM_ERR_BAD_DTYPE = 3,  /* dtype not in norm_dtype                          */
    NORM_ERR_BAD_EPS = 4,    /* eps negative, NaN or infinite                    */
    NORM_ERR_BAD_ARG = 5,    /* misaligned pointer; beta or mean given to an
                                RMSNorm; a bad FP8 scale                      */
    NORM_ERR_ALIAS = 6,      /* two of the buffers overlap                       */
    NORM_ERR_HIP = 7,        /* a HIP runtime call or kernel launch failed       */
    NORM_ERR_SCRATCH = 8     /* norm_fwd_noalloc: the call needs more scratch
                                than its fixed buffer holds                    */
} norm_status;

/* LayerNorm forward.  Returns a norm_status. */
int ln_fwd(const void *x, const void *gamma, const void *beta, void *y,
           float *mean, float *rstd, int64_t M, int64_t N, float eps,
           int dtype, void *stream);

/* RMSNorm forward.  beta and mean must be NULL.  Returns a norm_status. */
int rms_fwd(const void *x, const void *gamma, const void *beta, void *y,
            float *mean, float *rstd, int64_t M, int64_t N, float eps,
            int dtype, void *stream);

/*
 * Residual add, then RMSNorm.  x, residual, y, residual_out: [M, N] of
 * `dtype`; gamma [N] or NULL; rstd fp32 [M] or NULL.  residual_out receives
 * x + residual (rounded to dtype), y the RMSNorm of it.  In-place use is
 * allowed exactly as the fused step is used in a transformer block:
 * residual_out may be residual itself and y may be x itself (the very same
 * pointers; a partial overlap, or any other overlap, is NORM_ERR_ALIAS).
 * Rows too long for one workgroup read residual_out back in a second pass
 * (so the caller must not read or write it until the stream has passed the
 * call, as for every output).  Other conventions as above.  Returns a
 * norm_status.
 */
int add_rms_fwd(const void *x, const void *residual, const void *gamma, void *y,
                void *residual_out, float *rstd, int64_t M, int64_t N, float eps,
                int dtype, void *stream);

/*
 * RMSNorm with FP8 E4M3 output.  y: [M, N] bytes (E4M3 codes); scale: the
 * static dequantisation scale (finite, > 0, with 1/scale finite, else
 * NORM_ERR_BAD_ARG); the codes are of y_norm / scale.  No in-place use.  A
 * result of exactly zero may be coded as +0 or -0.  Other conventions as for
 * rms_fwd.  Returns a norm_status.
 */
int rms_fp8_fwd(const void *x, const void *gamma, void *y, float *rstd,
                int64_t M, int64_t N, float eps, float scale, int dtype, void *stream);

/*
 * Residual add, then RMSNorm with FP8 E4M3 output: residual_out receives
 * x + residual in `dtype` (it may be residual itself), y the E4M3 codes of
 * the norm of it divided by scale.  Other conventions as for add_rms_fwd and
 * rms_fp8_fwd.  Returns a norm_status.
 */
int add_rms_fp8_fwd(const void *x, const void *residual, const void *gamma, void *y,
                    void *residual_out, float *rstd, int64_t M, int64_t N, float eps,
                    float scale, int dtype, void *stream);

/*
 * Every operation above, with row strides (non-contiguous rows, such as a
 * slice of columns of a wider matrix, without a copy).
 */
typedef enum {
    NORM_OP_LN = 0,           /* ln_fwd          */
    NORM_OP_RMS = 1,          /* rms_fwd         */
    NORM_OP_ADD_RMS = 2,      /* add_rms_fwd     */
    NORM_OP_RMS_FP8 = 3,      /* rms_fp8_fwd     */
    NORM_OP_ADD_RMS_FP8 = 4   /* add_rms_fp8_fwd */
} norm_op;

typedef struct {
    int op;                       /* norm_op                                       */
    int dtype;                    /* norm_dtype of every matrix but an FP8 y        */
    int64_t M, N;
    const void *x;                /* row r at x + r * ld_x elements                 */
    int64_t ld_x;                 /* row stride in elements, >= N; 0 means N        */
    const void *residual;         /* add_rms ops only, else NULL                    */
    int64_t ld_residual;
    const void *gamma;            /* [N] or NULL                                    */
    const void *beta;             /* [N] or NULL; LayerNorm only                    */
    void *y;
    int64_t ld_y;                 /* elements of y's type (bytes for FP8 codes)     */
    void *residual_out;           /* add_rms ops only, else NULL                    */
    int64_t ld_residual_out;
    float *mean;                  /* fp32 [M] or NULL; LayerNorm only               */
    float *rstd;                  /* fp32 [M] or NULL                               */
    float eps;
    float scale;                  /* FP8 ops only (ignored otherwise)               */
} norm_args;

/*
 * Runs args->op with the conventions of its entry point above, rows being
 * ld_* elements apart (ld_* < N, or an ld_* so large that the matrix does
 * not fit 2^63 bytes, is NORM_ERR_BAD_SHAPE; NULL args is NORM_ERR_NULL_ARG).
 * The 16-byte vector path is taken when every row start is 16-byte aligned
 * (EPV-byte for FP8 codes); for LayerNorm, RMSNorm and RMSNorm with FP8
 * output also when only the rows of x are not (any ld_x; split rows then
 * take the two kernels); otherwise the element-wise path.  Overlaps are
 * checked row by row when the two matrices share a stride or one is a
 * vector (interleaved matrices that share no byte are accepted), and over
 * their whole spans otherwise.  Returns a norm_status.
 */
int norm_fwd(const norm_args *args, void *stream);

/*
 * norm_fwd without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and conventions as norm_fwd, and the same
 * kernels, but rows too long for one workgroup always run the two-kernel
 * schedule, with their per-chunk partial statistics in a fixed 1 MiB device
 * array that the library holds on every GPU it runs on until the process
 * exits (its address is looked up on the first call on each device, with
 * that device current), instead of in a workspace it allocates.  Where
 * norm_fwd picks the two kernels the results are its bits; where it picks
 * the single pass (RMSNorm, fp32 LayerNorm; see norm_describe) the two
 * forms chunk rows differently and agree within rounding.  1 MiB covers
 * every shape of the two-kernel schedule at its default batch (at most
 * about 576 KiB of partials per batch of rows); a call needing more (a
 * larger MI355NORM_SPLIT_BATCH) returns NORM_ERR_SCRATCH, and an explicit
 * request for the single pass (MI355NORM_PATH=splitpass) NORM_ERR_BAD_ARG,
 * both before any launch.  No hipMalloc, hipFree or
 * allocating routine is called.  Calls on one GPU share the array: calls
 * that overlap in time on one GPU (different streams, or graph replays
 * overlapping eager calls) race on it and must be ordered by the caller.
 * Returns a norm_status.
 */
int norm_fwd_noalloc(const norm_args *args, void *stream);

/*
 * Backward of ln_fwd and rms_fwd ("CUDA 算子工程" ch. 7, section 7.7), from
 * the fp32 mean and rstd the forward stored per row.  With g = dy * gamma:
 *
 *   LayerNorm   xhat[r,i] = (x[r,i] - mean_r) * rstd_r
 *               dx[r,i]   = rstd_r * (g[r,i] - (1/N) sum_j g[r,j]
 *                                    - xhat[r,i] * (1/N) sum_j g[r,j] xhat[r,j])
 *               dgamma[i] = sum_r dy[r,i] * xhat[r,i],   dbeta[i] = sum_r dy[r,i]
 *   RMSNorm     dx[r,i]   = rstd_r * g[r,i]
 *                           - x[r,i] * rstd_r^3 * (1/N) sum_j g[r,j] x[r,j]
 *               dgamma[i] = sum_r dy[r,i] * x[r,i] * rstd_r
 *
 *   dy, x, dx   device pointers to contiguous [M, N] arrays of `dtype`.  dx
 *               may be exactly dy or x (in place); any other overlap of an
 *               output with an input or another output is NORM_ERR_ALIAS.
 *   gamma       [N] of `dtype`, or NULL meaning gamma = 1.
 *   mean, rstd  fp32 [M] as ln_fwd / rms_fwd wrote them (mean: LayerNorm only).
 *               Required when M > 0 (NORM_ERR_NULL_ARG otherwise).
 *   dgamma,     fp32 [N] device pointers, or NULL: not computed.  Written
 *   dbeta       (zeros when M == 0); dbeta exists for LayerNorm only.
 *   M, N        M >= 0; 1 <= N <= 2^24.  Rows up to 32768 elements (16384
 *               unless dy, x, gamma and dx rows are 16-byte aligned and N *
 *               element size is a multiple of 16) are handled one workgroup
 *               per row (fp32 rows longer than 16384 for RMSNorm and 24576
 *               for LayerNorm excepted); longer ones are split across
 *               workgroups: chunk sums, row sums, then dx and the column
 *               sums' partial rows (three kernels; dy and x read twice).
 *
 * Arithmetic is fp32; dx is rounded to `dtype` (round-to-nearest-even).
 * dgamma and dbeta are summed in a fixed order (per-workgroup partial rows,
 * then a column sum over them), so repeated calls on one device give the
 * same bits.  The partial rows (fp32 [grid, N] each; with the split rows
 * also 8 bytes per row per 512-vector chunk and 8 per row) live in a workspace the
 * library keeps per (device, stream), grown when a call needs more; growing
 * waits for the stream.  Calls run asynchronously on `stream`.  Returns a
 * norm_status.
 */
int ln_bwd(const void *dy, const void *x, const void *gamma, const float *mean, const float *rstd,
           void *dx, float *dgamma, float *dbeta, int64_t M, int64_t N, int dtype, void *stream);

int rms_bwd(const void *dy, const void *x, const void *gamma, const float *rstd, void *dx,
            float *dgamma, int64_t M, int64_t N, int dtype, void *stream);

/*
 * ln_bwd (op NORM_OP_LN) or rms_bwd (op NORM_OP_RMS) with row strides: row r
 * of dy, x and dx starts ld_* elements after row r - 1 (0 means N; ld_* < N,
 * or so large that a matrix does not fit 2^63 bytes, is NORM_ERR_BAD_SHAPE).
 * dx may be written over dy or x only with the same pointer and stride.  The
 * 16-byte vector path needs every row start 16-byte aligned.  Other
 * conventions as above; returns a norm_status.
 */
typedef struct {
    int op;                       /* NORM_OP_LN or NORM_OP_RMS                     */
    int dtype;
    int64_t M, N;
    const void *dy;
    int64_t ld_dy;
    const void *x;
    int64_t ld_x;
    const void *gamma;            /* [N] or NULL                                    */
    const float *mean;            /* fp32 [M]; LayerNorm only (NULL for RMSNorm)    */
    const float *rstd;            /* fp32 [M]                                       */
    void *dx;
    int64_t ld_dx;
    float *dgamma;                /* fp32 [N] or NULL                               */
    float *dbeta;                 /* fp32 [N] or NULL; LayerNorm only               */
} norm_bwd_args;

int norm_bwd(const norm_bwd_args *args, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *norm_status_str(int status);

/*
 * The HIP failure behind the calling thread's most recent NORM_ERR_HIP: the
 * failing call and HIP's error name and text ("" if none yet).  The string
 * belongs to the library and stays valid until that thread's next failing
 * call.
 */
const char *norm_last_error(void);

/*
 * Describe, without launching anything, how a call with these arguments
 * would be executed: path ("rows" or "split"), lanes per row, 16-byte vectors
 * per lane, workgroup size, grid size, and the vector width; for split rows
 * the mode: "pass" (one launch, x read once: RMSNorm and fp32 LayerNorm on
 * 16-byte vectors, when every chunk of a row can be resident on the current
 * device) or "two" (two kernels per batch of rows: LayerNorm with 16-bit
 * I/O, the residual add, element-wise rows, or no device present).  `op` is 0 for
 * LayerNorm, 1 for RMSNorm, 2 for residual add + RMSNorm, 3 and 4 for the
 * same two RMSNorms with FP8 output; `aligned` says whether every pointer is
 * 16-byte aligned (1) or not (0), or that only the rows of x are not (2: the
 * realigned row kernel where it applies, reported as "x=realigned").  Writes at most buflen bytes (NUL-terminated) into buf and
 * returns a norm_status.  For tests and the benchmark's reports.
 */
int norm_describe(int op, int64_t M, int64_t N, int dtype, int aligned,
                  char *buf, int buflen);

/*
 * As norm_describe, for ln_bwd (rms = 0) or rms_bwd (rms = 1): path ("bwd"
 * or "bwd_split"), lanes per row, vectors per lane, workgroup size, grid and
 * the number of partial rows of dgamma and dbeta; for split rows also the
 * mode ("three" kernels per batch, or "pass", the single pass in one launch:
 * for rows of 16-byte vectors, except LayerNorm with fp16 I/O, when a row's
 * chunks fit on the device at once and there are at least 32 rows per team
 * of them, or on request), chunks per row and rows per batch.
 */
int norm_bwd_describe(int rms, int64_t M, int64_t N, int dtype, int aligned,
                      char *buf, int buflen);

#ifdef __cplusplus
}
#endif

#endif /* MI355NORM_H */
