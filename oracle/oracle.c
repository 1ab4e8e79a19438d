/*
 * oracle.c -- plain, slow CPU reference for the row-wise LayerNorm and
 * RMSNorm forward pass, in IEEE double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; it shares no code, header, table or helper with the
 * HIP kernels.  Only the test suite, the smoke check and the bench's CPU
 * baseline load it.
 *
 * Built with: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FMA contraction, no reassociation: every sum below is a plain
 * left-to-right loop, so a reader can check it against the definitions).
 *
 * Definitions followed (page titles as printed on the pages):
 *   LayerNorm  -- "CUDA 算子工程" ch. 7, section 7.1 (the LN formula: mean over
 *                 the hidden dimension, biased variance divided by H, eps inside
 *                 the square root, per-feature gamma and beta) and section 7.2
 *                 (the plain mean pass, variance pass, normalise pass).
 *                 "T3 讲解：LayerNorm / RMSNorm 的 forward", part ② (divide by
 *                 the true N, biased variance, rstd = 1/sqrt(var + eps)).
 *   RMSNorm    -- "CUDA 算子工程" ch. 7, section 7.5 (y = x / sqrt(mean(x^2) +
 *                 eps) * gamma, no mean, no beta); "CUDA算子优化(2)：RMSNorm",
 *                 section 1 (same formula, eps inside the root);
 *                 "T3 讲解", part ③.
 *   Residual add + RMSNorm -- the fused step "CUDA 算子工程" ch. 7 (sections
 *                 7.9-7.10) and "T3 讲解" part ⑤ name after vLLM's
 *                 fused_add_rms_norm: read as exactly what a separate add
 *                 (whose rounded sum is stored as the new residual) followed by
 *                 RMSNorm of that stored sum computes.
 *   FP8 output -- "CUDA 算子工程" ch. 7, section 7.9: the norm fused with the
 *                 quantisation of its output for the next GEMM (vLLM's
 *                 rms_norm_static_fp8_quant and its fused-add variant): read
 *                 as code = FP8(clamp(y / scale, +-max)) with one static fp32
 *                 scale per call, FP8 being OCP E4M3 (the format gfx950
 *                 converts to natively), round-to-nearest-even.
 *   Backward     -- "CUDA 算子工程" ch. 7, section 7.7: the LayerNorm gradients
 *                 dgamma_i = sum_n dy_i xhat_i, dbeta_i = sum_n dy_i and
 *                 dx_i = rstd (g_i - mean(g) - xhat_i mean(g xhat)) with
 *                 g = dy * gamma and xhat = (x - mean) rstd, from the mean and
 *                 rstd the forward pass stored; RMSNorm's needs one in-row sum,
 *                 of dy gamma x (its formula is the derivative of the forward
 *                 definition, worked out below).
 *   Output rounding -- round-to-nearest-even from the double result straight
 *                 to the storage type (no intermediate float rounding).  The
 *                 pages only say the result is cast to the output dtype
 *                 ("T3 讲解" part ②); RNE is the reading taken.
 *
 * Parity status: every function here is pinned by the CPU test suite against
 * values printed on the pages, closed forms, exact rational brute force and
 * independent library routines; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Storage types understood by the oracle.  F64 exists only so that the tests
 * can feed the decimal example rows of the pages exactly as printed. */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

/* ---- exact widening of one stored element to double --------------------- */

static double bf16_bits_to_double(uint16_t b)
{
    /* bfloat16 is the upper half of an IEEE binary32 word */
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double f16_bits_to_double(uint16_t h)
{
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int fr = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);                 /* zero or subnormal */
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp((double)(fr | 0x400), ex - 25);   /* 1.fraction * 2^(ex-15) */
    return sign ? -v : v;
}

static double load_elem(const void *p, int64_t i, int dtype)
{
    switch (dtype) {
    case OR_F32: return (double)((const float *)p)[i];
    case OR_F16: return f16_bits_to_double(((const uint16_t *)p)[i]);
    case OR_BF16: return bf16_bits_to_double(((const uint16_t *)p)[i]);
    case OR_F64: return ((const double *)p)[i];
    }
    return NAN;
}

/* ---- direct round-to-nearest-even from double ---------------------------- */

/*
 * Round v to a binary format with `prec` significand bits (implicit bit
 * included) and minimum normal exponent `emin` (value 2^emin).  The quantum
 * of v is 2^(e - prec) for v in [2^(e-1), 2^e), but never below the
 * subnormal quantum 2^(emin - prec + 1).  Scaling by a power of two is exact
 * in double, and rint() rounds half to even in the default rounding mode.
 * Returns the rounded value (possibly +-inf is left to the caller).
 */
static double rne_to_format(double v, int prec, int emin)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    frexp(v, &e);                        /* |v| in [2^(e-1), 2^e) */
    int qexp = e - prec;
    int qmin = emin - prec + 1;
    if (qexp < qmin)
        qexp = qmin;
    double k = ldexp(v, -qexp);          /* exact */
    double r = rint(k);                  /* nearest integer, ties to even */
    return ldexp(r, qexp);
}

static uint16_t double_to_bf16_bits(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xffc0 : 0x7fc0);
    /* bfloat16: 8 significand bits, min normal 2^-126, max (2 - 2^-7) * 2^127 */
    double r = rne_to_format(v, 8, -126);
    const double maxv = ldexp(255.0, 120);
    if (r > maxv) r = INFINITY;
    if (r < -maxv) r = -INFINITY;
    float f = (float)r;                  /* exact: r is representable */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(w >> 16);
}

static uint16_t double_to_f16_bits(double v)
{
    if (isnan(v))
        return (uint16_t)(signbit(v) ? 0xfe00 : 0x7e00);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    /* binary16: 11 significand bits, min normal 2^-14, max 65504 */
    double r = rne_to_format(a, 11, -14);
    if (r > 65504.0)
        return (uint16_t)(sign | 0x7c00);
    if (r == 0.0)
        return sign;
    int e;
    double m = frexp(r, &e);             /* r = m * 2^e, m in [0.5, 1) */
    if (e - 1 < -14) {                   /* subnormal: r = frac * 2^-24 */
        uint16_t frac = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | frac);
    }
    uint16_t ex = (uint16_t)(e - 1 + 15);
    uint16_t frac = (uint16_t)(ldexp(m, 11) - 1024.0);
    return (uint16_t)(sign | (ex << 10) | frac);
}

/* Round n doubles to the storage type `dtype`; `out` holds n elements of it. */
void oracle_round(const double *v, int64_t n, int dtype, void *out)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (dtype) {
        case OR_F32: ((float *)out)[i] = (float)v[i]; break;   /* C cast: RNE */
        case OR_F16: ((uint16_t *)out)[i] = double_to_f16_bits(v[i]); break;
        case OR_BF16: ((uint16_t *)out)[i] = double_to_bf16_bits(v[i]); break;
        case OR_F64: ((double *)out)[i] = v[i]; break;
        }
    }
}

/* Widen n stored elements of `dtype` to double (exact for every format). */
void oracle_widen(const void *in, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = load_elem(in, i, dtype);
}

/* ---- LayerNorm forward ----------------------------------------------------
 *
 * For every row r of x[M, N] (row-major):
 *   mu    = (sum_i x_i) / N
 *   var   = (sum_i (x_i - mu)^2) / N            (biased)
 *   rstd  = 1 / sqrt(var + eps)
 *   y_i   = (x_i - mu) * rstd * gamma_i + beta_i
 * gamma == NULL means gamma_i = 1, beta == NULL means beta_i = 0.
 * y, mean and rstd are written in double; mean / rstd may be NULL.
 * `eps` is the exact value the kernel receives (a float widened to double).
 * Returns 0, or -1 on a bad dtype or shape.
 */
int oracle_ln_fwd(const void *x, const void *gamma, const void *beta, int dtype,
                  int64_t M, int64_t N, double eps,
                  double *y, double *mean, double *rstd)
{
    if (dtype < OR_F32 || dtype > OR_F64 || M < 0 || N < 1)
        return -1;
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double s = 0.0;
        for (int64_t i = 0; i < N; ++i)
            s += load_elem(x, base + i, dtype);
        double mu = s / (double)N;
        double q = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double d = load_elem(x, base + i, dtype) - mu;
            q += d * d;
        }
        double var = q / (double)N;
        double rs = 1.0 / sqrt(var + eps);
        if (y) {
            for (int64_t i = 0; i < N; ++i) {
                double g = gamma ? load_elem(gamma, i, dtype) : 1.0;
                double b = beta ? load_elem(beta, i, dtype) : 0.0;
                y[base + i] = (load_elem(x, base + i, dtype) - mu) * rs * g + b;
            }
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/* ---- RMSNorm forward ------------------------------------------------------
 *
 * For every row r of x[M, N]:
 *   ms    = (sum_i x_i^2) / N
 *   rstd  = 1 / sqrt(ms + eps)
 *   y_i   = x_i * rstd * gamma_i
 * gamma == NULL means gamma_i = 1.  rstd may be NULL.  Returns 0 or -1.
 */
int oracle_rms_fwd(const void *x, const void *gamma, int dtype,
                   int64_t M, int64_t N, double eps, double *y, double *rstd)
{
    if (dtype < OR_F32 || dtype > OR_F64 || M < 0 || N < 1)
        return -1;
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double q = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double v = load_elem(x, base + i, dtype);
            q += v * v;
        }
        double ms = q / (double)N;
        double rs = 1.0 / sqrt(ms + eps);
        if (y) {
            for (int64_t i = 0; i < N; ++i) {
                double g = gamma ? load_elem(gamma, i, dtype) : 1.0;
                y[base + i] = load_elem(x, base + i, dtype) * rs * g;
            }
        }
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/* ---- residual add, then RMSNorm --------------------------------------------
 *
 * For every element of x[M, N] and res[M, N]:
 *   h_i   = x_i + res_i, rounded to the storage type (the updated residual
 *           a separate add would store)
 * then RMSNorm of the stored h, row by row, as oracle_rms_fwd:
 *   rstd  = 1 / sqrt((sum_i h_i^2) / N + eps),   y_i = h_i * rstd * gamma_i
 * h is written in the storage type (it must not be NULL), y and rstd in
 * double; gamma == NULL means gamma_i = 1; rstd may be NULL.  Returns 0 or -1.
 */
static int64_t elem_size(int dtype)
{
    return dtype == OR_F64 ? 8 : dtype == OR_F32 ? 4 : 2;
}

int oracle_add_rms_fwd(const void *x, const void *res, const void *gamma, int dtype,
                       int64_t M, int64_t N, double eps, void *h, double *y, double *rstd)
{
    if (dtype < OR_F32 || dtype > OR_F64 || M < 0 || N < 1 || !h)
        return -1;
    for (int64_t i = 0; i < M * N; ++i) {
        double s = load_elem(x, i, dtype) + load_elem(res, i, dtype);
        oracle_round(&s, 1, dtype, (char *)h + i * elem_size(dtype));
    }
    return oracle_rms_fwd(h, gamma, dtype, M, N, eps, y, rstd);
}

/* ---- FP8 (OCP E4M3) output ------------------------------------------------
 *
 * E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; normal
 * values (1 + f/8) * 2^(e - 7) for e = 1..15 except the all-ones pattern
 * S.1111.111 (NaN); subnormals (f/8) * 2^-6; no infinities; largest finite
 * value 448.  Quantisation divides by the static scale, saturates to
 * +-448, rounds to nearest even; NaN stays NaN.
 */
static uint8_t double_to_e4m3_code(double v)
{
    if (isnan(v))
        return 0x7f;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a > 448.0)
        a = 448.0;
    double r = rne_to_format(a, 4, -6);
    if (r == 0.0)
        return sign;
    int e;
    frexp(r, &e);                        /* r in [2^(e-1), 2^e) */
    if (e - 1 < -6)                      /* subnormal: r = f * 2^-9 */
        return (uint8_t)(sign | (uint8_t)ldexp(r, 9));
    uint8_t f = (uint8_t)(ldexp(r, 3 - (e - 1)) - 8.0);    /* r / 2^(e-1) = 1 + f/8 */
    return (uint8_t)(sign | (uint8_t)((e - 1 + 7) << 3) | f);
}

/* code[i] = E4M3(clamp(v[i] / scale)) for n doubles. */
void oracle_quant_e4m3(const double *v, int64_t n, double scale, uint8_t *code)
{
    for (int64_t i = 0; i < n; ++i)
        code[i] = double_to_e4m3_code(v[i] / scale);
}

/* ---- LayerNorm backward ---------------------------------------------------
 *
 * For every row r, with mean_r and rstd_r as given (the forward pass's):
 *   xhat_i = (x_i - mean_r) * rstd_r,   g_i = dy_i * gamma_i
 *   gbar   = (sum_i g_i) / N,           gxbar = (sum_i g_i * xhat_i) / N
 *   dx_i   = rstd_r * (g_i - gbar - xhat_i * gxbar)
 * and over all rows
 *   dgamma_i = sum_r dy_i * xhat_i,     dbeta_i = sum_r dy_i
 * gamma == NULL means gamma_i = 1.  dx, dgamma, dbeta are written in double
 * and may each be NULL.  Returns 0 or -1.
 */
int oracle_ln_bwd(const void *dy, const void *x, const void *gamma, int dtype, int64_t M, int64_t N,
                  const double *mean, const double *rstd, double *dx, double *dgamma, double *dbeta)
{
    if (dtype < OR_F32 || dtype > OR_F64 || M < 0 || N < 1 || !mean || !rstd)
        return -1;
    if (dgamma) for (int64_t i = 0; i < N; ++i) dgamma[i] = 0.0;
    if (dbeta) for (int64_t i = 0; i < N; ++i) dbeta[i] = 0.0;
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double sg = 0.0, sgx = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double xhat = (load_elem(x, base + i, dtype) - mean[r]) * rstd[r];
            double g = load_elem(dy, base + i, dtype) * (gamma ? load_elem(gamma, i, dtype) : 1.0);
            sg += g;
            sgx += g * xhat;
        }
        double gbar = sg / (double)N, gxbar = sgx / (double)N;
        for (int64_t i = 0; i < N; ++i) {
            double d = load_elem(dy, base + i, dtype);
            double xhat = (load_elem(x, base + i, dtype) - mean[r]) * rstd[r];
            double g = d * (gamma ? load_elem(gamma, i, dtype) : 1.0);
            if (dx) dx[base + i] = rstd[r] * (g - gbar - xhat * gxbar);
            if (dgamma) dgamma[i] += d * xhat;
            if (dbeta) dbeta[i] += d;
        }
    }
    return 0;
}

/* ---- RMSNorm backward -----------------------------------------------------
 *
 * y_i = x_i * rstd * gamma_i with rstd = (sum_j x_j^2 / N + eps)^(-1/2), so
 * d rstd / d x_j = -rstd^3 x_j / N and, with g = dy * gamma,
 *   dx_i     = rstd * g_i - x_i * rstd^3 * (sum_j g_j x_j) / N
 *   dgamma_i = sum_r dy_i * x_i * rstd_r
 * rstd_r as given (the forward pass's).  dx, dgamma may be NULL.  Returns 0
 * or -1.
 */
int oracle_rms_bwd(const void *dy, const void *x, const void *gamma, int dtype, int64_t M, int64_t N,
                   const double *rstd, double *dx, double *dgamma)
{
    if (dtype < OR_F32 || dtype > OR_F64 || M < 0 || N < 1 || !rstd)
        return -1;
    if (dgamma) for (int64_t i = 0; i < N; ++i) dgamma[i] = 0.0;
    for (int64_t r = 0; r < M; ++r) {
        int64_t base = r * N;
        double sgx = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            double g = load_elem(dy, base + i, dtype) * (gamma ? load_elem(gamma, i, dtype) : 1.0);
            sgx += g * load_elem(x, base + i, dtype);
        }
        double rs = rstd[r];
        double c = rs * rs * rs * sgx / (double)N;
        for (int64_t i = 0; i < N; ++i) {
            double d = load_elem(dy, base + i, dtype);
            double xv = load_elem(x, base + i, dtype);
            double g = d * (gamma ? load_elem(gamma, i, dtype) : 1.0);
            if (dx) dx[base + i] = rs * g - xv * c;
            if (dgamma) dgamma[i] += d * xv * rs;
        }
    }
    return 0;
}
