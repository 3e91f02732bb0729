/*
 * oracle.c -- plain CPU reference for the fused GEMM + epilogue path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the GPU
 * library.
 *
 * Every step is a separate pass over fp64 arrays, in the order the pages
 * give, with no blocking, fusion or reordering:
 *
 *   unpack   (W4 only)  code = high / low nibble of each packed byte
 *                       (page "Fusion Thinking", Pattern 3 -- Dequant + GEMM)
 *   dequant  (W4 only)  w = (code - zero_point) * s[k / group][n]
 *                       (same section: zero-point 8 and per-group scales)
 *   gemm                acc[m][n] = sum_k A[m][k] * B[k][n], k ascending
 *   scale               t = alpha * acc                 (page "Fusion and
 *   C term              t += beta * C                    Epilogues", Epilogue
 *                                                        fusion: the axpby
 *                                                        ending alpha*AB+beta*C)
 *   bias                t += bias[n]    (pages "Kernel fusion" (Concept) and
 *   activation          u = act(t)       "Fusion and Epilogues": bias, then
 *   residual            v = u + R        activation, then residual add)
 *   swiglu              v = silu(g) * u  (page "Fusion Thinking", Pattern 2)
 *   add + rmsnorm       r = a + x; y = r / sqrt(mean(r^2) + eps) * w
 *                       (page "Fusion Thinking", Pattern 1)
 *
 * All arithmetic is IEEE fp64 (build with -ffp-contract=off); storage types
 * (fp32, bf16 bit patterns, fp64) are widened exactly on read.  Results are
 * returned in fp64 with no final rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2

#define OR_ACT_NONE 0
#define OR_ACT_RELU 1
#define OR_ACT_GELU_TANH 2
#define OR_ACT_SILU 3

/* Exact widening of one stored element to fp64. */
static double or_load(const void *p, int dtype, int64_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)p)[i];
    if (dtype == OR_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[i];
}

static int or_dtype_ok(int d) { return d == OR_F32 || d == OR_BF16 || d == OR_F64; }

/*
 * GEMM pass.  acc is a dense M x N fp64 array.
 *   A element (m, k) is at A[m * lda + k].
 *   b_layout 0 ("KN"): B element (k, n) at B[k * ldb + n];
 *   b_layout 1 ("NK"): B element (k, n) at B[n * ldb + k].
 * Each acc[m][n] is the sum over k = 0 .. K-1, in that order, of the
 * products A[m][k] * B[k][n].
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_gemm(int M, int N, int K, const void *A, int a_dtype, int64_t lda,
                const void *B, int b_dtype, int b_layout, int64_t ldb, double *acc)
{
    if (M < 0 || N < 0 || K < 0 || !or_dtype_ok(a_dtype) || !or_dtype_ok(b_dtype))
        return -1;
    if (b_layout != 0 && b_layout != 1)
        return -1;
    double *Bd = (double *)malloc(sizeof(double) * ((size_t)K * (size_t)N + 1));
    if (!Bd)
        return -1;
    /* widen B once into a dense [K][N] array (exact) */
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Bd[k * N + n] = b_layout == 0 ? or_load(B, b_dtype, k * ldb + n)
                                          : or_load(B, b_dtype, n * ldb + k);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *row = acc + m * (int64_t)N;
        for (int64_t n = 0; n < N; ++n)
            row[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = or_load(A, a_dtype, m * lda + k);
            const double *brow = Bd + k * (int64_t)N;
            for (int64_t n = 0; n < N; ++n)
                row[n] += a * brow[n];
        }
    }
    free(Bd);
    return 0;
}

/* Scale pass: t[i] = alpha * t[i]. */
void oracle_scale(int64_t count, double *t, double alpha)
{
    for (int64_t i = 0; i < count; ++i)
        t[i] = alpha * t[i];
}

/* Matrix term: t[m][n] += coef * X[m][n]  (X element (m, n) at X[m * ldx + n]). */
int oracle_add_matrix(int M, int N, double *t, const void *X, int x_dtype, int64_t ldx, double coef)
{
    if (!or_dtype_ok(x_dtype))
        return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            t[m * N + n] += coef * or_load(X, x_dtype, m * ldx + n);
    return 0;
}

/* Bias pass: t[m][n] += bias[n]. */
int oracle_add_bias(int M, int N, double *t, const void *bias, int b_dtype)
{
    if (!or_dtype_ok(b_dtype))
        return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            t[m * N + n] += or_load(bias, b_dtype, n);
    return 0;
}

/* Logistic sigmoid 1 / (1 + e^-x). */
static double or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Activation pass, elementwise:
 *   relu      max(t, 0)
 *   gelu_tanh 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3)))
 *             (tanh form of GELU, Hendrycks & Gimpel 2016)
 *   silu      t * sigmoid(t)   (the SiLU of the SwiGLU pattern)
 */
int oracle_activation(int64_t count, double *t, int act)
{
    const double c = sqrt(2.0 / M_PI);
    switch (act) {
    case OR_ACT_NONE:
        return 0;
    case OR_ACT_RELU:
        for (int64_t i = 0; i < count; ++i)
            t[i] = t[i] > 0.0 ? t[i] : 0.0;
        return 0;
    case OR_ACT_GELU_TANH:
        for (int64_t i = 0; i < count; ++i) {
            const double x = t[i];
            t[i] = 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
        }
        return 0;
    case OR_ACT_SILU:
        for (int64_t i = 0; i < count; ++i)
            t[i] = t[i] * or_sigmoid(t[i]);
        return 0;
    default:
        return -1;
    }
}

/* Elementwise product: out[i] = a[i] * b[i]. */
void oracle_mul(int64_t count, double *out, const double *a, const double *b)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = a[i] * b[i];
}

/*
 * Unpack pass.  Wq is K rows of N/2 bytes (row stride ldq bytes); each byte
 * holds the codes of two adjacent columns.  High nibble first (default):
 * code[k][2j] = byte >> 4, code[k][2j+1] = byte & 0xF.  lo_first swaps them.
 * codes is a dense K x N uint8 array.
 */
int oracle_w4_unpack(int K, int N, const uint8_t *Wq, int64_t ldq, int lo_first, uint8_t *codes)
{
    if (K < 0 || N < 0 || (N & 1))
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N / 2; ++j) {
            const uint8_t b = Wq[k * ldq + j];
            const uint8_t hi = (uint8_t)(b >> 4), lo = (uint8_t)(b & 0x0F);
            codes[k * N + 2 * j] = lo_first ? lo : hi;
            codes[k * N + 2 * j + 1] = lo_first ? hi : lo;
        }
    return 0;
}

/*
 * Dequant pass.  W[k][n] = (code[k][n] - zero_point) * s[k / group][n],
 * exact in fp64; scale element (g, n) at scales[g * lds + n].
 */
int oracle_w4_dequant(int K, int N, const uint8_t *codes, const void *scales, int s_dtype,
                      int64_t lds, int group, int zero_point, double *W)
{
    if (group <= 0 || K % group || !or_dtype_ok(s_dtype))
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const double s = or_load(scales, s_dtype, (k / group) * lds + n);
            W[k * N + n] = ((double)codes[k * N + n] - (double)zero_point) * s;
        }
    return 0;
}

/*
 * 8-bit weights (one code per byte, W stored [K, N] like dense B), the wider
 * formats next to the pages' int4 loader ("Fusion Thinking", Pattern 3: codes
 * dequantised with a per-group scale before the product):
 *   fmt 1, unsigned 8-bit integer:  W[k][n] = (q - zero_point) * s[k / group][n]
 *   fmt 2, OCP fp8 E4M3 ("fn": no infinities; S.1111.111 is NaN):
 *          W[k][n] = value(q) * s[k / group][n], where for sign bit S, exponent
 *          field E (4 bits, bias 7) and mantissa field F (3 bits)
 *            E = 0:  (-1)^S * 2^-6 * F / 8         (subnormal)
 *            E > 0:  (-1)^S * 2^(E - 7) * (1 + F / 8)
 * Exact in fp64.
 */
static double or_fp8_e4m3(uint8_t q)
{
    const int sign = q >> 7, e = (q >> 3) & 15, f = q & 7;
    double v;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)f / 8.0, -6);
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 7);
    return sign ? -v : v;
}

int oracle_w8_dequant(int K, int N, const uint8_t *Wq, int64_t ldq, int fmt, int zero_point,
                      const void *scales, int s_dtype, int64_t lds, int group, double *W)
{
    if (group <= 0 || K % group || !or_dtype_ok(s_dtype) || (fmt != 1 && fmt != 2))
        return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t q = Wq[k * ldq + n];
            const double s = or_load(scales, s_dtype, (k / group) * lds + n);
            const double v = fmt == 1 ? (double)q - (double)zero_point : or_fp8_e4m3(q);
            W[k * N + n] = v * s;
        }
    return 0;
}

/*
 * Fused residual add + RMSNorm reference, one row at a time:
 *   r = a + x                  (stored to resid)
 *   rrms = 1 / sqrt(sum(r^2) / N + eps)
 *   y = r * rrms * w[n]        (stored to out)
 */
int oracle_add_rmsnorm(int M, int N, const void *a, int a_dtype, const void *x, int x_dtype,
                       const void *w, int w_dtype, double eps, double *resid, double *out)
{
    if (!or_dtype_ok(a_dtype) || !or_dtype_ok(x_dtype) || !or_dtype_ok(w_dtype) || N <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double r = or_load(a, a_dtype, m * N + n) + or_load(x, x_dtype, m * N + n);
            resid[m * N + n] = r;
            ss += r * r;
        }
        const double rrms = 1.0 / sqrt(ss / (double)N + eps);
        for (int64_t n = 0; n < N; ++n)
            out[m * N + n] = resid[m * N + n] * rrms * or_load(w, w_dtype, n);
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
