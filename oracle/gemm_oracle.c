/*
 * CPU oracle for the half-precision GEMM with optional bias + erf-GELU epilogue (and the
 * tutorial's element-wise vector add, oracle_vector_add, row-wise softmax, oracle_softmax,
 * and attention forward, oracle_attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or call
 * this file; only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no fusion, no reordering):
 *
 *   C[i][j] = fp16_rne( epi( sum_{k=0}^{K-1} A[i][k] * B[k][j]  (+ bias[j]) ) )
 *
 * with A (M x K) and B (K x N) row-major half-precision matrices, C (M x N) row-major
 * half precision, following "Designing High-Performance GPU Kernels with TileLang:
 * Tensor-Core GEMM, Fused Softmax, FlashAttention, and Autotuning" (thecryptopost.io
 * page), section 2 "Memory hierarchy - tiled tensor-core GEMM": make_matmul's
 * problem statement (A: (M, K), B: (K, N), C: (M, N), all float16, accumulation in
 * "float").  The oracle accumulates in fp64 instead of fp32 so that it is strictly
 * tighter than any fp32 implementation; every fp16*fp16 product is exact in fp64.
 *
 * The epilogue follows the same tutorial's fused-epilogue paragraph (ainovat.com
 * page, the paragraph that extends the matrix multiply): the bias is added to the
 * accumulator and GELU is applied before the single write of the output.  Readings
 * taken where the page is silent:
 *   - bias is one value per output column j (length N), added before GELU;
 *   - GELU is the exact form x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2));
 *   - the result is rounded to fp16 once, round-to-nearest-even, directly from fp64.
 *
 * Epilogue codes: 0 = none, 1 = bias, 2 = bias then GELU.
 *
 * fp16 <-> fp64 conversion is written out here from the IEEE 754 binary16 format
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0 encodes
 * zeros and subnormals, exponent 31 encodes infinities and NaNs).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (see oracle/__init__.py).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* Threads the OpenMP loops below will use (reported with CPU timings). */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* Threads for the following calls (for single-thread timings); n < 1 is ignored. */
void oracle_set_num_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

/* binary16 -> double, exact for every bit pattern. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);              /* zero or subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double that is an exact multiple of 1/2 or finer to the
 * nearest integer, ties to even.  n is exact (a power-of-two scaling of the input). */
static double round_half_even(double n)
{
    double fl = floor(n);
    double d = n - fl;                 /* exact: n and fl share the binade or fl = 0 */
    if (d > 0.5) return fl + 1.0;
    if (d < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* double -> binary16, IEEE round-to-nearest-even, a single rounding. */
uint16_t oracle_f64_to_f16(double x)
{
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* 65520 = 65504 + half an ulp of the top binade: at or above it, RNE gives inf. */
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a rounded count of 1024 is the smallest
         * normal, whose encoding 0x0400 is exactly 1024 in the low bits. */
        double n = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)n;
    }
    int ex;
    frexp(a, &ex);                      /* a = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;                     /* a in [2^E, 2^(E+1)), E in [-14, 15] */
    double n = round_half_even(ldexp(a, 10 - E));   /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; E += 1; }
    return sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024));
}

/* GELU(x) = x * Phi(x) with Phi the standard normal CDF.  Phi(x) = 0.5 (1 + erf(x/sqrt2))
 * = 0.5 erfc(-x/sqrt2); the erfc form is used for x < 0, where 1 + erf would cancel. */
double oracle_gelu(double x)
{
    if (x < 0.0) return 0.5 * x * erfc(-x / sqrt(2.0));
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

static double apply_epilogue(double s, double bias_j, int epi)
{
    if (epi == 0) return s;
    double v = s + bias_j;
    if (epi == 2) v = oracle_gelu(v);
    return v;
}

/* One output element: the k-ordered fp64 dot product of row i of A and column j of B,
 * then the epilogue, then one rounding to fp16. */
static uint16_t element(int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                        const uint16_t *bias, int epi, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += oracle_f16_to_f64(A[i * K + k]) * oracle_f16_to_f64(B[k * N + j]);
    double bj = (epi != 0) ? oracle_f16_to_f64(bias[j]) : 0.0;
    return oracle_f64_to_f16(apply_epilogue(s, bj, epi));
}

/* Full product.  Step 1 converts both operands to fp64 (exact).  Step 2 forms each row
 * of C: rows are independent, so they are spread over OpenMP threads; within a row every
 * element is summed over k in increasing order, exactly as element() does, so the full
 * and the sampled entry points give bit-identical values. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, const uint16_t *A, const uint16_t *B,
                const uint16_t *bias, int epi, uint16_t *C)
{
    if (M < 0 || N < 0 || K < 0 || epi < 0 || epi > 2) return 1;
    if (epi != 0 && bias == NULL && N > 0) return 1;
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *Bd = (double *)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (Ad == NULL || Bd == NULL) { free(Ad); free(Bd); return 2; }
    #pragma omp parallel for
    for (int64_t t = 0; t < M * K; ++t) Ad[t] = oracle_f16_to_f64(A[t]);
    #pragma omp parallel for
    for (int64_t t = 0; t < K * N; ++t) Bd[t] = oracle_f16_to_f64(B[t]);
    #pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = Ad[i * K + k];
                for (int64_t j = 0; j < N; ++j) acc[j] += a * Bd[k * N + j];
            }
            for (int64_t j = 0; j < N; ++j) {
                double bj = (epi != 0) ? oracle_f16_to_f64(bias[j]) : 0.0;
                C[i * N + j] = oracle_f64_to_f16(apply_epilogue(acc[j], bj, epi));
            }
        }
        free(acc);
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* Selected elements only: out[s] = C[rows[s]][cols[s]].  Used where the full product is
 * too large for the CPU (e.g. 8192^3). */
int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K, const uint16_t *A,
                        const uint16_t *B, const uint16_t *bias, int epi, int64_t count,
                        const int64_t *rows, const int64_t *cols, uint16_t *out)
{
    if (M < 0 || N < 0 || K < 0 || epi < 0 || epi > 2 || count < 0) return 1;
    if (epi != 0 && bias == NULL && count > 0) return 1;
    for (int64_t s = 0; s < count; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N) return 1;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < count; ++s)
        out[s] = element(N, K, A, B, bias, epi, rows[s], cols[s]);
    return 0;
}

/* Element-wise sum of two half-precision vectors, the tutorial's first kernel (the
 * ainovat.com page's first paragraph: a vector-add kernel whose bandwidth is compared with
 * PyTorch's).  c[i] = fp16_rne(a[i] + b[i]): the sum of two binary16 values is exact in
 * binary64 (their exponents differ by at most 39, so it needs at most 51 significant bits),
 * so this is the correctly rounded sum, one rounding. */
int oracle_vector_add(int64_t n, const uint16_t *a, const uint16_t *b, uint16_t *c)
{
    if (n < 0) return 1;
    for (int64_t i = 0; i < n; ++i)
        c[i] = oracle_f64_to_f16(oracle_f16_to_f64(a[i]) + oracle_f16_to_f64(b[i]));
    return 0;
}

/* Row-wise softmax, the tutorial's fused softmax (the ainovat.com page's third paragraph:
 * a row-wise softmax with maximum and sum reductions over each row).  For each row i of
 * the M x N half-precision input, in fp64:
 *   m = max_j x[i][j]                 (NaN entries skipped, as fmax does)
 *   e_j = exp(x[i][j] - m),  s = sum_j e_j  (j in increasing order)
 *   y[i][j] = fp16_rne(e_j / s)
 * Subtracting the row maximum changes nothing mathematically (exp(x - m) / sum exp(x - m)
 * = exp(x) / sum exp(x)) and keeps every exponent <= 0.  IEEE rules give the edge cases:
 * a row of -inf has m = -inf and -inf - -inf = NaN, so every output is NaN; a +inf entry
 * gives NaN the same way; a NaN entry makes the sum, and every output, NaN. */
int oracle_softmax(int64_t M, int64_t N, const uint16_t *x, uint16_t *y)
{
    if (M < 0 || N < 0) return 1;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t *xr = x + i * N;
        uint16_t *yr = y + i * N;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j) m = fmax(m, oracle_f16_to_f64(xr[j]));
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) s += exp(oracle_f16_to_f64(xr[j]) - m);
        for (int64_t j = 0; j < N; ++j)
            yr[j] = oracle_f64_to_f16(exp(oracle_f16_to_f64(xr[j]) - m) / s);
    }
    return 0;
}

/* Attention forward, the tutorial's FlashAttention (the ainovat.com page, the paragraph
 * on the fused FlashAttention forward kernel: scores of query and key tiles, a softmax
 * over the keys, weights applied to the value tiles, causal and non-causal, checked
 * against PyTorch's scaled dot-product attention).  This is the plain definition the
 * tiled kernel must reach; none of its tiling or online rescaling appears here.
 *
 * q: (BH, Sq, D), k and v: (BH, Sk, D), o: (BH, Sq, D), half precision, row-major, one
 * (batch, head) pair after another.  For row i of pair b, in fp64:
 *   keys j allowed: 0 <= j < Sk, and j <= i when causal (the upper-left aligned mask of
 *     PyTorch's is_causal: query i sees keys 0..i);
 *   s_j = scale * sum_{d=0}^{D-1} q[i][d] * k[j][d]      (d in increasing order)
 *   m = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j   (j in increasing order)
 *   o[i][d] = fp16_rne( sum_j p_j v[j][d] / l )
 *   lse[i]  = m + log(l)              (log of sum_j exp(s_j); may be NULL)
 *   err[i][d] = sum_j p_j |v[j][d]| / l   (may be NULL): the scale against which an fp16
 *     rounding of every weight shows in o, used by the tests to set their tolerance.
 * Subtracting m changes nothing mathematically and keeps every exponent <= 0.  Sk == 0
 * leaves the softmax undefined and is rejected (return 1). */
static void attention_row(int64_t Sk, int64_t D, const uint16_t *qi, const uint16_t *kb,
                          const uint16_t *vb, double scale, int64_t nkeys, double *sbuf,
                          uint16_t *oi, double *lse_i, double *err_i)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += oracle_f16_to_f64(qi[d]) * oracle_f16_to_f64(kb[j * D + d]);
        sbuf[j] = scale * dot;
        m = fmax(m, sbuf[j]);
    }
    double l = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        sbuf[j] = exp(sbuf[j] - m);
        l += sbuf[j];
    }
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, mag = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            const double vj = oracle_f16_to_f64(vb[j * D + d]);
            acc += sbuf[j] * vj;
            mag += sbuf[j] * fabs(vj);
        }
        oi[d] = oracle_f64_to_f16(acc / l);
        if (err_i) err_i[d] = mag / l;
    }
    if (lse_i) *lse_i = m + log(l);
    (void)Sk;
}

static int64_t allowed_keys(int64_t i, int64_t Sk, int causal)
{
    return (causal && i + 1 < Sk) ? i + 1 : Sk;
}

int oracle_attention(int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const uint16_t *q,
                     const uint16_t *k, const uint16_t *v, double scale, int causal,
                     uint16_t *o, double *lse, double *err)
{
    if (BH < 0 || Sq < 0 || Sk < 0 || D < 0) return 1;
    if (BH == 0 || Sq == 0) return 0;
    if (Sk == 0) return 1;
    #pragma omp parallel
    {
        double *sbuf = (double *)malloc((size_t)Sk * sizeof(double));
        #pragma omp for schedule(dynamic, 4) collapse(2)
        for (int64_t b = 0; b < BH; ++b)
            for (int64_t i = 0; i < Sq; ++i)
                attention_row(Sk, D, q + (b * Sq + i) * D, k + b * Sk * D, v + b * Sk * D, scale,
                              allowed_keys(i, Sk, causal), sbuf, o + (b * Sq + i) * D,
                              lse ? lse + b * Sq + i : NULL, err ? err + (b * Sq + i) * D : NULL);
        free(sbuf);
    }
    return 0;
}

/* The same rows one by one: n selected (pair, row) indices, outputs packed n x D (and n
 * for lse), each computed exactly as oracle_attention computes it. */
int oracle_attention_rows(int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const uint16_t *q,
                          const uint16_t *k, const uint16_t *v, double scale, int causal,
                          int64_t n, const int64_t *pair, const int64_t *row, uint16_t *o,
                          double *lse, double *err)
{
    if (BH < 0 || Sq < 0 || Sk <= 0 || D < 0 || n < 0) return 1;
    for (int64_t t = 0; t < n; ++t)
        if (pair[t] < 0 || pair[t] >= BH || row[t] < 0 || row[t] >= Sq) return 1;
    #pragma omp parallel
    {
        double *sbuf = (double *)malloc((size_t)Sk * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            const int64_t b = pair[t], i = row[t];
            attention_row(Sk, D, q + (b * Sq + i) * D, k + b * Sk * D, v + b * Sk * D, scale,
                          allowed_keys(i, Sk, causal), sbuf, o + t * D, lse ? lse + t : NULL,
                          err ? err + t * D : NULL);
        }
        free(sbuf);
    }
    return 0;
}

/* Element-wise helpers exposed for the oracle's own pins. */
void oracle_f16_to_f64_array(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}

void oracle_f64_to_f16_array(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(in[i]);
}

void oracle_gelu_array(int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_gelu(in[i]);
}
