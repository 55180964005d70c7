/*
 * sdt oracle: a plain, slow, obviously correct CPU reference for the fp16
 * GEMM C = A.B and the M=1 GEMV y = x.B (weights stored either way round).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It is used by the test suite, by the smoke check
 * and by the benchmark's CPU-baseline leg, and by nothing else.  It shares no
 * header, codec, table or helper with the GPU library.
 *
 * What it computes (the plain definition, no reordering):
 *   C(m,n) = sum_{k=0}^{K-1} dec(A[m*lda + k]) * dec(B[n*ldb + k])
 * summed in fp64 in ascending k.  A is row-major (M x K), B is stored with K
 * contiguous ("K-major": row n of the buffer is column n of the math B), C is
 * row-major.  This is the transposed-B ("TN") product C = A @ B_T.T that the
 * FlyDSL pull request "Speed up the RDNA3 GEMM up to 1.85x by choosing the
 * tile from the shape" benchmarks (its Performance section), on the fp16
 * square shapes of "Beating hipBLASLt on a Gaming GPU" (section "The result")
 * and the M=1, K=4096, N=12288 decode shape of the mojo-baro project page
 * (section "Four rounds on the decode shape").
 *
 * Precision: every product of two binary16 values is exact in fp64 (11-bit x
 * 11-bit significands), so the only rounding is in the K-1 fp64 additions;
 * the result is far more exact than any fp32-accumulating GPU kernel.  Loop
 * order over (m, n) and the thread count never change an element's sum,
 * which is always taken in ascending k, so results are bit-identical for any
 * number of threads.
 *
 * The fp16 codec below is written from the IEEE 754-2008 binary16 definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits; exponent 0 is
 * the subnormal range with quantum 2^-24; exponent 31 is inf/NaN).  The
 * pages do not say how the GPU's fp32 results become fp16; the reading taken
 * is IEEE round-to-nearest, ties to even, with overflow to +-inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* ---- binary16 codec ---------------------------------------------------- */

double sdt_oracle_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);            /* zero and subnormals */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25); /* 1.f * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* Round x to the nearest binary16 value, ties to even.
 *
 * With E = max(floor(log2|x|), -14), every binary16 value in the binade of
 * |x| (or in the subnormal range when E = -14) is r * 2^(E-10) for an
 * integer r.  The encoding of r * 2^(E-10) is (E+14)*1024 + r for every
 * r in [0, 2048]: r < 1024 only happens for E = -14 and gives a subnormal,
 * r = 2048 gives the first value of the next binade.  So rounding reduces to
 * rounding the exact quotient |x| / 2^(E-10) to an integer. */
uint16_t sdt_oracle_f16_encode_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    double a = fabs(x);
    /* 65504 is the largest finite value; its fraction 0x3ff is odd, so the
     * midpoint 65520 between it and 2^16 rounds up, out of range. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);           /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                /* a in [2^E, 2^(E+1)) */
    if (E < -14)
        E = -14;
    double n = ldexp(a, 10 - E);   /* exact: scaling by a power of two */
    double fl = floor(n);
    double d = n - fl;             /* exact: n < 2^53 */
    double r = fl;
    if (d > 0.5 || (d == 0.5 && fmod(fl, 2.0) != 0.0))
        r = fl + 1.0;
    long bits = (long)(E + 14) * 1024L + (long)r;
    return (uint16_t)(sign | (uint16_t)bits);
}

/* ---- bfloat16 codec ------------------------------------------------------
 * The upper half of an IEEE 754 binary32: 1 sign bit, 8 exponent bits with
 * bias 127, 7 fraction bits; exponent 0 is the subnormal range with quantum
 * 2^-133, exponent 255 is inf/NaN. */

double sdt_oracle_bf16_decode(uint16_t h)
{
    int neg = (h >> 15) & 1;
    int ebits = (h >> 7) & 0xff;
    int man = h & 0x7f;
    double v;
    if (ebits == 0) {
        v = ldexp((double)man, -133);              /* zero and subnormals */
    } else if (ebits == 255) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + man), ebits - 134); /* 1.m * 2^(e-127) */
    }
    return neg ? -v : v;
}

/* Round x to the nearest bfloat16 value, ties to even.  Same construction as
 * the binary16 encoder: with P = max(floor(log2|x|), -126) every value of the
 * binade (or of the subnormal range) is q * 2^(P-7), encoded as
 * (P+126)*128 + q for q in [0, 256]. */
uint16_t sdt_oracle_bf16_encode_rne(double x)
{
    uint16_t sgn = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sgn | 0x7fc0);
    double mag = fabs(x);
    /* the largest finite value is 255 * 2^120 (odd significand), so the
     * midpoint 255.5 * 2^120 rounds up, out of range */
    if (mag >= ldexp(255.5, 120))
        return (uint16_t)(sgn | 0x7f80);
    if (mag == 0.0)
        return sgn;
    int e2;
    (void)frexp(mag, &e2);
    int P = e2 - 1;
    if (P < -126)
        P = -126;
    double q = ldexp(mag, 7 - P);   /* exact */
    double lo = floor(q);
    double rem = q - lo;            /* exact */
    double qr = lo;
    if (rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) == 1.0))
        qr = lo + 1.0;
    long code = (long)(P + 126) * 128L + (long)qr;
    return (uint16_t)(sgn | (uint16_t)code);
}

static double g_dec[65536];        /* binary16 bit pattern -> value */
static double g_dec_bf16[65536];   /* bfloat16 bit pattern -> value */
static int g_dec_ready = 0;

static void build_decode_table(void)
{
    #pragma omp critical(sdt_oracle_table)
    {
        if (!g_dec_ready) {
            for (int h = 0; h < 65536; ++h) {
                g_dec[h] = sdt_oracle_f16_decode((uint16_t)h);
                g_dec_bf16[h] = sdt_oracle_bf16_decode((uint16_t)h);
            }
            g_dec_ready = 1;
        }
    }
}

/* The decode table of element type `dtype`: 0 binary16, 1 bfloat16. */
static const double* table_of(int dtype)
{
    build_decode_table();
    return dtype == 1 ? g_dec_bf16 : (dtype == 0 ? g_dec : 0);
}

void sdt_oracle_decode_array(const uint16_t* in, double* out, int64_t n)
{
    build_decode_table();
    for (int64_t i = 0; i < n; ++i)
        out[i] = g_dec[in[i]];
}

void sdt_oracle_encode_array(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sdt_oracle_f16_encode_rne(in[i]);
}

void sdt_oracle_bf16_decode_array(const uint16_t* in, double* out, int64_t n)
{
    build_decode_table();
    for (int64_t i = 0; i < n; ++i)
        out[i] = g_dec_bf16[in[i]];
}

void sdt_oracle_bf16_encode_array(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sdt_oracle_bf16_encode_rne(in[i]);
}

int sdt_oracle_max_threads(void)
{
    return omp_get_max_threads();
}

/* ---- GEMM and GEMV ----------------------------------------------------- */

/* Every entry point below takes `dtype` (0 binary16, 1 bfloat16), which
 * only selects the decode table: the sums are the same for both.  Products
 * of two bfloat16 values are exact in fp64 as well (8-bit significands). */

/* One output element: the plain dot product of row m of A with row n of the
 * K-contiguous B buffer, in ascending k, in fp64. */
static double dot_f64(const double* dec, const uint16_t* a, const uint16_t* b, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += dec[a[k]] * dec[b[k]];
    return s;
}

/* C (fp64, row-major, ldc) = A.B for the whole M x N output.
 * Returns 0, or -1 for an invalid argument.  threads <= 0 uses the OpenMP
 * default. */
int sdt_oracle_gemm_t(int dtype, int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb,
                      double* C, int64_t ldc, int threads)
{
    const double* dec = table_of(dtype);
    if (!dec || M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N)
        return -1;
    int nt = threads > 0 ? threads : omp_get_max_threads();
    #pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            C[m * ldc + n] = dot_f64(dec, A + m * lda, B + n * ldb, K);
    return 0;
}

/* The same definition at `count` chosen output elements (rows[i], cols[i]);
 * out[i] receives C(rows[i], cols[i]).  Used where the full product is too
 * large for the host. */
int sdt_oracle_gemm_sample_t(int dtype, int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t lda,
                             const uint16_t* B, int64_t ldb,
                             int64_t count, const int64_t* rows,
                             const int64_t* cols, double* out, int threads)
{
    const double* dec = table_of(dtype);
    if (!dec || M < 0 || N < 0 || K < 0 || lda < K || ldb < K || count < 0)
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N)
            return -1;
    int nt = threads > 0 ? threads : omp_get_max_threads();
    #pragma omp parallel for schedule(dynamic, 64) num_threads(nt)
    for (int64_t i = 0; i < count; ++i)
        out[i] = dot_f64(dec, A + rows[i] * lda, B + cols[i] * ldb, K);
    return 0;
}

/* y(n) = sum_k dec(x[k]) * dec(B[n*ldb + k]) for n in [0, N): the M=1 decode
 * product of the mojo-baro page ("Four rounds on the decode shape"), with
 * the weights stored K-contiguous per output column. */
int sdt_oracle_gemv_m1_t(int dtype, int64_t N, int64_t K, const uint16_t* x,
                         const uint16_t* B, int64_t ldb, double* y, int threads)
{
    const double* dec = table_of(dtype);
    if (!dec || N < 0 || K < 0 || ldb < K)
        return -1;
    int nt = threads > 0 ? threads : omp_get_max_threads();
    #pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        const uint16_t* col = B + n * ldb;
        for (int64_t k = 0; k < K; ++k)
            s += dec[x[k]] * dec[col[k]];
        y[n] = s;
    }
    return 0;
}

/* y(n) = sum_k dec(x[k]) * dec(B[k*ldb + n]) for n in [0, N): the same decode
 * product with the weights stored the other way round, K rows of ldb >= N
 * elements, the N of one row contiguous (the "B-layout" the mojo-baro page
 * reaches by transposing the weights at load, section "Four rounds on the
 * decode shape", rounds v1-v3).  Same fp64 ascending-k sum per column. */
int sdt_oracle_gemv_kn_t(int dtype, int64_t N, int64_t K, const uint16_t* x,
                         const uint16_t* B, int64_t ldb, double* y, int threads)
{
    const double* dec = table_of(dtype);
    if (!dec || N < 0 || K < 0 || (K > 0 && ldb < N))
        return -1;
    int nt = threads > 0 ? threads : omp_get_max_threads();
    #pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += dec[x[k]] * dec[B[k * ldb + n]];
        y[n] = s;
    }
    return 0;
}
