/*
 * oracle_gemm.c -- plain CPU reference for the multi-precision square GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or constant with the GPU path.
 *
 * What it computes: C = A * B, written out as the textbook triple loop.
 *   - "Hand-Written PTX Tensor-Core GEMM Kernels: A Multi-Precision Study on
 *     NVIDIA L4": the abstract and Section I (Introduction) define the work as
 *     GEMM in FP16, INT8 and INT4; Section II-A states the operation as
 *     D = AB + C (here with C = 0); Section VI says the quantized kernels
 *     return INT32 accumulations with no dequantization or scaling.
 *   - Listing 2 of the same page (the m16n8k64 .row.col .s4 instruction)
 *     fixes the operand roles: A is read along its rows ("row"), B along its
 *     columns ("col"), both contiguous in K, and the 4-bit type is signed.
 *   - "PTX Programming from Your First Kernel to Tensor Cores", section
 *     "Multiply one tile with a full warp": FP16 inputs, FP32 accumulators,
 *     with a worked 16x8x16 example that the tests check.
 *
 * Accumulation precision: integers in int64 (exact for every size this
 * library accepts), FP16 in fp64.  A product of two binary16 values is exact
 * in fp64 (11+11 significant bits), so only the fp64 summation rounds.
 * Alongside each FP16 result the oracle returns S = sum_k |a_ik * b_kj|, the
 * scale of the per-element error bound |C - R| <= 1e-3 * S.
 *
 * Layout (the library's operand contract; the pages leave C's layout open and
 * the reading taken is row-major):
 *   A[i*lda + k]      A is M x K row-major
 *   B[j*ldb + k]      B is K x N column-major ("non-transposed" B)
 *   C[i*ldc + j]      C is M x N row-major
 * INT4: two signed 4-bit values per byte along K; element k of a row sits in
 * byte k/2, in the low nibble when k is even and the high nibble when k is
 * odd; lda/ldb count 4-bit elements (the pages do not give the nibble order;
 * low-nibble-first is the reading taken).
 *
 * The *_rowb functions take B row-major instead: element (k, j) at
 * B[k*ldb + j] with ldb >= N, the "transposed B" layout of the paper's
 * Section IV-D loader ablation (Run 4), which it finds slower.  INT4 B then
 * packs two values per byte along N: element j of row k sits in byte j/2 of
 * that row, low nibble for even j.
 *
 * Parallelism: output rows are split over POSIX threads; each element is the
 * same sequential k loop, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds
 * zero and the subnormals fraction * 2^-24; exponent 31 holds inf and NaN. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

/* Signed 4-bit element k of a packed row (two's complement, low nibble = even k). */
static int s4_at(const uint8_t *row, int64_t k)
{
    uint8_t byte = row[k >> 1];
    int v = (k & 1) ? (byte >> 4) : (byte & 0x0f);
    return v < 8 ? v : v - 16;
}

/* Element (k, j) of B in either layout. */
static double b_f16(const void *B, int64_t ldb, int rowmajor, int64_t k, int64_t j)
{
    const uint16_t *b = (const uint16_t *)B;
    return oracle_half_to_double(rowmajor ? b[k * ldb + j] : b[j * ldb + k]);
}

static int64_t b_i8(const void *B, int64_t ldb, int rowmajor, int64_t k, int64_t j)
{
    const int8_t *b = (const int8_t *)B;
    return rowmajor ? b[k * ldb + j] : b[j * ldb + k];
}

static int64_t b_i4(const void *B, int64_t ldb, int rowmajor, int64_t k, int64_t j)
{
    const uint8_t *b = (const uint8_t *)B;
    return rowmajor ? s4_at(b + k * (ldb / 2), j) : s4_at(b + j * (ldb / 2), k);
}

/* ----------------------------------------------------------------------- */
/* Full-matrix products, row-parallel.                                      */

enum prec { P_F16, P_I8, P_I4 };

struct job {
    enum prec p;
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const void *B;
    int64_t ldb;
    int b_rowmajor; /* B layout: 0 column-major (K contiguous), 1 row-major */
    void *C;        /* int64_t* (int) or double* R (f16) */
    double *S;      /* f16 only */
    int64_t ldc;
    int64_t row0, row1;
};

static void one_row(const struct job *jb, int64_t i)
{
    int64_t j, k;
    const int rm = jb->b_rowmajor;
    if (jb->p == P_F16) {
        const uint16_t *a = (const uint16_t *)jb->A + i * jb->lda;
        double *r = (double *)jb->C + i * jb->ldc;
        double *s = jb->S + i * jb->ldc;
        for (j = 0; j < jb->N; ++j) {
            double acc = 0.0, mag = 0.0;
            for (k = 0; k < jb->K; ++k) {
                double prod = oracle_half_to_double(a[k]) * b_f16(jb->B, jb->ldb, rm, k, j);
                acc += prod;
                mag += fabs(prod);
            }
            r[j] = acc;
            s[j] = mag;
        }
    } else if (jb->p == P_I8) {
        const int8_t *a = (const int8_t *)jb->A + i * jb->lda;
        int64_t *c = (int64_t *)jb->C + i * jb->ldc;
        for (j = 0; j < jb->N; ++j) {
            int64_t acc = 0;
            for (k = 0; k < jb->K; ++k)
                acc += (int64_t)a[k] * b_i8(jb->B, jb->ldb, rm, k, j);
            c[j] = acc;
        }
    } else {
        const uint8_t *a = (const uint8_t *)jb->A + i * (jb->lda / 2);
        int64_t *c = (int64_t *)jb->C + i * jb->ldc;
        for (j = 0; j < jb->N; ++j) {
            int64_t acc = 0;
            for (k = 0; k < jb->K; ++k)
                acc += (int64_t)s4_at(a, k) * b_i4(jb->B, jb->ldb, rm, k, j);
            c[j] = acc;
        }
    }
}

static void *run_rows(void *arg)
{
    const struct job *jb = (const struct job *)arg;
    for (int64_t i = jb->row0; i < jb->row1; ++i)
        one_row(jb, i);
    return NULL;
}

static int run(struct job base, int nthreads)
{
    if (base.M < 0 || base.N < 0 || base.K < 0)
        return ORACLE_EINVAL;
    if (base.M == 0 || base.N == 0)
        return ORACLE_OK;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > base.M)
        nthreads = (int)base.M;
    struct job *jobs = (struct job *)calloc((size_t)nthreads, sizeof(struct job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return ORACLE_EINVAL;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].row0 = base.M * t / nthreads;
        jobs[t].row1 = base.M * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_rows, &jobs[t]);
    run_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return ORACLE_OK;
}

/* FP16 inputs, fp64 result R and magnitude sum S (both M x N, row stride ldr). */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                    const uint16_t *B, int64_t ldb, double *R, double *S, int64_t ldr,
                    int nthreads)
{
    struct job jb = {P_F16, M, N, K, A, lda, B, ldb, 0, R, S, ldr, 0, 0};
    return run(jb, nthreads);
}

/* INT8 inputs, exact int64 sums. */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                   const int8_t *B, int64_t ldb, int64_t *C, int64_t ldc, int nthreads)
{
    struct job jb = {P_I8, M, N, K, A, lda, B, ldb, 0, C, NULL, ldc, 0, 0};
    return run(jb, nthreads);
}

/* Packed INT4 inputs (K, lda, ldb in 4-bit elements; lda, ldb even), exact int64 sums. */
int oracle_gemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                   const uint8_t *B, int64_t ldb, int64_t *C, int64_t ldc, int nthreads)
{
    if ((lda & 1) || (ldb & 1))
        return ORACLE_EINVAL;
    struct job jb = {P_I4, M, N, K, A, lda, B, ldb, 0, C, NULL, ldc, 0, 0};
    return run(jb, nthreads);
}

/* The same three products with B row-major (element (k, j) at B[k*ldb + j],
 * ldb >= N; INT4 packed two per byte along N, ldb in 4-bit elements). */
int oracle_gemm_f16_rowb(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb, double *R, double *S, int64_t ldr,
                         int nthreads)
{
    struct job jb = {P_F16, M, N, K, A, lda, B, ldb, 1, R, S, ldr, 0, 0};
    return run(jb, nthreads);
}

int oracle_gemm_i8_rowb(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                        const int8_t *B, int64_t ldb, int64_t *C, int64_t ldc, int nthreads)
{
    struct job jb = {P_I8, M, N, K, A, lda, B, ldb, 1, C, NULL, ldc, 0, 0};
    return run(jb, nthreads);
}

int oracle_gemm_i4_rowb(int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda,
                        const uint8_t *B, int64_t ldb, int64_t *C, int64_t ldc, int nthreads)
{
    if ((lda & 1) || (ldb & 1))
        return ORACLE_EINVAL;
    struct job jb = {P_I4, M, N, K, A, lda, B, ldb, 1, C, NULL, ldc, 0, 0};
    return run(jb, nthreads);
}

/* ----------------------------------------------------------------------- */
/* Single entries C[rows[t]][cols[t]] for t < count: the same sums, one at  */
/* a time, for checking sampled outputs of products too large to form.     */

int oracle_entries_f16(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                       int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                       double *R, double *S)
{
    for (int64_t t = 0; t < count; ++t) {
        const uint16_t *a = A + rows[t] * lda;
        const uint16_t *b = B + cols[t] * ldb;
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = oracle_half_to_double(a[k]) * oracle_half_to_double(b[k]);
            acc += prod;
            mag += fabs(prod);
        }
        R[t] = acc;
        S[t] = mag;
    }
    return ORACLE_OK;
}

int oracle_entries_i8(int64_t K, const int8_t *A, int64_t lda, const int8_t *B,
                      int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                      int64_t *C)
{
    for (int64_t t = 0; t < count; ++t) {
        const int8_t *a = A + rows[t] * lda;
        const int8_t *b = B + cols[t] * ldb;
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k)
            acc += (int64_t)a[k] * (int64_t)b[k];
        C[t] = acc;
    }
    return ORACLE_OK;
}

int oracle_entries_i4(int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                      int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                      int64_t *C)
{
    if ((lda & 1) || (ldb & 1))
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < count; ++t) {
        const uint8_t *a = A + rows[t] * (lda / 2);
        const uint8_t *b = B + cols[t] * (ldb / 2);
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k)
            acc += (int64_t)s4_at(a, k) * (int64_t)s4_at(b, k);
        C[t] = acc;
    }
    return ORACLE_OK;
}

/* Single entries with B row-major (layout as for the *_rowb products). */
int oracle_entries_f16_rowb(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                            int64_t ldb, int64_t count, const int64_t *rows,
                            const int64_t *cols, double *R, double *S)
{
    for (int64_t t = 0; t < count; ++t) {
        const uint16_t *a = A + rows[t] * lda;
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double prod = oracle_half_to_double(a[k]) * b_f16(B, ldb, 1, k, cols[t]);
            acc += prod;
            mag += fabs(prod);
        }
        R[t] = acc;
        S[t] = mag;
    }
    return ORACLE_OK;
}

int oracle_entries_i8_rowb(int64_t K, const int8_t *A, int64_t lda, const int8_t *B,
                           int64_t ldb, int64_t count, const int64_t *rows,
                           const int64_t *cols, int64_t *C)
{
    for (int64_t t = 0; t < count; ++t) {
        const int8_t *a = A + rows[t] * lda;
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k)
            acc += (int64_t)a[k] * b_i8(B, ldb, 1, k, cols[t]);
        C[t] = acc;
    }
    return ORACLE_OK;
}

int oracle_entries_i4_rowb(int64_t K, const uint8_t *A, int64_t lda, const uint8_t *B,
                           int64_t ldb, int64_t count, const int64_t *rows,
                           const int64_t *cols, int64_t *C)
{
    if ((lda & 1) || (ldb & 1))
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < count; ++t) {
        const uint8_t *a = A + rows[t] * (lda / 2);
        int64_t acc = 0;
        for (int64_t k = 0; k < K; ++k)
            acc += (int64_t)s4_at(a, k) * b_i4(B, ldb, 1, k, cols[t]);
        C[t] = acc;
    }
    return ORACLE_OK;
}

/* ----------------------------------------------------------------------- */
/* Dequantizing epilogue for the integer products.                          */
/*                                                                          */
/* The paper ("Hand-Written PTX Tensor-Core GEMM Kernels ...", Section VI)  */
/* returns INT32 sums without dequantization or scaling; this is the step   */
/* that follows it in an inference pipeline.  The library's definition is   */
/*     C[i][j] = ((float)S_ij * scale_a[i]) * scale_b[j]                    */
/* in IEEE binary32 arithmetic (round to nearest even, in that order), then */
/* optionally rounded to binary16 (round to nearest even, overflow to inf). */
/* S_ij is the exact integer sum computed above.                            */

/* binary32 -> binary16 bits, round to nearest even, from the formats'
 * definitions (no library conversion). */
uint16_t oracle_float_to_half(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    int expo = (int)((x >> 23) & 0xff);
    uint32_t mant = x & 0x7fffffu;
    if (expo == 0xff)                              /* inf or NaN */
        return (uint16_t)(sign | 0x7c00u | (mant ? 0x200u : 0u));
    int e = expo - 127;                            /* unbiased exponent */
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);         /* overflow */
    uint32_t sig = mant | (expo ? 0x800000u : 0u); /* 24-bit significand */
    /* value = sig * 2^(e - 23); a half keeps 11 significant bits, or fewer
     * below 2^-14 (subnormals, quantum 2^-24) */
    int shift;
    if (e >= -14)
        shift = 13;                                /* keep the top 11 of 24 bits */
    else
        shift = 13 + (-14 - e);                    /* subnormal: quantum 2^-24 */
    if (expo == 0 || shift > 24 + 1)
        return (uint16_t)sign;                     /* below half of the smallest subnormal */
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1u;                                   /* round to nearest, ties to even */
    if (e >= -14) {
        /* q in [2^10, 2^11]; a carry to 2^11 moves to the next binade */
        int he = e + 15;
        if (q == 0x800u) {
            q = 0x400u;
            he += 1;
        }
        if (he >= 31)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | ((uint32_t)he << 10) | (q & 0x3ffu));
    }
    /* subnormal: q counts 2^-24; q == 2^10 is the smallest normal */
    return (uint16_t)(sign | q);
}

static float dequant(int64_t s, float sa, float sb)
{
    volatile float c = (float)s; /* volatile: one binary32 rounding per step */
    c = c * sa;
    c = c * sb;
    return c;
}

/* Dequantize int64 sums S (M x N, row stride lds) into C: binary32 when
 * half_out == 0 (C is float*), binary16 bits when half_out != 0 (uint16_t*). */
int oracle_dequant(int64_t M, int64_t N, const int64_t *S, int64_t lds, const float *scale_a,
                   const float *scale_b, void *C, int64_t ldc, int half_out)
{
    if (M < 0 || N < 0)
        return ORACLE_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            float c = dequant(S[i * lds + j], scale_a[i], scale_b[j]);
            if (half_out)
                ((uint16_t *)C)[i * ldc + j] = oracle_float_to_half(c);
            else
                ((float *)C)[i * ldc + j] = c;
        }
    return ORACLE_OK;
}

/* The same per-element dequantization for n listed entries: C[t] from the
 * sum S[t] with the row scale sa[t] and the column scale sb[t]. */
int oracle_dequant_entries(int64_t n, const int64_t *S, const float *sa, const float *sb, void *C,
                           int half_out)
{
    if (n < 0)
        return ORACLE_EINVAL;
    for (int64_t t = 0; t < n; ++t) {
        float c = dequant(S[t], sa[t], sb[t]);
        if (half_out)
            ((uint16_t *)C)[t] = oracle_float_to_half(c);
        else
            ((float *)C)[t] = c;
    }
    return ORACLE_OK;
}
