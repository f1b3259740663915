/*
 * CPU oracle for the dense matrix product C = A·B (row-major operands).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library or
 * its Python binding) may link, load or call this file; only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark use it.  It shares
 * no code, header or constant with the HIP kernels.
 *
 * What it computes (the plain definition of the product, written out):
 *   The subject of the pages is the matrix multiply itself: the ladder of
 *   kernels on "Bare Metal Bard" (page 1, first paragraph) and "Writing a
 *   Fast Matmul in CUDA, Step by Step" (vidyal.ai, Part 5) all compute
 *       C[i][j] = sum_{k<K} A[i][k] * B[k][j]
 *   and the correctness gate of this library additionally needs the
 *   magnitude sum
 *       D[i][j] = sum_{k<K} |A[i][k] * B[k][j]|
 *   so that a result c is judged by max_ij |c_ij - C_ij| / D_ij.
 *
 * Precision: every product of two fp32 (or two bf16) values is exact in
 * fp64 (24 + 24 significand bits <= 53), so the only rounding is the fp64
 * running sum, whose error is at most K * 2^-53 * D[i][j].  bf16 operands
 * are given as raw 16-bit patterns and decoded here (the pattern is the top
 * half of an IEEE binary32 value).
 *
 * Loop order is i-k-j (a row of B is contiguous), rows are split into
 * contiguous static blocks over POSIX threads.  Each output row is computed
 * by exactly one thread in a fixed order, so the result does not depend on
 * the thread count.  Build with -O2 -ffp-contract=off and no fast-math so the
 * compiler neither fuses the multiply into the add nor reorders the sums.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* Compile-time planted mistakes, used only by the oracle's own sensitivity
 * tests (the pins must reject each of them).  The default build defines none.
 *   ORACLE_MUTANT_DROP_LAST_K  - the last k term is left out of both sums
 *   ORACLE_MUTANT_TRANSPOSE_B  - B is read as B[j][k] instead of B[k][j]
 *   ORACLE_MUTANT_SIGNED_D     - D sums signed products instead of |products|
 *   ORACLE_MUTANT_BF16_SWAP    - bf16 decode takes the pattern byte-swapped
 *   ORACLE_MUTANT_IGNORE_TA    - a transposed A is read as if it were not
 *   ORACLE_MUTANT_BATCH_B0     - every product of a batch reads the first B
 *   ORACLE_MUTANT_F16_BIAS     - fp16 decode uses an exponent bias of 16
 *   ORACLE_MUTANT_E4M3_NAN     - e4m3 decode treats exponent 15 as infinity/NaN
 *   ORACLE_MUTANT_F16_ROWS_BF16 - the fp16 row-sampled entry decodes its
 *                                 operands as bf16 patterns
 *   ORACLE_MUTANT_MX_BLOCK16   - MX scales applied per 16 elements of K, not 32
 *   ORACLE_MUTANT_E8M0_BIAS    - E8M0 scale exponent biased by 128, not 127
 */

static double decode_bf16(uint16_t bits)
{
#ifdef ORACLE_MUTANT_BF16_SWAP
    bits = (uint16_t)((bits >> 8) | (bits << 8));
#endif
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* IEEE binary16 pattern -> fp64: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is zero or subnormal (fraction * 2^-24), 31 is
 * infinity or NaN.  Written from the format's definition. */
static double decode_f16(uint16_t bits)
{
    int bias = 15;
#ifdef ORACLE_MUTANT_F16_BIAS
    bias = 16;
#endif
    const int sign = bits >> 15, e = (bits >> 10) & 31, f = bits & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, 1 - bias - 10);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - bias - 10);
    return sign ? -v : v;
}

/* 8-bit floating point patterns (the OCP 8-bit formats), decoded from their
 * definitions.  e4m3: sign, 4-bit exponent (bias 7), 3-bit fraction; no
 * infinities, the only NaN patterns are S.1111.111 (so exponent 15 carries
 * ordinary values up to 448).  e5m2: sign, 5-bit exponent (bias 15), 2-bit
 * fraction, IEEE-style infinities and NaNs at exponent 31.  Exponent 0 is
 * zero or subnormal in both. */
static double decode_e4m3(uint8_t bits)
{
    const int sign = bits >> 7, e = (bits >> 3) & 15, f = bits & 7;
    double v;
#ifdef ORACLE_MUTANT_E4M3_NAN
    if (e == 15) return f ? NAN : (sign ? -INFINITY : INFINITY);
#endif
    if (e == 15 && f == 7) return NAN;
    if (e == 0) v = ldexp((double)f, 1 - 7 - 3);
    else v = ldexp((double)(8 + f), e - 7 - 3);
    return sign ? -v : v;
}

static double decode_e5m2(uint8_t bits)
{
    const int sign = bits >> 7, e = (bits >> 2) & 31, f = bits & 3;
    double v;
    if (e == 0) v = ldexp((double)f, 1 - 15 - 2);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(4 + f), e - 15 - 2);
    return sign ? -v : v;
}

/* OCP microscaling (MX) block scale, E8M0: an 8-bit biased exponent and
 * nothing else, the value 2^(e - 127); the all-ones pattern is NaN.  One
 * scale covers a block of 32 consecutive elements along K. */
static double decode_e8m0(uint8_t e)
{
    int bias = 127;
#ifdef ORACLE_MUTANT_E8M0_BIAS
    bias = 128;
#endif
    if (e == 255) return NAN;
    return ldexp(1.0, (int)e - bias);
}

static int64_t mx_block(int64_t k)
{
#ifdef ORACLE_MUTANT_MX_BLOCK16
    return k / 16;
#else
    return k / 32;
#endif
}

enum { KIND_F32 = 0, KIND_BF16 = 1, KIND_F16 = 2, KIND_E4M3 = 3, KIND_E5M2 = 4 };

static double decode_byte(int kind, uint8_t bits)
{
    return kind == KIND_E4M3 ? decode_e4m3(bits) : decode_e5m2(bits);
}

static double decode_kind(int kind, uint16_t bits)
{
    return kind == KIND_F16 ? decode_f16(bits) : decode_bf16(bits);
}

typedef struct {
    int kind;
    int64_t M, N, K;
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    double *C; double *D; int64_t ldo;
    const int64_t *rows;   /* NULL: output row r is input row r */
    int64_t nrows;
    int64_t r0, r1;        /* this worker's block of output rows */
    int ta, tb;            /* operand stored transposed: A as K x M, B as N x K */
    int kind_b;            /* B's element type when it differs from A's (8-bit formats) */
    const double *Bd;      /* B's values decoded once into a K x N fp64 array, or NULL */
    const uint8_t *sa, *sb;  /* MX block scales of A and B (E8M0), or NULL: scale of block
                                kb of row i of A at sa[kb * ld_sa + i], of column n of B
                                at sb[kb * ld_sb + n] */
    int64_t ld_sa, ld_sb;
} job_t;

/* Element (i, k) of the M x K left factor.  Stored as written (row i at
 * A + i*lda) or transposed (stored K x M: element (i, k) at A[k*lda + i]). */
static double load_a(const job_t *j, int64_t i, int64_t k)
{
    int64_t at = j->ta ? k * j->lda + i : i * j->lda + k;
#ifdef ORACLE_MUTANT_IGNORE_TA
    /* row-major indexing of transposed storage, wrapped to stay inside it */
    if (j->ta) at = (i * j->lda + k) % ((j->K - 1) * j->lda + j->M);
#endif
    if (j->kind == KIND_F32)
        return (double)((const float *)j->A)[at];
    if (j->kind >= KIND_E4M3) {
        const double v = decode_byte(j->kind, ((const uint8_t *)j->A)[at]);
        return j->sa ? v * decode_e8m0(j->sa[mx_block(k) * j->ld_sa + i]) : v;
    }
    return decode_kind(j->kind, ((const uint16_t *)j->A)[at]);
}

/* Forced inline: it runs once per multiply, and a call there halves the
 * oracle's speed. */
static inline __attribute__((always_inline))
double load_b_stored(const job_t *j, int64_t k, int64_t n)
{
#ifdef ORACLE_MUTANT_TRANSPOSE_B
    int64_t t = k; k = n % j->K; n = t % j->N;
#endif
    /* Element (k, n) of the K x N right factor; stored as written (row k at
     * B + k*ldb) or transposed (stored N x K: element (k, n) at B[n*ldb + k]). */
    int64_t at = j->tb ? n * j->ldb + k : k * j->ldb + n;
    if (j->kind == KIND_F32)
        return (double)((const float *)j->B)[at];
    if (j->kind >= KIND_E4M3) {
        const double v = decode_byte(j->kind_b, ((const uint8_t *)j->B)[at]);
        return j->sb ? v * decode_e8m0(j->sb[mx_block(k) * j->ld_sb + n]) : v;
    }
    return decode_kind(j->kind, ((const uint16_t *)j->B)[at]);
}

/* One output row: acc and den start at zero, then for each k the row of B is
 * scaled by A[i][k] and added (signed into C, absolute into D).  Row k of B
 * comes from the decoded copy when there is one (fp16 and 8-bit patterns,
 * whose decode is the slow part, and any B stored transposed; the copy holds
 * exactly the values load_b_stored returns), else straight from storage. */
static void one_row(const job_t *j, int64_t i, double *crow, double *drow)
{
    for (int64_t n = 0; n < j->N; ++n) { crow[n] = 0.0; drow[n] = 0.0; }
    int64_t kend = j->K;
#ifdef ORACLE_MUTANT_DROP_LAST_K
    if (kend > 0) kend -= 1;
#endif
    const double *bd = j->Bd;
    for (int64_t k = 0; k < kend; ++k) {
        double a = load_a(j, i, k);
        for (int64_t n = 0; n < j->N; ++n) {
            double p = a * (bd ? bd[k * j->N + n] : load_b_stored(j, k, n));
            crow[n] += p;
#ifdef ORACLE_MUTANT_SIGNED_D
            drow[n] += p;
#else
            drow[n] += fabs(p);
#endif
        }
    }
}

static void *worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int64_t i = j->rows ? j->rows[r] : r;
        one_row(j, i, j->C + r * j->ldo, j->D + r * j->ldo);
    }
    return NULL;
}

static int default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

static int run(job_t base, int nthreads)
{
    if (base.M < 0 || base.N < 0 || base.K < 0 || base.nrows < 0) return 1;
    if (base.nrows == 0 || base.N == 0) return 0;
    if (base.ldo < base.N) return 1;
    if (base.K > 0 && (base.lda < (base.ta ? base.M : base.K) ||
                       base.ldb < (base.tb ? base.K : base.N))) return 1;
    if (base.rows)
        for (int64_t r = 0; r < base.nrows; ++r)
            if (base.rows[r] < 0 || base.rows[r] >= base.M) return 1;
    if (nthreads <= 0) nthreads = default_threads();
    if (nthreads > base.nrows) nthreads = (int)base.nrows;
    if (nthreads > 1024) nthreads = 1024;

    double *bd = NULL;
    if (base.K > 0 && (base.kind == KIND_F16 || base.kind >= KIND_E4M3 || base.tb)) {
        bd = (double *)malloc(sizeof(double) * (size_t)base.K * (size_t)base.N);
        if (!bd) return 2;
        for (int64_t k = 0; k < base.K; ++k)
            for (int64_t n = 0; n < base.N; ++n) bd[k * base.N + n] = load_b_stored(&base, k, n);
        base.Bd = bd;
    }

    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!jobs || !tids) { free(jobs); free(tids); free(bd); return 2; }
    int64_t per = base.nrows / nthreads, extra = base.nrows % nthreads, r = 0;
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].r0 = r;
        r += per + (t < extra ? 1 : 0);
        jobs[t].r1 = r;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, worker, &jobs[t]) != 0) { rc = 2; break; }
        started = t;
    }
    if (rc == 0) worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    free(jobs);
    free(tids);
    free(bd);
    return rc;
}

/* Full product.  C and D are M x N row-major fp64 with leading dimension ldo.
 * Returns 0 on success, 1 on invalid arguments, 2 on a thread/alloc failure.
 * nthreads <= 0 uses every online core. */
int oracle_gemm_f32(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    double *C, double *D, int64_t ldo, int nthreads)
{
    job_t j = {KIND_F32, M, N, K, A, lda, B, ldb, C, D, ldo, NULL, M, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
    return run(j, nthreads);
}

int oracle_gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                     double *C, double *D, int64_t ldo, int nthreads)
{
    job_t j = {KIND_BF16, M, N, K, A, lda, B, ldb, C, D, ldo, NULL, M, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
    return run(j, nthreads);
}

/* Selected rows only: output row r (of nrows) is the product's row rows[r].
 * Used where the full product is too slow on a CPU (8192-cubed workloads). */
int oracle_gemm_f32_rows(int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda, const float *B, int64_t ldb,
                         const int64_t *rows, int64_t nrows,
                         double *C, double *D, int64_t ldo, int nthreads)
{
    job_t j = {KIND_F32, M, N, K, A, lda, B, ldb, C, D, ldo, rows, nrows, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
    return run(j, nthreads);
}

int oracle_gemm_bf16_rows(int64_t M, int64_t N, int64_t K,
                          const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                          const int64_t *rows, int64_t nrows,
                          double *C, double *D, int64_t ldo, int nthreads)
{
    job_t j = {KIND_BF16, M, N, K, A, lda, B, ldb, C, D, ldo, rows, nrows, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
    return run(j, nthreads);
}

/* A strided batch of products with either factor optionally stored
 * transposed: for b < batch,
 *     C_b[i][j] = sum_k op(A)_b[i][k] * op(B)_b[k][j]
 * where op(A)_b is the M x K matrix at A + b*sa (stored M x K with row
 * stride lda, or K x M when ta != 0) and op(B)_b the K x N matrix at
 * B + b*sb (stored K x N, or N x K when tb != 0).  These are the layouts a
 * training step's backward pass multiplies ("Bare Metal Bard", page 1,
 * second paragraph: the GPT trained on the same kernels, whose gradients
 * are products with one factor transposed).  A stride of 0 reuses one
 * matrix for every product.  C and D are batch consecutive M x ldo fp64
 * matrices.  kind is 0 for fp32 operands, 1 for bf16 patterns.  Same
 * return codes as above. */
int oracle_gemm_batched(int kind, int ta, int tb, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, int64_t sa,
                        const void *B, int64_t ldb, int64_t sb, int64_t batch,
                        double *C, double *D, int64_t ldo, int nthreads)
{
    if (kind != KIND_F32 && kind != KIND_BF16 && kind != KIND_F16) return 1;
    if (batch < 0 || sa < 0 || sb < 0 || M < 0 || N < 0) return 1;
    const int64_t es = kind == KIND_F32 ? 4 : 2;
    for (int64_t b = 0; b < batch; ++b) {
        int64_t bb = b;
#ifdef ORACLE_MUTANT_BATCH_B0
        bb = 0;
#endif
        job_t j = {kind, M, N, K,
                   (const char *)A + b * sa * es, lda,
                   (const char *)B + bb * sb * es, ldb,
                   C + b * M * ldo, D + b * M * ldo, ldo, NULL, M, 0, 0, ta != 0, tb != 0, 0, NULL, NULL, NULL, 0, 0};
        int rc = run(j, nthreads);
        if (rc != 0) return rc;
    }
    return 0;
}

/* fp16 operands (raw IEEE binary16 patterns): the full product and
 * selected rows, as for bf16 above. */
int oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                    double *C, double *D, int64_t ldo, int nthreads)
{
    job_t j = {KIND_F16, M, N, K, A, lda, B, ldb, C, D, ldo, NULL, M, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
    return run(j, nthreads);
}

int oracle_gemm_f16_rows(int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                         const int64_t *rows, int64_t nrows,
                         double *C, double *D, int64_t ldo, int nthreads)
{
#ifdef ORACLE_MUTANT_F16_ROWS_BF16
    job_t j = {KIND_BF16, M, N, K, A, lda, B, ldb, C, D, ldo, rows, nrows, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
#else
    job_t j = {KIND_F16, M, N, K, A, lda, B, ldb, C, D, ldo, rows, nrows, 0, 0, 0, 0, 0, NULL, NULL, NULL, 0, 0};
#endif
    return run(j, nthreads);
}

/* bf16 pattern -> fp64, exposed so tests can pin the decoder on its own. */
void oracle_decode_bf16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_bf16(in[i]);
}

/* 8-bit operands: A in format fmt_a, B in fmt_b (0: e4m3, 1: e5m2), either
 * stored transposed, a strided batch as in oracle_gemm_batched (strides and
 * leading dimensions in bytes = elements). */
int oracle_gemm_fp8_batched(int fmt_a, int fmt_b, int ta, int tb, int64_t M, int64_t N,
                            int64_t K, const uint8_t *A, int64_t lda, int64_t sa,
                            const uint8_t *B, int64_t ldb, int64_t sb, int64_t batch,
                            double *C, double *D, int64_t ldo, int nthreads)
{
    if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return 1;
    if (batch < 0 || sa < 0 || sb < 0 || M < 0 || N < 0) return 1;
    for (int64_t b = 0; b < batch; ++b) {
        job_t j = {KIND_E4M3 + fmt_a, M, N, K, A + b * sa, lda, B + b * sb, ldb,
                   C + b * M * ldo, D + b * M * ldo, ldo, NULL, M, 0, 0, ta != 0, tb != 0,
                   KIND_E4M3 + fmt_b, NULL, NULL, NULL, 0, 0};
        int rc = run(j, nthreads);
        if (rc != 0) return rc;
    }
    return 0;
}

/* 8-bit operands with MX block scales (OCP microscaling: every 32
 * consecutive elements along K of a row of A, or of a column of B, share
 * one E8M0 scale): A stored M x K as written, B given transposed (stored
 * N x K, row n at Bt + n*ldb),
 *     C[i][n] = sum_k (a_ik * 2^(SA[k/32][i] - 127)) * (b_kn * 2^(SB[k/32][n] - 127))
 * with the scale of block kb of row i of A at SA[kb*ld_sa + i] and of
 * column n of B at SB[kb*ld_sb + n].  Each scaled element is exact in fp64
 * (a power of two times a value of at most 4 significant bits), so the only
 * rounding is the fp64 sum, as for the unscaled product. */
int oracle_gemm_mxfp8(int fmt_a, int fmt_b, int64_t M, int64_t N, int64_t K,
                      const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ld_sa,
                      const uint8_t *Bt, int64_t ldb, const uint8_t *SB, int64_t ld_sb,
                      double *C, double *D, int64_t ldo, int nthreads)
{
    if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return 1;
    if (M < 0 || N < 0 || K < 0 || ld_sa < M || ld_sb < N) return 1;
    if (K > 0 && (!SA || !SB)) return 1;
    job_t j = {KIND_E4M3 + fmt_a, M, N, K, A, lda, Bt, ldb, C, D, ldo, NULL, M, 0, 0, 0, 1,
               KIND_E4M3 + fmt_b, NULL, SA, SB, ld_sa, ld_sb};
    return run(j, nthreads);
}

/* 8-bit pattern -> fp64 (fmt 0: e4m3, 1: e5m2), exposed to pin the decoders. */
void oracle_decode_fp8(int fmt, const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_byte(KIND_E4M3 + fmt, in[i]);
}

/* E8M0 scale pattern -> fp64, exposed for the same reason. */
void oracle_decode_e8m0(const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_e8m0(in[i]);
}

/* fp16 pattern -> fp64, exposed for the same reason. */
void oracle_decode_f16(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_f16(in[i]);
}
