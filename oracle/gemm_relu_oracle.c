/*
 * CPU oracle for the fused GEMM + ReLU with fp16 storage, and for its
 * variants: bf16 storage, B stored as (N,K), a per-column bias, no activation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (the definition, written out; no blocking or reordering):
 *
 *   for every batch b, row i < M, column j < N:
 *     s  = sum_{k=0}^{K-1} dec(A[b][i*lda + k]) * dec(B[b][k*ldb + j])
 *          accumulated in IEEE binary64, k ascending
 *     r  = s if s > 0 else +0.0                                    (ReLU)
 *     C[b][i*ldc + j] = enc(r)          binary64 -> binary16, round to nearest,
 *                                       ties to even; |r| >= 65520 -> inf
 *
 * Sources on the pages:
 *  - "TileLang paper reading" (hotelren.com page), section 2: the matmul_relu
 *    tile program: A is a (M,K) fp16 tensor, B a (K,N) fp16 tensor, the block
 *    accumulator is an fp32 fragment cleared to zero, K is walked tile by tile
 *    and added into it, the accumulator is clamped at zero with a max against
 *    0, then copied out to the fp16 C.  On a CPU the tile grid is only a pair
 *    of outer loops, so tiling does not change the value computed.
 *  - "tilelang practitioner's notes" (dpshk.com page), section 3.2: the K loop
 *    is a serial accumulation into one accumulator, and the accumulator is kept
 *    in a wider type than fp16 because fp16 accumulation is too inexact.
 * The oracle accumulates in binary64 (wider than the kernel's fp32), so it is
 * the exact sum up to binary64 rounding; the kernel is expected to agree within
 * fp32 summation error plus one fp16 rounding.
 *
 * Readings where the pages are silent:
 *  - ReLU maps s <= 0 (and NaN) to +0.0, the behaviour of max(x, 0) taken as
 *    "x if x > 0 else 0".
 *  - The fp16 store rounds to nearest even (the IEEE default conversion).
 *  - Subnormal fp16 inputs and outputs are exact (no flushing).
 *
 * Variants (oracle_gemm_ex), each a plain generalisation of the definition:
 *  - element type bf16 instead of fp16: dec and enc use the bfloat16 format
 *    (8 exponent bits, 7 stored significand bits); bf16 products are exact in
 *    binary64 too (two 8-bit significands).
 *  - B stored as an (N,K) row-major array: B(k,j) is read at B[j*ldb + k]
 *    (the (BN,BK) B tile of section 3.2 of the practitioner's notes page).
 *  - a bias vector of N values of the element type, added to every row's sum
 *    before the activation: r = act(s + bias[j]).  The fusion of neighbouring
 *    operators into the GEMM's epilogue is what section 2.2 of that page
 *    describes; the bias-add is the plainest such neighbour.
 *  - activation none (r = s) or ReLU.
 *
 * Weight-only int4 variant (oracle_gemm_w4), the W_INT4/A_FP16 dequantize
 * GEMM named in section 5 of the "TileLang paper reading" page.  The page
 * gives no format; the reading taken: the weight is an (N,K) array of signed
 * 4-bit integers q in [-8, 7] (two's complement), two per byte along k (even
 * k in the low nibble, row n at Wq[n*ldw], ldw in bytes); each group of G
 * consecutive k of row n has one scale s[n][k/G] of the element type (row n
 * at S[n*lds]); the weight's value is s * q, exactly; then
 *     C[i][j] = store(act(sum_k A[i][k] * s[j][k/G] * q[j][k] + bias[j])).
 *
 * Also exported: dec/enc on arrays (for the pins in the tests), a sampled
 * variant that computes chosen (b, i, j) outputs one by one, and the optional
 * per-element s and sum_k |A_ik * B_kj| (+ |bias_j|) used by the fp32
 * error-bound gate.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* binary16 bit pattern -> exact binary64 value. */
static double dec16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e < 31)
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    else
        v = m ? NAN : INFINITY;
    return sign ? -v : v;
}

/* Round a non-negative binary64 value q to an integer, ties to even.  q is at
 * most 2^12 here, so q - floor(q) is exact. */
static double round_half_even(double q)
{
    double f = floor(q);
    double d = q - f;
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* binary64 -> binary16 bit pattern, round to nearest, ties to even. */
static uint16_t enc16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* 65504 is the largest finite half; 65520 is the midpoint to 2^16 and ties
     * to the even neighbour, which is 2^16, i.e. infinity. */
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24.  A result of 1024 is the
         * smallest normal, whose encoding is exactly 0x0400. */
        double q = round_half_even(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    double q = round_half_even(ldexp(a, 11 - e));   /* in [1024, 2048] */
    /* biased exponent of a is (e - 1) + 15; q == 2048 carries into it. */
    uint32_t bits = ((uint32_t)(e + 14) << 10) + ((uint32_t)q - 1024u);
    return sign | (uint16_t)bits;
}

/* bfloat16 bit pattern -> exact binary64 value. */
static double decbf16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* subnormal: m * 2^-133 */
    else if (e < 255)
        v = ldexp((double)(128 + m), e - 134);     /* (1 + m/128) * 2^(e-127) */
    else
        v = m ? NAN : INFINITY;
    return sign ? -v : v;
}

/* binary64 -> bfloat16 bit pattern, round to nearest, ties to even (directly
 * from binary64: no intermediate binary32 rounding). */
static uint16_t encbf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: the quantum is 2^-133; 128 quanta are the smallest
         * normal, encoded 0x0080 */
        double q = round_half_even(ldexp(a, 133));
        return sign | (uint16_t)q;
    }
    if (isinf(a))
        return sign | 0x7f80;
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    double q = round_half_even(ldexp(a, 8 - e));    /* in [128, 256] */
    /* biased exponent of a is (e - 1) + 127; q == 256 carries into it, and a
     * carry out of the largest finite binade gives 0x7f80, infinity */
    uint32_t bits = ((uint32_t)(e + 126) << 7) + ((uint32_t)q - 128u);
    if (bits >= 0x7f80u)
        return sign | 0x7f80;
    return sign | (uint16_t)bits;
}

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { B_KN = 0, B_NK = 1 };
enum { ACT_NONE = 0, ACT_RELU = 1 };

static double dec(int dtype, uint16_t h) { return dtype == DT_BF16 ? decbf16(h) : dec16(h); }

/* The activation on the exact value, then the store in the element type. */
static uint16_t act_store(int dtype, int act, double s)
{
    double r = (act == ACT_RELU) ? ((s > 0.0) ? s : 0.0) : s;
    return dtype == DT_BF16 ? encbf16(r) : enc16(r);
}

/* ReLU on the exact accumulator, then the fp16 store. */
static uint16_t relu_store(double s)
{
    return act_store(DT_F16, ACT_RELU, s);
}

/* The K-sum for one output: a[k] * b[k], k ascending, in binary64. */
static double dot_k(const double *a, const double *b, int64_t K, double *abs_out)
{
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = a[k] * b[k];   /* exact: two 11-bit significands */
        s += p;
        sa += fabs(p);
    }
    if (abs_out)
        *abs_out = sa;
    return s;
}

/* ------------------------------------------------------------------------ */

void oracle_dec16_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dec16(in[i]);
}

void oracle_enc16_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = enc16(in[i]);
}

void oracle_relu_store_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = relu_store(in[i]);
}

void oracle_decbf16_array(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = decbf16(in[i]);
}

void oracle_encbf16_array(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = encbf16(in[i]);
}

/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *A, *B;
    uint16_t *C;
    double *S, *Sabs;         /* optional, batch*M*N, contiguous */
    int64_t M, N, K, lda, ldb, ldc, sA, sB, sC;
    int dtype, act;
    const double *bias;       /* decoded bias (N values) or NULL */
    const double *Bt;         /* this batch's B decoded and laid out as (N,K) */
    int64_t b;                /* current batch */
    int nthreads;
    int tid;
} job_t;

static void *row_worker(void *p)
{
    job_t *j = (job_t *)p;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    const uint16_t *A = j->A + j->b * j->sA;
    uint16_t *C = j->C + j->b * j->sC;
    for (int64_t i = j->tid; i < j->M; i += j->nthreads) {
        for (int64_t k = 0; k < j->K; ++k)
            arow[k] = dec(j->dtype, A[i * j->lda + k]);
        for (int64_t n = 0; n < j->N; ++n) {
            double sabs;
            double s = dot_k(arow, j->Bt + n * j->K, j->K, &sabs);
            if (j->bias) {
                s += j->bias[n];
                sabs += fabs(j->bias[n]);
            }
            C[i * j->ldc + n] = act_store(j->dtype, j->act, s);
            if (j->S) {
                int64_t o = (j->b * j->M + i) * j->N + n;
                j->S[o] = s;
                j->Sabs[o] = sabs;
            }
        }
    }
    free(arow);
    return NULL;
}

static int clamp_threads(int nthreads)
{
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 256)
        nthreads = 256;
    return nthreads;
}

/*
 * Full computation of every output.  Strides and leading dimensions are in
 * elements.  dtype: 0 fp16, 1 bf16; b_layout: 0 B is (K,N) row-major, 1 B is
 * (N,K) row-major; act: 0 none, 1 ReLU; bias: N values of the element type
 * shared by every row and batch, or NULL.  S and Sabs may be NULL; when given
 * they receive the binary64 value before the activation (sum plus bias) and
 * the sum of absolute products (plus |bias|) for every (b, i, j), laid out
 * contiguously as [batch][M][N].  Returns 0, -1 when memory runs out, -2 for
 * an unknown dtype, layout or activation.
 */
int oracle_gemm_ex(int dtype, int b_layout, int act,
                   const uint16_t *A, const uint16_t *B, uint16_t *C, const uint16_t *bias,
                   int64_t M, int64_t N, int64_t K,
                   int64_t lda, int64_t ldb, int64_t ldc,
                   int64_t sA, int64_t sB, int64_t sC, int64_t batch,
                   double *S, double *Sabs, int nthreads)
{
    if ((dtype != DT_F16 && dtype != DT_BF16) || (b_layout != B_KN && b_layout != B_NK) ||
        (act != ACT_NONE && act != ACT_RELU))
        return -2;
    nthreads = clamp_threads(nthreads);
    if (M <= 0 || N <= 0 || batch <= 0)
        return 0;
    double *Bt = (double *)malloc(sizeof(double) * (size_t)N * (size_t)(K > 0 ? K : 1));
    double *biasd = bias ? (double *)malloc(sizeof(double) * (size_t)N) : NULL;
    if (!Bt || (bias && !biasd)) {
        free(Bt);
        free(biasd);
        return -1;
    }
    for (int64_t n = 0; bias && n < N; ++n)
        biasd[n] = dec(dtype, bias[n]);
    pthread_t th[256];
    job_t jobs[256];
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *Bb = B + b * sB;
        /* a copy of B in (N,K) order, so that each output's k-loop reads
         * contiguous memory; the values and their order of use are unchanged */
        for (int64_t k = 0; k < K; ++k)
            for (int64_t n = 0; n < N; ++n)
                Bt[n * K + k] = dec(dtype, b_layout == B_KN ? Bb[k * ldb + n] : Bb[n * ldb + k]);
        int nt = (int)(M < nthreads ? M : nthreads);
        for (int t = 0; t < nt; ++t) {
            job_t *j = &jobs[t];
            j->A = A; j->B = B; j->C = C; j->S = S; j->Sabs = Sabs;
            j->M = M; j->N = N; j->K = K; j->lda = lda; j->ldb = ldb; j->ldc = ldc;
            j->sA = sA; j->sB = sB; j->sC = sC; j->Bt = Bt; j->b = b;
            j->dtype = dtype; j->act = act; j->bias = biasd;
            j->nthreads = nt; j->tid = t;
            if (nt == 1)
                row_worker(j);
            else
                pthread_create(&th[t], NULL, row_worker, j);
        }
        if (nt > 1)
            for (int t = 0; t < nt; ++t)
                pthread_join(th[t], NULL);
    }
    free(Bt);
    free(biasd);
    return 0;
}

/* The fp16 GEMM + ReLU itself: oracle_gemm_ex with fp16, (K,N) B, no bias. */
int oracle_gemm_relu_f16(const uint16_t *A, const uint16_t *B, uint16_t *C,
                         int64_t M, int64_t N, int64_t K,
                         int64_t lda, int64_t ldb, int64_t ldc,
                         int64_t sA, int64_t sB, int64_t sC, int64_t batch,
                         double *S, double *Sabs, int nthreads)
{
    return oracle_gemm_ex(DT_F16, B_KN, ACT_RELU, A, B, C, NULL, M, N, K, lda, ldb, ldc, sA, sB,
                          sC, batch, S, Sabs, nthreads);
}

/*
 * Sampled computation: out[q] = C[b][i][j] for the q-th triple (b, i, j) in
 * idx (3*n int64 values).  s_out / abs_out (optional) receive the binary64
 * value before the activation and the sum of absolute products (plus |bias|).
 * Same arithmetic as the full version.
 */
typedef struct {
    const uint16_t *A, *B, *bias;
    int64_t K, lda, ldb, sA, sB;
    int dtype, b_layout, act;
    const int64_t *idx;
    int64_t n;
    uint16_t *out;
    double *s_out, *abs_out;
    int nthreads, tid;
} sjob_t;

static void *sample_worker(void *p)
{
    sjob_t *j = (sjob_t *)p;
    int64_t K = j->K;
    double *a = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *bcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    for (int64_t q = j->tid; q < j->n; q += j->nthreads) {
        int64_t b = j->idx[3 * q], i = j->idx[3 * q + 1], c = j->idx[3 * q + 2];
        const uint16_t *Ar = j->A + b * j->sA + i * j->lda;
        const uint16_t *Bb = j->B + b * j->sB;
        for (int64_t k = 0; k < K; ++k) {
            a[k] = dec(j->dtype, Ar[k]);
            bcol[k] = dec(j->dtype, j->b_layout == B_KN ? Bb[k * j->ldb + c] : Bb[c * j->ldb + k]);
        }
        double sabs;
        double s = dot_k(a, bcol, K, &sabs);
        if (j->bias) {
            double bv = dec(j->dtype, j->bias[c]);
            s += bv;
            sabs += fabs(bv);
        }
        j->out[q] = act_store(j->dtype, j->act, s);
        if (j->s_out)
            j->s_out[q] = s;
        if (j->abs_out)
            j->abs_out[q] = sabs;
    }
    free(a);
    free(bcol);
    return NULL;
}

int oracle_gemm_ex_sampled(int dtype, int b_layout, int act,
                           const uint16_t *A, const uint16_t *B, const uint16_t *bias,
                           int64_t K, int64_t lda, int64_t ldb,
                           int64_t sA, int64_t sB,
                           const int64_t *idx, int64_t n,
                           uint16_t *out, double *s_out, double *abs_out,
                           int nthreads)
{
    if ((dtype != DT_F16 && dtype != DT_BF16) || (b_layout != B_KN && b_layout != B_NK) ||
        (act != ACT_NONE && act != ACT_RELU))
        return -2;
    nthreads = clamp_threads(nthreads);
    if (n <= 0)
        return 0;
    int nt = (int)(n < nthreads ? n : nthreads);
    pthread_t th[256];
    sjob_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        sjob_t *j = &jobs[t];
        j->A = A; j->B = B; j->bias = bias; j->K = K; j->lda = lda; j->ldb = ldb;
        j->sA = sA; j->sB = sB; j->dtype = dtype; j->b_layout = b_layout; j->act = act;
        j->idx = idx; j->n = n; j->out = out;
        j->s_out = s_out; j->abs_out = abs_out; j->nthreads = nt; j->tid = t;
        if (nt == 1)
            sample_worker(j);
        else
            pthread_create(&th[t], NULL, sample_worker, j);
    }
    if (nt > 1)
        for (int t = 0; t < nt; ++t)
            pthread_join(th[t], NULL);
    return 0;
}

int oracle_gemm_relu_f16_sampled(const uint16_t *A, const uint16_t *B,
                                 int64_t K, int64_t lda, int64_t ldb,
                                 int64_t sA, int64_t sB,
                                 const int64_t *idx, int64_t n,
                                 uint16_t *out, double *s_out, double *abs_out,
                                 int nthreads)
{
    return oracle_gemm_ex_sampled(DT_F16, B_KN, ACT_RELU, A, B, NULL, K, lda, ldb, sA, sB, idx,
                                  n, out, s_out, abs_out, nthreads);
}

/* ------------------------------------------------------------------------ */

/* The signed value of nibble `hi` (0: bits 0-3, 1: bits 4-7) of a byte. */
static int nibble_s4(uint8_t b, int hi)
{
    int v = hi ? (b >> 4) : (b & 15);
    return v >= 8 ? v - 16 : v;
}

void oracle_s4_decode_array(const uint8_t *in, int8_t *lo, int8_t *hi, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        lo[i] = (int8_t)nibble_s4(in[i], 0);
        hi[i] = (int8_t)nibble_s4(in[i], 1);
    }
}

typedef struct {
    const uint16_t *A, *S, *bias;
    const uint8_t *W;
    uint16_t *C;
    double *Sum, *Sabs;
    int64_t M, N, K, G, lda, ldw, lds, ldc;
    int dtype, act, nthreads, tid;
} w4job_t;

static void *w4_worker(void *p)
{
    w4job_t *j = (w4job_t *)p;
    int64_t K = j->K;
    double *a = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    /* threads take columns: each dequantizes its weight rows once */
    for (int64_t n = j->tid; n < j->N; n += j->nthreads) {
        for (int64_t k = 0; k < K; ++k) {
            int q = nibble_s4(j->W[n * j->ldw + k / 2], (int)(k & 1));
            w[k] = dec(j->dtype, j->S[n * j->lds + k / j->G]) * (double)q;   /* exact */
        }
        double bv = j->bias ? dec(j->dtype, j->bias[n]) : 0.0;
        for (int64_t i = 0; i < j->M; ++i) {
            for (int64_t k = 0; k < K; ++k)
                a[k] = dec(j->dtype, j->A[i * j->lda + k]);
            double sabs;
            double s = dot_k(a, w, K, &sabs);
            if (j->bias) {
                s += bv;
                sabs += fabs(bv);
            }
            j->C[i * j->ldc + n] = act_store(j->dtype, j->act, s);
            if (j->Sum) {
                j->Sum[i * j->N + n] = s;
                j->Sabs[i * j->N + n] = sabs;
            }
        }
    }
    free(a);
    free(w);
    return NULL;
}

/*
 * Weight-only int4 GEMM (see the header): A (M,K) of the element type dtype,
 * Wq the (N, ldw-byte) packed weight, S the (N, lds) scales, group size G
 * (K a multiple of G), optional bias, act 0 none / 1 ReLU.  Sum and Sabs as
 * for oracle_gemm_ex, laid out [M][N].  Returns 0, -1 (memory), -2 (mode).
 */
int oracle_gemm_w4(int dtype, int act, const uint16_t *A, const uint8_t *Wq, const uint16_t *S,
                   uint16_t *C, const uint16_t *bias, int64_t M, int64_t N, int64_t K, int64_t G,
                   int64_t lda, int64_t ldw, int64_t lds, int64_t ldc, double *Sum, double *Sabs,
                   int nthreads)
{
    if ((dtype != DT_F16 && dtype != DT_BF16) || (act != ACT_NONE && act != ACT_RELU) || G <= 0)
        return -2;
    nthreads = clamp_threads(nthreads);
    if (M <= 0 || N <= 0)
        return 0;
    int nt = (int)(N < nthreads ? N : nthreads);
    pthread_t th[256];
    w4job_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        w4job_t *j = &jobs[t];
        j->A = A; j->S = S; j->bias = bias; j->W = Wq; j->C = C; j->Sum = Sum; j->Sabs = Sabs;
        j->M = M; j->N = N; j->K = K; j->G = G; j->lda = lda; j->ldw = ldw; j->lds = lds;
        j->ldc = ldc; j->dtype = dtype; j->act = act; j->nthreads = nt; j->tid = t;
        if (nt == 1)
            w4_worker(j);
        else
            pthread_create(&th[t], NULL, w4_worker, j);
    }
    if (nt > 1)
        for (int t = 0; t < nt; ++t)
            pthread_join(th[t], NULL);
    return 0;
}
