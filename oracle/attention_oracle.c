/*
 * CPU oracle for the fused attention forward (scaled dot-product attention).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library.
 *
 * The pages name fused attention kernels (FlashAttention, MLA) among the tile
 * programs they measure ("TileLang paper reading" page, section 5; the
 * "80-line MLA article" page) but give no formula.  The reading taken is the
 * standard definition, written out: for every batch b, head h and query i,
 * with kv = h / (H / Hkv) the key/value head that query head h reads,
 *
 *   s_j   = scale * sum_d Q[b][i][h][d] * K[b][j][kv][d]    (binary64, d ascending)
 *   keys j visible to i: all j < Sk, or with `causal` only j <= i + (Sk - Sq)
 *   p_j   = exp(s_j - max_visible s) / sum_visible exp(s - max s)
 *   O[b][i][h][d] = enc16( sum_j p_j * V[b][j][kv][d] )     (binary64, j ascending)
 *
 * Q, O are fp16 (bit patterns) laid out (batch, seq, heads, head_dim), K, V
 * (batch, seq, kv_heads, head_dim), contiguously; kv_heads = heads is
 * multi-head attention, fewer key/value heads each shared by a group of
 * consecutive query heads is grouped-query attention (one: multi-query).  A
 * query with no visible key (causal, Sk < Sq) gets O = 0.
 * exp is the C library's binary64 exp.  The result is exact up to binary64
 * rounding; the GPU kernel (fp32 scores and sums, an online maximum,
 * exp2-based exponentials, fp16 probabilities) is expected to agree within a
 * tolerance derived from those steps.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <unistd.h>

static double a_dec16(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e < 31)
        v = ldexp((double)(1024 + m), e - 25);
    else
        v = m ? NAN : INFINITY;
    return sign ? -v : v;
}

static double a_rhe(double q)
{
    double f = floor(q), d = q - f;
    if (d > 0.5)
        return f + 1.0;
    if (d < 0.5)
        return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

static uint16_t a_enc16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14))
        return sign | (uint16_t)a_rhe(ldexp(a, 24));
    int e;
    frexp(a, &e);
    double q = a_rhe(ldexp(a, 11 - e));
    return sign | (uint16_t)(((uint32_t)(e + 14) << 10) + ((uint32_t)q - 1024u));
}

typedef struct {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    double *rowmax, *rowsum;   /* optional, [b][h][i] */
    int64_t B, Sq, Sk, H, Hkv, D;
    double scale;
    int causal, nthreads, tid;
} ajob_t;

static void *attn_worker(void *p)
{
    ajob_t *j = (ajob_t *)p;
    const int64_t D = j->D, Sk = j->Sk, H = j->H, Hkv = j->Hkv, group = H / Hkv;
    double *q = (double *)malloc(sizeof(double) * (size_t)D);
    double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    const int64_t rows = j->B * H * j->Sq;
    for (int64_t r = j->tid; r < rows; r += j->nthreads) {
        const int64_t b = r / (H * j->Sq), h = (r / j->Sq) % H, i = r % j->Sq;
        for (int64_t d = 0; d < D; ++d)
            q[d] = a_dec16(j->Q[((b * j->Sq + i) * H + h) * D + d]);
        int64_t visible = Sk;
        if (j->causal) {
            visible = i + (Sk - j->Sq) + 1;
            if (visible < 0)
                visible = 0;
            if (visible > Sk)
                visible = Sk;
        }
        double mx = -INFINITY;
        for (int64_t k = 0; k < visible; ++k) {
            const uint16_t *kr = j->K + ((b * Sk + k) * Hkv + h / group) * D;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                acc += q[d] * a_dec16(kr[d]);
            s[k] = j->scale * acc;
            if (s[k] > mx)
                mx = s[k];
        }
        double sum = 0.0;
        for (int64_t k = 0; k < visible; ++k) {
            s[k] = exp(s[k] - mx);
            sum += s[k];
        }
        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t k = 0; k < visible; ++k) {
            const uint16_t *vr = j->V + ((b * Sk + k) * Hkv + h / group) * D;
            const double pk = s[k] / sum;
            for (int64_t d = 0; d < D; ++d)
                o[d] += pk * a_dec16(vr[d]);
        }
        for (int64_t d = 0; d < D; ++d)
            j->O[((b * j->Sq + i) * H + h) * D + d] = a_enc16(o[d]);
        if (j->rowmax) {
            j->rowmax[(b * H + h) * j->Sq + i] = mx;
            j->rowsum[(b * H + h) * j->Sq + i] = sum;
        }
    }
    free(q);
    free(s);
    free(o);
    return NULL;
}

/* Returns 0, or -2 for a bad size (kv_heads must divide heads). */
int oracle_attention_gqa_f16(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                             uint16_t *O, int64_t B, int64_t Sq, int64_t Sk, int64_t H,
                             int64_t Hkv, int64_t D, double scale, int causal, double *rowmax,
                             double *rowsum, int nthreads)
{
    if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || D <= 0)
        return -2;
    if (H == 0)
        return 0;
    if (Hkv <= 0 || H % Hkv != 0)
        return -2;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 256)
        nthreads = 256;
    const int64_t rows = B * H * Sq;
    if (rows == 0)
        return 0;
    int nt = (int)(rows < nthreads ? rows : nthreads);
    pthread_t th[256];
    ajob_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        ajob_t *j = &jobs[t];
        j->Q = Q; j->K = K; j->V = V; j->O = O; j->rowmax = rowmax; j->rowsum = rowsum;
        j->B = B; j->Sq = Sq; j->Sk = Sk; j->H = H; j->Hkv = Hkv; j->D = D; j->scale = scale;
        j->causal = causal; j->nthreads = nt; j->tid = t;
        if (nt == 1)
            attn_worker(j);
        else
            pthread_create(&th[t], NULL, attn_worker, j);
    }
    if (nt > 1)
        for (int t = 0; t < nt; ++t)
            pthread_join(th[t], NULL);
    return 0;
}

/* Multi-head attention: as many key/value heads as query heads. */
int oracle_attention_f16(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O,
                         int64_t B, int64_t Sq, int64_t Sk, int64_t H, int64_t D, double scale,
                         int causal, double *rowmax, double *rowsum, int nthreads)
{
    return oracle_attention_gqa_f16(Q, K, V, O, B, Sq, Sk, H, H, D, scale, causal, rowmax, rowsum,
                                    nthreads);
}

/*
 * Latent-attention decode (the MLA decode the pages measure: the "TileLang
 * paper reading" page, section 5, and the "80-line MLA article" page, which
 * give its head size of 512 + 64 but no formula).  The reading taken is the
 * absorbed DeepSeek form, written out: every cached token j of sequence b
 * holds one row c_j of Dl + Dr fp16 values, the first Dl a latent vector
 * shared by all heads as key and as value, the last Dr a rotary key part;
 * each query head h holds q of Dl + Dr values (latent part, then rotary
 * part), and with n = seqlens[b] (all Sk when seqlens is NULL)
 *
 *   s_j = scale * sum_{d < Dl+Dr} q[d] * c_j[d]      (binary64, d ascending)
 *   p_j = exp(s_j - max_{j<n} s) / sum_{j<n} exp(s - max s)
 *   O[b][h][d] = enc16( sum_{j<n} p_j * c_j[d] )     (d < Dl; binary64, j ascending)
 *
 * Q is (batch, heads, Dl + Dr), the cache KV (batch, Sk, Dl + Dr) and O
 * (batch, heads, Dl), contiguously; n = 0 gives O = 0.  rowmax / rowsum,
 * when given, receive max s and the sum of exp(s - max s) per (b, h).
 * Returns 0, or -2 for a bad size or a seqlens entry outside [0, Sk].
 */
typedef struct {
    const uint16_t *Q, *KV;
    uint16_t *O;
    const int32_t *seqlens;
    double *rowmax, *rowsum;
    int64_t B, H, Sk, Dl, Dr;
    double scale;
    int nthreads, tid;
} mjob_t;

static void *mla_worker(void *p)
{
    mjob_t *j = (mjob_t *)p;
    const int64_t Dq = j->Dl + j->Dr, Sk = j->Sk;
    double *q = (double *)malloc(sizeof(double) * (size_t)Dq);
    double *s = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)(j->Dl > 0 ? j->Dl : 1));
    for (int64_t r = j->tid; r < j->B * j->H; r += j->nthreads) {
        const int64_t b = r / j->H, h = r % j->H;
        const int64_t n = j->seqlens ? j->seqlens[b] : Sk;
        for (int64_t d = 0; d < Dq; ++d)
            q[d] = a_dec16(j->Q[(b * j->H + h) * Dq + d]);
        double mx = -INFINITY;
        for (int64_t k = 0; k < n; ++k) {
            const uint16_t *c = j->KV + (b * Sk + k) * Dq;
            double acc = 0.0;
            for (int64_t d = 0; d < Dq; ++d)
                acc += q[d] * a_dec16(c[d]);
            s[k] = j->scale * acc;
            if (s[k] > mx)
                mx = s[k];
        }
        double sum = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            s[k] = exp(s[k] - mx);
            sum += s[k];
        }
        for (int64_t d = 0; d < j->Dl; ++d)
            o[d] = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            const uint16_t *c = j->KV + (b * Sk + k) * Dq;
            const double pk = s[k] / sum;
            for (int64_t d = 0; d < j->Dl; ++d)
                o[d] += pk * a_dec16(c[d]);
        }
        for (int64_t d = 0; d < j->Dl; ++d)
            j->O[(b * j->H + h) * j->Dl + d] = a_enc16(o[d]);
        if (j->rowmax) {
            j->rowmax[b * j->H + h] = mx;
            j->rowsum[b * j->H + h] = sum;
        }
    }
    free(q);
    free(s);
    free(o);
    return NULL;
}

int oracle_mla_decode_f16(const uint16_t *Q, const uint16_t *KV, uint16_t *O,
                          const int32_t *seqlens, int64_t B, int64_t H, int64_t Sk, int64_t Dl,
                          int64_t Dr, double scale, double *rowmax, double *rowsum, int nthreads)
{
    if (B < 0 || H < 0 || Sk < 0 || Dl < 0 || Dr < 0 || Dl + Dr <= 0)
        return -2;
    if (seqlens)
        for (int64_t b = 0; b < B; ++b)
            if (seqlens[b] < 0 || seqlens[b] > Sk)
                return -2;
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > 256)
        nthreads = 256;
    const int64_t rows = B * H;
    if (rows == 0)
        return 0;
    int nt = (int)(rows < nthreads ? rows : nthreads);
    pthread_t th[256];
    mjob_t jobs[256];
    for (int t = 0; t < nt; ++t) {
        mjob_t *j = &jobs[t];
        j->Q = Q; j->KV = KV; j->O = O; j->seqlens = seqlens;
        j->rowmax = rowmax; j->rowsum = rowsum;
        j->B = B; j->H = H; j->Sk = Sk; j->Dl = Dl; j->Dr = Dr; j->scale = scale;
        j->nthreads = nt; j->tid = t;
        if (nt == 1)
            mla_worker(j);
        else
            pthread_create(&th[t], NULL, mla_worker, j);
    }
    if (nt > 1)
        for (int t = 0; t < nt; ++t)
            pthread_join(th[t], NULL);
    return 0;
}
