/*
 * CPU oracle for the k-quant prefill GEMM (q4_K / q6_K weights x q8_1 activations).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this
 * file: it exists so that tests, the smoke check and the benchmark's CPU-baseline leg
 * can judge the HIP kernels. It shares no code, header, table or helper with them.
 *
 * It is deliberately plain and slow: every quantity is decoded from the block bytes
 * one element at a time, integer sub-block sums are exact int32 loops, and the scale
 * fold is done in fp64, where every individual term is exact (see the fold below), so
 * the only rounding is the fp64 summation itself.
 *
 * Sources (the pages of the minfer CUDA optimisation log):
 *   [r28]  "31 - r28 - Direction-A raw-nibble NB kernel, 2 blocks/SM"
 *   [r29]  "32 - r29 - NB kd-loop unroll"
 *   [r14]  "19 - r14 - B fragments via ldmatrix + widened scale reads"
 *   [r40]  "43 - r40 - __launch_bounds__(256,3) third resident block"
 * and, where the pages do not print a layout, the public GGUF block formats.
 *
 * Pinned by tests/test_oracle.py (closed forms, layout sweeps, brute force, invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QO_QK_K 256
#define QO_Q4K_BYTES 144
#define QO_Q6K_BYTES 210
#define QO_QK8 32

/* ------------------------------------------------------------------------------ */
/* IEEE binary16 conversions, written out from the format definition.             */
/* ------------------------------------------------------------------------------ */

/* binary16 bits -> exact double. */
double qo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);      /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* float -> binary16 bits, round to nearest, ties to even; overflow -> inf. */
uint16_t qo_f32_to_f16(float xf)
{
    double x = (double)xf;                 /* exact */
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(a))
        return sign | 0x7e00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer number of 2^-24 units, rounded to even */
        double q = rint(a * ldexp(1.0, 24)); /* a*2^24 is exact; rint = RNE */
        return sign | (uint16_t)q;           /* q == 1024 is the smallest normal */
    }
    int ex;
    double fr = frexp(a, &ex);             /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;                         /* a = (2*fr) * 2^e, 2*fr in [1, 2) */
    double mant = rint(ldexp(fr, 11));      /* 11 significant bits, RNE */
    if (mant == 2048.0) { mant = 1024.0; e += 1; }
    if (e > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)mant - 1024));
}

static double rd_f16(const uint8_t* p)
{
    return qo_f16_to_f64((uint16_t)(p[0] | (p[1] << 8)));
}

/* ------------------------------------------------------------------------------ */
/* q8_1 activation quantisation                                                   */
/* ------------------------------------------------------------------------------ */
/*
 * Per 32-value block of a token row: amax = max|x|, d = amax/127 (f32 division),
 * q = round(x * (1/d)) to int8 (ties away from zero), ssum = sum of q, and the stored
 * scale dh = fp16(d). The header pairs (fp16 d, int16 ssum) in one 32-bit word per
 * token and chunk ([r28] sec. 3.2 smem map; [r14] sec. 3.2(d) decodes the low half as
 * the fp16 scale and the high half as the signed sum). The pages do not show the
 * quantiser itself; the rounding rule is the plain reading recorded with the tests.
 * d == 0 (an all-zero block) gives q = 0 and ssum = 0. When 1/d overflows (a block
 * of tiny values, d < 2^-128) the product x*(1/d) is infinite: it saturates to +-127,
 * and x = 0 gives q = 0 (reading: the saturating limit of the same formula).
 */
int qo_quantize_q8_1(const float* x, int64_t M, int64_t K,
                     int8_t* q, uint16_t* dh, int16_t* ssum)
{
    if (!x || !q || !dh || !ssum || M < 0 || K < 0 || K % QO_QK8)
        return -1;
    const int64_t nc = K / QO_QK8;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t c = 0; c < nc; ++c) {
            const float* xb = x + i * K + c * QO_QK8;
            float amax = 0.0f;
            for (int l = 0; l < QO_QK8; ++l) {
                float a = fabsf(xb[l]);
                if (a > amax) amax = a;
            }
            volatile float d = amax / 127.0f;        /* IEEE single division */
            volatile float id = (d != 0.0f) ? 1.0f / d : 0.0f;
            int sum = 0;
            for (int l = 0; l < QO_QK8; ++l) {
                volatile float v = xb[l] * id;       /* single-precision product */
                int qi;
                if (v != v)                          /* 0 * inf: x = 0 in a block whose 1/d overflowed */
                    qi = 0;
                else if (v >= 127.0f)                /* saturate (covers +inf) */
                    qi = 127;
                else if (v <= -127.0f)
                    qi = -127;
                else
                    qi = (int)roundf(v);             /* half away from zero */
                q[i * K + c * QO_QK8 + l] = (int8_t)qi;
                sum += qi;
            }
            dh[i * nc + c] = qo_f32_to_f16(d);
            ssum[i * nc + c] = (int16_t)sum;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* Block decoders                                                                 */
/* ------------------------------------------------------------------------------ */
/*
 * q4_K (144 B). qs starts at +16 and holds 256 4-bit values, two per byte; sub-block
 * s (32 weights) reads byte group s>>1, the low nibble for even s and the high nibble
 * for odd s, and element l of the sub-block is byte l of the group ([r29] sec. 3.2 and
 * [r28] sec. 3.2, B unpack: p = sg>>1, is_hi = sg&1). d and dmin are the fp16 words at
 * +0 and +2 and the eight (scale, min) 6-bit pairs are packed in the 12 bytes at +4
 * (GGUF q4_K): for s < 4 the low 6 bits of byte s / byte s+4; for s >= 4 the low /
 * high nibble of byte s+4 plus the top two bits of byte s-4 / byte s.
 * Weight value: d*sc_s*nib - dmin*m_s ([r28] sec. 2.3).
 */
void qo_decode_q4K(const uint8_t* blk, double* d, double* dmin,
                   int sc[8], int m[8], int nib[256])
{
    const uint8_t* S = blk + 4;
    const uint8_t* qs = blk + 16;
    *d = rd_f16(blk + 0);
    *dmin = rd_f16(blk + 2);
    for (int s = 0; s < 8; ++s) {
        if (s < 4) {
            sc[s] = S[s] & 63;
            m[s] = S[s + 4] & 63;
        } else {
            sc[s] = (S[s + 4] & 15) | ((S[s - 4] >> 6) << 4);
            m[s] = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
        }
    }
    for (int s = 0; s < 8; ++s) {
        for (int l = 0; l < 32; ++l) {
            int byte = qs[32 * (s >> 1) + l];
            nib[32 * s + l] = (s & 1) ? (byte >> 4) : (byte & 15);
        }
    }
}

/*
 * q6_K (210 B, GGUF q6_K). ql[128] at +0, qh[64] at +128, 16 int8 scales at +192 (one
 * per 16 weights), fp16 d at +208. Element e: half h = e/128, r = e%128, quarter
 * g = r/32, l = r%32; low 4 bits come from ql[64h + 32(g&1) + l] shifted by 4*(g>>1),
 * high 2 bits from qh[32h + l] shifted by 2g; v = (low | high<<4) - 32 in [-32, 31].
 * Weight value: d*sc[e/16]*v. The 16-wide scale granularity is the pages' "KSPLIT=2":
 * two 16-k products per 32-k chunk ([r40] sec. 5).
 */
void qo_decode_q6K(const uint8_t* blk, double* d, int sc[16], int v[256])
{
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    for (int u = 0; u < 16; ++u)
        sc[u] = (int8_t)blk[192 + u];
    *d = rd_f16(blk + 208);
    for (int e = 0; e < 256; ++e) {
        int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
        int lo = (ql[64 * h + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15;
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        v[e] = (lo | (hi << 4)) - 32;
    }
}

/* Dequantised weights, fp64 [N][K]. */
int qo_dequant_q4K(const uint8_t* w, int64_t N, int64_t K, double* out)
{
    if (!w || !out || N < 0 || K <= 0 || K % QO_QK_K) return -1;
    const int64_t nsb = K / QO_QK_K;
    double d, dmin;
    int sc[8], m[8], nib[256];
    for (int64_t j = 0; j < N; ++j)
        for (int64_t b = 0; b < nsb; ++b) {
            qo_decode_q4K(w + (j * nsb + b) * QO_Q4K_BYTES, &d, &dmin, sc, m, nib);
            for (int e = 0; e < 256; ++e)
                out[j * K + b * 256 + e] = d * sc[e / 32] * nib[e] - dmin * m[e / 32];
        }
    return 0;
}

int qo_dequant_q6K(const uint8_t* w, int64_t N, int64_t K, double* out)
{
    if (!w || !out || N < 0 || K <= 0 || K % QO_QK_K) return -1;
    const int64_t nsb = K / QO_QK_K;
    double d;
    int sc[16], v[256];
    for (int64_t j = 0; j < N; ++j)
        for (int64_t b = 0; b < nsb; ++b) {
            qo_decode_q6K(w + (j * nsb + b) * QO_Q6K_BYTES, &d, sc, v);
            for (int e = 0; e < 256; ++e)
                out[j * K + b * 256 + e] = d * sc[e / 16] * v[e];
        }
    return 0;
}

/* ------------------------------------------------------------------------------ */
/* Row-parallel driver                                                            */
/* ------------------------------------------------------------------------------ */

typedef struct {
    int kind;                 /* 0 isums q4K, 1 isums q6K, 2 mmq q4K, 3 mmq q6K */
    const uint8_t* w;
    const int8_t* q;
    const uint16_t* dh;
    const int16_t* ssum;
    int64_t M, N, K;
    int64_t j0, j1;           /* weight rows [j0, j1) */
    int32_t* s;
    double* y;
} qo_job;

/*
 * One weight row j of q4_K against every token i.
 *   I[i,j,c] = sum over the 32 k of chunk c of nib[j,k] * q[i,k]   (exact int32)
 *   y[i,j]   = sum_c  da_ic * dsv_jc * I  +  da_ic * ssum_ic * dmv_jc
 * with dsv = d*sc and dmv = -dmin*m per (row, chunk) and da = fp16 scale of the token's
 * chunk: the two-term fold of [r28] sec. 2.3 (and its inner loop in sec. 3.2). The
 * sum equals dequant(W) . dequant(q8_1(X))^T exactly in real arithmetic. In fp64 each
 * term is exact: da (11 significant bits) * dsv (17) * I (17) needs <= 45 bits and
 * da * ssum * dmv <= 41 bits, so only the fp64 additions round.
 */
static void row_q4K(const qo_job* jb, int64_t j, int32_t* isum_out, double* y_out)
{
    const int64_t K = jb->K, nsb = K / QO_QK_K, nc = K / QO_QK8;
    int* nib = (int*)malloc(sizeof(int) * K);
    double* dsv = (double*)malloc(sizeof(double) * nc);
    double* dmv = (double*)malloc(sizeof(double) * nc);
    for (int64_t b = 0; b < nsb; ++b) {
        double d, dmin;
        int sc[8], m[8];
        qo_decode_q4K(jb->w + (j * nsb + b) * QO_Q4K_BYTES, &d, &dmin, sc, m, nib + b * 256);
        for (int s = 0; s < 8; ++s) {
            dsv[b * 8 + s] = d * sc[s];
            dmv[b * 8 + s] = -(dmin * m[s]);
        }
    }
    for (int64_t i = 0; i < jb->M; ++i) {
        const int8_t* qi = jb->q + i * K;
        double acc = 0.0;
        for (int64_t c = 0; c < nc; ++c) {
            int32_t I = 0;
            for (int l = 0; l < QO_QK8; ++l)
                I += nib[c * QO_QK8 + l] * (int32_t)qi[c * QO_QK8 + l];
            if (isum_out)
                isum_out[(i * jb->N + j) * nc + c] = I;
            if (y_out) {
                double da = qo_f16_to_f64(jb->dh[i * nc + c]);
                double ss = (double)jb->ssum[i * nc + c];
                acc += da * dsv[c] * (double)I;
                acc += da * ss * dmv[c];
            }
        }
        if (y_out)
            y_out[i * jb->N + j] = acc;
    }
    free(nib);
    free(dsv);
    free(dmv);
}

/*
 * One weight row j of q6_K against every token i.
 *   J[i,j,u] = sum over the 16 k of sub-block u of v[j,k] * q[i,k]   (exact int32)
 *   y[i,j]   = sum_u  da_{i,u/2} * d_{j,u/16} * sc_{j,u} * J
 * (q6_K has no min term; its scale granularity is 16, two products per q8_1 chunk.)
 * Each fp64 term is exact: 11 + 11 + 7 + 17 bits.
 */
static void row_q6K(const qo_job* jb, int64_t j, int32_t* isum_out, double* y_out)
{
    const int64_t K = jb->K, nsb = K / QO_QK_K, nc = K / QO_QK8, nu = K / 16;
    int* v = (int*)malloc(sizeof(int) * K);
    double* dsc = (double*)malloc(sizeof(double) * nu);
    for (int64_t b = 0; b < nsb; ++b) {
        double d;
        int sc[16];
        qo_decode_q6K(jb->w + (j * nsb + b) * QO_Q6K_BYTES, &d, sc, v + b * 256);
        for (int u = 0; u < 16; ++u)
            dsc[b * 16 + u] = d * sc[u];
    }
    for (int64_t i = 0; i < jb->M; ++i) {
        const int8_t* qi = jb->q + i * K;
        double acc = 0.0;
        for (int64_t u = 0; u < nu; ++u) {
            int32_t J = 0;
            for (int l = 0; l < 16; ++l)
                J += v[u * 16 + l] * (int32_t)qi[u * 16 + l];
            if (isum_out)
                isum_out[(i * jb->N + j) * nu + u] = J;
            if (y_out) {
                double da = qo_f16_to_f64(jb->dh[i * nc + u / 2]);
                acc += da * dsc[u] * (double)J;
            }
        }
        if (y_out)
            y_out[i * jb->N + j] = acc;
    }
    free(v);
    free(dsc);
}

static void* run_job(void* arg)
{
    const qo_job* jb = (const qo_job*)arg;
    for (int64_t j = jb->j0; j < jb->j1; ++j) {
        switch (jb->kind) {
        case 0: row_q4K(jb, j, jb->s, NULL); break;
        case 1: row_q6K(jb, j, jb->s, NULL); break;
        case 2: row_q4K(jb, j, NULL, jb->y); break;
        case 3: row_q6K(jb, j, NULL, jb->y); break;
        }
    }
    return NULL;
}

static int run_rows(qo_job base, int nthreads)
{
    if (base.M < 0 || base.N < 0 || base.K <= 0 || base.K % QO_QK_K || !base.w || !base.q)
        return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (base.N < nthreads) nthreads = base.N > 0 ? (int)base.N : 1;
    pthread_t th[256];
    qo_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].j0 = base.N * t / nthreads;
        jobs[t].j1 = base.N * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, run_job, &jobs[t]);
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    return 0;
}

/* Exact int32 sub-block sums. s is [M][N][K/32] for q4_K, [M][N][K/16] for q6_K. */
int qo_isums_q4K(const uint8_t* w, const int8_t* q, int64_t M, int64_t N, int64_t K,
                 int32_t* s, int nthreads)
{
    if (!s) return -1;
    qo_job jb = {0, w, q, NULL, NULL, M, N, K, 0, 0, s, NULL};
    return run_rows(jb, nthreads);
}

int qo_isums_q6K(const uint8_t* w, const int8_t* q, int64_t M, int64_t N, int64_t K,
                 int32_t* s, int nthreads)
{
    if (!s) return -1;
    qo_job jb = {1, w, q, NULL, NULL, M, N, K, 0, 0, s, NULL};
    return run_rows(jb, nthreads);
}

/* y[M][N] (fp64) from q8_1 activations (q [M][K], dh/ssum [M][K/32]). */
int qo_mmq_q4K(const uint8_t* w, const int8_t* q, const uint16_t* dh, const int16_t* ssum,
               int64_t M, int64_t N, int64_t K, double* y, int nthreads)
{
    if (!dh || !ssum || !y) return -1;
    qo_job jb = {2, w, q, dh, ssum, M, N, K, 0, 0, NULL, y};
    return run_rows(jb, nthreads);
}

int qo_mmq_q6K(const uint8_t* w, const int8_t* q, const uint16_t* dh, const int16_t* ssum,
               int64_t M, int64_t N, int64_t K, double* y, int nthreads)
{
    if (!dh || !y) return -1;
    (void)ssum;
    qo_job jb = {3, w, q, dh, ssum, M, N, K, 0, 0, NULL, y};
    return run_rows(jb, nthreads);
}
