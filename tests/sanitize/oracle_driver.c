/* Host-sanitizer driver of the CPU oracle (tests/test_sanitize.py builds it together with
 * oracle/oracle.c under -fsanitize=address,undefined): every oracle function on small seeded
 * inputs, including the edge blocks of the q8_1 quantiser, plus its argument rejections.
 * Exit status 0 when every call returned what it should; the sanitizers abort on their own
 * findings. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double qo_f16_to_f64(uint16_t h);
uint16_t qo_f32_to_f16(float x);
int qo_quantize_q8_1(const float* x, int64_t M, int64_t K, int8_t* q, uint16_t* dh, int16_t* ssum);
void qo_decode_q4K(const uint8_t* blk, double* d, double* dmin, int sc[8], int m[8], int nib[256]);
void qo_decode_q6K(const uint8_t* blk, double* d, int sc[16], int v[256]);
int qo_dequant_q4K(const uint8_t* w, int64_t N, int64_t K, double* out);
int qo_dequant_q6K(const uint8_t* w, int64_t N, int64_t K, double* out);
int qo_isums_q4K(const uint8_t* w, const int8_t* q, int64_t M, int64_t N, int64_t K, int32_t* s, int nthreads);
int qo_isums_q6K(const uint8_t* w, const int8_t* q, int64_t M, int64_t N, int64_t K, int32_t* s, int nthreads);
int qo_mmq_q4K(const uint8_t* w, const int8_t* q, const uint16_t* dh, const int16_t* ssum, int64_t M, int64_t N,
               int64_t K, double* y, int nthreads);
int qo_mmq_q6K(const uint8_t* w, const int8_t* q, const uint16_t* dh, const int16_t* ssum, int64_t M, int64_t N,
               int64_t K, double* y, int nthreads);

static uint32_t state = 12345u;
static uint32_t rnd(void) { state = state * 1664525u + 1013904223u; return state >> 8; }

#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); return 1; } } while (0)

int main(void)
{
    enum { M = 7, N = 5, K = 512, NC = K / 32 };
    float* x = malloc(sizeof(float) * M * K);
    for (int i = 0; i < M * K; ++i) x[i] = ((int)(rnd() % 20001) - 10000) * 1e-3f;
    for (int l = 0; l < 32; ++l) { x[l] = 0.0f; x[32 + l] = 1e-39f * (float)(l - 16); x[64 + l] = (float)l + 0.5f; }
    int8_t* q = malloc(M * K);
    uint16_t* dh = malloc(sizeof(uint16_t) * M * NC);
    int16_t* ss = malloc(sizeof(int16_t) * M * NC);
    CHECK(qo_quantize_q8_1(x, M, K, q, dh, ss) == 0);
    CHECK(qo_quantize_q8_1(x, M, 48, q, dh, ss) == -1);          /* K % 32 */
    CHECK(qo_quantize_q8_1(NULL, M, K, q, dh, ss) == -1);
    for (uint32_t h = 0; h < 65536; h += 97) (void)qo_f16_to_f64((uint16_t)h);
    (void)qo_f32_to_f16(65520.0f); (void)qo_f32_to_f16(-1e-8f); (void)qo_f32_to_f16(0.0f);

    const int nsb = K / 256;
    uint8_t* w4 = malloc(N * nsb * 144);
    uint8_t* w6 = malloc(N * nsb * 210);
    for (int i = 0; i < N * nsb * 144; ++i) w4[i] = (uint8_t)rnd();
    for (int i = 0; i < N * nsb * 210; ++i) w6[i] = (uint8_t)rnd();
    double d, dmin;
    int sc[16], m[8], v[256];
    qo_decode_q4K(w4, &d, &dmin, sc, m, v);
    qo_decode_q6K(w6, &d, sc, v);
    double* deq = malloc(sizeof(double) * N * K);
    CHECK(qo_dequant_q4K(w4, N, K, deq) == 0);
    CHECK(qo_dequant_q6K(w6, N, K, deq) == 0);
    CHECK(qo_dequant_q4K(w4, N, 300, deq) == -1);
    int32_t* s = malloc(sizeof(int32_t) * M * N * (K / 16));
    double* y = malloc(sizeof(double) * M * N);
    for (int th = 1; th <= 4; th += 3) {
        CHECK(qo_isums_q4K(w4, q, M, N, K, s, th) == 0);
        CHECK(qo_isums_q6K(w6, q, M, N, K, s, th) == 0);
        CHECK(qo_mmq_q4K(w4, q, dh, ss, M, N, K, y, th) == 0);
        CHECK(qo_mmq_q6K(w6, q, dh, ss, M, N, K, y, th) == 0);
    }
    CHECK(qo_isums_q4K(w4, q, M, N, K, NULL, 2) == -1);
    CHECK(qo_mmq_q6K(w6, q, NULL, ss, M, N, K, y, 2) == -1);
    CHECK(qo_mmq_q4K(w4, q, dh, ss, M, N, 288, y, 2) == -1);
    free(x); free(q); free(dh); free(ss); free(w4); free(w6); free(deq); free(s); free(y);
    printf("oracle driver: ok\n");
    return 0;
}
