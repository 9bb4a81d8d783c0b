/*
 * Host-side fuzz driver for the plain C oracle (oracle/kqref.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py.  Every buffer is allocated at its exact size,
 * so a read or write past any end is reported.  Prints "ok" and exits 0 when
 * every call returns its expected status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double kqref_f16_to_f64(uint16_t h);
void kqref_decode_q4k(const uint8_t *b, double *d, double *dmin, int32_t sc[8], int32_t mn[8],
                      int32_t q[256]);
void kqref_decode_q6k(const uint8_t *b, double *d, int32_t sc[16], int32_t q[256]);
void kqref_decode_tq(const uint8_t *b, double *d, int32_t t[128]);
void kqref_decode_tq2(const uint8_t *b, double *d, int32_t t[128]);
int kqref_dequant_rows(int fmt, const uint8_t *W, int64_t N, int64_t K, double *out);
int kqref_int_operands(int fmt, const uint8_t *W, int64_t N, int64_t K, int32_t *out);
int kqref_quantize_act(int act_fmt, const float *x, int64_t M, int64_t K, int8_t *qs, float *d,
                       int16_t *bsums);
int kqref_gemm_rows(int fmt, const uint8_t *W, const int8_t *qs, const float *d_a, int64_t M,
                    int64_t N, int64_t K, const int64_t *rows, int64_t n_rows, float *out,
                    double *tol);
int kqref_subsums(int fmt, const uint8_t *W, const int8_t *qs, int64_t M, int64_t N, int64_t K,
                  int32_t *S);

static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (uint32_t)(rs >> 16);
}

static const int QK[5] = {0, 256, 256, 128, 128}, BB[5] = {0, 144, 210, 28, 34};
static const int SUB[5] = {0, 32, 16, 128, 128};
static const int ACT[5] = {0, 1, 1, 2, 2}, ABS_[5] = {0, 256, 256, 128, 128};

static int failures = 0;
#define EXPECT(c)                                                   \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
            failures++;                                             \
        }                                                           \
    } while (0)

/* fp16 scale values the fuzz blocks take, including zero, negative and
 * subnormal ones */
static const uint16_t F16S[] = {0x0000, 0x8000, 0x0001, 0x03FF, 0x1C00, 0x2E66, 0xB400, 0x3C00, 0x7BFF};

static void fill_blocks(int fmt, uint8_t *W, int64_t nblocks) {
    for (int64_t i = 0; i < nblocks; i++) {
        uint8_t *b = W + i * BB[fmt];
        for (int j = 0; j < BB[fmt]; j++) b[j] = (uint8_t)rnd();
        uint16_t d = F16S[rnd() % (sizeof F16S / sizeof F16S[0])];
        if (fmt == 1) {
            memcpy(b, &d, 2);
            d = F16S[rnd() % (sizeof F16S / sizeof F16S[0])];
            memcpy(b + 2, &d, 2);
        } else if (fmt == 2) {
            memcpy(b + 208, &d, 2);
        } else if (fmt == 4) {
            for (int j = 0; j < 32; j++) {
                uint32_t v = 0;
                for (int p = 0; p < 4; p++) v |= (rnd() % 3) << (2 * p);
                b[j] = (uint8_t)v;
            }
            memcpy(b + 32, &d, 2);
        } else {
            for (int j = 0; j < 25; j++) b[j] = (uint8_t)(rnd() % 243);
            b[25] = (uint8_t)(108 + rnd() % 27);
            memcpy(b + 26, &d, 2);
        }
    }
}

static float act_value(void) {
    switch (rnd() % 8) {
        case 0: return 0.0f;
        case 1: return -0.0f;
        case 2: return 1e-40f; /* subnormal */
        case 3: return (rnd() & 1 ? 1.0f : -1.0f) * 3e30f;
        default: return ((float)(rnd() % 2001) - 1000.0f) / 37.0f;
    }
}

int main(void) {
    /* decoders on arbitrary bytes */
    for (int it = 0; it < 4000; it++) {
        uint8_t b4[144], b6[210], bt[28];
        for (int j = 0; j < 144; j++) b4[j] = (uint8_t)rnd();
        for (int j = 0; j < 210; j++) b6[j] = (uint8_t)rnd();
        for (int j = 0; j < 28; j++) bt[j] = (uint8_t)rnd();
        double d, dm;
        int32_t sc[16], mn[8], q[256];
        kqref_decode_q4k(b4, &d, &dm, sc, mn, q);
        for (int k = 0; k < 256; k++) EXPECT(q[k] >= 0 && q[k] <= 15);
        for (int j = 0; j < 8; j++) EXPECT(sc[j] >= 0 && sc[j] <= 63 && mn[j] >= 0 && mn[j] <= 63);
        kqref_decode_q6k(b6, &d, sc, q);
        for (int k = 0; k < 256; k++) EXPECT(q[k] >= 0 && q[k] <= 63);
        kqref_decode_tq(bt, &d, q);
        uint8_t b2[34];
        for (int j = 0; j < 34; j++) b2[j] = (uint8_t)rnd();
        kqref_decode_tq2(b2, &d, q);
        for (int k = 0; k < 128; k++) EXPECT(q[k] >= -1 && q[k] <= 2);
    }
    for (uint32_t h = 0; h < 65536; h++) {
        double v = kqref_f16_to_f64((uint16_t)h);
        EXPECT(isnan(v) || isinf(v) || fabs(v) <= 65504.0);
    }

    /* every entry point on ragged shapes; exact-size buffers */
    static const int64_t Ms[] = {1, 3, 33}, Ns[] = {1, 2, 7};
    for (int fmt = 1; fmt <= 4; fmt++) {
        for (int kk = 1; kk <= 3; kk++) {
            const int64_t K = kk * QK[fmt];
            for (int mi = 0; mi < 3; mi++) {
                for (int ni = 0; ni < 3; ni++) {
                    const int64_t M = Ms[mi], N = Ns[ni], nb = K / QK[fmt];
                    uint8_t *W = malloc((size_t)(N * nb * BB[fmt]));
                    float *x = malloc(sizeof(float) * (size_t)(M * K));
                    int8_t *qs = malloc((size_t)(M * K));
                    float *da = malloc(sizeof(float) * (size_t)(M * (K / ABS_[fmt])));
                    int16_t *bs = ACT[fmt] == 1 ? malloc(sizeof(int16_t) * (size_t)(M * (K / 16))) : NULL;
                    double *deq = malloc(sizeof(double) * (size_t)(N * K));
                    int32_t *qi = malloc(sizeof(int32_t) * (size_t)(N * K));
                    float *out = malloc(sizeof(float) * (size_t)(M * N));
                    double *tol = malloc(sizeof(double) * (size_t)(M * N));
                    float *out2 = malloc(sizeof(float) * (size_t)(M * 2));
                    int32_t *S = malloc(sizeof(int32_t) * (size_t)(M * N * (K / SUB[fmt])));
                    int64_t rows[2] = {N - 1, 0};
                    fill_blocks(fmt, W, N * nb);
                    for (int64_t i = 0; i < M * K; i++) x[i] = act_value();
                    if (M > 1)
                        for (int64_t k = 0; k < K; k++) x[K + k] = 0.0f; /* an all-zero row */
                    EXPECT(kqref_quantize_act(ACT[fmt], x, M, K, qs, da, bs) == 0);
                    for (int64_t i = 0; i < M * K; i++) EXPECT(qs[i] >= -127 && qs[i] <= 127);
                    EXPECT(kqref_dequant_rows(fmt, W, N, K, deq) == 0);
                    EXPECT(kqref_int_operands(fmt, W, N, K, qi) == 0);
                    EXPECT(kqref_gemm_rows(fmt, W, qs, da, M, N, K, NULL, 0, out, tol) == 0);
                    EXPECT(kqref_gemm_rows(fmt, W, qs, da, M, N, K, rows, 2, out2, NULL) == 0);
                    /* the listed rows give the same values as the full product */
                    for (int64_t m = 0; m < M; m++)
                        EXPECT(out2[m * 2] == out[m * N + N - 1] && out2[m * 2 + 1] == out[m * N]);
                    EXPECT(kqref_subsums(fmt, W, qs, M, N, K, S) == 0);
                    /* K not a multiple of the block: refused */
                    EXPECT(kqref_quantize_act(ACT[fmt], x, M, K - 16, qs, da, bs) == -1);
                    EXPECT(kqref_gemm_rows(fmt, W, qs, da, M, N, K - 16, NULL, 0, out, tol) == -1);
                    EXPECT(kqref_subsums(fmt, W, qs, M, N, K - 16, S) == -1);
                    free(W); free(x); free(qs); free(da); free(bs); free(deq); free(qi);
                    free(out); free(tol); free(out2); free(S);
                }
            }
        }
    }
    EXPECT(kqref_dequant_rows(7, NULL, 0, 256, NULL) == -1);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
