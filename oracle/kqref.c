/*
 * kqref.c -- plain, slow CPU oracle for the block-quantized weight x
 * quantized-activation matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP path
 * never links, calls or reads it, and it shares no code, header or table
 * with the HIP path.
 *
 * What it computes (the method of the vllm.cpp PR "cooperative-tile WMMA
 * kernels -- Shared rejected, BigTile accepted" and the llama.cpp PR
 * "branch-free PTQ1_0 MMQ tile loader": activations are quantized to int8
 * superblocks with an fp32 scale, weights are stored as k-quant / ternary
 * blocks, and the product is taken over those integers with the block scales
 * and mins folded in):
 *
 *   out[m][n] = fp32( sum_k W^[n][k] * A^[m][k] )      (fp64 accumulation)
 *
 * where W^ is the dequantized weight (decoded here from the block bytes) and
 * A^[m][k] = d_a[m][block] * qs[m][k] comes from the Q8 rule below, which
 * runs in fp32 because it decides integers (the kernel decides them in fp32
 * too).  The oracle also emits the per-sub-block integer dot sums and the
 * per-element tolerance 1e-4 * sum_k |W^ A^| + 1e-6.
 *
 * Block layouts are this project's own (the pages fix only block sizes:
 * 292 bytes per 256 activations for the Q8_K block in the vllm.cpp PR, a
 * 28-byte block per 128 ternary weights in the llama.cpp PR, which also
 * names PQ2_0, the same trits at two bits each).  The decoders below state
 * each layout in full.
 *
 * Every routine is written for clarity: bit-by-bit field extraction, plain
 * loops, no blocking.  Build: gcc -O2 -fopenmp -ffp-contract=off (no
 * fast-math), so x*s is a single fp32 multiply and rintf rounds half to even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KQREF_Q4_K 1
#define KQREF_Q6_K 2
#define KQREF_TQ 3
#define KQREF_TQ2 4
#define KQREF_ACT_Q8_K 1
#define KQREF_ACT_Q8_128 2

int kqref_version(void) { return 1; }

/* ---------------------------------------------------------------------- */
/* fp16 -> fp64, exact.  IEEE binary16: 1 sign, 5 exponent (bias 15), 10
 * fraction bits.  Subnormals are frac * 2^-24.                            */
double kqref_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), e - 25);
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---------------------------------------------------------------------- */
/* Q4_K block, 144 bytes, 256 weights in 8 sub-blocks of 32.
 *   [0,2) fp16 d   [2,4) fp16 dmin   [4,16) twelve bytes = a little-endian
 *   96-bit integer whose bits [6f, 6f+6) hold field f: f < 8 is the scale
 *   sc_f of sub-block f, f >= 8 is the min m_(f-8).
 *   [16,144) nibbles: byte 16+32c+t has weight 64c+t in bits 0..3 and weight
 *   64c+32+t in bits 4..7 (c = 0..3, t = 0..31).
 *   W^_k = d * sc_j * q_k - dmin * m_j with j = k / 32.                    */
void kqref_decode_q4k(const uint8_t *b, double *d, double *dmin, int32_t sc[8],
                      int32_t mn[8], int32_t q[256])
{
    *d = kqref_f16_to_f64(rd16(b + 0));
    *dmin = kqref_f16_to_f64(rd16(b + 2));
    for (int f = 0; f < 16; f++) {
        int v = 0;
        for (int bit = 0; bit < 6; bit++) {
            int pos = 6 * f + bit;
            v |= ((b[4 + pos / 8] >> (pos % 8)) & 1) << bit;
        }
        if (f < 8)
            sc[f] = v;
        else
            mn[f - 8] = v;
    }
    for (int c = 0; c < 4; c++)
        for (int t = 0; t < 32; t++) {
            int byte = b[16 + 32 * c + t];
            q[64 * c + t] = byte & 15;
            q[64 * c + 32 + t] = (byte >> 4) & 15;
        }
}

/* Q6_K block, 210 bytes, 256 weights in 16 sub-blocks of 16.
 *   [0,128) ql: byte 64h+t has the low 4 bits of weight 128h+t in bits 0..3
 *           and of weight 128h+64+t in bits 4..7 (h = 0..1, t = 0..63).
 *   [128,192) qh: bits 2u..2u+1 of byte 128+32h+t are the high 2 bits of
 *           weight 128h+32u+t (t = 0..31, u = 0..3).
 *   [192,208) signed 8-bit scales sc_j.   [208,210) fp16 d.
 *   W^_k = d * sc_j * (q_k - 32) with j = k / 16.                          */
void kqref_decode_q6k(const uint8_t *b, double *d, int32_t sc[16], int32_t q[256])
{
    for (int h = 0; h < 2; h++) {
        for (int t = 0; t < 64; t++) {
            int v = b[64 * h + t];
            q[128 * h + t] = v & 15;
            q[128 * h + 64 + t] = (v >> 4) & 15;
        }
        for (int t = 0; t < 32; t++) {
            int v = b[128 + 32 * h + t];
            for (int u = 0; u < 4; u++)
                q[128 * h + 32 * u + t] |= ((v >> (2 * u)) & 3) << 4;
        }
    }
    for (int j = 0; j < 16; j++)
        sc[j] = (int8_t)b[192 + j];
    *d = kqref_f16_to_f64(rd16(b + 208));
}

/* Ternary block, 28 bytes, 128 weights.
 *   [0,26): weight k is digit e_k = t_k + 1 at base-3 position k mod 5 of
 *   byte k / 5, i.e. byte b = sum_p e_(5b+p) 3^p.  [26,28): fp16 d.
 *   W^_k = d * t_k.                                                        */
void kqref_decode_tq(const uint8_t *b, double *d, int32_t t[128])
{
    for (int k = 0; k < 128; k++) {
        int v = b[k / 5];
        for (int p = 0; p < k % 5; p++)
            v /= 3;
        t[k] = v % 3 - 1;
    }
    *d = kqref_f16_to_f64(rd16(b + 26));
}

/* Ternary block at two bits per weight (the PQ2_0 packing the llama.cpp PR
 * names: the same trits as above, two bits each), 34 bytes, 128 weights.
 *   [0,32): weight k has code c_k = t_k + 1 in bits 2*(k/32) .. 2*(k/32)+1
 *   of byte k % 32, i.e. byte j holds weights j, j+32, j+64, j+96 from its
 *   low bits up.  Code 3 is not a valid trit.  [32,34): fp16 d.
 *   W^_k = d * t_k.                                                        */
void kqref_decode_tq2(const uint8_t *b, double *d, int32_t t[128])
{
    for (int k = 0; k < 128; k++) {
        int c = (b[k % 32] >> (2 * (k / 32))) & 3;
        t[k] = c - 1;
    }
    *d = kqref_f16_to_f64(rd16(b + 32));
}

static int ternary(int fmt) { return fmt == KQREF_TQ || fmt == KQREF_TQ2; }
static int qk_of(int fmt) { return ternary(fmt) ? 128 : 256; }
static int bb_of(int fmt)
{
    return fmt == KQREF_Q4_K ? 144 : fmt == KQREF_Q6_K ? 210 : fmt == KQREF_TQ ? 28
         : fmt == KQREF_TQ2 ? 34 : 0;
}
static int sub_of(int fmt)
{
    return fmt == KQREF_Q4_K ? 32 : fmt == KQREF_Q6_K ? 16 : ternary(fmt) ? 128 : 0;
}

/* Dequantize one block to fp64 (QK values), plus the integer operand that the
 * int8 contraction uses for each weight (Q4_K: q in [0,15]; Q6_K: q-32;
 * ternary: t).  Either output may be NULL.                                 */
static void dequant_block(int fmt, const uint8_t *b, double *w, int32_t *qint)
{
    int32_t q[256], sc[16], mn[8];
    double d, dmin;
    if (fmt == KQREF_Q4_K) {
        kqref_decode_q4k(b, &d, &dmin, sc, mn, q);
        for (int k = 0; k < 256; k++) {
            int j = k / 32;
            if (w) w[k] = d * sc[j] * q[k] - dmin * mn[j];
            if (qint) qint[k] = q[k];
        }
    } else if (fmt == KQREF_Q6_K) {
        kqref_decode_q6k(b, &d, sc, q);
        for (int k = 0; k < 256; k++) {
            int j = k / 16;
            if (w) w[k] = d * sc[j] * (q[k] - 32);
            if (qint) qint[k] = q[k] - 32;
        }
    } else {
        if (fmt == KQREF_TQ2)
            kqref_decode_tq2(b, &d, q);
        else
            kqref_decode_tq(b, &d, q);
        for (int k = 0; k < 128; k++) {
            if (w) w[k] = d * q[k];
            if (qint) qint[k] = q[k];
        }
    }
}

/* Dequantize N rows of stored blocks into fp64 [N][K]. */
int kqref_dequant_rows(int fmt, const uint8_t *W, int64_t N, int64_t K, double *out)
{
    int qk = qk_of(fmt), bb = bb_of(fmt);
    if (!bb || K % qk) return -1;
    int64_t nb = K / qk;
    for (int64_t n = 0; n < N; n++)
        for (int64_t s = 0; s < nb; s++)
            dequant_block(fmt, W + (n * nb + s) * bb, out + n * K + s * qk, NULL);
    return 0;
}

/* Integer operands of N rows, int32 [N][K] (see dequant_block). */
int kqref_int_operands(int fmt, const uint8_t *W, int64_t N, int64_t K, int32_t *out)
{
    int qk = qk_of(fmt), bb = bb_of(fmt);
    if (!bb || K % qk) return -1;
    int64_t nb = K / qk;
    for (int64_t n = 0; n < N; n++)
        for (int64_t s = 0; s < nb; s++)
            dequant_block(fmt, W + (n * nb + s) * bb, NULL, out + n * K + s * qk);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Q8 activation rule, per block of `bs` values (256 for Q8_K, 128 for
 * Q8_128), in fp32:
 *   amax = max |x_i|; if amax == 0 or 127/amax is not finite: d = 0, q = 0.
 *   else d = amax/127, s = 127/amax, q_i = clamp(rint(x_i * s), -127, 127).
 * Q8_K also stores bsums[g] = sum of q over each 16-wide group.            */
static void quant_block(const float *x, int bs, int8_t *qs, float *d, int16_t *bsums)
{
    float amax = 0.0f;
    for (int i = 0; i < bs; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float s = 127.0f / amax;
    if (amax == 0.0f || !isfinite(s)) {
        for (int i = 0; i < bs; i++) qs[i] = 0;
        *d = 0.0f;
    } else {
        *d = amax / 127.0f;
        for (int i = 0; i < bs; i++) {
            float v = rintf(x[i] * s);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            qs[i] = (int8_t)v;
        }
    }
    if (bsums)
        for (int g = 0; g < bs / 16; g++) {
            int sum = 0;
            for (int i = 0; i < 16; i++) sum += qs[16 * g + i];
            bsums[g] = (int16_t)sum;
        }
}

/* x fp32 [M][K] -> qs int8 [M][K], d fp32 [M][K/bs], bsums int16 [M][K/16]
 * (bsums only for Q8_K; pass NULL for Q8_128).                             */
int kqref_quantize_act(int act_fmt, const float *x, int64_t M, int64_t K, int8_t *qs,
                       float *d, int16_t *bsums)
{
    int bs = act_fmt == KQREF_ACT_Q8_K ? 256 : act_fmt == KQREF_ACT_Q8_128 ? 128 : 0;
    if (!bs || K % bs) return -1;
    int64_t nb = K / bs;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < nb; b++)
            quant_block(x + m * K + b * bs, bs, qs + m * K + b * bs, d + m * nb + b,
                        (act_fmt == KQREF_ACT_Q8_K && bsums) ? bsums + m * (K / 16) + b * 16
                                                             : NULL);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* The product, the slow way.  qs/d_a are the quantized activations (Q8_K
 * for Q4_K and Q6_K weights, Q8_128 for ternary).  Rows of W are decoded to
 * fp64 one at a time; A^ is expanded once to fp64 [M][K].  Writes
 * out fp32 [M][N] and, when tol != NULL, tol fp64 [M][N].
 * `rows`, when not NULL, lists n_rows output rows (columns of out) to
 * compute; out/tol then have shape [M][n_rows].                            */
int kqref_gemm_rows(int fmt, const uint8_t *W, const int8_t *qs, const float *d_a,
                    int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t n_rows,
                    float *out, double *tol)
{
    int qk = qk_of(fmt), bb = bb_of(fmt);
    int abs_ = ternary(fmt) ? 128 : 256;          /* activation block size */
    if (!bb || K % qk) return -1;
    int64_t nb = K / qk, na = K / abs_;
    int64_t ncols = rows ? n_rows : N;
    double *A = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!A) return -2;
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++)
            A[m * K + k] = (double)d_a[m * na + k / abs_] * (double)qs[m * K + k];
    int err = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t c = 0; c < ncols; c++) {
                int64_t n = rows ? rows[c] : c;
                for (int64_t s = 0; s < nb; s++)
                    dequant_block(fmt, W + (n * nb + s) * bb, w + s * qk, NULL);
                for (int64_t m = 0; m < M; m++) {
                    const double *a = A + m * K;
                    double acc = 0.0, mag = 0.0;
                    for (int64_t k = 0; k < K; k++) {
                        double p = w[k] * a[k];
                        acc += p;
                        mag += fabs(p);
                    }
                    out[m * ncols + c] = (float)acc;
                    if (tol) tol[m * ncols + c] = 1e-4 * mag + 1e-6;
                }
            }
            free(w);
        }
    }
    free(A);
    return err;
}

int kqref_gemm(int fmt, const uint8_t *W, const int8_t *qs, const float *d_a, int64_t M,
               int64_t N, int64_t K, float *out, double *tol)
{
    return kqref_gemm_rows(fmt, W, qs, d_a, M, N, K, NULL, 0, out, tol);
}

/* Per-sub-block integer dot sums S[m][n][j] = sum_{k in sub-block j}
 * qint[n][k] * qs[m][k], int32 [M][N][K/sub] with sub = 32 (Q4_K), 16 (Q6_K),
 * 128 (ternary).  Sums are formed in int64 and checked to fit int32.      */
int kqref_subsums(int fmt, const uint8_t *W, const int8_t *qs, int64_t M, int64_t N,
                  int64_t K, int32_t *S)
{
    int qk = qk_of(fmt), bb = bb_of(fmt), sub = sub_of(fmt);
    if (!bb || K % qk) return -1;
    int64_t nb = K / qk, nj = K / sub;
    int err = 0;
#pragma omp parallel
    {
        int32_t *qi = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
        if (!qi) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < N; n++) {
                for (int64_t s = 0; s < nb; s++)
                    dequant_block(fmt, W + (n * nb + s) * bb, NULL, qi + s * qk);
                for (int64_t m = 0; m < M; m++)
                    for (int64_t j = 0; j < nj; j++) {
                        int64_t acc = 0;
                        for (int64_t k = j * sub; k < (j + 1) * sub; k++)
                            acc += (int64_t)qi[k] * (int64_t)qs[m * K + k];
                        if (acc > INT32_MAX || acc < INT32_MIN) {
#pragma omp atomic write
                            err = -3;
                        }
                        S[(m * N + n) * nj + j] = (int32_t)acc;
                    }
            }
            free(qi);
        }
    }
    return err;
}
