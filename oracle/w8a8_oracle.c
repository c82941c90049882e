/*
 * W8A8 linear layer: plain, slow CPU oracle (test infrastructure only).
 *
 * Same status as sagesla_oracle.c: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it; it shares no code with the GPU library.
 *
 * What the method computes (TurboDiffusion explainer, news.qq.com, "Third key"): both the
 * weights and the activations of the linear layers are 8-bit integers, so that the whole
 * product runs in the INT8 domain. The weights are quantized offline in blocks of
 * 128 x 128, each block with one scale factor; the activations are quantized on the fly
 * at inference. The page does not say how the activations are grouped; the reading here
 * is one scale per token and 128-channel block (the K extent of the weight blocks).
 *
 *   activations x [M][K] bf16:  s_x[m][b] = amax_x(m, b) / 127,  q_x = rne(x * 127/amax)
 *   weights     w [N][K] bf16:  s_w[n/128][b] = amax_w(block) / 127, q_w likewise
 *   y[m][n] = sum_b s_x[m][b] s_w[n/128][b] sum_{k in block b} q_x[m][k] q_w[n][k]  (+ bias[n])
 *
 * Every fp32 expression that decides an integer code is the same as in the attention
 * oracle (inv = 127.0f/amax, product in fp32, round half to even, clamp to +-127;
 * amax = 0 gives zero codes and scale 0). The integer sums are exact (int64); scaling
 * and the sum over blocks are fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float w8_bf16f(uint16_t h)
{
    union {
        uint32_t u;
        float f;
    } v;
    v.u = (uint32_t)h << 16;
    return v.f;
}

static int8_t w8_q(float x, float inv)
{
    float y = x * inv; /* fp32 product */
    float r = nearbyintf(y); /* round half to even (default rounding mode) */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* Activations: one scale per (row m, 128-column block b). K is a multiple of 128.
 * q: [M][K] int8, s: [M][K/128] fp32. */
void oracle_w8a8_quant_act(const uint16_t *x, int M, int K, int8_t *q, float *s)
{
    int KB = K / 128;
    for (int m = 0; m < M; m++)
        for (int b = 0; b < KB; b++) {
            const uint16_t *row = x + (size_t)m * K + 128 * b;
            float amax = 0.0f;
            for (int c = 0; c < 128; c++) {
                float a = fabsf(w8_bf16f(row[c]));
                if (a > amax)
                    amax = a;
            }
            float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
            s[(size_t)m * KB + b] = amax > 0.0f ? amax / 127.0f : 0.0f;
            for (int c = 0; c < 128; c++)
                q[(size_t)m * K + 128 * b + c] = w8_q(w8_bf16f(row[c]), inv);
        }
}

/* Weights: one scale per 128 x 128 block (rows n, columns k). N, K multiples of 128.
 * q: [N][K] int8, s: [N/128][K/128] fp32. */
void oracle_w8a8_quant_weight(const uint16_t *w, int N, int K, int8_t *q, float *s)
{
    int NB = N / 128, KB = K / 128;
    for (int a = 0; a < NB; a++)
        for (int b = 0; b < KB; b++) {
            float amax = 0.0f;
            for (int r = 0; r < 128; r++)
                for (int c = 0; c < 128; c++) {
                    float v = fabsf(w8_bf16f(w[(size_t)(128 * a + r) * K + 128 * b + c]));
                    if (v > amax)
                        amax = v;
                }
            float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
            s[(size_t)a * KB + b] = amax > 0.0f ? amax / 127.0f : 0.0f;
            for (int r = 0; r < 128; r++)
                for (int c = 0; c < 128; c++) {
                    size_t e = (size_t)(128 * a + r) * K + 128 * b + c;
                    q[e] = w8_q(w8_bf16f(w[e]), inv);
                }
        }
}

/* y[m][n] = sum_b s_x[m][b] s_w[n/128][b] (exact int dot over block b) (+ bias[n]).
 * rows m0 .. m1-1 only (the rest of y is not written); bias may be NULL. y: [M][N] fp64. */
void oracle_w8a8_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw,
                      const uint16_t *bias, int M, int N, int K, int m0, int m1, double *y)
{
    int KB = K / 128;
    (void)M;
    for (int m = m0; m < m1; m++)
        for (int n = 0; n < N; n++) {
            double acc = 0.0;
            for (int b = 0; b < KB; b++) {
                int64_t dot = 0;
                const int8_t *xa = qx + (size_t)m * K + 128 * b;
                const int8_t *wb = qw + (size_t)n * K + 128 * b;
                for (int c = 0; c < 128; c++)
                    dot += (int64_t)xa[c] * (int64_t)wb[c];
                acc += (double)dot * (double)sx[(size_t)m * KB + b] * (double)sw[(size_t)(n / 128) * KB + b];
            }
            if (bias)
                acc += (double)w8_bf16f(bias[n]);
            y[(size_t)m * N + n] = acc;
        }
}
