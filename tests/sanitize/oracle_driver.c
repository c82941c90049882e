/*
 * Drives the C oracle (oracle/sagesla_oracle.c, oracle/w8a8_oracle.c) on small, ragged
 * inputs for a build with the address and undefined-behaviour sanitizers: every entry
 * point the tests use runs at least once, and a few invariants are checked so that a
 * wrong result also fails. Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t h);
uint16_t oracle_double_to_bf16(double x);
double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float x);
int oracle_num_blocks(int N, int blk);
int oracle_ksel(double topk, int Nb);
void oracle_scores(const double *qbar, const double *kbar, int nq, int nk, int d, double *scores);
void oracle_select(const double *scores, int nq, int Nb, int ksel, int32_t *idx);
int oracle_sagesla_head(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *w, int N,
                        int d, int blk, double topk, int quant, const int32_t *qblocks, int nqb, double *out,
                        double *out_s, double *out_l, int32_t *idx_out);
void oracle_w8a8_quant_act(const uint16_t *x, int M, int K, int8_t *q, float *s);
void oracle_w8a8_quant_weight(const uint16_t *w, int N, int K, int8_t *q, float *s);
void oracle_w8a8_gemm(const int8_t *qx, const float *sx, const int8_t *qw, const float *sw, const uint16_t *bias,
                      int M, int N, int K, int m0, int m1, double *y);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void) /* splitmix64 -> [0, 1) */
{
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (double)((z ^ (z >> 31)) >> 11) / 9007199254740992.0;
}
static double gauss(void) { return sqrt(-2.0 * log(1.0 - unif())) * cos(6.283185307179586 * unif()); }
static void fill_bf16(uint16_t *a, size_t n, double scale)
{
    for (size_t i = 0; i < n; i++)
        a[i] = oracle_double_to_bf16(scale * gauss());
}

#define CHECK(c)                                                                                 \
    do {                                                                                         \
        if (!(c)) {                                                                              \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);                      \
            return 1;                                                                            \
        }                                                                                        \
    } while (0)

int main(void)
{
    /* every finite e4m3 code survives a decode/encode round trip */
    for (int c = 0; c < 256; c++) {
        double x = oracle_e4m3_decode((uint8_t)c);
        if (x != x)
            continue;
        CHECK(oracle_e4m3_encode((float)x) == (uint8_t)c || (x == 0.0 && (c == 0 || c == 0x80)));
    }
    /* selection against a full sort on a small score matrix */
    enum { NQ = 5, NB = 9, DD = 16 };
    double qb[NQ * DD], kb[NB * DD], sc[NQ * NB];
    for (int i = 0; i < NQ * DD; i++) qb[i] = gauss();
    for (int i = 0; i < NB * DD; i++) kb[i] = gauss();
    oracle_scores(qb, kb, NQ, NB, DD, sc);
    int32_t idx[NQ * 3];
    oracle_select(sc, NQ, NB, 3, idx);
    for (int i = 0; i < NQ; i++)
        for (int a = 0; a < 3; a++) {
            int better = 0;
            for (int j = 0; j < NB; j++)
                better += sc[i * NB + j] > sc[i * NB + idx[i * 3 + a]];
            CHECK(better < 3);
        }
    /* whole heads: ragged length, with and without the linear branch, quantized or not */
    const int d = 128, blk = 64;
    const int Ns[3] = {37, 200, 300};
    for (int t = 0; t < 3; t++) {
        int N = Ns[t], Nb = oracle_num_blocks(N, blk);
        uint16_t *q = malloc(sizeof(uint16_t) * N * d), *k = malloc(sizeof(uint16_t) * N * d);
        uint16_t *v = malloc(sizeof(uint16_t) * N * d), *w = malloc(sizeof(uint16_t) * d * d);
        fill_bf16(q, (size_t)N * d, 1.0);
        fill_bf16(k, (size_t)N * d, 1.0);
        fill_bf16(v, (size_t)N * d, 1.0);
        fill_bf16(w, (size_t)d * d, 1.0 / sqrt((double)d));
        int32_t *qbl = malloc(sizeof(int32_t) * Nb);
        for (int b = 0; b < Nb; b++) qbl[b] = b;
        double topk = 0.5;
        int ks = oracle_ksel(topk, Nb);
        double *out = malloc(sizeof(double) * Nb * blk * d), *os = malloc(sizeof(double) * Nb * blk * d);
        double *ol = malloc(sizeof(double) * Nb * blk * d);
        int32_t *id = malloc(sizeof(int32_t) * Nb * ks);
        for (int quant = 0; quant < 2; quant++)
            for (int lin = 0; lin < 2; lin++) {
                CHECK(oracle_sagesla_head(q, k, v, lin ? w : NULL, N, d, blk, topk, quant, qbl, Nb, out, os, ol, id) == ks);
                for (int r = 0; r < N; r++)
                    for (int c = 0; c < d; c++) CHECK(isfinite(out[(size_t)r * d + c]));
                for (int b = 0; b < Nb; b++)
                    for (int u = 0; u < ks; u++) CHECK(id[b * ks + u] >= 0 && id[b * ks + u] < Nb);
            }
        free(q); free(k); free(v); free(w); free(qbl); free(out); free(os); free(ol); free(id);
    }
    /* the W8A8 oracle on a ragged row count */
    {
        int M = 3, K = 256, N = 256;
        uint16_t *x = malloc(sizeof(uint16_t) * M * K), *wt = malloc(sizeof(uint16_t) * N * K);
        uint16_t *bias = malloc(sizeof(uint16_t) * N);
        fill_bf16(x, (size_t)M * K, 1.0);
        fill_bf16(wt, (size_t)N * K, 0.06);
        fill_bf16(bias, N, 0.02);
        int8_t *qx = malloc((size_t)M * K), *qw = malloc((size_t)N * K);
        float *sx = malloc(sizeof(float) * M * (K / 128)), *sw = malloc(sizeof(float) * (N / 128) * (K / 128));
        double *y = malloc(sizeof(double) * M * N);
        oracle_w8a8_quant_act(x, M, K, qx, sx);
        oracle_w8a8_quant_weight(wt, N, K, qw, sw);
        oracle_w8a8_gemm(qx, sx, qw, sw, bias, M, N, K, 0, M, y);
        for (int e = 0; e < M * N; e++) CHECK(isfinite(y[e]));
        free(x); free(wt); free(bias); free(qx); free(qw); free(sx); free(sw); free(y);
    }
    printf("oracle driver ok\n");
    return 0;
}
