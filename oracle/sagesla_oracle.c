/*
 * SageSLA attention forward: plain, slow CPU oracle (test infrastructure only).
 *
 * This file is the reference that the GPU path is checked against. Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark may load it. It
 * shares no code with the GPU library: it is plain scalar C, fp64 wherever no
 * rounding is being replicated and fp32 exactly where the GPU's fp32 rounding
 * decides an integer code (INT8/FP8 quantization), built with -ffp-contract=off.
 *
 * What the method computes (sources):
 *  - SageSLA = sparse-linear attention (SLA) combined with SageAttention low-bit
 *    quantization, swapped in for trained SLA at inference (TurboDiffusion explainer,
 *    news.qq.com, sections "First key: attention" and "From training to deployment").
 *  - SLA first quickly scores how strongly pairs are related, keeps the top fraction
 *    (Top-K ratio 0.1, 0.1-0.15 recommended) exactly, and skips the rest from the
 *    exact computation (same page, "First key"); the remainder goes to a linear-
 *    attention branch (bonega.ai blog, SLA paragraph; tiemojia.cn article, 2.2.1).
 *  - SageAttention quantizes to 8-bit integers (news.qq.com, "First key"); outliers
 *    are smoothed into the normal range before quantization and restored after
 *    (news.qq.com, "Third key"); every small block is quantized with a single
 *    scale of its own (news.qq.com, "Third key").
 * The pages give no formulas. Every step below that they leave open follows one
 * stated reading (block granularity 64, mean pooling, scores qbar.kbar/sqrt(d),
 * ceil(topk*Nb) blocks per query block, K-mean smoothing, per-block INT8 Q/K,
 * per-channel FP8 e4m3 V, e4m3(448 p) probabilities normalised by their own sum,
 * kept blocks processed best first, phi = softmax over channels,
 * O = O_s + O_l W_proj). Parity of those choices is unpinned by the pages; the
 * implementation of each is pinned by the tests in tests/test_oracle_*.py.
 *
 * Layout: one head at a time. q, k, v are bf16 bit patterns, [N][d] row-major.
 * Token blocks are blk consecutive tokens; the last block may hold fewer (n_i).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- number formats */

/* bf16 -> value: the top 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static float bf16f(uint16_t h) { return (float)oracle_bf16_to_double(h); }

/* value -> bf16, round to nearest even (NaN not expected). */
uint16_t oracle_double_to_bf16(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * OCP 8-bit floating point, E4M3FN variant (OCP "8-bit Floating Point Specification
 * (OFP8)"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 1.75*2^8 = 448, smallest normal 2^-6,
 * subnormals m*2^-9 for m = 1..7.
 */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* The decode above evaluated once for all 256 codes when the library loads (used in
 * the inner loops; filled before any thread can call in). */
static double e4m3_table[256];

__attribute__((constructor)) static void e4m3_table_init(void)
{
    for (int i = 0; i < 256; i++)
        e4m3_table[i] = oracle_e4m3_decode((uint8_t)i);
}

static double dec8(uint8_t c) { return e4m3_table[c]; }

/* fp32 -> e4m3, round to nearest with ties to even, saturating to +-448 (finite in). */
uint8_t oracle_e4m3_encode(float xf)
{
    double x = (double)xf;
    uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7E;
    /* spacing of representable values around a */
    int e;
    double quantum;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
        quantum = ldexp(1.0, (e - 1) - 3);
    }
    double n = nearbyint(a / quantum); /* exact division by a power of two; ties-to-even */
    double r = n * quantum;
    if (r >= 448.0)
        return sign | 0x7E;
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))
        return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: m in 1..7 (8 -> normal) */
    int er;
    double fr = frexp(r, &er);                     /* r = fr*2^er, fr in [0.5,1) */
    int exp_field = (er - 1) + 7;
    int mant = (int)((fr * 2.0 - 1.0) * 8.0 + 0.5);
    return sign | (uint8_t)(exp_field << 3) | (uint8_t)mant;
}

/* ---------------------------------------------------------------- block geometry */

int oracle_num_blocks(int N, int blk) { return (N + blk - 1) / blk; }

static int block_len(int i, int N, int blk)
{
    int rem = N - i * blk;
    return rem < blk ? rem : blk;
}

/*
 * Number of key blocks kept per query block: the Top-K ratio applied to the number of
 * key blocks, rounded up, at least 1 and at most all (reading of keeping the top tenth,
 * news.qq.com, "First key"). The 1e-9 guards products such as 0.1*30 that land a hair
 * above an integer in binary.
 */
int oracle_ksel(double topk, int Nb)
{
    double x = ceil(topk * (double)Nb - 1e-9);
    int k = (int)x;
    if (k < 1)
        k = 1;
    if (k > Nb)
        k = Nb;
    return k;
}

/* ---------------------------------------------------------------- O1: pooling */

/* Block means of x over the valid tokens of each block, fp64. out: [Nb][d]. */
void oracle_pool(const uint16_t *x, int N, int d, int blk, double *out)
{
    int Nb = oracle_num_blocks(N, blk);
    for (int i = 0; i < Nb; i++) {
        int n = block_len(i, N, blk);
        for (int c = 0; c < d; c++) {
            double s = 0.0;
            for (int t = 0; t < n; t++)
                s += oracle_bf16_to_double(x[(size_t)(i * blk + t) * d + c]);
            out[(size_t)i * d + c] = s / n;
        }
    }
}

/* ---------------------------------------------------------------- O2, O3: score and select */

/* s_ij = qbar_i . kbar_j / sqrt(d), fp64. qbar: [nq][d], kbar: [nk][d], scores: [nq][nk]. */
void oracle_scores(const double *qbar, const double *kbar, int nq, int nk, int d, double *scores)
{
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < nq; i++)
        for (int j = 0; j < nk; j++) {
            double s = 0.0;
            for (int c = 0; c < d; c++)
                s += qbar[(size_t)i * d + c] * kbar[(size_t)j * d + c];
            scores[(size_t)i * nk + j] = s * inv;
        }
}

/*
 * For every query block keep the ksel key blocks with the largest score; equal scores
 * prefer the lower key index. The kept indices are written in ascending order.
 * Plain selection: ksel passes, each picking the best not-yet-taken block.
 * scores: [nq][Nb], idx: [nq][ksel].
 */
void oracle_select(const double *scores, int nq, int Nb, int ksel, int32_t *idx)
{
    char *taken = (char *)malloc((size_t)Nb);
    for (int i = 0; i < nq; i++) {
        const double *row = scores + (size_t)i * Nb;
        memset(taken, 0, (size_t)Nb);
        for (int r = 0; r < ksel; r++) {
            int best = -1;
            for (int j = 0; j < Nb; j++) {
                if (taken[j])
                    continue;
                if (best < 0 || row[j] > row[best])
                    best = j; /* strict '>' keeps the lower index on ties */
            }
            taken[best] = 1;
        }
        int w = 0;
        for (int j = 0; j < Nb; j++)
            if (taken[j])
                idx[(size_t)i * ksel + w++] = j;
    }
    free(taken);
}

/*
 * Processing order of a row's kept blocks (reading): the block with the highest score
 * first (lowest index on ties), then the other kept blocks in ascending index order.
 * The running softmax maximum then starts at (almost always) its final value.
 * row: one score row [Nb]; kept: the ksel kept indices in ascending order (rewritten).
 */
void oracle_order_best_first(const double *row, int ksel, int32_t *kept)
{
    int best = 0;
    for (int u = 1; u < ksel; u++)
        if (row[kept[u]] > row[kept[best]])
            best = u; /* strict '>' keeps the lower index on ties */
    int32_t jb = kept[best];
    for (int u = best; u > 0; u--)
        kept[u] = kept[u - 1];
    kept[0] = jb;
}

/* ---------------------------------------------------------------- adaptive k_sel */

/*
 * Content-adaptive number of kept blocks per head. The pages list sparsity that adapts
 * to the content as future work and give no rule (news.qq.com explainer, the section on
 * the method's limits, sixth challenge; 0.1-0.15 of the blocks at inference, section
 * "From training to deployment"). Reading: the block scores s_ij already estimate the
 * attention logits of the block pair, so the pooled attention mass of key block j for
 * query block i is w_ij = n_j exp(s_ij - max_j s_ij) (n_j valid tokens), and query block
 * i needs k_i = the fewest blocks, taken in selection order (score descending, lower
 * index on ties), whose mass reaches tau of its row's total sum_j w_ij. A head keeps
 * k_sel = clamp(ceil(sum_i k_i / nq), kmin, kmax) blocks for every query block
 * (the same count for all of a head's query blocks).
 *
 * scores: [nq][Nb] (the selection scores), n_j from N and blk. k_rows: [nq]. margin
 * (may be NULL): [nq], the distance of tau from the nearer of the two prefix masses
 * around the decision, |prefix(k_i) - tau W| and |prefix(k_i - 1) - tau W|, over W;
 * a decision closer than rounding can change is a near-tie.
 * Plain: a full sort of each row by (score desc, index asc), then a running sum.
 */
typedef struct {
    double s;
    int j;
} scored_block;

/* selection order: higher score first, lower index on equal scores */
static int adaptive_cmp(const void *a, const void *b)
{
    const scored_block *x = (const scored_block *)a, *y = (const scored_block *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return x->j < y->j ? -1 : (x->j > y->j ? 1 : 0);
}

void oracle_adaptive_k(const double *scores, int nq, int Nb, int N, int blk, double tau, int32_t *k_rows,
                       double *margin)
{
    scored_block *order = (scored_block *)malloc(sizeof(scored_block) * (size_t)Nb);
    double *w = (double *)malloc(sizeof(double) * (size_t)Nb);
    for (int i = 0; i < nq; i++) {
        const double *row = scores + (size_t)i * Nb;
        double mx = -INFINITY;
        for (int j = 0; j < Nb; j++)
            if (row[j] > mx)
                mx = row[j];
        double W = 0.0;
        for (int j = 0; j < Nb; j++) {
            w[j] = (double)block_len(j, N, blk) * exp(row[j] - mx);
            W += w[j];
        }
        for (int j = 0; j < Nb; j++) {
            order[j].s = row[j];
            order[j].j = j;
        }
        qsort(order, (size_t)Nb, sizeof(scored_block), adaptive_cmp);
        const double T = tau * W;
        double prefix = 0.0, before = 0.0;
        int k = Nb;
        for (int r = 0; r < Nb; r++) {
            before = prefix;
            prefix += w[order[r].j];
            if (prefix >= T) {
                k = r + 1;
                break;
            }
        }
        k_rows[i] = k;
        if (margin) {
            double a = fabs(prefix - T), b = fabs(before - T);
            margin[i] = (a < b ? a : b) / W;
        }
    }
    free(order);
    free(w);
}

/* Per-head count from the rows' counts: clamp(ceil(sum k_i / nq), kmin, kmax), the
 * ceiling taken on integers. */
int oracle_adaptive_ksel(const int32_t *k_rows, int nq, int kmin, int kmax)
{
    long long sum = 0;
    for (int i = 0; i < nq; i++)
        sum += k_rows[i];
    int k = (int)((sum + nq - 1) / nq);
    if (k < kmin)
        k = kmin;
    if (k > kmax)
        k = kmax;
    return k;
}

/* ---------------------------------------------------------------- O4: K smoothing */

/*
 * Per-channel mean of K over all N tokens, fp64 sum then rounded to fp32 (the outlier
 * smoothing of news.qq.com, "Third key", read as subtracting the channel mean of K;
 * it leaves softmax(q.k) unchanged because q.mu is the same for every key of a row).
 */
void oracle_k_mean(const uint16_t *k, int N, int d, float *mu)
{
    for (int c = 0; c < d; c++) {
        double s = 0.0;
        for (int t = 0; t < N; t++)
            s += oracle_bf16_to_double(k[(size_t)t * d + c]);
        mu[c] = (float)(s / N);
    }
}

/* ---------------------------------------------------------------- O5, O6: quantization */

/* INT8 code of x with multiplier inv: round half to even, clamp to [-127, 127] (fp32). */
static int8_t q_int8(float x, float inv)
{
    float y = x * inv;
    float r = nearbyintf(y);
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/*
 * Per-block symmetric INT8 of fp32 values x: [N][d] (one scale per block of blk tokens
 * over all d channels; one scale per small block, news.qq.com,
 * "Third key"). amax over the valid tokens; inv = 127/amax, scale = amax/127 (fp32
 * IEEE divisions); amax = 0 gives zero codes and scale 0. Padded rows are 0.
 * q8: [Nb*blk][d], scale: [Nb].
 */
void oracle_quant_blocks(const float *x, int N, int d, int blk, int8_t *q8, float *scale)
{
    int Nb = oracle_num_blocks(N, blk);
    memset(q8, 0, (size_t)Nb * blk * d);
    for (int i = 0; i < Nb; i++) {
        int n = block_len(i, N, blk);
        float amax = 0.0f;
        for (int t = 0; t < n; t++)
            for (int c = 0; c < d; c++) {
                float a = fabsf(x[(size_t)(i * blk + t) * d + c]);
                if (a > amax)
                    amax = a;
            }
        float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        scale[i] = amax > 0.0f ? amax / 127.0f : 0.0f;
        for (int t = 0; t < n; t++)
            for (int c = 0; c < d; c++)
                q8[(size_t)(i * blk + t) * d + c] = q_int8(x[(size_t)(i * blk + t) * d + c], inv);
    }
}

/*
 * Per-channel FP8 e4m3 of V over all N tokens: inv = 448/amax_c, scale = amax_c/448,
 * code = e4m3(v*inv) (fp32 product). v8: [N][d], sv: [d].
 */
void oracle_quant_v(const uint16_t *v, int N, int d, uint8_t *v8, float *sv)
{
    for (int c = 0; c < d; c++) {
        float amax = 0.0f;
        for (int t = 0; t < N; t++) {
            float a = fabsf(bf16f(v[(size_t)t * d + c]));
            if (a > amax)
                amax = a;
        }
        float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        sv[c] = amax > 0.0f ? amax / 448.0f : 0.0f;
        for (int t = 0; t < N; t++)
            v8[(size_t)t * d + c] = oracle_e4m3_encode(bf16f(v[(size_t)t * d + c]) * inv);
    }
}

/* ---------------------------------------------------------------- O7: sparse softmax */

/*
 * Exact integer dot product of two INT8 rows (|S| <= d*127*127 fits int32).
 */
int32_t oracle_dot_i8(const int8_t *a, const int8_t *b, int d)
{
    int32_t s = 0;
    for (int c = 0; c < d; c++)
        s += (int32_t)a[c] * (int32_t)b[c];
    return s;
}

/*
 * Quantized sparse attention for the rows of query block qb (reading of SageAttention
 * on the kept blocks): for each kept key block j in the row's processing order,
 *   S = q8 . k8 (int32), a = (s_q[i]*s_k[j]) * c0 with c0 = fp32(log2(e)/sqrt(d)),
 *   x = fp32(S)*a, the reference m' = max(m, ceil(max x)): the running row maximum
 *     rounded up to an integer (in log2 units), so that every change of reference is an
 *     exact power of two, alpha = exp2f(m - m') (0 for the first block),
 *   w = exp2f(fmaf(F, a, c)) with F = 1.5*2^23 + S (an integer below 2^24, exact in
 *     fp32), c = (L - m') - fp32(1.5*2^23 * a) and L = fp32(log2(448)); in exact
 *     arithmetic F*a + c = S*a + L - m', so w = 448 p for p = 2^(x - m') up to the fp32
 *     roundings of c and of the fused product (the exponent argument is formed in fp32
 *     exactly as the FP8 code decision is taken on the GPU, whose integer accumulators
 *     start from the bit pattern of 1.5*2^23); the row maximum gets a weight in (224, 448],
 *   p8 = e4m3(w) (saturating),
 *   l = l*alpha + sum dec(p8), acc = acc*alpha + sum dec(p8)*dec(v8) (fp64), m = m'.
 * Output row: acc[c] * sv[c] / l, i.e. the average of the dequantized V rows weighted by
 * the FP8 probabilities actually used. Keys past N are skipped.
 * out: [blk][d] (rows past N left untouched). l_out, ref_out (may be NULL): [blk], each
 * row's final l and reference m.
 */
void oracle_sparse_block(const int8_t *q8, const int8_t *k8, const uint8_t *v8,
                         const float *sq, const float *sk, const float *sv,
                         const int32_t *idx, int ksel, int N, int d, int blk, int qb,
                         double *out, double *l_out, float *ref_out)
{
    const float c0 = (float)(1.4426950408889634 / sqrt((double)d));
    const float L = (float)log2(448.0);
    int nq = block_len(qb, N, blk);
    const int32_t *crit = idx + (size_t)qb * ksel;
    float *sf = (float *)malloc(sizeof(float) * blk);
    double *acc = (double *)malloc(sizeof(double) * d);
    for (int r = 0; r < nq; r++) {
        const int8_t *qrow = q8 + (size_t)(qb * blk + r) * d;
        float m = -INFINITY;
        double l = 0.0;
        for (int c = 0; c < d; c++)
            acc[c] = 0.0;
        for (int u = 0; u < ksel; u++) {
            int j = crit[u];
            int nk = block_len(j, N, blk);
            float a = (sq[qb] * sk[j]) * c0;
            float mb = -INFINITY;
            for (int t = 0; t < nk; t++) {
                sf[t] = (float)oracle_dot_i8(qrow, k8 + (size_t)(j * blk + t) * d, d);
                float x = sf[t] * a;
                if (x > mb)
                    mb = x;
            }
            float mbr = ceilf(mb);
            float mn = m > mbr ? m : mbr;
            float alpha = exp2f(m - mn);
            float c = (L - mn) - 12582912.0f * a;
            l *= (double)alpha;
            for (int c = 0; c < d; c++)
                acc[c] *= (double)alpha;
            for (int t = 0; t < nk; t++) {
                double pq = dec8(oracle_e4m3_encode(exp2f(fmaf(12582912.0f + sf[t], a, c))));
                l += pq;
                const uint8_t *vrow = v8 + (size_t)(j * blk + t) * d;
                for (int c = 0; c < d; c++)
                    acc[c] += pq * dec8(vrow[c]);
            }
            m = mn;
        }
        for (int c = 0; c < d; c++)
            out[(size_t)r * d + c] = acc[c] * (double)sv[c] / l;
        if (l_out)
            l_out[r] = l;
        if (ref_out)
            ref_out[r] = m;
    }
    free(sf);
    free(acc);
}

/*
 * Unquantized variant of the same computation (fp64 throughout, raw bf16 Q and K, no
 * smoothing): softmax over the kept keys of q.k/sqrt(d), times V. With every block
 * kept this is textbook softmax attention.
 */
void oracle_sparse_block_fp64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *idx, int ksel, int N, int d, int blk, int qb,
                              double *out)
{
    double inv = 1.0 / sqrt((double)d);
    int nq = block_len(qb, N, blk);
    const int32_t *crit = idx + (size_t)qb * ksel;
    double *acc = (double *)malloc(sizeof(double) * d);
    double *xs = (double *)malloc(sizeof(double) * blk);
    for (int r = 0; r < nq; r++) {
        size_t qrow = (size_t)(qb * blk + r) * d;
        double m = -INFINITY, l = 0.0;
        for (int c = 0; c < d; c++)
            acc[c] = 0.0;
        for (int u = 0; u < ksel; u++) {
            int j = crit[u];
            int nk = block_len(j, N, blk);
            double mb = -INFINITY;
            for (int t = 0; t < nk; t++) {
                double s = 0.0;
                size_t krow = (size_t)(j * blk + t) * d;
                for (int c = 0; c < d; c++)
                    s += oracle_bf16_to_double(q[qrow + c]) * oracle_bf16_to_double(k[krow + c]);
                xs[t] = s * inv;
                if (xs[t] > mb)
                    mb = xs[t];
            }
            double mn = m > mb ? m : mb;
            double alpha = exp(m - mn);
            l *= alpha;
            for (int c = 0; c < d; c++)
                acc[c] *= alpha;
            for (int t = 0; t < nk; t++) {
                double p = exp(xs[t] - mn);
                l += p;
                size_t vrow = (size_t)(j * blk + t) * d;
                for (int c = 0; c < d; c++)
                    acc[c] += p * oracle_bf16_to_double(v[vrow + c]);
            }
            m = mn;
        }
        for (int c = 0; c < d; c++)
            out[(size_t)r * d + c] = acc[c] / l;
    }
    free(acc);
    free(xs);
}

/* ---------------------------------------------------------------- O8: linear branch */

/* phi(x) = softmax over the d channels of a raw bf16 row, fp64, max-subtracted. */
void oracle_phi(const uint16_t *x, int d, double *out)
{
    double mx = -INFINITY;
    for (int c = 0; c < d; c++) {
        double a = oracle_bf16_to_double(x[c]);
        if (a > mx)
            mx = a;
    }
    double s = 0.0;
    for (int c = 0; c < d; c++) {
        out[c] = exp(oracle_bf16_to_double(x[c]) - mx);
        s += out[c];
    }
    for (int c = 0; c < d; c++)
        out[c] /= s;
}

/*
 * Per key block j: H_j[a][c] = sum_{t in j} phi(k_t)[a] * v_t[c] and
 * z_j[a] = sum_{t in j} phi(k_t)[a], fp64 (linear-attention states of the SLA branch).
 * H: [Nb][d][d], z: [Nb][d].
 */
void oracle_linear_states(const uint16_t *k, const uint16_t *v, int N, int d, int blk,
                          double *H, double *z)
{
    int Nb = oracle_num_blocks(N, blk);
    double *ph = (double *)malloc(sizeof(double) * d);
    memset(H, 0, sizeof(double) * (size_t)Nb * d * d);
    memset(z, 0, sizeof(double) * (size_t)Nb * d);
    for (int t = 0; t < N; t++) {
        int j = t / blk;
        oracle_phi(k + (size_t)t * d, d, ph);
        double *Hj = H + (size_t)j * d * d;
        for (int a = 0; a < d; a++) {
            z[(size_t)j * d + a] += ph[a];
            for (int c = 0; c < d; c++)
                Hj[(size_t)a * d + c] += ph[a] * oracle_bf16_to_double(v[(size_t)t * d + c]);
        }
    }
    free(ph);
}

/*
 * Linear-branch output for the rows of query block qb: the complement state is summed
 * directly over the blocks NOT kept for qb,
 *   Hc = sum_{j not kept} H_j,  zc = sum_{j not kept} z_j,
 *   O_l[r] = phi(q_r) Hc / (phi(q_r) . zc),
 * or 0 when every block is kept. out: [blk][d].
 */
void oracle_linear_block(const uint16_t *q, const double *H, const double *z,
                         const int32_t *idx, int ksel, int N, int d, int blk, int qb,
                         double *out)
{
    int Nb = oracle_num_blocks(N, blk);
    int nq = block_len(qb, N, blk);
    if (ksel >= Nb) {
        for (int r = 0; r < nq; r++)
            for (int c = 0; c < d; c++)
                out[(size_t)r * d + c] = 0.0;
        return;
    }
    char *kept = (char *)calloc((size_t)Nb, 1);
    for (int u = 0; u < ksel; u++)
        kept[idx[(size_t)qb * ksel + u]] = 1;
    double *Hc = (double *)calloc((size_t)d * d, sizeof(double));
    double *zc = (double *)calloc((size_t)d, sizeof(double));
    for (int j = 0; j < Nb; j++) {
        if (kept[j])
            continue;
        for (int e = 0; e < d * d; e++)
            Hc[e] += H[(size_t)j * d * d + e];
        for (int a = 0; a < d; a++)
            zc[a] += z[(size_t)j * d + a];
    }
    double *ph = (double *)malloc(sizeof(double) * d);
    for (int r = 0; r < nq; r++) {
        oracle_phi(q + (size_t)(qb * blk + r) * d, d, ph);
        double den = 0.0;
        for (int a = 0; a < d; a++)
            den += ph[a] * zc[a];
        for (int c = 0; c < d; c++) {
            double num = 0.0;
            for (int a = 0; a < d; a++)
                num += ph[a] * Hc[(size_t)a * d + c];
            out[(size_t)r * d + c] = num / den;
        }
    }
    free(ph);
    free(Hc);
    free(zc);
    free(kept);
}

/* ---------------------------------------------------------------- O9: projection */

/* y[r] = ol[r] W, W row-major [d][d] bf16 (row vector times matrix), fp64. */
void oracle_project(const double *ol, const uint16_t *w, int rows, int d, double *y)
{
    for (int r = 0; r < rows; r++)
        for (int c = 0; c < d; c++) {
            double s = 0.0;
            for (int a = 0; a < d; a++)
                s += ol[(size_t)r * d + a] * oracle_bf16_to_double(w[(size_t)a * d + c]);
            y[(size_t)r * d + c] = s;
        }
}

/* ---------------------------------------------------------------- whole head */

/*
 * SageSLA forward of one head for the query blocks listed in qblocks, keeping ksel key
 * blocks per query block:
 *   O = O_s + O_l W_proj,
 * O_s from the quantized sparse softmax (quant = 1) or its fp64 form (quant = 0),
 * O_l from the linear branch over the blocks that were not kept (skipped when w is
 * NULL or every block is kept). Outputs for listed block b go to rows
 * [b_pos*blk, b_pos*blk + n_b) of out, out_s, out_l (each [nqb*blk][d]; out_s / out_l
 * may be NULL). idx_out (may be NULL, [Nb][kstride], kstride >= ksel) receives the kept
 * blocks of every listed query block in its row, -1 past ksel; rows of query blocks
 * that are not listed are all -1. Scores and selection are evaluated only for the listed
 * query blocks.
 */
static void head_core(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *w,
                      int N, int d, int blk, int ksel, int kstride, int quant, const int32_t *qblocks,
                      int nqb, double *out, double *out_s, double *out_l, int32_t *idx_out)
{
    int Nb = oracle_num_blocks(N, blk);

    /* O1-O3: pooling, scores and selection for the listed query blocks */
    double *qbar = (double *)malloc(sizeof(double) * (size_t)Nb * d);
    double *kbar = (double *)malloc(sizeof(double) * (size_t)Nb * d);
    double *srow = (double *)malloc(sizeof(double) * (size_t)Nb);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)Nb * ksel);
    for (size_t e = 0; e < (size_t)Nb * ksel; e++)
        idx[e] = -1;
    oracle_pool(q, N, d, blk, qbar);
    oracle_pool(k, N, d, blk, kbar);
    for (int b = 0; b < nqb; b++) {
        int qb = qblocks[b];
        if (qb < 0 || qb >= Nb)
            continue;
        oracle_scores(qbar + (size_t)qb * d, kbar, 1, Nb, d, srow);
        oracle_select(srow, 1, Nb, ksel, idx + (size_t)qb * ksel);
        oracle_order_best_first(srow, ksel, idx + (size_t)qb * ksel);
    }
    if (idx_out)
        for (int i = 0; i < Nb; i++)
            for (int r = 0; r < kstride; r++)
                idx_out[(size_t)i * kstride + r] = r < ksel ? idx[(size_t)i * ksel + r] : -1;
    free(qbar);
    free(kbar);
    free(srow);

    /* O4-O6: smoothing and quantization */
    int8_t *q8 = NULL, *k8 = NULL;
    uint8_t *v8 = NULL;
    float *sq = NULL, *sk = NULL, *sv = NULL;
    if (quant) {
        float *xf = (float *)malloc(sizeof(float) * (size_t)N * d);
        float *mu = (float *)malloc(sizeof(float) * d);
        q8 = (int8_t *)malloc((size_t)Nb * blk * d);
        k8 = (int8_t *)malloc((size_t)Nb * blk * d);
        v8 = (uint8_t *)malloc((size_t)N * d);
        sq = (float *)malloc(sizeof(float) * Nb);
        sk = (float *)malloc(sizeof(float) * Nb);
        sv = (float *)malloc(sizeof(float) * d);
        for (size_t e = 0; e < (size_t)N * d; e++)
            xf[e] = bf16f(q[e]);
        oracle_quant_blocks(xf, N, d, blk, q8, sq);
        oracle_k_mean(k, N, d, mu);
        for (size_t e = 0; e < (size_t)N * d; e++)
            xf[e] = bf16f(k[e]) - mu[e % d];
        oracle_quant_blocks(xf, N, d, blk, k8, sk);
        oracle_quant_v(v, N, d, v8, sv);
        free(xf);
        free(mu);
    }

    /* O8 states */
    double *H = NULL, *z = NULL;
    int linear = (w != NULL) && ksel < Nb;
    if (linear) {
        H = (double *)malloc(sizeof(double) * (size_t)Nb * d * d);
        z = (double *)malloc(sizeof(double) * (size_t)Nb * d);
        oracle_linear_states(k, v, N, d, blk, H, z);
    }

    /* O7-O10 per listed query block */
    double *os = (double *)malloc(sizeof(double) * (size_t)blk * d);
    double *ol = (double *)malloc(sizeof(double) * (size_t)blk * d);
    double *y = (double *)malloc(sizeof(double) * (size_t)blk * d);
    for (int b = 0; b < nqb; b++) {
        int qb = qblocks[b];
        if (qb < 0 || qb >= Nb)
            continue;
        int nq = block_len(qb, N, blk);
        if (quant)
            oracle_sparse_block(q8, k8, v8, sq, sk, sv, idx, ksel, N, d, blk, qb, os, NULL, NULL);
        else
            oracle_sparse_block_fp64(q, k, v, idx, ksel, N, d, blk, qb, os);
        if (linear) {
            oracle_linear_block(q, H, z, idx, ksel, N, d, blk, qb, ol);
            oracle_project(ol, w, nq, d, y);
        } else {
            memset(ol, 0, sizeof(double) * (size_t)blk * d);
            memset(y, 0, sizeof(double) * (size_t)blk * d);
        }
        for (int r = 0; r < nq; r++)
            for (int c = 0; c < d; c++) {
                size_t o = ((size_t)b * blk + r) * d + c;
                out[o] = os[(size_t)r * d + c] + y[(size_t)r * d + c];
                if (out_s)
                    out_s[o] = os[(size_t)r * d + c];
                if (out_l)
                    out_l[o] = ol[(size_t)r * d + c];
            }
    }
    free(os);
    free(ol);
    free(y);
    free(idx);
    free(q8);
    free(k8);
    free(v8);
    free(sq);
    free(sk);
    free(sv);
    free(H);
    free(z);
}

/* The forward of one head at the Top-K ratio topk (ksel = oracle_ksel(topk, Nb)); outputs
 * as for head_core with kstride = ksel. Returns ksel, or -1 on bad arguments. */
int oracle_sagesla_head(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const uint16_t *w, int N, int d, int blk, double topk, int quant,
                        const int32_t *qblocks, int nqb, double *out, double *out_s,
                        double *out_l, int32_t *idx_out)
{
    if (N < 1 || d < 1 || blk < 1 || !(topk > 0.0 && topk <= 1.0))
        return -1;
    int ksel = oracle_ksel(topk, oracle_num_blocks(N, blk));
    head_core(q, k, v, w, N, d, blk, ksel, ksel, quant, qblocks, nqb, out, out_s, out_l, idx_out);
    return ksel;
}

/*
 * The forward of one head with its content-adaptive count: scores of every query block
 * (oracle_pool, oracle_scores), k_rows = oracle_adaptive_k at tau, the head's count
 * ksel = oracle_adaptive_ksel(k_rows, oracle_ksel(topk_min), oracle_ksel(topk_max)),
 * then head_core with kstride = oracle_ksel(topk_max). k_rows (may be NULL): [Nb].
 * Returns ksel, or -1 on bad arguments.
 */
int oracle_sagesla_head_adaptive(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *w, int N, int d, int blk, double topk_min,
                                 double topk_max, double tau, int quant, const int32_t *qblocks,
                                 int nqb, double *out, double *out_s, double *out_l,
                                 int32_t *idx_out, int32_t *k_rows)
{
    if (N < 1 || d < 1 || blk < 1 || !(topk_min > 0.0 && topk_min <= topk_max && topk_max <= 1.0) ||
        !(tau > 0.0 && tau <= 1.0))
        return -1;
    int Nb = oracle_num_blocks(N, blk);
    int kmin = oracle_ksel(topk_min, Nb), kmax = oracle_ksel(topk_max, Nb);
    double *qbar = (double *)malloc(sizeof(double) * (size_t)Nb * d);
    double *kbar = (double *)malloc(sizeof(double) * (size_t)Nb * d);
    double *S = (double *)malloc(sizeof(double) * (size_t)Nb * Nb);
    int32_t *kr = (int32_t *)malloc(sizeof(int32_t) * (size_t)Nb);
    oracle_pool(q, N, d, blk, qbar);
    oracle_pool(k, N, d, blk, kbar);
    oracle_scores(qbar, kbar, Nb, Nb, d, S);
    oracle_adaptive_k(S, Nb, Nb, N, blk, tau, kr, NULL);
    int ksel = oracle_adaptive_ksel(kr, Nb, kmin, kmax);
    if (k_rows)
        memcpy(k_rows, kr, sizeof(int32_t) * (size_t)Nb);
    free(qbar);
    free(kbar);
    free(S);
    free(kr);
    head_core(q, k, v, w, N, d, blk, ksel, kmax, quant, qblocks, nqb, out, out_s, out_l, idx_out);
    return ksel;
}

/* ---------------------------------------------------------------- array helpers */

void oracle_e4m3_encode_n(const float *x, uint8_t *c, size_t n)
{
    for (size_t i = 0; i < n; i++)
        c[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_n(const uint8_t *c, double *x, size_t n)
{
    for (size_t i = 0; i < n; i++)
        x[i] = oracle_e4m3_decode(c[i]);
}
