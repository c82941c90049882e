/*
 * sagesla.h — C ABI of the SageSLA attention forward for AMD Instinct MI355X (gfx950).
 *
 * SageSLA is sparse-linear attention (SLA) combined with SageAttention's low-bit
 * quantization, swapped in for trained SLA at inference time (TurboDiffusion explainer,
 * news.qq.com, sections "First key: attention" and "From training to deployment").
 * SLA scores how strongly pairs of positions are related, computes only the top
 * fraction exactly (Top-K ratio 0.1; 0.1-0.15 recommended) and hands the rest to a
 * linear-attention branch; SageAttention runs the exact part on 8-bit data (same page;
 * bonega.ai blog, SLA paragraph; tiemojia.cn article, sections 2.2.1-2.2.2).
 *
 * The pages give no formulas. This library computes, per (batch, head):
 *   1. pooling + selection: mean-pool Q and K over 64-token blocks, score block pairs
 *      s_ij = Qbar_i . Kbar_j / sqrt(d) (fp64, compared exactly), keep the
 *      ksel = ceil(topk * Nb) best key blocks of every query block (ties: lower index),
 *      stored best first (highest score, lowest index on ties), then the rest ascending;
 *   2. quantization: K smoothed by its per-channel mean over all tokens; Q and K to INT8
 *      per 64-token block (scale amax/127, round half to even); V to FP8 e4m3 per
 *      channel (scale amax/448);
 *   3. sparse attention over the kept blocks: INT8 QK^T, online softmax in fp32,
 *      probabilities as e4m3(p*448), FP8 PV;
 *   4. linear branch over the other blocks: phi = softmax over the d channels,
 *      per-key-block states H_j = phi(K_j)^T V_j and z_j = colsum phi(K_j), the
 *      complement total minus kept, O_l = phi(q) H^c / (phi(q) . z^c);
 *   5. output O = O_s + O_l W_proj (bf16).
 *
 * Conventions (all entry points):
 *  - Tensors are device pointers to contiguous row-major data. q, k, v, out are bf16
 *    [B, H, N, d]; proj is bf16 [d, d] applied as (row vector) x W.
 *  - This version supports d = 128 and block = 64 only (others: SAGESLA_ERR_UNSUPPORTED),
 *    1 <= N <= 1048576, B*H*ceil(N/64) < 2^31, 0 < topk <= 1.
 *  - Every pointer must be 16-byte aligned. The caller owns all memory; the library
 *    allocates nothing and keeps no state other than a per-device architecture check.
 *  - Arguments are validated on the host before anything is enqueued; on any error
 *    nothing is launched and the status says why. Launch failures return
 *    SAGESLA_ERR_HIP. Faults inside kernels surface at the caller's next synchronize.
 *  - All work is enqueued on `stream` (0 = the null stream); calls never synchronize.
 *    Inputs must stay alive until the stream has passed the call.
 *  - Calls on different streams with different workspaces may run concurrently.
 */
#ifndef SAGESLA_H
#define SAGESLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *sagesla_stream_t; /* a hipStream_t */

typedef enum {
    SAGESLA_OK = 0,
    SAGESLA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or ratio */
    SAGESLA_ERR_UNSUPPORTED = 2,      /* d != 128, block != 64, or not a gfx950 device */
    SAGESLA_ERR_WORKSPACE = 3,        /* workspace smaller than sagesla_workspace_size */
    SAGESLA_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed */
} sagesla_status;

/* Workspace regions (indices into the offsets array of sagesla_workspace_layout). */
enum {
    SAGESLA_WS_QBAR = 0,  /* fp64 [BH][Nb][d]   block means of Q                          */
    SAGESLA_WS_KBART,     /* fp64 [BH][d][Nb]   block means of K, channel-major            */
    SAGESLA_WS_KSUM,      /* fp64 [BH][Nb][d]   block column sums of K                     */
    SAGESLA_WS_VAMAXB,    /* fp32 [BH][Nb][d]   block column max |V|                       */
    SAGESLA_WS_KMEAN,     /* fp32 [BH][d]       per-channel mean of K over all N           */
    SAGESLA_WS_VAMAX,     /* fp32 [BH][d]       per-channel max |V| over all N             */
    SAGESLA_WS_Q8,        /* int8 [BH][Nb][8192] Q codes, MFMA operand order (see below)   */
    SAGESLA_WS_SQ,        /* fp32 [BH][Nb]      Q block scales                             */
    SAGESLA_WS_K8,        /* int8 [BH][Nb][8192] smoothed-K codes, MFMA operand order      */
    SAGESLA_WS_SK,        /* fp32 [BH][Nb]      K block scales                             */
    SAGESLA_WS_V8,        /* e4m3 [BH][Nb][8192] V codes, MFMA operand order               */
    SAGESLA_WS_IDX,       /* int32 [BH][Nb][ksel] kept key blocks: best first, then ascending */
    SAGESLA_WS_HS,        /* bf16 [BH][Nb][129][d] state S_j: rows c<128 = H_j^T, row 128 = z_j */
    SAGESLA_WS_HPART,     /* fp32 [BH][Nc][129][d] sums of 16 consecutive S_j (linear)      */
    SAGESLA_WS_HTOT,      /* fp32 [BH][129][d]  sum of all S_j                  (linear)   */
    SAGESLA_WS_ULIST,     /* int32 [BH][Ng][Nb] union of kept blocks of each query group   */
    SAGESLA_WS_UMASK,     /* u32 [BH][Ng][ceil(Nb/32)][256] per query block: bits over union positions */
    SAGESLA_WS_UCOUNT,    /* int32 [BH][Ng]     union sizes                     (linear)   */
    SAGESLA_WS_HC,        /* bf16 [BH][Nb][129][d] complement states total - kept (linear) */
    SAGESLA_WS_Y,         /* bf16 [BH][N][d]    O_l W_proj                      (linear)   */
    SAGESLA_WS_KEYS,      /* u64 [BH][Nb][Nb]   block scores as order-preserving keys (the
                             fp64 bits, negatives complemented, positives with the sign bit
                             set); only in the adaptive forward's workspace               */
    SAGESLA_WS_COUNT
};
/*
 * Code layouts (one 64-token block = 8192 bytes; lane l in 0..63, g = l/32, r = l%32):
 *  Q8/K8: byte ((t*4 + s)*64 + l)*16 + e holds row 32*t + r, channel 64*g + 16*s + e
 *         (t in 0..1, s in 0..3, e in 0..15); rows past N are 0.
 *  V8:    byte ((dt*2 + e/16)*64 + l)*16 + e%16 holds channel 32*dt + r of token
 *         32*(e/16) + 8*((e%16)/4) + 4*g + e%4 (dt in 0..3, e in 0..31); rows past N are 0.
 * H_j[a][c] = sum_t phi(k_t)[a] v_t[c], z_j[a] = sum_t phi(k_t)[a] over the tokens of block j.
 * Nc = ceil(Nb/16) partial sums; Ng = ceil(Nb/256) query-block groups.
 */

int sagesla_version(void);
const char *sagesla_status_string(sagesla_status s);

/* Tensor descriptors for sagesla_fwd_tensors: element type, rank, sizes and strides (in
 * elements). The library accepts only contiguous row-major tensors (a dimension of size 1
 * may carry any stride) of the element type each argument needs; anything else returns
 * SAGESLA_ERR_INVALID_ARGUMENT before any work is enqueued. */
typedef enum {
    SAGESLA_BF16 = 0,
    SAGESLA_F32 = 1,
    SAGESLA_I8 = 2,
    SAGESLA_FP8E4M3 = 3,
    SAGESLA_I32 = 4,
    SAGESLA_U8 = 5
} sagesla_dtype;

typedef struct {
    void *data;          /* device pointer, 16-byte aligned */
    sagesla_dtype dtype;
    int ndim;            /* 1..4 */
    int64_t shape[4];
    int64_t stride[4];
} sagesla_tensor;

/* Number of kept key blocks per query block: clamp(ceil(topk*Nb - 1e-9), 1, Nb). */
sagesla_status sagesla_ksel(int N, int block, double topk, int *ksel);

/* Bytes of workspace sagesla_fwd needs (linear = 0 when proj will be NULL). Host only. */
sagesla_status sagesla_workspace_size(int B, int H, int N, int d, int block, double topk,
                                      int linear, size_t *bytes);

/* Byte offsets of the SAGESLA_WS_* regions inside the workspace (unused regions get the
 * total size). Host only. */
sagesla_status sagesla_workspace_layout(int B, int H, int N, int d, int block, double topk,
                                        int linear, size_t offsets[SAGESLA_WS_COUNT]);

/*
 * Full forward: out = SageSLA(q, k, v) (+ linear branch through proj when proj != NULL
 * and ksel < Nb). workspace: device memory of at least sagesla_workspace_size bytes;
 * its contents on return are the SAGESLA_WS_* intermediates of this call.
 * Streams: the whole call is ordered on `stream`. Inside it, the key-block selection (and,
 * with the linear branch, the union of the kept lists) runs on a second stream the library
 * owns per device (default priority, created by the first call on that device outside a
 * graph capture, kept until the process ends), forked from `stream` after the head
 * statistics and joined back before the masked complement product. The
 * call may be captured into a HIP graph (a first call on a device that is itself being
 * captured runs on `stream` alone), and calls from several host threads are safe.
 * sagesla_fwd_prepared and sagesla_fwd_tensors do the same; sagesla_fwd_noalloc runs on
 * `stream` alone.
 */
sagesla_status sagesla_fwd(const void *q, const void *k, const void *v, const void *proj,
                           int B, int H, int N, int d, double topk, int block, void *out,
                           void *workspace, size_t workspace_bytes, sagesla_stream_t stream);

/* The same forward with tensor descriptors: q, k, v, out bf16 [B, H, N, d]; proj bf16
 * [d, d] or NULL (linear branch off); workspace u8 [bytes]. Each descriptor's type, rank,
 * shape and contiguity are checked first (SAGESLA_ERR_INVALID_ARGUMENT on a mismatch);
 * then the call is sagesla_fwd. */
sagesla_status sagesla_fwd_tensors(const sagesla_tensor *q, const sagesla_tensor *k,
                                   const sagesla_tensor *v, const sagesla_tensor *proj, double topk,
                                   int block, sagesla_tensor *out, const sagesla_tensor *workspace,
                                   sagesla_stream_t stream);

/* ---- forward without allocation ---------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sagesla_fwd with the workspace in a
 * fixed device array of SAGESLA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on, until the process ends. The caller still passes q, k, v, proj, out. Shapes
 * whose workspace (sagesla_workspace_size) exceeds the array return SAGESLA_ERR_WORKSPACE
 * before anything is enqueued. No step needs the array cleared (every region is written
 * before it is read). All calls on one GPU share its array, which keeps the last call's
 * intermediates: calls that overlap on one GPU (other streams, other threads) race and
 * must not be issued; calls on one stream are ordered and safe. */
#define SAGESLA_NOALLOC_SCRATCH_BYTES (256u << 20) /* 256 MiB */

sagesla_status sagesla_fwd_noalloc(const void *q, const void *k, const void *v, const void *proj,
                                   int B, int H, int N, int d, double topk, int block, void *out,
                                   sagesla_stream_t stream);

/* ---- content-adaptive kept-block count ------------------------------------------------
 * The pages fix a Top-K ratio (0.1-0.15 at inference: news.qq.com explainer, "From training
 * to deployment") and name sparsity that follows the input as open work, without a rule
 * (same page, "The limits of the technique", sixth challenge). Here the count follows the
 * scores: with s_ij the block scores and n_j the valid tokens of key block j, query block i
 * needs k_i = the fewest blocks, in selection order (score descending, lower index on
 * ties), whose mass n_j exp(s_ij - max_j s_ij) reaches tau of its row's total; a head keeps
 * k_head = clamp(ceil(sum_i k_i / Nb), kmin, kmax) blocks for every query block, where kmin
 * and kmax are sagesla_ksel of topk_min and topk_max. The masses are fp64; a row whose
 * prefix mass lies within rounding of tau times its total may resolve either way.
 * Requires 0 < topk_min <= topk_max <= 1, 0 < tau <= 1 and Nb <= 8192 (N <= 524288;
 * SAGESLA_ERR_UNSUPPORTED beyond).
 *
 * sagesla_adaptive_ksel: from the pooled means (QBAR, KBART as sagesla_pool writes them),
 * k_rows int32 [BH][Nb] and k_head int32 [BH] (device, written).
 *
 * sagesla_fwd_adaptive: the forward with each head at its own count: the same steps as
 * sagesla_fwd, with the counts computed after pooling. k_rows and k_head as above (device,
 * written). The workspace holds the SAGESLA_WS_* regions at the offsets of
 * sagesla_adaptive_workspace_layout; its IDX region is int32 [BH][Nb][kmax] with the head's
 * k_head entries first in each row (best first, then ascending) and -1 after them. With
 * proj, the linear branch runs for every head that leaves blocks out; a head at k_head = Nb
 * adds nothing. Each head's output equals sagesla_fwd's on that head alone with
 * topk = k_head / Nb. */
sagesla_status sagesla_adaptive_workspace_size(int B, int H, int N, int d, int block, double topk_min,
                                               double topk_max, int linear, size_t *bytes);

sagesla_status sagesla_adaptive_workspace_layout(int B, int H, int N, int d, int block,
                                                 double topk_min, double topk_max, int linear,
                                                 size_t offsets[SAGESLA_WS_COUNT]);

sagesla_status sagesla_adaptive_ksel(const void *qbar, const void *kbart, int B, int H, int N,
                                     int d, int block, double topk_min, double topk_max,
                                     double tau, void *k_rows, void *k_head,
                                     sagesla_stream_t stream);

sagesla_status sagesla_fwd_adaptive(const void *q, const void *k, const void *v, const void *proj,
                                    int B, int H, int N, int d, double topk_min, double topk_max,
                                    double tau, int block, void *out, void *k_rows, void *k_head,
                                    void *workspace, size_t workspace_bytes,
                                    sagesla_stream_t stream);

/* ---- producer-side fusion -------------------------------------------------------------
 * The pages fuse the rewritten LayerNorm/RMSNorm kernels with their neighbours (news.qq.com
 * explainer, "Fourth key"). sagesla_prepare takes the QKV projection output qkv bf16
 * [B, N, 3, H, d] (token-major, as a linear layer writes it) and, in one pass over it,
 * RMS-normalizes q and k over their model width D = H*d (per token:
 * r = fp32(1/sqrt(mean(x^2) + eps)) with the mean in fp64; out = bf16(bf16(x r) g) with the
 * learned weights gq, gk bf16 [D]), writes q, k, v bf16 [B, H, N, d], and fills the pool
 * regions of a forward workspace (QBAR, KBART, KSUM, VAMAXB, Q8, SQ) from them.
 * sagesla_fwd_prepared then runs the forward from the next stage on, on the same q, k, v,
 * sizes and topk; its result equals sagesla_fwd's on those q, k, v. The workspace is sized
 * by sagesla_workspace_size with the same topk and linear flag. */
sagesla_status sagesla_prepare(const void *qkv, const void *gq, const void *gk, double eps, int B,
                               int H, int N, int d, double topk, int block, int linear, void *q,
                               void *k, void *v, void *workspace, size_t workspace_bytes,
                               sagesla_stream_t stream);

sagesla_status sagesla_fwd_prepared(const void *q, const void *k, const void *v, const void *proj,
                                    int B, int H, int N, int d, double topk, int block, void *out,
                                    void *workspace, size_t workspace_bytes,
                                    sagesla_stream_t stream);

/* ---- stages ("friends"): the same conventions; buffers as in the workspace table ----
 * sagesla_fwd runs, in order: pool, head_stats, select, quant_kv (codes and, with the
 * linear branch, its states), linear_total and linear_complement (linear branch only),
 * sparse_attn. Three grouped calls cover the same launches by purpose:
 * sagesla_pool_select = pool + head_stats + select, sagesla_quantize = quant_kv without
 * states, sagesla_linear_states = quant_kv with states + linear_total. */

/* Pooling and selection together: the block means of Q and K, the per-head K channel
 * mean and V channel max, and the kept key blocks of every query block (SLA's quick
 * scoring of how strongly blocks are related and its Top-K choice: news.qq.com
 * explainer, "First key: attention"). Q's INT8 codes are made in the same pass, which
 * reads Q anyway. Outputs as in the workspace table (QBAR, KBART, KSUM, VAMAXB, Q8, SQ,
 * KMEAN, VAMAX, IDX). */
sagesla_status sagesla_pool_select(const void *q, const void *k, const void *v, int B, int H, int N,
                                   int d, int block, double topk, void *qbar, void *kbart,
                                   void *ksum, void *vamax_blk, void *q8, void *sq, void *kmean,
                                   void *vamax, void *idx, sagesla_stream_t stream);

/* SageAttention's quantization of K and V (news.qq.com explainer, "First key" and "Third
 * key": 8-bit data, outliers smoothed before quantizing, one scale per small block): K
 * minus its channel mean to INT8 per 64-token block, V to FP8 e4m3 per channel. */
sagesla_status sagesla_quantize(const void *k, const void *v, const void *kmean,
                                const void *vamax, int B, int H, int N, int d, int block, void *k8,
                                void *sk, void *v8, sagesla_stream_t stream);

/* The linear-attention states of every key block and their totals (the SLA branch that
 * carries the blocks not computed exactly: bonega.ai blog, SLA paragraph; tiemojia.cn
 * article, 2.2.1). They are formed in the same pass over K and V as the K/V codes, so this
 * call fills k8, sk, v8 too (as sagesla_quantize would), then hs, hpart and htot. */
sagesla_status sagesla_linear_states(const void *k, const void *v, const void *kmean,
                                     const void *vamax, int B, int H, int N, int d, int block,
                                     void *k8, void *sk, void *v8, void *hs, void *hpart,
                                     void *htot, sagesla_stream_t stream);

/* Block pooling of Q and K (fp64 sums of the bf16 inputs), K block sums, V block max,
 * and INT8 quantization of Q per block (pooling for SLA's quick block scoring and
 * SageAttention's per-block INT8: news.qq.com explainer, "First key" and "Third key"). */
sagesla_status sagesla_pool(const void *q, const void *k, const void *v, int B, int H, int N,
                            int d, int block, void *qbar, void *kbart, void *ksum,
                            void *vamax_blk, void *q8, void *sq, sagesla_stream_t stream);

/* Per-head reductions: K channel mean (from block sums) and V channel max: the smoothing
 * offset and the FP8 range of SageAttention's quantization (news.qq.com explainer, "Third
 * key"). */
sagesla_status sagesla_head_stats(const void *ksum, const void *vamax_blk, int B, int H, int N,
                                  int d, int block, void *kmean, void *vamax,
                                  sagesla_stream_t stream);

/* Block scores (fp64) and top-ksel selection per query block (SLA's Top-K of the block
 * scores: news.qq.com explainer, "First key"; kept list best first, then ascending). */
sagesla_status sagesla_select(const void *qbar, const void *kbart, int B, int H, int N, int d,
                              int block, double topk, void *idx, sagesla_stream_t stream);

/* K smoothing + INT8, V FP8 (news.qq.com explainer, "Third key"), and (when hs != NULL)
 * the linear-branch states S_j and their 16-block fp32 partial sums (bonega.ai blog, SLA
 * paragraph). */
sagesla_status sagesla_quant_kv(const void *k, const void *v, const void *kmean,
                                const void *vamax, int B, int H, int N, int d, int block,
                                void *k8, void *sk, void *v8, void *hs, void *hpart,
                                sagesla_stream_t stream);

/* Totals S_total = sum_j S_j (fp32) from the partial sums: the linear branch's state over
 * all key blocks, from which each query block's complement is taken (tiemojia.cn article,
 * 2.2.1). */
sagesla_status sagesla_linear_total(const void *hpart, int B, int H, int N, int d, int block,
                                    void *htot, sagesla_stream_t stream);

/* Linear branch (the blocks SLA does not compute exactly go to linear attention:
 * bonega.ai blog, SLA paragraph; tiemojia.cn article, 2.2.1): per group of 256 query
 * blocks the union of their kept sets (ulist,
 * umask, ucount), the complement states hc = S_total - sum_kept S_j (a 0/1-mask product
 * on the matrix cores), and y = O_l W with O_l = phi(q) H^c / (phi(q) . z^c). When more
 * than half the blocks are kept (2 ksel > Nb) the lists and masks describe the blocks
 * NOT kept and hc is their direct sum (no cancellation against the total). */
sagesla_status sagesla_linear_complement(const void *q, const void *idx, const void *hs,
                                         const void *htot, const void *proj, int B, int H,
                                         int N, int d, int block, double topk, void *ulist,
                                         void *umask, void *ucount, void *hc, void *y,
                                         sagesla_stream_t stream);

/* Sparse attention over the kept blocks, on the 8-bit matrix cores (news.qq.com explainer,
 * "First key": the exact part at 8-bit precision), and the epilogue out = O_s (+ y if
 * y != NULL; y is bf16 [B,H,N,d]). */
sagesla_status sagesla_sparse_attn(const void *q8, const void *sq, const void *k8,
                                   const void *sk, const void *v8, const void *vamax,
                                   const void *idx, const void *y, int B, int H, int N, int d,
                                   int block, double topk, void *out, sagesla_stream_t stream);

/* ------------------------------------------------------------------ SLA training path
 *
 * Trainable sparse-linear attention, unquantized: SLA is fine-tuned so that the model
 * learns which connections matter, and SageSLA replaces it only at inference (news.qq.com
 * explainer, "First key: attention" and "From training to deployment"). Per (batch, head),
 * with the same pooling, selection and linear branch as above:
 *   O_s = softmax(Q K_J^T / sqrt(d)) V_J over the tokens J of the kept key blocks, in bf16
 *   products with fp32 accumulation and an fp32 online softmax;  O = O_s + O_l W.
 * The backward takes the kept sets as fixed (the selection is piecewise constant) and
 * returns dQ, dK, dV (and dW) of L = sum(dO * O):
 *   sparse part: dS = P * (dP - D), dP = dO V^T, D = rowsum(dO * O_s);
 *     dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO;
 *   linear part (u = phi(q) H^c, s = phi(q) . z^c, O_l = u / s): dO_l = dO W^T,
 *     du = dO_l / s, ds = -(dO_l . O_l) / s, dphi(q) = du H^c^T + ds z^c, and through the
 *     channel softmax to dQ; the complement gradients dH^c_i = sum phi(q)^T du, dz^c_i =
 *     sum phi(q) ds pass to every key block the query block leaves out, then through
 *     H_j = phi(K_j)^T V_j and z_j to dK and dV; dW = sum O_l^T dO.
 * On the GPU the key blocks' gradients are formed as the total minus the query blocks that
 * keep them (or as the direct sum when 2 ksel > Nb), on the same masked product as the
 * forward's complement.
 *
 * The training workspace holds the forward regions (SAGESLA_WS_*, same meaning) and
 * these; sagesla_sla_bwd reads what sagesla_sla_fwd left there for the same inputs. */
typedef enum {
    SAGESLA_SLA_WS_LSE = SAGESLA_WS_COUNT, /* fp32 [BH][N] row log-sum-exp of the scores
                                              s/sqrt(d), base 2: log2 sum_j 2^(s_ij log2(e)/sqrt(d)) */
    SAGESLA_SLA_WS_OS,    /* fp32 [BH][N][d]     O_s                                      */
    SAGESLA_SLA_WS_KT,    /* bf16 [BH][Nb][8192] tiles (below): K head-dim-reduction (forward),
                             phi(q) token-reduction (backward, linear part)                */
    SAGESLA_SLA_WS_VT,    /* bf16 [BH][Nb][8192] V token-reduction (forward); V head-dim-
                             reduction, then O_l token-reduction (backward)                */
    SAGESLA_SLA_WS_QT,    /* bf16 [BH][Nb][8192] du token-reduction tiles (backward, linear) */
    SAGESLA_SLA_WS_DOT,   /* bf16 [BH][Nb][8192] dO token-reduction tiles (backward, dW)  */
    SAGESLA_SLA_WS_DSUM,  /* fp32 [BH][N]        D = rowsum(dO * O_s) (backward)          */
    SAGESLA_SLA_WS_MASK,  /* u32 [BH][Nb][ceil(Nb/32)] bit i of row j: query block i keeps j */
    SAGESLA_SLA_WS_H0,    /* bf16 [BH][Nb][8192] head-dim-reduction tiles (below) of K, then of Q */
    SAGESLA_SLA_WS_H1,    /* bf16 [BH][Nb][8192] head-dim-reduction tiles of dO (backward) */
    SAGESLA_SLA_WS_PHQ,   /* bf16 [BH][N][d] phi(q)                          (linear)   */
    SAGESLA_SLA_WS_DU,    /* bf16 [BH][N][d] du = dO_l / s                   (linear)   */
    SAGESLA_SLA_WS_OL,    /* bf16 [BH][N][d] O_l                             (linear)   */
    SAGESLA_SLA_WS_DS,    /* fp32 [BH][N]    ds = -(dO_l . O_l) / s          (linear)   */
    SAGESLA_SLA_WS_DWP,   /* fp32 [512][d][d] partial sums of dW             (linear)   */
    SAGESLA_SLA_WS_COUNT
} sagesla_sla_ws_region;
/* Token-reduction tiles of a [N][d] tensor X, per 64-token block: element
 * ((tt*4 + ct)*2 + t)*512 + l*8 + e holds X[32*tt + 16*t + 8*(e/4) + 4*g + e%4][32*ct + r]
 * (l in 0..63, r = l%32, g = l/32; tt, t in 0..1, ct in 0..3, e in 0..7; tokens past N are
 * 0). Head-dim-reduction tiles: element (tt*8 + s)*512 + p*8 + e, with
 * p = l ^ (4*(s%2) + 8*(l/32)), holds X[32*tt + r][16*s + 8*g + e] (s in 0..7). The forward
 * leaves K's head-dim-reduction tiles in SAGESLA_SLA_WS_KT and the backward rewrites the
 * tile regions. */

/* Bytes of the training workspace (linear = 0 when proj will be NULL). Host only. */
sagesla_status sagesla_sla_workspace_size(int B, int H, int N, int d, int block, double topk,
                                          int linear, size_t *bytes);

/* Byte offsets of the SAGESLA_WS_* and SAGESLA_SLA_WS_* regions. Host only. */
sagesla_status sagesla_sla_workspace_layout(int B, int H, int N, int d, int block, double topk,
                                            int linear, size_t offsets[SAGESLA_SLA_WS_COUNT]);

/* SLA forward (unquantized): out bf16 [B,H,N,d] = O_s (+ O_l W when proj != NULL and
 * ksel < Nb); leaves lse, O_s and the kept sets in the workspace for the backward. */
sagesla_status sagesla_sla_fwd(const void *q, const void *k, const void *v, const void *proj,
                               int B, int H, int N, int d, double topk, int block, void *out,
                               void *workspace, size_t workspace_bytes, sagesla_stream_t stream);

/* SLA backward: dq, dk, dv fp32 [B,H,N,d] (overwritten) from dout bf16 [B,H,N,d] and the
 * workspace of the sagesla_sla_fwd call on the same q, k, v, proj, sizes and topk (its
 * forward regions are overwritten). dproj: fp32 [d, d] (overwritten), required exactly
 * when proj != NULL; it is the sum over all batches and heads. */
sagesla_status sagesla_sla_bwd(const void *q, const void *k, const void *v, const void *proj,
                               const void *dout, int B, int H, int N, int d, double topk,
                               int block, void *dq, void *dk, void *dv, void *dproj,
                               void *workspace, size_t workspace_bytes, sagesla_stream_t stream);

/* ------------------------------------------------------------------ W8A8 linear layer
 *
 * y = x W^T (+ bias) with 8-bit weights and activations, the layer computed in the INT8
 * domain (TurboDiffusion explainer, news.qq.com, "Third key": both weights and activations
 * of the linear layers are quantized to 8-bit integers; the weights offline in 128 x 128
 * blocks that each share one scale factor, the activations dynamically at inference).
 * Activation grouping (not given there): one scale per token and 128-channel block.
 *
 * Quantization of a group G (weight block or activation token-block), in fp32:
 *   amax = max |x| over G;  s = amax / 127;  code = clamp(rne(x * (127 / amax)), -127, 127);
 *   amax = 0 gives s = 0 and zero codes.
 * Product:  y[m][n] = sum_kb sx[kb][m] sw[n/128][kb] (sum_{k in kb} x8[m][k] w8[n][k]) (+ bias[n]),
 *   the integer sums exact (int32), scaling and the sum over blocks in fp32, y rounded to bf16.
 *
 * Shapes: x bf16 [M][K], W bf16 [N][K] (row-major, as a torch Linear weight), bias bf16 [N]
 * or NULL, y bf16 [M][N]. K a multiple of 128 (<= 65536), N a multiple of 256 (<= 65536),
 * 1 <= M <= 2^24. Rows are padded to Mp = 256 * ceil(M / 256).
 *
 * Code layout of x8 and w8: tiles of 32 rows x 128 channels (4096 bytes) in MFMA operand
 * order, byte (s*64 + lane)*16 + e <-> row 32*tile + lane % 32 and channel
 * 128*kb + 64*(lane / 32) + 16*s + e, stored block-major: tile (kb, rt) at byte
 * (kb * RT + rt) * 4096 with RT = Mp / 32 (x8) or N / 32 (w8). Scales: sx fp32 [K/128][Mp]
 * (rows past M: 0), sw fp32 [N/128][K/128]. All buffers are the caller's (16-byte aligned
 * device memory, sizes from sagesla_w8a8_sizes); calls enqueue on the stream and return.
 * Errors: SAGESLA_ERR_INVALID_ARGUMENT for shapes or pointers out of these bounds,
 * SAGESLA_ERR_UNSUPPORTED off gfx950, SAGESLA_ERR_HIP for a failed launch. */
sagesla_status sagesla_w8a8_sizes(int M, int N, int K, size_t *x8_bytes, size_t *sx_bytes,
                                  size_t *w8_bytes, size_t *sw_bytes);

/* Weight codes w8 and block scales sw of W (done once per weight). */
sagesla_status sagesla_w8a8_quant_weight(const void *w, int N, int K, void *w8, void *sw,
                                         sagesla_stream_t stream);

/* Activation codes x8 and scales sx of x (each call). */
sagesla_status sagesla_w8a8_quant_act(const void *x, int M, int K, void *x8, void *sx,
                                      sagesla_stream_t stream);

/* The block-scaled INT8 product y = x W^T (+ bias) from the codes and scales. */
sagesla_status sagesla_w8a8_gemm(const void *x8, const void *sx, const void *w8, const void *sw,
                                 const void *bias, int M, int N, int K, void *y,
                                 sagesla_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SAGESLA_H */
