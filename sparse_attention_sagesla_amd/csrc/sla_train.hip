// Trainable sparse-linear attention (SLA, unquantized): the forward with the row
// log-sum-exp saved, and the backward of its sparse part.
//
// SLA is fine-tuned so that the model learns which connections matter; SageSLA only
// replaces it at inference (news.qq.com explainer, "First key: attention" and "From
// training to deployment"). Training needs the unquantized forward and its gradients:
//   O_s = softmax(Q K_J^T / sqrt(d)) V_J over the tokens J of the kept key blocks,
//   lse = the row log-sum-exp (saved, here in the base-2 domain of the scaled scores),
//   dS = P * (dP - D) with dP = dO V^T and D = rowsum(dO * O_s),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO.
// The selection is piecewise constant in the inputs; the backward takes the kept lists
// as fixed.
//
// All products run on v_mfma_f32_32x32x16_bf16 with bf16 operands and fp32 accumulators.
// Layout conventions (lane l, r = l % 32, g = l / 32):
//  * operands with the head dimension as the reduction index are read straight from the
//    row-major [N][128] tensors: lane (row r, g) takes channels 16s + 8g .. +7 for step s;
//  * operands with tokens as the reduction index use the "token-reduction tiles" written
//    by sla_relayout_kernel: per 64-token block, chunk ((tt*4 + ct)*2 + t)*64 + l holds the
//    8 bf16 of channel 32ct + r at tokens 32tt + 16t + 8(e/4) + 4g + e%4, e = 0..7;
//  * a 32x32 accumulator D[row][col] holds col = r and rows 8(v/4) + 4g + v%4, v = 0..15,
//    so its registers v = 8t .. 8t+7 are exactly the B operand of a token-reduction step t
//    (the same token assignment as the tiles above): probabilities and score gradients
//    feed the next product without moving between lanes.
#include "common.h"

namespace sagesla {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kTrTile = kBlk * kD;        // bf16 elements of one block's token-reduction tiles
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v8bf ld8(const uint16_t* p) { return __builtin_bit_cast(v8bf, *(const v4i*)p); }

__device__ __forceinline__ v8bf pack8(const float* x) {
  v4i r;
  r.x = (int)pack_bf16x2(x[0], x[1]);
  r.y = (int)pack_bf16x2(x[2], x[3]);
  r.z = (int)pack_bf16x2(x[4], x[5]);
  r.w = (int)pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(v8bf, r);
}

__device__ __forceinline__ v16f mfma(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ token-reduction tiles
// X [BH][N][128] bf16 -> Xt [BH][Nb][kTrTile] bf16 (tokens past N are zero). One workgroup
// per block: the block is staged in LDS, then each thread gathers 8 values per chunk.
__global__ __launch_bounds__(256) void sla_relayout_kernel(const uint16_t* __restrict__ x, int N, int Nb,
                                                           uint16_t* __restrict__ xt) {
  __shared__ uint16_t s[kBlk][kD + 8];
  const int bh = blockIdx.x / Nb, blk = blockIdx.x % Nb, t = threadIdx.x;
  const int n = block_len(blk, N);
  const uint16_t* src = x + ((size_t)bh * N + (size_t)blk * kBlk) * kD;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int c = t + 256 * k, row = c >> 4, col = (c & 15) * 8;
    v4i val = (v4i){0, 0, 0, 0};
    if (row < n) val = *(const v4i*)(src + (size_t)row * kD + col);
    *(v4i*)&s[row][col] = val;
  }
  __syncthreads();
  uint16_t* dst = xt + ((size_t)bh * Nb + blk) * kTrTile;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int c = t + 256 * k;  // chunk ((tt*4 + ct)*2 + st)*64 + l
    const int l = c & 63, st = (c >> 6) & 1, ct = (c >> 7) & 3, tt = c >> 9;
    const int r = l & 31, g = l >> 5;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int tok0 = 32 * tt + 16 * st + 8 * (e >> 2) + 4 * g + (e & 3);
      w[e >> 1] = (uint32_t)s[tok0][32 * ct + r] | ((uint32_t)s[tok0 + 1][32 * ct + r] << 16);
    }
    *(v4i*)(dst + (size_t)c * 8) = (v4i){(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  }
}

// ------------------------------------------------------------------ transposed kept sets
// mask[bh][j][i / 32] bit i % 32 set when query block i keeps key block j.
__global__ __launch_bounds__(256) void sla_fill_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

__global__ __launch_bounds__(256) void sla_kept_mask_kernel(const int* __restrict__ idx, int BH, int Nb, int ksel,
                                                            int nw, uint32_t* __restrict__ mask) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)BH * Nb * ksel) return;
  const size_t row = e / ksel;  // bh * Nb + i
  const int bh = (int)(row / Nb), i = (int)(row % Nb);
  const int j = idx[e];
  atomicOr(mask + ((size_t)bh * Nb + j) * nw + (i >> 5), 1u << (i & 31));
}

// ------------------------------------------------------------------ forward
// One workgroup (2 waves) per (head, query block); wave w owns query rows 32w .. +31, one
// per lane column. Per kept key block: S^T = K Q^T (two 32-key tiles), online softmax in
// the base-2 domain, O^T += V^T P^T. Epilogue: O_s (bf16), lse, and out = O_s + y.
__global__ __launch_bounds__(128) void sla_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ vt, const int* __restrict__ idx,
                                                      const uint16_t* __restrict__ y, int BH, int N, int Nb, int ksel,
                                                      int per_xcd, uint16_t* __restrict__ out,
                                                      uint16_t* __restrict__ os, float* __restrict__ lse) {
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int qi = kBlk * i + 32 * w + r;
  const bool qvalid = qi < N;
  const uint16_t* Qh = q + (size_t)bh * N * kD;
  const uint16_t* Kh = k + (size_t)bh * N * kD;
  const float c = kLog2e * 0.08838834764831845f;  // log2(e) / sqrt(128)

  v8bf qop[8];
#pragma unroll
  for (int s = 0; s < 8; s++)
    qop[s] = qvalid ? ld8(Qh + (size_t)qi * kD + 16 * s + 8 * g) : (v8bf){};

  float m = -INFINITY, lsum = 0.f;
  v16f o[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) o[ct] = (v16f){};

  const int* irow = idx + ((size_t)bh * Nb + i) * ksel;
  for (int kk = 0; kk < ksel; kk++) {
    const int j = irow[kk];
    const int nj = block_len(j, N);
    float sc[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      const int kr = 32 * kt + r;
      const uint16_t* krow = Kh + ((size_t)j * kBlk + kr) * kD + 8 * g;
      v16f acc = (v16f){};
#pragma unroll
      for (int s = 0; s < 8; s++) acc = mfma(kr < nj ? ld8(krow + 16 * s) : (v8bf){}, qop[s], acc);
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int key = 32 * kt + 8 * (v >> 2) + 4 * g + (v & 3);
        sc[kt][v] = key < nj ? acc[v] * c : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int v = 0; v < 16; v++) mx = fmaxf(mx, sc[kt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        sc[kt][v] = exp2f(sc[kt][v] - mn);
        rs += sc[kt][v];
      }
    rs += __shfl_xor(rs, 32);
    lsum = lsum * alpha + rs;
    m = mn;
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v = 0; v < 16; v++) o[ct][v] *= alpha;
    const uint16_t* vb = vt + ((size_t)bh * Nb + j) * kTrTile + l * 8;
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const v8bf pb = pack8(&sc[kt][8 * t]);
#pragma unroll
        for (int ct = 0; ct < 4; ct++) o[ct] = mfma(ld8(vb + ((kt * 4 + ct) * 2 + t) * 512), pb, o[ct]);
      }
  }

  if (!qvalid) return;
  const float inv = 1.f / lsum;
  if (g == 0) lse[(size_t)bh * N + qi] = m + log2f(lsum);
  const size_t rowoff = ((size_t)bh * N + qi) * kD;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * ct + 8 * v4 + 4 * g;
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; e++) a[e] = o[ct][4 * v4 + e] * inv;
      uint2 pk;
      pk.x = pack_bf16x2(a[0], a[1]);
      pk.y = pack_bf16x2(a[2], a[3]);
      *(uint2*)(os + rowoff + ch) = pk;
      if (y) {
        const uint2 yy = *(const uint2*)(y + rowoff + ch);
        a[0] += __uint_as_float(yy.x << 16);
        a[1] += __uint_as_float(yy.x & 0xFFFF0000u);
        a[2] += __uint_as_float(yy.y << 16);
        a[3] += __uint_as_float(yy.y & 0xFFFF0000u);
        pk.x = pack_bf16x2(a[0], a[1]);
        pk.y = pack_bf16x2(a[2], a[3]);
      }
      *(uint2*)(out + rowoff + ch) = pk;
    }
}

// ------------------------------------------------------------------ backward: dQ (and D)
// One workgroup (2 waves) per (head, query block), lanes = query rows as in the forward.
// D = rowsum(dO * O_s) first (stored for the dK/dV pass), then per kept key block and
// 32-key tile: S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T.
__global__ __launch_bounds__(128) void sla_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const uint16_t* __restrict__ kt_,
                                                         const uint16_t* __restrict__ dout, const uint16_t* __restrict__ os,
                                                         const float* __restrict__ lse, const int* __restrict__ idx,
                                                         int BH, int N, int Nb, int ksel, int per_xcd,
                                                         float* __restrict__ dsum, float* __restrict__ dq) {
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int qi = kBlk * i + 32 * w + r;
  const bool qvalid = qi < N;
  const size_t hoff = (size_t)bh * N * kD;
  const float c = kLog2e * 0.08838834764831845f;

  v8bf qop[8], dop[8];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const size_t e = hoff + (size_t)qi * kD + 16 * s + 8 * g;
    qop[s] = qvalid ? ld8(q + e) : (v8bf){};
    dop[s] = qvalid ? ld8(dout + e) : (v8bf){};
    if (qvalid) {
      const v8bf ov = ld8(os + e);
#pragma unroll
      for (int x = 0; x < 8; x++) dpart += (float)dop[s][x] * (float)ov[x];
    }
  }
  const float D = dpart + __shfl_xor(dpart, 32);
  const float L = qvalid ? lse[(size_t)bh * N + qi] : 0.f;
  if (qvalid && g == 0) dsum[(size_t)bh * N + qi] = D;

  v16f acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) acc[ct] = (v16f){};

  const int* irow = idx + ((size_t)bh * Nb + i) * ksel;
  for (int kk = 0; kk < ksel; kk++) {
    const int j = irow[kk];
    const int nj = block_len(j, N);
    const uint16_t* kb = kt_ + ((size_t)bh * Nb + j) * kTrTile + l * 8;
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
      const int kr = 32 * kt + r;
      const size_t roff = hoff + ((size_t)j * kBlk + kr) * kD + 8 * g;
      v16f s_ = (v16f){}, dp = (v16f){};
#pragma unroll
      for (int s = 0; s < 8; s++) {
        const bool kv = kr < nj;
        s_ = mfma(kv ? ld8(k + roff + 16 * s) : (v8bf){}, qop[s], s_);
        dp = mfma(kv ? ld8(v + roff + 16 * s) : (v8bf){}, dop[s], dp);
      }
      float ds[16];
#pragma unroll
      for (int x = 0; x < 16; x++) {
        const int key = 32 * kt + 8 * (x >> 2) + 4 * g + (x & 3);
        const float p = (key < nj && qvalid) ? exp2f(s_[x] * c - L) : 0.f;
        ds[x] = p * (dp[x] - D);
      }
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const v8bf b = pack8(&ds[8 * t]);
#pragma unroll
        for (int ct = 0; ct < 4; ct++) acc[ct] = mfma(ld8(kb + ((kt * 4 + ct) * 2 + t) * 512), b, acc[ct]);
      }
    }
  }

  if (!qvalid) return;
  const float sc = 0.08838834764831845f;  // 1 / sqrt(128)
  float* drow = dq + hoff + (size_t)qi * kD;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * ct + 8 * v4 + 4 * g;
      *(float4*)(drow + ch) = make_float4(acc[ct][4 * v4] * sc, acc[ct][4 * v4 + 1] * sc, acc[ct][4 * v4 + 2] * sc,
                                          acc[ct][4 * v4 + 3] * sc);
    }
}

// ------------------------------------------------------------------ backward: dK, dV
// One workgroup (2 waves) per (head, key block j); wave w owns keys 32w .. +31, one per
// lane column. The query blocks that keep j come from the transposed mask, ascending. Per
// 32-query tile: S = Q K^T, dP = dO V^T (lanes = keys, registers = queries), P and dS from
// the saved lse and D, then dV^T += dO^T P and dK^T += Q^T dS on the token-reduction tiles
// of dO and Q. The wave's K and V operands stay in registers.
__global__ __launch_bounds__(128) void sla_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, const uint16_t* __restrict__ qt_,
                                                           const uint16_t* __restrict__ dout,
                                                           const uint16_t* __restrict__ dot_, const float* __restrict__ lse,
                                                           const float* __restrict__ dsum, const uint32_t* __restrict__ mask,
                                                           int BH, int N, int Nb, int nw, int per_xcd,
                                                           float* __restrict__ dk, float* __restrict__ dv) {
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, j = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int kj = kBlk * j + 32 * w + r;
  const bool kvalid = kj < N;
  const size_t hoff = (size_t)bh * N * kD;
  const float c = kLog2e * 0.08838834764831845f;

  v8bf kop[8], vop[8];
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const size_t e = hoff + (size_t)kj * kD + 16 * s + 8 * g;
    kop[s] = kvalid ? ld8(k + e) : (v8bf){};
    vop[s] = kvalid ? ld8(v + e) : (v8bf){};
  }
  v16f dka[4], dva[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) dka[ct] = dva[ct] = (v16f){};

  const uint32_t* mrow = mask + ((size_t)bh * Nb + j) * nw;
  for (int wi = 0; wi < nw; wi++) {
    uint32_t bits = mrow[wi];
    while (bits) {
      const int i = 32 * wi + __builtin_ctz(bits);
      bits &= bits - 1;
      const int ni = block_len(i, N);
      const uint16_t* qb = qt_ + ((size_t)bh * Nb + i) * kTrTile + l * 8;
      const uint16_t* db = dot_ + ((size_t)bh * Nb + i) * kTrTile + l * 8;
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        const int qr = 32 * qt + r;
        const size_t roff = hoff + ((size_t)i * kBlk + qr) * kD + 8 * g;
        v16f s_ = (v16f){}, dp = (v16f){};
#pragma unroll
        for (int s = 0; s < 8; s++) {
          const bool qv = qr < ni;
          s_ = mfma(qv ? ld8(q + roff + 16 * s) : (v8bf){}, kop[s], s_);
          dp = mfma(qv ? ld8(dout + roff + 16 * s) : (v8bf){}, vop[s], dp);
        }
        // registers x hold query rows 32qt + 8(x/4) + 4g + x%4: four runs of four
        const float* lrow = lse + (size_t)bh * N + (size_t)i * kBlk + 32 * qt + 4 * g;
        const float* drow = dsum + (size_t)bh * N + (size_t)i * kBlk + 32 * qt + 4 * g;
        float p[16], ds[16];
#pragma unroll
        for (int x4 = 0; x4 < 4; x4++) {
          const int q0 = 32 * qt + 8 * x4 + 4 * g;  // within the block
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int x = 4 * x4 + e;
            const bool ok = q0 + e < ni;
            const float Lq = ok ? lrow[8 * x4 + e] : 0.f;
            const float Dq = ok ? drow[8 * x4 + e] : 0.f;
            p[x] = ok ? exp2f(s_[x] * c - Lq) : 0.f;
            ds[x] = p[x] * (dp[x] - Dq);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; t++) {
          const v8bf pb = pack8(&p[8 * t]), sb = pack8(&ds[8 * t]);
#pragma unroll
          for (int ct = 0; ct < 4; ct++) {
            const int off = ((qt * 4 + ct) * 2 + t) * 512;
            dva[ct] = mfma(ld8(db + off), pb, dva[ct]);
            dka[ct] = mfma(ld8(qb + off), sb, dka[ct]);
          }
        }
      }
    }
  }

  if (!kvalid) return;
  const float sc = 0.08838834764831845f;
  float* krow = dk + hoff + (size_t)kj * kD;
  float* vrow = dv + hoff + (size_t)kj * kD;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * ct + 8 * v4 + 4 * g;
      *(float4*)(krow + ch) = make_float4(dka[ct][4 * v4] * sc, dka[ct][4 * v4 + 1] * sc, dka[ct][4 * v4 + 2] * sc,
                                          dka[ct][4 * v4 + 3] * sc);
      *(float4*)(vrow + ch) = make_float4(dva[ct][4 * v4], dva[ct][4 * v4 + 1], dva[ct][4 * v4 + 2], dva[ct][4 * v4 + 3]);
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_sla_relayout(const void* x, int BH, int N, int Nb, void* xt, hipStream_t st) {
  hipLaunchKernelGGL(sla_relayout_kernel, dim3(BH * Nb), dim3(256), 0, st, (const uint16_t*)x, N, Nb, (uint16_t*)xt);
  return hipGetLastError();
}

hipError_t launch_sla_kept_mask(const void* idx, int BH, int Nb, int ksel, void* mask, hipStream_t st) {
  const int nw = (Nb + 31) / 32;
  const size_t words = (size_t)BH * Nb * nw;
  const int fill_blocks = (int)((words + 255) / 256 < 65536 ? (words + 255) / 256 : 65536);
  hipLaunchKernelGGL(sla_fill_kernel, dim3(fill_blocks), dim3(256), 0, st, (uint32_t*)mask, words);
  const size_t pairs = (size_t)BH * Nb * ksel;
  hipLaunchKernelGGL(sla_kept_mask_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, st, (const int*)idx,
                     BH, Nb, ksel, nw, (uint32_t*)mask);
  return hipGetLastError();
}

hipError_t launch_sla_fwd(const void* q, const void* k, const void* vt, const void* idx, const void* y, int BH, int N,
                          int Nb, int ksel, void* out, void* os, void* lse, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sla_fwd_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)vt, (const int*)idx, (const uint16_t*)y, BH, N, Nb, ksel, per_xcd,
                     (uint16_t*)out, (uint16_t*)os, (float*)lse);
  return hipGetLastError();
}

hipError_t launch_sla_bwd_dq(const void* q, const void* k, const void* v, const void* kt, const void* dout,
                             const void* os, const void* lse, const void* idx, int BH, int N, int Nb, int ksel,
                             void* dsum, void* dq, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sla_bwd_dq_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)kt, (const uint16_t*)dout, (const uint16_t*)os,
                     (const float*)lse, (const int*)idx, BH, N, Nb, ksel, per_xcd, (float*)dsum, (float*)dq);
  return hipGetLastError();
}

hipError_t launch_sla_bwd_dkdv(const void* q, const void* k, const void* v, const void* qt, const void* dout,
                               const void* dot, const void* lse, const void* dsum, const void* mask, int BH, int N,
                               int Nb, void* dk, void* dv, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8, nw = (Nb + 31) / 32;
  hipLaunchKernelGGL(sla_bwd_dkdv_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)qt, (const uint16_t*)dout,
                     (const uint16_t*)dot, (const float*)lse, (const float*)dsum, (const uint32_t*)mask, BH, N, Nb, nw,
                     per_xcd, (float*)dk, (float*)dv);
  return hipGetLastError();
}

}  // namespace sagesla
