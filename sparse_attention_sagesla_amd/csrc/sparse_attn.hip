// Block-sparse quantized attention over the kept key blocks, with the fused epilogue
// out = O_s + y (y = O_l W_proj from the linear branch, optional).
//
// SLA computes only the top ~10 % of block pairs exactly and skips about 90 % of the
// work (TurboDiffusion explainer, news.qq.com, "First key: attention"); SageAttention
// runs that exact part on 8-bit data at the matrix cores' 8-bit peak (same section).
// Here QK^T is INT8 MFMA (v_mfma_i32_32x32x32_i8) and PV is FP8 e4m3 MFMA
// (v_mfma_f32_32x32x64_f8f6f4), with the online softmax in fp32 registers.
//
// Per query block i (64 rows) and kept key block j (ascending), for each row:
//   S = q8 . k8 (int32), a = (s_q[i] * s_k[j]) * c0 with c0 = fp32(log2(e)/sqrt(d)),
//   m' = max(m, max float(S)*a), alpha = 2^(m - m'),
//   P8 = e4m3(2^fma(float(S), a, log2(448) - m'))  (= e4m3(448 p), p = 2^(x - m')),
//   l = l*alpha + sum P8, acc = acc*alpha + P8 . V8   (l on the matrix cores too).
// Epilogue: O = acc * s_v / l (+ y), rounded to bf16: the average of the dequantized V
// rows weighted by the FP8 probabilities actually used. Kept blocks arrive best first.
//
// Work split: one workgroup of 2 waves per (bh, i); wave w owns query rows 32w..32w+31.
// The K/V code tiles go through an LDS ring filled by direct global-to-LDS loads.
// S^T = K8 Q8^T is computed so that each lane holds one query and 32 of the 64 keys:
// the row max and row sum stay in registers plus one exchange with lane l^32, and the
// probabilities are already in the B-operand layout of O^T = V8^T P8^T (the V8 code
// block is stored in the matching key order).
#include <math.h>

#include "common.h"

namespace sagesla {

constexpr float kLog2_448 = 8.807354922057604f;  // fp32(log2(448))

// c0 = fp32(log2(e) / sqrt(d)), rounded once from double
static float log2e_over_sqrt_d() { return (float)(1.4426950408889634 / sqrt((double)kD)); }

__device__ __forceinline__ int key_of_slot(int g, int t, int v) { return 32 * t + 8 * (v >> 2) + 4 * g + (v & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Per-wave state of the online softmax for 32 query rows (one per lane pair l, l^32).
struct RowState {
  float m, l;   // running max; sum of the FP8 weights (filled in at the end)
  v16f acc[4];  // O^T accumulators (4 tiles of 32 channels)
  v4f lacc;     // running row sums on the matrix cores: lanes 0..15, element 0 (query l), 1 (query l + 16)
};

// Online softmax of one 64-key tile (S^T accumulators) -> FP8 probabilities in the
// B-operand layout of O^T = V8^T P8^T. Keys masked out hold INT_MIN.
__device__ __forceinline__ v8i softmax_tile(RowState& st, v16i (&S)[2], float a) {
  int mx = INT_MIN;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int v = 0; v < 16; v++) mx = max(mx, S[tt][v]);
  {
    // the builtin returns unsigned lanes: compare as signed
    auto sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = max((int)sw[0], (int)sw[1]);
  }
  const float mn = fmaxf(st.m, (float)mx * a);
  // rescale only when some row's running max moved (alpha == 1 otherwise)
  if (__builtin_amdgcn_ballot_w64(mn > st.m) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
#pragma unroll
    for (int d = 0; d < 4; d++) st.acc[d] *= alpha;
    // lane j < 16 holds the sums of queries j (element 0) and j + 16 (element 1)
    const float alpha_hi = __shfl(alpha, (__lane_id() & 15) + 16);
    st.lacc[0] *= alpha;
    st.lacc[1] *= alpha_hi;
  }
  st.m = mn;
  // 448 p = 2^fma(S, a, log2(448) - m'). For the row maximum the fused product may land
  // a few ulps above log2(448); the FP8 conversion saturates (448, 464] to 448.
  const float bias = kLog2_448 - mn;
  v8i pb;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int sv = S[tt][4 * v4 + e];
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sv, a, bias));
      }
      // the first conversion keeps the high half of its third operand, which the second
      // overwrites: any register will do (p[0]'s bits; a constant would cost a move)
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
      pb[4 * tt + v4] = wd;
    }
  return pb;
}

// One workgroup of 2 waves per (bh, query block i); wave w owns query rows 32w..32w+31.
// The K and V code tiles of each kept block are DMA-loaded straight into an LDS ring of
// two stages (wave 0 the K tile, wave 1 the V tile, 8 x 1 KB each) one block ahead, and
// both waves read their MFMA operands from there. The loop is unrolled by two so every
// LDS access names its stage statically; all LDS reads of a step precede its DMA.
__global__ __launch_bounds__(128, 2) void sparse_attn_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ sq, const int8_t* __restrict__ k8,
    const float* __restrict__ sk, const uint8_t* __restrict__ v8, const float* __restrict__ vamax,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ y, int N, int Nb, int ksel, int tiles,
    int per_xcd, float c0, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_k0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_v0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_k1[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_v1[kBlkBytes];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= tiles) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int t = threadIdx.x, l = t & 63, g = l >> 5, r = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index (uniform)
  const size_t hb = (size_t)bh * Nb;
  const int32_t* crit = idx + (hb + i) * ksel;
  // wave 0 streams K code tiles, wave 1 V code tiles
  const uint8_t* src_base = w == 0 ? (const uint8_t*)k8 : v8;
  auto issue = [&](uint8_t* dk, uint8_t* dv, int j) {
    const uint8_t* src = src_base + (hb + j) * kBlkBytes + l * 16;
    // one LDS object per DMA instruction (wave-uniform branch)
    if (w == 0) {
#pragma unroll
      for (int n = 0; n < 8; n++)
        __builtin_amdgcn_global_load_lds((const void*)(src + n * 1024), (lds_ptr_t)(dk + n * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int n = 0; n < 8; n++)
        __builtin_amdgcn_global_load_lds((const void*)(src + n * 1024), (lds_ptr_t)(dv + n * 1024), 16, 0, 0);
    }
  };

  issue(s_k0, s_v0, crit[0]);
  // Q8 B-operand for query tile w: 4 steps of 16 bytes
  v4i qb[4];
  {
    const int8_t* qsrc = q8 + (hb + i) * kBlkBytes;
#pragma unroll
    for (int s = 0; s < 4; s++) qb[s] = *(const v4i*)(qsrc + ((w * 4 + s) * 64 + l) * 16);
  }
  const float sqi = sq[hb + i];
  const int nlast = block_len(Nb - 1, N);  // valid keys in the last block

  RowState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.lacc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < 4; d++) st.acc[d] = (v16f){};

  // Row sums on v_mfma_f32_16x16x128_f8f6f4 with P8 as its B operand: lane l's 32 bytes
  // are column l % 16 over keys 32 (l / 16) .., and lane l holds query l % 32. The A
  // operand (lane l: row l % 16 over keys 32 (l / 16) ..) is e4m3 1.0 in row 0 over the
  // key ranges of lanes 0..15 and 32..47 (queries 0..15) and in row 1 over those of lanes
  // 16..31 and 48..63 (queries 16..31), zero elsewhere: result rows 0 and 1 are the sums.
  const int lr = l & 15, lq = (l >> 4) & 1;
  const int one8 = ((lr == 0 && lq == 0) || (lr == 1 && lq == 1)) ? 0x38383838 : 0;
  const v8i lsel = {one8, one8, one8, one8, one8, one8, one8, one8};

  // one kept block: tile in (ck, cv), next block's DMA into (nk, nv)
  auto step = [&](int u, const uint8_t* ck, const uint8_t* cv, uint8_t* nk, uint8_t* nv) {
    const int j = crit[u];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tile of block u has landed (and Q)
    __syncthreads();                // and the other wave's
    // every LDS read of this block precedes the next block's DMA, so no read waits on it
    v4i ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int s = 0; s < 4; s++) ka[tt][s] = *(const v4i*)(ck + ((tt * 4 + s) * 64 + l) * 16);
    v8i va[4];
#pragma unroll
    for (int d = 0; d < 4; d++) {
      // V operand: two lane-contiguous 16-byte halves (conflict-free LDS reads)
      const v4i lo = *(const v4i*)(cv + ((2 * d) * 64 + l) * 16);
      const v4i hi = *(const v4i*)(cv + ((2 * d + 1) * 64 + l) * 16);
      va[d] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if (u + 1 < ksel) issue(nk, nv, crit[u + 1]);
    v16i S[2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
      S[tt] = (v16i){};
#pragma unroll
      for (int s = 0; s < 4; s++) S[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[tt][s], qb[s], S[tt], 0, 0, 0);
    }
    const float a = (sqi * sk[hb + j]) * c0;
    // The partial last block: keys at or past nlast take no part. Their scores are set
    // to INT_MIN before the softmax (out of the row maximum) and their FP8 weights to
    // zero after it. (One softmax body for both cases: a second copy of it doubles the
    // loop's register demand.)
    const bool partial = j == Nb - 1 && nlast < kBlk;
    if (partial) {
#pragma unroll
      for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int v = 0; v < 16; v++)
          if (key_of_slot(g, tt, v) >= nlast) S[tt][v] = INT_MIN;
    }
    v8i pb = softmax_tile(st, S, a);
    if (partial) {
#pragma unroll
      for (int tt = 0; tt < 2; tt++)
#pragma unroll
        for (int v4 = 0; v4 < 4; v4++) {
          uint32_t keep = 0u;
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (key_of_slot(g, tt, 4 * v4 + e) < nlast) keep |= 0xFFu << (8 * e);
          pb[4 * tt + v4] &= (int)keep;
        }
    }
#pragma unroll
    for (int d = 0; d < 4; d++)
      st.acc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[d], pb, st.acc[d], 0, 0, 0, 0, 0, 0);
    // this block's row sums of the FP8 weights, accumulated on the matrix cores
    st.lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pb, st.lacc, 0, 0, 0, 0, 0, 0);
  };

  int u = 0;
  for (; u + 1 < ksel; u += 2) {
    step(u, s_k0, s_v0, s_k1, s_v1);
    step(u + 1, s_k1, s_v1, s_k0, s_v0);
  }
  if (u < ksel) step(u, s_k0, s_v0, s_k1, s_v1);

  {
    // query r's sum: lane r & 15, element 0 for r < 16, element 1 otherwise
    const float l0 = __shfl(st.lacc[0], r & 15), l1 = __shfl(st.lacc[1], r & 15);
    st.l = r < 16 ? l0 : l1;
  }
  const float inv_l = 1.0f / st.l;
  const int qrow = i * kBlk + 32 * w + r;
  if (qrow < N) {
    uint16_t* orow = out + ((size_t)bh * N + qrow) * kD;
    const uint16_t* yrow = y ? y + ((size_t)bh * N + qrow) * kD : nullptr;
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int c = 32 * d + 8 * v4 + 4 * g;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = st.acc[d][4 * v4 + e] * ((vamax[(size_t)bh * kD + c + e] / 448.0f) * inv_l);
        if (yrow) {
          const uint2 yv = *(const uint2*)(yrow + c);
          o[0] += bf16_to_f32((uint16_t)(yv.x & 0xffff));
          o[1] += bf16_to_f32((uint16_t)(yv.x >> 16));
          o[2] += bf16_to_f32((uint16_t)(yv.y & 0xffff));
          o[3] += bf16_to_f32((uint16_t)(yv.y >> 16));
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *(uint2*)(orow + c) = pk;
      }
  }
}

hipError_t launch_sparse_attn(const void* q8, const void* sq, const void* k8, const void* sk,
                              const void* v8, const void* vamax, const void* idx, const void* y, int BH,
                              int N, int Nb, int ksel, void* out, hipStream_t st) {
  const int tiles = BH * Nb;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const int8_t*)q8,
                     (const float*)sq, (const int8_t*)k8, (const float*)sk, (const uint8_t*)v8,
                     (const float*)vamax, (const int32_t*)idx, (const uint16_t*)y, N, Nb, ksel, tiles,
                     per_xcd, log2e_over_sqrt_d(), (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace sagesla
