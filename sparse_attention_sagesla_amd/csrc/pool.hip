// Block pooling of Q/K, V block max, and per-block INT8 quantization of Q.
//
// SLA first makes a quick estimate of how strongly positions relate before deciding
// what to compute exactly (TurboDiffusion explainer, news.qq.com, "First key:
// attention"); here that estimate is made on 64-token block means. SageAttention's
// 8-bit quantization with one scale per small block (same page, "First key" and
// "Third key") is applied to Q in the same pass, since Q needs no smoothing.
#include "common.h"

namespace sagesla {

// One workgroup (256 threads) per (bh, block). Thread t covers rows t/16 + 16m
// (m = 0..3) and channels 8*(t%16) .. +7.
__global__ __launch_bounds__(256) void pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int N, int Nb, double* __restrict__ qbar, double* __restrict__ kbart, double* __restrict__ ksum,
    float* __restrict__ vamax_blk, int8_t* __restrict__ q8, float* __restrict__ sq) {
  __shared__ double s_q[16][kD];
  __shared__ double s_k[16][kD];
  __shared__ float s_v[16][kD];
  __shared__ float s_amax[4];

  const int tile = blockIdx.x;
  const int bh = tile / Nb, i = tile % Nb;
  const int n = block_len(i, N);
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15;
  const size_t base = ((size_t)bh * N + (size_t)i * kBlk) * kD;

  double sumq[8], sumk[8];
  float mv[8];
  float qv[4][8];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) { sumq[e] = 0.0; sumk[e] = 0.0; mv[e] = 0.f; }
#pragma unroll
  for (int m = 0; m < 4; m++) {
    int row = rg + 16 * m;
    uint4 qa = {0, 0, 0, 0}, ka = {0, 0, 0, 0}, va = {0, 0, 0, 0};
    if (row < n) {
      size_t off = base + (size_t)row * kD + ch * 8;
      qa = *(const uint4*)(q + off);
      ka = *(const uint4*)(k + off);
      va = *(const uint4*)(v + off);
    }
    const uint16_t* qh = (const uint16_t*)&qa;
    const uint16_t* kh = (const uint16_t*)&ka;
    const uint16_t* vh = (const uint16_t*)&va;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float xq = bf16_to_f32(qh[e]);
      qv[m][e] = xq;
      sumq[e] += (double)xq;
      sumk[e] += (double)bf16_to_f32(kh[e]);
      mv[e] = fmaxf(mv[e], fabsf(bf16_to_f32(vh[e])));
      amax = fmaxf(amax, fabsf(xq));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; e++) {
    s_q[rg][ch * 8 + e] = sumq[e];
    s_k[rg][ch * 8 + e] = sumk[e];
    s_v[rg][ch * 8 + e] = mv[e];
  }
  // block-wide max |q|
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((t & 63) == 0) s_amax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));

  if (t < kD) {
    double a = 0.0, b = 0.0;
    float mx = 0.f;
    for (int r = 0; r < 16; r++) {  // fixed order: exact for bf16 inputs of moderate range
      a += s_q[r][t];
      b += s_k[r][t];
      mx = fmaxf(mx, s_v[r][t]);
    }
    size_t o = ((size_t)bh * Nb + i) * kD + t;
    qbar[o] = a / n;
    ksum[o] = b;
    kbart[((size_t)bh * kD + t) * Nb + i] = b / n;
    vamax_blk[o] = mx;
  }

  // INT8 codes of Q with one scale per block
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  if (t == 0) sq[(size_t)bh * Nb + i] = amax > 0.f ? amax / 127.0f : 0.f;
  int8_t* dst = q8 + ((size_t)bh * Nb + i) * kBlkBytes;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    int row = rg + 16 * m;
    uint32_t lo = 0, hi = 0;
    if (row < n) {
#pragma unroll
      for (int e = 0; e < 4; e++) lo |= (uint32_t)(uint8_t)q_int8(qv[m][e], inv) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; e++) hi |= (uint32_t)(uint8_t)q_int8(qv[m][e + 4], inv) << (8 * e);
    }
    *(uint2*)(dst + qk_code_offset(row, ch * 8)) = make_uint2(lo, hi);
  }
}

// Per head: K channel mean over all N tokens (fp64 sum of block sums, rounded to fp32)
// and V channel max |v|. 16 workgroups per head, each 8 channels x 32 block-strided
// parts, reduced in a fixed order (the block sums are exact, so is their sum).
__global__ __launch_bounds__(256) void head_stats_kernel(const double* __restrict__ ksum,
                                                         const float* __restrict__ vamax_blk, int N,
                                                         int Nb, float* __restrict__ kmean,
                                                         float* __restrict__ vamax) {
  __shared__ double s_s[32][8];
  __shared__ float s_m[32][8];
  const int bh = blockIdx.x >> 4, c = (blockIdx.x & 15) * 8 + (threadIdx.x & 7), part = threadIdx.x >> 3;
  double s = 0.0;
  float mx = 0.f;
  for (int i = part; i < Nb; i += 32) {
    size_t o = ((size_t)bh * Nb + i) * kD + c;
    s += ksum[o];
    mx = fmaxf(mx, vamax_blk[o]);
  }
  s_s[part][threadIdx.x & 7] = s;
  s_m[part][threadIdx.x & 7] = mx;
  __syncthreads();
  if (threadIdx.x < 8) {
    double tot = 0.0;
    float m = 0.f;
    for (int p = 0; p < 32; p++) {
      tot += s_s[p][threadIdx.x];
      m = fmaxf(m, s_m[p][threadIdx.x]);
    }
    kmean[(size_t)bh * kD + c] = (float)(tot / N);
    vamax[(size_t)bh * kD + c] = m;
  }
}

hipError_t launch_pool(const void* q, const void* k, const void* v, int BH, int N, int Nb, void* qbar,
                       void* kbart, void* ksum, void* vamax_blk, void* q8, void* sq, hipStream_t st) {
  hipLaunchKernelGGL(pool_kernel, dim3(BH * Nb), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, N, Nb, (double*)qbar, (double*)kbart,
                     (double*)ksum, (float*)vamax_blk, (int8_t*)q8, (float*)sq);
  return hipGetLastError();
}

hipError_t launch_head_stats(const void* ksum, const void* vamax_blk, int BH, int N, int Nb,
                             void* kmean, void* vamax, hipStream_t st) {
  hipLaunchKernelGGL(head_stats_kernel, dim3(BH * 16), dim3(256), 0, st, (const double*)ksum,
                     (const float*)vamax_blk, N, Nb, (float*)kmean, (float*)vamax);
  return hipGetLastError();
}

}  // namespace sagesla
