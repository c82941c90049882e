// Linear branch of SLA for one query block: complement state = total - kept blocks,
// O_l = phi(q) H^c / (phi(q) . z^c), then y = O_l W_proj.
//
// SLA sends what it does not compute exactly to a linear-attention variant
// (bonega.ai blog, SLA paragraph; tiemojia.cn article, 2.2.1); the per-key-block states
// and the "total minus kept" complement make the cost independent of how many blocks
// are not kept. phi is the softmax over the d channels of the raw bf16 row.
#include "common.h"

namespace sagesla {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kLs = 136;  // LDS row stride (bf16) for 128-wide tiles: 272 B, 16-B aligned

// One workgroup (256 threads, 4 waves) per (bh, query block).
__global__ __launch_bounds__(256) void linear_complement_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, const float* __restrict__ hs,
    const float* __restrict__ zs, const float* __restrict__ htot, const float* __restrict__ ztot,
    const uint16_t* __restrict__ proj, int N, int Nb, int ksel, int tiles, int per_xcd,
    float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kD * kLs];   // H^c transposed, then W transposed
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kBlk * kLs];  // phi(Q), then O_l
  __shared__ float s_zc[kD];
  __shared__ float s_den[kBlk];

  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= tiles) return;  // grid is rounded up to a multiple of 8
  const int bh = tile / Nb, i = tile % Nb;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 5, r = lane & 31;
  const int n = block_len(i, N);

  // ---- complement H^c = H_total - sum_{kept} H_j (thread owns 16 float4 chunks)
  v4f acc[16];
  const float* ht = htot + (size_t)bh * kD * kD;
#pragma unroll
  for (int m = 0; m < 16; m++) acc[m] = *(const v4f*)(ht + 4 * (t + 256 * m));
  v4f zacc = {0.f, 0.f, 0.f, 0.f};
  if (t < 32) zacc = *(const v4f*)(ztot + (size_t)bh * kD + 4 * t);
  const int32_t* crit = idx + ((size_t)bh * Nb + i) * ksel;
  for (int u = 0; u < ksel; u++) {
    const int j = crit[u];
    const float* hj = hs + ((size_t)bh * Nb + j) * kD * kD;
#pragma unroll
    for (int m = 0; m < 16; m++) acc[m] -= *(const v4f*)(hj + 4 * (t + 256 * m));
    if (t < 32) zacc -= *(const v4f*)(zs + ((size_t)bh * Nb + j) * kD + 4 * t);
  }
  // H^c[a][c] with a = (t + 256m)/32, c = 4*(t%32) + e -> LDS transposed [c][a] as bf16
#pragma unroll
  for (int m = 0; m < 16; m++) {
    const int a = (t >> 5) + 8 * m, c0 = 4 * (t & 31);
#pragma unroll
    for (int e = 0; e < 4; e++) s_b[(c0 + e) * kLs + a] = f32_to_bf16(acc[m][e]);
  }
  if (t < 32) {
#pragma unroll
    for (int e = 0; e < 4; e++) s_zc[4 * t + e] = zacc[e];
  }
  __syncthreads();

  // ---- phi(q) rows (16 lanes per row) -> LDS bf16, and den = phi(q) . z^c in fp32
  {
    const int rg = t >> 4, ch = t & 15;
#pragma unroll
    for (int mm = 0; mm < 4; mm++) {
      const int row = rg + 16 * mm;
      float x[8];
      uint4 qa = {0, 0, 0, 0};
      if (row < n) qa = *(const uint4*)(q + ((size_t)bh * N + (size_t)i * kBlk + row) * kD + ch * 8);
      const uint16_t* qh = (const uint16_t*)&qa;
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = bf16_to_f32(qh[e]);
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; e++) mx = fmaxf(mx, x[e]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) { x[e] = expf(x[e] - mx); s += x[e]; }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
      float den = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float ph = x[e] / s;
        den += ph * s_zc[ch * 8 + e];
        s_a[row * kLs + ch * 8 + e] = f32_to_bf16(ph);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) den += __shfl_xor(den, o);
      if (ch == 0) s_den[row] = den;
    }
  }
  __syncthreads();

  // ---- numerator phi(Q) H^c on MFMA: wave w -> rows 32*(w%2).., column tiles 2*(w/2), +1
  const int rt = w & 1, ct0 = 2 * (w >> 1);
  v16f num[2] = {(v16f){}, (v16f){}};
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const int kk = 16 * s + 8 * g;
    v8bf a = *(const v8bf*)(s_a + (32 * rt + r) * kLs + kk);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      v8bf b = *(const v8bf*)(s_b + (32 * (ct0 + c) + r) * kLs + kk);
      num[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, num[c], 0, 0, 0);
    }
  }
  __syncthreads();
  // O_l = num / den -> LDS (row-major bf16); W transposed -> s_b
#pragma unroll
  for (int c = 0; c < 2; c++)
#pragma unroll
    for (int qq = 0; qq < 16; qq++) {
      const int row = 32 * rt + 8 * (qq >> 2) + 4 * g + (qq & 3);
      const int col = 32 * (ct0 + c) + r;
      const float den = s_den[row];
      s_a[row * kLs + col] = f32_to_bf16(den != 0.f ? num[c][qq] / den : 0.f);
    }
  for (int e = t; e < kD * kD / 8; e += 256) {
    const int a = e / 16, c0 = (e % 16) * 8;  // W[a][c0..c0+7]
    uint4 wv = *(const uint4*)(proj + a * kD + c0);
    const uint16_t* wh = (const uint16_t*)&wv;
#pragma unroll
    for (int x = 0; x < 8; x++) s_b[(c0 + x) * kLs + a] = wh[x];
  }
  __syncthreads();
  // ---- y = O_l W on MFMA
  v16f yo[2] = {(v16f){}, (v16f){}};
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const int kk = 16 * s + 8 * g;
    v8bf a = *(const v8bf*)(s_a + (32 * rt + r) * kLs + kk);
#pragma unroll
    for (int c = 0; c < 2; c++) {
      v8bf b = *(const v8bf*)(s_b + (32 * (ct0 + c) + r) * kLs + kk);
      yo[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, yo[c], 0, 0, 0);
    }
  }
  float* ydst = y + ((size_t)bh * N + (size_t)i * kBlk) * kD;
#pragma unroll
  for (int c = 0; c < 2; c++)
#pragma unroll
    for (int qq = 0; qq < 16; qq++) {
      const int row = 32 * rt + 8 * (qq >> 2) + 4 * g + (qq & 3);
      if (row < n) ydst[(size_t)row * kD + 32 * (ct0 + c) + r] = yo[c][qq];
    }
}

hipError_t launch_linear_complement(const void* q, const void* idx, const void* hs, const void* zs,
                                    const void* htot, const void* ztot, const void* proj, int BH,
                                    int N, int Nb, int ksel, void* y, hipStream_t st) {
  const int tiles = BH * Nb;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(linear_complement_kernel, dim3(per_xcd * 8), dim3(256), 0, st,
                     (const uint16_t*)q, (const int32_t*)idx, (const float*)hs, (const float*)zs,
                     (const float*)htot, (const float*)ztot, (const uint16_t*)proj, N, Nb, ksel,
                     tiles, per_xcd, (float*)y);
  return hipGetLastError();
}

}  // namespace sagesla
