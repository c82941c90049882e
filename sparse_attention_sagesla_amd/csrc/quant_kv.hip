// K smoothing + INT8, V to FP8 e4m3, and the linear-branch states per key block.
//
// SageAttention smooths outliers into range before quantizing and undoes the transform
// afterwards (TurboDiffusion explainer, news.qq.com, "Third key"); for K this is the
// subtraction of the per-channel mean over all tokens, which leaves softmax(q.k)
// unchanged. Q and K share one scale per 64-token block ("each small block shares one
// scale factor", same section); V is FP8 e4m3 with one scale per channel.
// The linear half of SLA (bonega.ai blog, SLA paragraph; tiemojia.cn article, 2.2.1)
// needs, per key block j, H_j = phi(K_j)^T V_j and z_j = colsum phi(K_j) with
// phi = softmax over the d channels of the raw K row; they are computed here from the
// same loads, on bf16 MFMA with phi split into bf16 hi + lo parts (V is exact in bf16).
// Each block's state is stored transposed, in bf16, with z as one more row:
// S_j[c][a] = H_j[a][c] for c < 128 and S_j[128][a] = z_j[a] (129 x 128), which is the
// operand order of the complement kernels; fp32 sums of 16 consecutive blocks feed the
// exact totals.
#include "common.h"

namespace sagesla {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTs = 72;  // LDS row stride (bf16) of the transposed tiles: 144 B, 16-B aligned

// One workgroup (256 threads, 4 waves) per (bh, chunk of 16 key blocks).
__global__ __launch_bounds__(256) void quant_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ kmean,
    const float* __restrict__ vamax, int N, int Nb, int Nc, int8_t* __restrict__ k8,
    float* __restrict__ sk, uint8_t* __restrict__ v8, uint16_t* __restrict__ hs,
    float* __restrict__ hpart) {
  __shared__ __attribute__((aligned(16))) uint8_t s_v8[kBlkBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_phi_hi[kD * kTs];
  __shared__ __attribute__((aligned(16))) uint16_t s_phi_lo[kD * kTs];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[kD * kTs];
  __shared__ float s_z[16][kD];
  __shared__ float s_amax[4];

  const int bh = blockIdx.x / Nc, chunk = blockIdx.x % Nc;
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15;
  const int lane = t & 63, w = t >> 6, g = lane >> 5, r = lane & 31;
  const bool states = hs != nullptr;

  float mu[8], inv_v[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    mu[e] = kmean[(size_t)bh * kD + ch * 8 + e];
    float am = vamax[(size_t)bh * kD + ch * 8 + e];
    inv_v[e] = am > 0.f ? 448.0f / am : 0.f;
  }

  v16f part[4];
  float zp = 0.f;
#pragma unroll
  for (int c = 0; c < 4; c++) part[c] = (v16f){};

  const int j0 = chunk * kChunk, j1 = min(Nb, j0 + kChunk);
  for (int j = j0; j < j1; j++) {
    const int n = block_len(j, N);
    const size_t base = ((size_t)bh * N + (size_t)j * kBlk) * kD;
    float kr[4][8], vr[4][8];
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      int row = rg + 16 * m;
      uint4 ka = {0, 0, 0, 0}, va = {0, 0, 0, 0};
      if (row < n) {
        size_t off = base + (size_t)row * kD + ch * 8;
        ka = *(const uint4*)(k + off);
        va = *(const uint4*)(v + off);
      }
      const uint16_t* kh = (const uint16_t*)&ka;
      const uint16_t* vh = (const uint16_t*)&va;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        kr[m][e] = bf16_to_f32(kh[e]);
        vr[m][e] = bf16_to_f32(vh[e]);
        if (row < n) amax = fmaxf(amax, fabsf(kr[m][e] - mu[e]));
      }
    }
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) s_amax[w] = amax;
    // V codes into LDS in operand order
#pragma unroll
    for (int m = 0; m < 4; m++) {
      int row = rg + 16 * m;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        int pk = 0;
        if (row < n) pk = __builtin_amdgcn_cvt_pk_fp8_f32(vr[m][e] * inv_v[e], vr[m][e + 1] * inv_v[e + 1], 0, false);
        s_v8[v_code_offset(row, ch * 8 + e)] = (uint8_t)(pk & 0xff);
        s_v8[v_code_offset(row, ch * 8 + e + 1)] = (uint8_t)((pk >> 8) & 0xff);
      }
    }
    __syncthreads();
    amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    if (t == 0) sk[(size_t)bh * Nb + j] = amax > 0.f ? amax / 127.0f : 0.f;
    int8_t* kdst = k8 + ((size_t)bh * Nb + j) * kBlkBytes;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      int row = rg + 16 * m;
      uint32_t lo = 0, hi = 0;
      if (row < n) {
#pragma unroll
        for (int e = 0; e < 4; e++) lo |= (uint32_t)(uint8_t)q_int8(kr[m][e] - mu[e], inv) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; e++) hi |= (uint32_t)(uint8_t)q_int8(kr[m][e + 4] - mu[e + 4], inv) << (8 * e);
      }
      *(uint2*)(kdst + qk_code_offset(row, ch * 8)) = make_uint2(lo, hi);
    }
    {
      uint8_t* vdst = v8 + ((size_t)bh * Nb + j) * kBlkBytes;
      *(uint4*)(vdst + t * 32) = *(const uint4*)(s_v8 + t * 32);
      *(uint4*)(vdst + t * 32 + 16) = *(const uint4*)(s_v8 + t * 32 + 16);
    }
    if (states) {
      // phi = softmax over channels of each raw K row (16 lanes share a row)
      float zc[8];
#pragma unroll
      for (int e = 0; e < 8; e++) zc[e] = 0.f;
#pragma unroll
      for (int m = 0; m < 4; m++) {
        int row = rg + 16 * m;
        float mx = kr[m][0];
#pragma unroll
        for (int e = 1; e < 8; e++) mx = fmaxf(mx, kr[m][e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float ex[8], s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { ex[e] = expf(kr[m][e] - mx); s += ex[e]; }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          float ph = row < n ? ex[e] / s : 0.f;
          zc[e] += ph;
          uint16_t hb = f32_to_bf16(ph);
          uint16_t lb = f32_to_bf16(ph - bf16_to_f32(hb));
          int c = ch * 8 + e;
          s_phi_hi[c * kTs + row] = hb;
          s_phi_lo[c * kTs + row] = lb;
          s_vt[c * kTs + row] = row < n ? f32_to_bf16(vr[m][e]) : (uint16_t)0;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; e++) s_z[rg][ch * 8 + e] = zc[e];
      __syncthreads();
      float zsum_t = 0.f;
      if (t < kD) {
        for (int q = 0; q < 16; q++) zsum_t += s_z[q][t];
        zp += zsum_t;
      }
      // H_j^T = V^T phi on MFMA: wave w owns rows c in [32w, 32w+32), all 4 column tiles a
      v16f acc[4];
#pragma unroll
      for (int c = 0; c < 4; c++) acc[c] = (v16f){};
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const int tok = 16 * s + 8 * g;
        v8bf av = *(const v8bf*)(s_vt + (32 * w + r) * kTs + tok);
#pragma unroll
        for (int c = 0; c < 4; c++) {
          v8bf bh_ = *(const v8bf*)(s_phi_hi + (32 * c + r) * kTs + tok);
          v8bf bl_ = *(const v8bf*)(s_phi_lo + (32 * c + r) * kTs + tok);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh_, acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl_, acc[c], 0, 0, 0);
        }
      }
      uint16_t* hdst = hs + ((size_t)bh * Nb + j) * kStateElems;
#pragma unroll
      for (int c = 0; c < 4; c++)
#pragma unroll
        for (int q = 0; q < 16; q++) {
          const int row = 32 * w + 8 * (q >> 2) + 4 * g + (q & 3);  // channel c of V
          hdst[row * kD + 32 * c + r] = f32_to_bf16(acc[c][q]);
          part[c][q] += acc[c][q];
        }
      if (t < kD) hdst[kD * kD + t] = f32_to_bf16(zsum_t);
    }
    __syncthreads();
  }
  if (states) {
    float* pdst = hpart + ((size_t)bh * Nc + chunk) * kStateElems;
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const int row = 32 * w + 8 * (q >> 2) + 4 * g + (q & 3);
        pdst[row * kD + 32 * c + r] = part[c][q];
      }
    if (t < kD) pdst[kD * kD + t] = zp;
  }
}

// Totals over the partial sums: htot[bh][e] = sum_c hpart[bh][c][e], e < 129*128.
// One workgroup of 256 threads per (bh, 1024 elements).
__global__ __launch_bounds__(256) void linear_total_kernel(const float* __restrict__ hpart, int Nc,
                                                           float* __restrict__ htot) {
  constexpr int kParts = (kStateElems + 1023) / 1024;
  const int bh = blockIdx.x / kParts, part = blockIdx.x % kParts, t = threadIdx.x;
  const int e = part * 1024 + t * 4;
  if (e >= kStateElems) return;
  v4f s = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < Nc; c++) s += *(const v4f*)(hpart + ((size_t)bh * Nc + c) * kStateElems + e);
  *(v4f*)(htot + (size_t)bh * kStateElems + e) = s;
}

hipError_t launch_quant_kv(const void* k, const void* v, const void* kmean, const void* vamax, int BH,
                           int N, int Nb, void* k8, void* sk, void* v8, void* hs, void* hpart, hipStream_t st) {
  const int Nc = (Nb + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(quant_kv_kernel, dim3(BH * Nc), dim3(256), 0, st, (const uint16_t*)k,
                     (const uint16_t*)v, (const float*)kmean, (const float*)vamax, N, Nb, Nc,
                     (int8_t*)k8, (float*)sk, (uint8_t*)v8, (uint16_t*)hs, (float*)hpart);
  return hipGetLastError();
}

hipError_t launch_linear_total(const void* hpart, int BH, int Nb, void* htot, hipStream_t st) {
  const int Nc = (Nb + kChunk - 1) / kChunk;
  constexpr int kParts = (kStateElems + 1023) / 1024;
  hipLaunchKernelGGL(linear_total_kernel, dim3(BH * kParts), dim3(256), 0, st, (const float*)hpart, Nc,
                     (float*)htot);
  return hipGetLastError();
}

}  // namespace sagesla
