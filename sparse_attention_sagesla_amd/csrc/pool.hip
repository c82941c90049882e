// Block pooling of Q/K, V block max, and per-block INT8 quantization of Q.
//
// SLA first makes a quick estimate of how strongly positions relate before deciding
// what to compute exactly (TurboDiffusion explainer, news.qq.com, "First key:
// attention"); here that estimate is made on 64-token block means. SageAttention's
// 8-bit quantization with one scale per small block (same page, "First key" and
// "Third key") is applied to Q in the same pass, since Q needs no smoothing.
#include "buffer.h"
#include "common.h"

namespace sagesla {

// Where the pool pass reads its rows from. Plain: q, k, v as [B, H, N, d]. From the
// projection (the producer-side fusion): the QKV projection output [B, N, 3, H, d]; q and k
// are RMS-normalized on the way in (scale r per token from rms_scale_kernel, then the
// learned weight, each product rounded to bf16), and all three are written out as
// [B, H, N, d] for the rest of the attention.
struct ProjSrc {
  const uint16_t* qkv;  // [B][N][3][H][d]
  const float* rs;      // [2][B][N]: r of q, then of k
  const uint16_t* gq;   // [H*d]
  const uint16_t* gk;   // [H*d]
  uint16_t *q, *k, *v;  // [B][H][N][d] outputs
  int H;
};

// bf16(bf16(x * r) * g) for 8 channels
__device__ __forceinline__ uint4 rms_apply(uint4 x, float r, uint4 g) {
  const uint16_t* xh = (const uint16_t*)&x;
  const uint16_t* gh = (const uint16_t*)&g;
  uint4 o;
  uint16_t* oh = (uint16_t*)&o;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint16_t nb = f32_to_bf16(bf16_to_f32(xh[e]) * r);
    oh[e] = f32_to_bf16(bf16_to_f32(nb) * bf16_to_f32(gh[e]));
  }
  return o;
}

// x summed with the value of lane l ^ 16 and then of l ^ 32 (the wave's four row groups of
// one channel), through the VALU lane swaps: every lane ends with the same total.
__device__ __forceinline__ double wave_rows_sum(double x) {
  int lo = __double2loint(x), hi = __double2hiint(x);
  {
    const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    x = __hiloint2double((int)sh[0], (int)sl[0]) + __hiloint2double((int)sh[1], (int)sl[1]);
  }
  lo = __double2loint(x);
  hi = __double2hiint(x);
  const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return __hiloint2double((int)sh[0], (int)sl[0]) + __hiloint2double((int)sh[1], (int)sl[1]);
}
__device__ __forceinline__ float wave_rows_max(float x) {
  {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = fmaxf(__int_as_float((int)s[0]), __int_as_float((int)s[1]));
  }
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float((int)s[0]), __int_as_float((int)s[1]));
}

// One workgroup (256 threads) per (bh, block). Thread t covers rows t/16 + 16m
// (m = 0..3) and channels 8*(t%16) .. +7. The channel sums (fp64: exact for bf16 inputs
// of moderate range, so their order is immaterial) and maxima are reduced within each
// wave by lane swaps and across the 4 waves through LDS.
template <bool kFromProj>
__global__ __launch_bounds__(256) void pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    ProjSrc ps, int N, int Nb, double* __restrict__ qbar, double* __restrict__ kbart, double* __restrict__ ksum,
    float* __restrict__ vamax_blk, int8_t* __restrict__ q8, float* __restrict__ sq) {
  __shared__ double s_q[4][kD];
  __shared__ double s_k[4][kD];
  __shared__ float s_v[4][kD];
  __shared__ float s_amax[4];

  const int tile = blockIdx.x;
  const int bh = __builtin_amdgcn_readfirstlane(tile / Nb), i = __builtin_amdgcn_readfirstlane(tile - bh * Nb);
  const int n = block_len(i, N);
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15, w = t >> 6;
  const size_t base = ((size_t)bh * N + (size_t)i * kBlk) * kD;

  uint4 qa[4], ka[4], va[4];
  if constexpr (kFromProj) {
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int row = rg + 16 * m;
      qa[m] = ka[m] = va[m] = make_uint4(0, 0, 0, 0);
      if (row < n) {
        const size_t off = base + (size_t)row * kD + ch * 8;
        const int b = bh / ps.H, h = bh % ps.H, tok = i * kBlk + row, D = ps.H * kD;
        const uint16_t* src = ps.qkv + ((size_t)b * N + tok) * 3 * D + h * kD + ch * 8;
        const size_t rr = (size_t)b * N + tok, BN = (size_t)(gridDim.x / Nb / ps.H) * N;
        qa[m] = rms_apply(*(const uint4*)src, ps.rs[rr], *(const uint4*)(ps.gq + h * kD + ch * 8));
        ka[m] = rms_apply(*(const uint4*)(src + D), ps.rs[BN + rr], *(const uint4*)(ps.gk + h * kD + ch * 8));
        va[m] = *(const uint4*)(src + 2 * D);
        *(uint4*)(ps.q + off) = qa[m];
        *(uint4*)(ps.k + off) = ka[m];
        *(uint4*)(ps.v + off) = va[m];
      }
    }
  } else {
    // one head's rows through buffer resources: 32-bit lane offsets, and rows past N
    // (past the resource's end) read zero
    const size_t h0 = scalar_off((size_t)bh * N * kD);
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(q + h0, (uint32_t)N * kD * 2);
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + h0, (uint32_t)N * kD * 2);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + h0, (uint32_t)N * kD * 2);
    const int sb = i * kBlk * kD * 2;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int off = (rg + 16 * m) * kD * 2 + ch * 16;
      qa[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, sb, 0));
      ka[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, sb, 0));
      va[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, sb, 0));
    }
  }
  // K, then Q, then V: one set of per-channel partials live at a time
  float amax = 0.f;
  {
    double sk_[8];
#pragma unroll
    for (int e = 0; e < 8; e++) sk_[e] = 0.0;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint16_t* kh = (const uint16_t*)&ka[m];
#pragma unroll
      for (int e = 0; e < 8; e++) sk_[e] += (double)bf16_to_f32(kh[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; e++) sk_[e] = wave_rows_sum(sk_[e]);
    if (rg % 4 == 0) {
#pragma unroll
      for (int e = 0; e < 8; e++) s_k[w][ch * 8 + e] = sk_[e];
    }
  }
  {
    double sq_[8];
#pragma unroll
    for (int e = 0; e < 8; e++) sq_[e] = 0.0;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint16_t* qh = (const uint16_t*)&qa[m];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float xq = bf16_to_f32(qh[e]);
        sq_[e] += (double)xq;
        amax = fmaxf(amax, fabsf(xq));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) sq_[e] = wave_rows_sum(sq_[e]);
    if (rg % 4 == 0) {
#pragma unroll
      for (int e = 0; e < 8; e++) s_q[w][ch * 8 + e] = sq_[e];
    }
  }
  {
    float mv[8];
#pragma unroll
    for (int e = 0; e < 8; e++) mv[e] = 0.f;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint16_t* vh = (const uint16_t*)&va[m];
#pragma unroll
      for (int e = 0; e < 8; e++) mv[e] = fmaxf(mv[e], fabsf(bf16_to_f32(vh[e])));
    }
#pragma unroll
    for (int e = 0; e < 8; e++) mv[e] = wave_rows_max(mv[e]);
    if (rg % 4 == 0) {
#pragma unroll
      for (int e = 0; e < 8; e++) s_v[w][ch * 8 + e] = mv[e];
    }
  }
  // block-wide max |q|
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((t & 63) == 0) s_amax[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));

  if (t < kD) {
    const double a = (s_q[0][t] + s_q[1][t]) + (s_q[2][t] + s_q[3][t]);
    const double b = (s_k[0][t] + s_k[1][t]) + (s_k[2][t] + s_k[3][t]);
    const float mx = fmaxf(fmaxf(s_v[0][t], s_v[1][t]), fmaxf(s_v[2][t], s_v[3][t]));
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
    const int row = rg + 16 * m;
    const uint16_t* qh = (const uint16_t*)&qa[m];
    uint32_t lo = 0, hi = 0;
    if (row < n) {
#pragma unroll
      for (int e = 0; e < 4; e++) lo |= (uint32_t)(uint8_t)q_int8(bf16_to_f32(qh[e]), inv) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; e++) hi |= (uint32_t)(uint8_t)q_int8(bf16_to_f32(qh[e + 4]), inv) << (8 * e);
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
  // one head's rows are addressed by 32-bit buffer offsets
  if ((uint64_t)N * kD * 2 > UINT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pool_kernel<false>, dim3(BH * Nb), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, ProjSrc{}, N, Nb, (double*)qbar, (double*)kbart,
                     (double*)ksum, (float*)vamax_blk, (int8_t*)q8, (float*)sq);
  return hipGetLastError();
}

// ---------------------------------------------------------------- producer-side fusion
// Per token: r = fp32(1 / sqrt(mean(x^2) + eps)) of its q row and of its k row (D = H*d
// channels each), the squares and their sum in fp64 (exact for bf16 inputs of ordinary
// range, so the sum does not depend on its order), one wave per (q or k, token).
__global__ __launch_bounds__(256) void rms_scale_kernel(const uint16_t* __restrict__ qkv, int BN, int D, double eps,
                                                        float* __restrict__ rs) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (wv >= 2 * BN) return;
  const int part = wv / BN, row = wv % BN;  // part 0: q, 1: k
  const uint16_t* src = qkv + (size_t)row * 3 * D + (size_t)part * D;
  double ss = 0.0;
  for (int c = l * 8; c < D; c += 512) {
    const uint4 x = *(const uint4*)(src + c);
    const uint16_t* xh = (const uint16_t*)&x;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const double f = (double)bf16_to_f32(xh[e]);
      ss += f * f;
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (l == 0) rs[(size_t)part * BN + row] = (float)(1.0 / sqrt(ss / (double)D + eps));
}

hipError_t launch_prepare(const void* qkv, const void* gq, const void* gk, double eps, int B, int H, int N, int Nb,
                          void* rs, void* q, void* k, void* v, void* qbar, void* kbart, void* ksum, void* vamax_blk,
                          void* q8, void* sq, hipStream_t st) {
  const int BN = B * N, D = H * kD;
  hipLaunchKernelGGL(rms_scale_kernel, dim3((2 * BN + 3) / 4), dim3(256), 0, st, (const uint16_t*)qkv, BN, D, eps,
                     (float*)rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProjSrc ps{(const uint16_t*)qkv, (const float*)rs, (const uint16_t*)gq, (const uint16_t*)gk,
             (uint16_t*)q,       (uint16_t*)k,      (uint16_t*)v,        H};
  hipLaunchKernelGGL(pool_kernel<true>, dim3(B * H * Nb), dim3(256), 0, st, nullptr, nullptr, nullptr, ps, N, Nb,
                     (double*)qbar, (double*)kbart, (double*)ksum, (float*)vamax_blk, (int8_t*)q8, (float*)sq);
  return hipGetLastError();
}

hipError_t launch_head_stats(const void* ksum, const void* vamax_blk, int BH, int N, int Nb,
                             void* kmean, void* vamax, hipStream_t st) {
  hipLaunchKernelGGL(head_stats_kernel, dim3(BH * 16), dim3(256), 0, st, (const double*)ksum,
                     (const float*)vamax_blk, N, Nb, (float*)kmean, (float*)vamax);
  return hipGetLastError();
}

}  // namespace sagesla
