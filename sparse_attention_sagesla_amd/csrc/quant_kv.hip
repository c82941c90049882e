// K smoothing + INT8, V to FP8 e4m3, and the linear-branch states per key block.
//
// SageAttention smooths outliers into range before quantizing and undoes the transform
// afterwards (TurboDiffusion explainer, news.qq.com, "Third key"); for K this is the
// subtraction of the per-channel mean over all tokens, which leaves softmax(q.k)
// unchanged. Q and K take one scale per 64-token block (the page has every small block
// share a single scale, same section); V is FP8 e4m3 with one scale per channel.
// The linear half of SLA (bonega.ai blog, SLA paragraph; tiemojia.cn article, 2.2.1)
// needs, per key block j, H_j = phi(K_j)^T V_j and z_j = colsum phi(K_j) with
// phi = softmax over the d channels of the raw K row; they are computed here from the
// same loads, on bf16 MFMA with phi split into bf16 hi + lo parts (V is exact in bf16).
// Each block's state is stored transposed, in bf16, with z as one more row:
// S_j[c][a] = H_j[a][c] for c < 128 and S_j[128][a] = z_j[a] (129 x 128), which is the
// operand order of the complement kernels; fp32 sums of 16 consecutive blocks feed the
// exact totals.
#include "buffer.h"
#include "common.h"

namespace sagesla {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_* lds_v4s_ptr;

constexpr int kTp = 144;  // LDS row pitch (bf16) of the [token][channel] tiles: 288 B (bank spread)
constexpr int kSp = 136;  // LDS row pitch (bf16) of the staged state tile: 272 B
static_assert((kD + 1) * kSp <= 2 * 64 * kTp, "the staged state must fit in the phi area");

// gfx950 transposing LDS read: within each group of 16 lanes, lanes 4a..4a+3 each name
// 4 consecutive 16-bit elements of row a of a 4 x 16 tile, and lane j receives column j.
__device__ __forceinline__ v4s_ lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p));
}

// 8 consecutive tokens t0..t0+7 of channel column (16-lane group base c0 + lane%16) of a
// row-major [token][channel] bf16 tile: the K=8 slice of a bf16 MFMA operand.
__device__ __forceinline__ v8bf tile_col8(const uint16_t* tile, int t0, int c0, int lane) {
  const int j = lane & 15, a = j >> 2, b = j & 3;
  const v4s_ r0 = lds_read_tr16(tile + (t0 + a) * kTp + c0 + 4 * b);
  const v4s_ r1 = lds_read_tr16(tile + (t0 + 4 + a) * kTp + c0 + 4 * b);
  const v8s v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(v8bf, v);
}

constexpr int kQkThreads = 512;

// One workgroup (512 threads, 8 waves) per (bh, chunk of 16 key blocks). Thread t
// covers rows t/16 + 32m (m = 0, 1) and channels 8*(t%16) .. +7 of each block. In the
// state product wave w owns rows c in [32(w%4), +32) and column tiles 2(w/4), 2(w/4)+1.
// All of one head's traffic goes through buffer resources with 32-bit offsets: the
// 128-register budget (two workgroups per CU) then holds without spills, whose reloads
// would wait on the prefetched rows.
__global__ __launch_bounds__(kQkThreads, 4) void quant_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ kmean,
    const float* __restrict__ vamax, int N, int Nb, int Nc, int8_t* __restrict__ k8,
    float* __restrict__ sk, uint8_t* __restrict__ v8, uint16_t* __restrict__ hs,
    float* __restrict__ hpart) {
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kBlk * kTp];       // V (bf16), [token][channel]
  __shared__ __attribute__((aligned(16))) uint16_t s_phi[2][kBlk * kTp];  // phi(K) hi, lo parts
  __shared__ float s_z[8][kD];
  __shared__ float s_amax[8];

  // the head and chunk are kept in scalar registers, so that every address derived
  // from them is scalar too
  const int bh = __builtin_amdgcn_readfirstlane(blockIdx.x / Nc);
  const int chunk = __builtin_amdgcn_readfirstlane(blockIdx.x - bh * Nc);
  const int t = threadIdx.x, rg = t >> 4, ch = t & 15;
  const int lane = t & 63, g = lane >> 5, r = lane & 31, hl = (lane >> 4) & 1;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wr = w & 3, wc = w >> 2;
  const bool states = hs != nullptr;

  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; e++) mu[e] = kmean[(size_t)bh * kD + ch * 8 + e];
  // V code chunk (dt, half) = (w/2, w%2); the lane's channel is 32*dt + r
  const int vdt = w >> 1, vhalf = w & 1;
  const float am_v = vamax[(size_t)bh * kD + 32 * vdt + r];
  const float inv_v = am_v > 0.f ? 448.0f / am_v : 0.f;

  v16f part[2];
  float zp = 0.f;
  part[0] = (v16f){};
  part[1] = (v16f){};

  const int j0 = chunk * kChunk, j1 = min(Nb, j0 + kChunk);
  const size_t tok0 = scalar_off((size_t)bh * N * kD), blk0 = scalar_off((size_t)bh * Nb);
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(k + tok0, (uint32_t)N * kD * 2);
  const __amdgpu_buffer_rsrc_t rv = buf_rsrc(v + tok0, (uint32_t)N * kD * 2);
  const __amdgpu_buffer_rsrc_t rk8 = buf_rsrc(k8 + blk0 * kBlkBytes, (uint32_t)Nb * kBlkBytes);
  const __amdgpu_buffer_rsrc_t rv8 = buf_rsrc(v8 + blk0 * kBlkBytes, (uint32_t)Nb * kBlkBytes);
  const __amdgpu_buffer_rsrc_t rhs = buf_rsrc(states ? hs + blk0 * kStateElems : hs, (uint32_t)Nb * kStateElems * 2);
  // Raw K and V rows of block jj; rows past N lie past the resource's end and read zero.
  // Each block's rows are fetched while the previous block is processed; every fetch is
  // unconditional (the chunk's last block is fetched again after itself), so that the
  // wait before a block's first use counts exactly the loads issued after it.
  uint4 kn[2], vn[2];
  auto fetch = [&](int jj) {
    const int sb = jj * kBlk * kD * 2;
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const int off = (rg + 32 * m) * kD * 2 + ch * 16;
      kn[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, sb, 0));
      vn[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, sb, 0));
    }
  };
  fetch(j0);
  for (int j = j0; j < j1; j++) {
    const int n = block_len(j, N);
    uint4 kraw[2], vraw[2];
#pragma unroll
    for (int m = 0; m < 2; m++) { kraw[m] = kn[m]; vraw[m] = vn[m]; }
    fetch(min(j + 1, j1 - 1));
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const int row = rg + 32 * m;
      // V row-major into LDS for the V codes and the state product
      *(uint4*)(s_v + row * kTp + ch * 8) = vraw[m];
      const uint16_t* kh = (const uint16_t*)&kraw[m];
      if (row < n) {
#pragma unroll
        for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf(bf16_to_f32(kh[e]) - mu[e]));
      }
    }
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) s_amax[w] = amax;
    // phi = softmax over channels of each raw K row (16 lanes share a row)
    if (states) {
      float zc[8];
#pragma unroll
      for (int e = 0; e < 8; e++) zc[e] = 0.f;
#pragma unroll
      for (int m = 0; m < 2; m++) {
        const int row = rg + 32 * m;
        const uint16_t* kh = (const uint16_t*)&kraw[m];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = bf16_to_f32(kh[e]);
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; e++) mx = fmaxf(mx, x[e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float ssum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { x[e] = __expf(x[e] - mx); ssum += x[e]; }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ssum += __shfl_xor(ssum, o);
        const float inv = row < n ? 1.0f / ssum : 0.f;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = x[e] * inv, p1 = x[e + 1] * inv;
          zc[e] += p0;
          zc[e + 1] += p1;
          hw[e / 2] = pack_bf16x2(p0, p1);
          lw[e / 2] = pack_bf16x2(p0 - bf16_to_f32((uint16_t)(hw[e / 2] & 0xffffu)),
                                  p1 - bf16_to_f32((uint16_t)(hw[e / 2] >> 16)));
        }
        *(uint4*)(s_phi[0] + row * kTp + ch * 8) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *(uint4*)(s_phi[1] + row * kTp + ch * 8) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      }
      // the wave's 4 row groups share channels: reduce over lanes ch, ch+16, ch+32, ch+48
#pragma unroll
      for (int e = 0; e < 8; e++) {
        zc[e] += __shfl_xor(zc[e], 16);
        zc[e] += __shfl_xor(zc[e], 32);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; e++) s_z[w][ch * 8 + e] = zc[e];
      }
    }
    __syncthreads();
    // K: smoothed INT8 codes with one scale per block
    amax = s_amax[0];
#pragma unroll
    for (int q = 1; q < 8; q++) amax = fmaxf(amax, s_amax[q]);
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    if (t == 0) sk[blk0 + j] = amax > 0.f ? amax / 127.0f : 0.f;
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const int row = rg + 32 * m;
      const uint16_t* kh = (const uint16_t*)&kraw[m];
      uint32_t lo = 0, hi = 0;
      if (row < n) {
#pragma unroll
        for (int e = 0; e < 4; e++) lo |= (uint32_t)(uint8_t)q_int8(bf16_to_f32(kh[e]) - mu[e], inv) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; e++) hi |= (uint32_t)(uint8_t)q_int8(bf16_to_f32(kh[e + 4]) - mu[e + 4], inv) << (8 * e);
      }
      __builtin_amdgcn_raw_buffer_store_b64((v2u){lo, hi}, rk8, qk_code_offset(row, ch * 8), j * kBlkBytes, 0);
    }
    // V: FP8 codes straight in operand order. Chunk (dt, half, lane) holds channel
    // 32*dt + r at tokens 32*half + 4*g + {0..3, 8..11, 16..19, 24..27}: four
    // transposing reads of 4 consecutive tokens each.
    {
      const int c0 = 32 * vdt + 16 * hl, jj = lane & 15, a = jj >> 2, b = jj & 3;
      uint32_t wd[4];
#pragma unroll
      for (int qd = 0; qd < 4; qd++) {
        const v4s_ rv = lds_read_tr16(s_v + (32 * vhalf + 4 * g + 8 * qd + a) * kTp + c0 + 4 * b);
        const float f0 = bf16_to_f32((uint16_t)rv[0]) * inv_v, f1 = bf16_to_f32((uint16_t)rv[1]) * inv_v;
        const float f2 = bf16_to_f32((uint16_t)rv[2]) * inv_v, f3 = bf16_to_f32((uint16_t)rv[3]) * inv_v;
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, pk, true);
        wd[qd] = (uint32_t)pk;
      }
      __builtin_amdgcn_raw_buffer_store_b128((v4u){wd[0], wd[1], wd[2], wd[3]}, rv8, t * 16, j * kBlkBytes, 0);
    }
    if (states) {
      float zsum_t = 0.f;
      if (t < kD) {
#pragma unroll
        for (int q = 0; q < 8; q++) zsum_t += s_z[q][t];
        zp += zsum_t;
      }
      // H_j^T = V^T phi on MFMA; both operands are 8-token slices read transposed from
      // the row-major tiles
      v16f acc[2];
      acc[0] = (v16f){};
      acc[1] = (v16f){};
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const int t0 = 16 * s + 8 * g;
        const v8bf av = tile_col8(s_v, t0, 32 * wr + 16 * hl, lane);
#pragma unroll
        for (int c = 0; c < 2; c++) {
          const int a0 = 32 * (2 * wc + c) + 16 * hl;
          const v8bf bh_ = tile_col8(s_phi[0], t0, a0, lane);
          const v8bf bl_ = tile_col8(s_phi[1], t0, a0, lane);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh_, acc[c], 0, 0, 0);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl_, acc[c], 0, 0, 0);
        }
      }
      // the block's state S_j (129 x 128 bf16) is staged in the phi area for 16-byte stores
      __syncthreads();  // every wave is done reading phi
      uint16_t* s_st = &s_phi[0][0];
#pragma unroll
      for (int c = 0; c < 2; c++)
#pragma unroll
        for (int q = 0; q < 16; q++) {
          const int row = 32 * wr + 8 * (q >> 2) + 4 * g + (q & 3);  // channel of V
          s_st[row * kSp + 32 * (2 * wc + c) + r] = f32_to_bf16(acc[c][q]);
          part[c][q] += acc[c][q];
        }
      if (t < kD) s_st[kD * kSp + t] = f32_to_bf16(zsum_t);
      __syncthreads();
      for (int e = t; e < (kD + 1) * 16; e += kQkThreads) {
        const int row = e >> 4, c8 = (e & 15) * 8;
        __builtin_amdgcn_raw_buffer_store_b128(*(const v4u*)(s_st + row * kSp + c8), rhs, (row * kD + c8) * 2,
                                               j * kStateElems * 2, 0);
      }
    }
    __syncthreads();
  }
  if (states) {
    float* pdst = hpart + ((size_t)bh * Nc + chunk) * kStateElems;
#pragma unroll
    for (int c = 0; c < 2; c++)
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const int row = 32 * wr + 8 * (q >> 2) + 4 * g + (q & 3);
        pdst[row * kD + 32 * (2 * wc + c) + r] = part[c][q];
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
  // one head's rows, codes and states are each addressed by 32-bit buffer offsets
  if ((uint64_t)N * kD * 2 > UINT32_MAX || (uint64_t)Nb * kStateElems * 2 > UINT32_MAX) return hipErrorInvalidValue;
  const int Nc = (Nb + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(quant_kv_kernel, dim3(BH * Nc), dim3(kQkThreads), 0, st, (const uint16_t*)k,
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
