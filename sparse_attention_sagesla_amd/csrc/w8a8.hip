// W8A8 linear layer on the INT8 matrix cores: y = x W^T (+ bias) with INT8 weights in
// 128 x 128 blocks (one fp32 scale per block, quantized once) and INT8 activations
// quantized on the fly, one fp32 scale per token and 128-channel block.
//
// TurboDiffusion explainer (news.qq.com, "Third key"): weights and activations of the
// linear layers are both 8-bit integers so that the whole layer runs in the INT8 domain;
// the weights are quantized offline in 128 x 128 blocks that each share one scale factor,
// the activations dynamically at inference. The activation grouping is not given; one
// scale per token and 128 channels (the K extent of a weight block) is the reading here.
//
// Code layout (both operands): tiles of 32 rows x 128 channels (4 KiB) in MFMA operand
// order, byte (s*64 + lane)*16 + e <-> row 32*tile + lane%32, channel 64*(lane/32) + 16*s + e
// of the 128-channel block, stored K-block major: tile (kb, rt) at (kb*RT + rt)*4096. One
// 16-byte chunk per lane is then one MFMA step's operand.
#include "common.h"

namespace sagesla {

constexpr int kW8Tile = 4096;  // bytes of one 32 x 128 code tile
typedef __attribute__((address_space(3))) void* lds_ptr_w8;

// One workgroup (4 waves) per (32-row tile, 128-channel block): thread (s, lane) holds
// channels 64*(lane/32) + 16*s .. +15 of row lane%32, that is its own 16-byte code chunk.
// Rows at or past M get zero codes and scale 0.
__global__ __launch_bounds__(256) void w8a8_quant_act_kernel(const uint16_t* __restrict__ x, int M, int K, int MT,
                                                            int Mp, int8_t* __restrict__ x8, float* __restrict__ sx) {
  __shared__ float s_am[4][32];
  const int kb = blockIdx.x / MT, mt = blockIdx.x % MT;
  const int t = threadIdx.x, s = t >> 6, lane = t & 63, r = lane & 31, g = lane >> 5;
  const int row = 32 * mt + r;
  float v[16];
  if (row < M) {
    const uint16_t* src = x + (size_t)row * K + 128 * kb + 64 * g + 16 * s;
    const uint4 a = *(const uint4*)src, b = *(const uint4*)(src + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; e++) v[e] = 0.f;
  }
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e++) am = fmaxf(am, fabsf(v[e]));
  am = fmaxf(am, __shfl_xor(am, 32));  // the row's other half (g)
  if (g == 0) s_am[s][r] = am;
  __syncthreads();
  am = fmaxf(fmaxf(s_am[0][r], s_am[1][r]), fmaxf(s_am[2][r], s_am[3][r]));
  const float inv = am > 0.f ? 127.0f / am : 0.f;
  uint32_t pk[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    uint32_t wd = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) wd |= (uint32_t)(uint8_t)(int8_t)q_int8(v[4 * e + b], inv) << (8 * b);
    pk[e] = wd;
  }
  *(uint4*)(x8 + ((size_t)kb * MT + mt) * kW8Tile + (s * 64 + lane) * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (t < 32) sx[(size_t)kb * Mp + 32 * mt + t] = am > 0.f ? am / 127.0f : 0.f;
}

// One workgroup per 128 x 128 weight block: thread (s, lane) holds its chunk of each of
// the block's four 32-row tiles.
__global__ __launch_bounds__(256) void w8a8_quant_weight_kernel(const uint16_t* __restrict__ w, int K, int NT,
                                                               int KB, int8_t* __restrict__ w8, float* __restrict__ sw) {
  __shared__ float s_am[4];
  const int nb = blockIdx.x / KB, kb = blockIdx.x % KB;
  const int t = threadIdx.x, s = t >> 6, lane = t & 63, r = lane & 31, g = lane >> 5;
  float v[4][16];
  float am = 0.f;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint16_t* src = w + (size_t)(128 * nb + 32 * q + r) * K + 128 * kb + 64 * g + 16 * s;
    const uint4 a = *(const uint4*)src, b = *(const uint4*)(src + 8);
    const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      v[q][2 * e] = __uint_as_float(wd[e] << 16);
      v[q][2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int e = 0; e < 16; e++) am = fmaxf(am, fabsf(v[q][e]));
  }
  for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if (lane == 0) s_am[s] = am;
  __syncthreads();
  am = fmaxf(fmaxf(s_am[0], s_am[1]), fmaxf(s_am[2], s_am[3]));
  const float inv = am > 0.f ? 127.0f / am : 0.f;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      uint32_t wd = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) wd |= (uint32_t)(uint8_t)(int8_t)q_int8(v[q][4 * e + b], inv) << (8 * b);
      pk[e] = wd;
    }
    *(uint4*)(w8 + ((size_t)kb * NT + 4 * nb + q) * kW8Tile + (s * 64 + lane) * 16) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
  if (t == 0) sw[(size_t)nb * KB + kb] = am > 0.f ? am / 127.0f : 0.f;
}

// y tile of 256 rows x 256 columns per workgroup (8 waves, 2 per SIMD, 1 workgroup per
// CU): wave (wm, wn) owns rows 64*wm .. +63 and columns 128*wn .. +127 (one 128-column
// weight block). Per 128-channel block kb: the 8 x-tiles, 8 w-tiles and the 256 activation
// scales go by DMA into a two-stage LDS ring, one block ahead. The wave's product is 8 x 4
// sub-tiles of 16 columns x 16 rows, each two INT8 16x16x64 MFMAs into an int32 tile
// D[n][m] (lane: row m = lane%16, columns 4*(lane/16) .. +3), added to the fp32 accumulator
// (in VGPRs: the VALU updates it) scaled by s_x[m][kb] s_w[nblock][kb].
//
// Operand chunks of a 16-row sub-tile for one 64-channel step t: lane 16g + r reads the
// 16-byte chunk (s = 2t + g/2, lane' = 32(g%2) + 16*half + r) of the 32-row code tile, a
// chunk of row r of that half. The chunks cover each row's 128 channels once over t and g,
// and the x and w operands use the same assignment, so each MFMA pair sums the block's
// products (the order of the K terms is immaterial to an exact integer sum).
__global__ __launch_bounds__(512) void w8a8_gemm_kernel(const int8_t* __restrict__ x8, const float* __restrict__ sx,
                                                        const int8_t* __restrict__ w8, const float* __restrict__ sw,
                                                        const uint16_t* __restrict__ bias, int M, int N, int KB,
                                                        int MT, int NT, int Mp, int tiles_n, int tiles,
                                                        int per_xcd, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(1024))) int8_t s_x0[8 * kW8Tile];
  __shared__ __attribute__((aligned(1024))) int8_t s_w0[8 * kW8Tile];
  __shared__ __attribute__((aligned(1024))) int8_t s_x1[8 * kW8Tile];
  __shared__ __attribute__((aligned(1024))) int8_t s_w1[8 * kW8Tile];
  __shared__ __attribute__((aligned(256))) float s_s0[256];
  __shared__ __attribute__((aligned(256))) float s_s1[256];

  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= tiles) return;
  // tiles in groups of 8 row tiles: consecutive tiles run through the group's row tiles for
  // one column tile, so that the 32 workgroups resident on an XCD read 8 x slices and 4 w
  // slices per block (the L2 then serves most operand reads; the whole weight, 26 MB for a
  // 5120 x 5120 layer, would otherwise be fetched again for every row tile)
  const int TM = tiles / tiles_n, grp = tile / (8 * tiles_n), gi = tile % (8 * tiles_n);
  const int gm = min(8, TM - grp * 8);
  const int tm = grp * 8 + gi % gm, tn = gi / gm;
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), wm = w & 3, wn = w >> 2;
  const int nblk = 2 * tn + wn;  // this wave's 128-column weight block

  // every wave issues 9 DMAs per block: its x tile (4 x 1 KiB), its w tile (4 x 1 KiB) and
  // 64 activation scales (waves 4..7 repeat waves 0..3's, into the same place)
  int lo = l * 16, ls = l * 4;  // this lane's DMA offsets (opaque: scalar-base addressing)
  auto issue = [&](int8_t* dx, int8_t* dw, float* ds, int kb) {
    asm volatile("" : "+v"(lo), "+v"(ls));
    const int8_t* xs = x8 + ((size_t)kb * MT + 8 * tm + w) * kW8Tile;
    const int8_t* ws = w8 + ((size_t)kb * NT + 8 * tn + w) * kW8Tile;
    const char* ss = (const char*)(sx + (size_t)kb * Mp + 256 * tm + 64 * (w & 3));
#pragma unroll
    for (int c = 0; c < 4; c++)
      __builtin_amdgcn_global_load_lds((const void*)(xs + (uint32_t)lo + c * 1024),
                                       (lds_ptr_w8)(dx + w * kW8Tile + c * 1024), 16, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; c++)
      __builtin_amdgcn_global_load_lds((const void*)(ws + (uint32_t)lo + c * 1024),
                                       (lds_ptr_w8)(dw + w * kW8Tile + c * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(ss + (uint32_t)ls), (lds_ptr_w8)(ds + 64 * (w & 3)), 4, 0, 0);
  };

  // accumulator of column sub-tile j (16 columns), row sub-tile h (16 rows) at acc[j][h]
  float acc[8][4][4];
  // The int32 tiles start from the bits of 1.5 * 2^23 (float), so the MFMA's integer sum
  // leaves the bits of the float 1.5 * 2^23 + dot (|dot| <= 127 * 127 * 128 < 2^22 keeps it
  // in [2^23, 2^24), where floats are the integers): one exact subtraction then gives
  // float(dot), in place of the slower int-to-float conversion.
  const v4i magic = (v4i){0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int h = 0; h < 4; h++)
#pragma unroll
      for (int v = 0; v < 4; v++) acc[j][h][v] = 0.f;

  // this lane's byte offset within a code tile (see above), and its operand bases (kept
  // opaque per block, so that the compiler adds the sub-tile and step offsets as immediates
  // instead of holding one address per stage, sub-tile and step)
  const int g = l >> 4, r = l & 15;
  const int lane_off = ((g >> 1) * 64 + 32 * (g & 1) + r) * 16;
  int xo = 2 * wm * kW8Tile + lane_off, wo = 4 * wn * kW8Tile + lane_off, so = 64 * wm + r;
  // The eight column groups go in a pipeline: the MFMAs of group j (four independent
  // two-MFMA chains, one per row sub-tile) are issued before group j-1 is scaled into its
  // accumulators, and the w operands of group j+1 are read from LDS meanwhile. The empty
  // asm statements keep that order (the compiler would otherwise issue every MFMA first and
  // hold all the int32 tiles): group j+1's operands pass through an asm placed after group
  // j-1's accumulators have been written, so at most two groups of int32 tiles are live.
  auto compute = [&](const int8_t* cx, const int8_t* cw, const float* cs, int kb) {
    asm volatile("" : "+v"(xo), "+v"(so), "+v"(wo));
    const float swv = sw[(size_t)nblk * KB + kb];
    v4i xb[4][2];
    float sc[4];
#pragma unroll
    for (int h = 0; h < 4; h++) {
#pragma unroll
      for (int t = 0; t < 2; t++) xb[h][t] = *(const v4i*)(cx + xo + (h >> 1) * kW8Tile + (h & 1) * 256 + t * 2048);
      sc[h] = cs[so + 16 * h] * swv;
    }
    auto w_op = [&](v4i* wa, int j) {
#pragma unroll
      for (int t = 0; t < 2; t++) wa[t] = *(const v4i*)(cw + wo + (j >> 1) * kW8Tile + (j & 1) * 256 + t * 2048);
    };
    auto scale_in = [&](const v4i* d, int j) {
#pragma unroll
      for (int h = 0; h < 4; h++)
#pragma unroll
        for (int v = 0; v < 4; v++) acc[j][h][v] = __builtin_fmaf(__int_as_float(d[h][v]) - kMagic, sc[h], acc[j][h][v]);
#pragma unroll
      for (int h = 0; h < 4; h++)
#pragma unroll
        for (int v = 0; v < 4; v++) asm volatile("" : "+v"(acc[j][h][v]));
    };
    v4i wa[2], wn_[2], dp[4];
    w_op(wa, 0);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      asm volatile("" : "+v"(xb[0][0]));
      if (j + 1 < 8) w_op(wn_, j + 1);
      v4i d[4];
#pragma unroll
      for (int h = 0; h < 4; h++) d[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[0], xb[h][0], magic, 0, 0, 0);
#pragma unroll
      for (int h = 0; h < 4; h++) d[h] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[1], xb[h][1], d[h], 0, 0, 0);
      if (j > 0) {
        scale_in(dp, j - 1);
#pragma unroll
        for (int k = 0; k < 8; k++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
#pragma unroll
      for (int h = 0; h < 4; h++) dp[h] = d[h];
      if (j + 1 < 8) {
        wa[0] = wn_[0];
        wa[1] = wn_[1];
      }
    }
    scale_in(dp, 7);
  };

  issue(s_x0, s_w0, s_s0, 0);
  for (int kb = 0; kb < KB; kb += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMAs of block kb have landed
    __syncthreads();                // and the other waves'; all reads of the other stage are done
    if (kb + 1 < KB) issue(s_x1, s_w1, s_s1, kb + 1);
    compute(s_x0, s_w0, s_s0, kb);
    if (kb + 1 < KB) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kb + 2 < KB) issue(s_x0, s_w0, s_s0, kb + 2);
      compute(s_x1, s_w1, s_s1, kb + 1);
    }
  }

  // D[n][m] of sub-tile (j, h): lane 16g + r holds row m = 16h + r, columns 16j + 4g .. +3.
  // The bias values go into registers before the first store: loads and stores share one
  // completion counter, so a load issued after stores would wait for all of them.
  const int m_lo = 256 * tm + 64 * wm + r;
  const int n_lo = 256 * tn + 128 * wn + 4 * g;
  uint2 bv[8];
#pragma unroll
  for (int j = 0; j < 8; j++) bv[j] = bias ? *(const uint2*)(bias + n_lo + 16 * j) : make_uint2(0u, 0u);
  // (one wait for all of them here, rather than one per guarded row group after stores)
#pragma unroll
  for (int j = 0; j < 8; j++) asm volatile("" : "+v"(bv[j].x), "+v"(bv[j].y));
#pragma unroll
  for (int h = 0; h < 4; h++) {
    const int m = m_lo + 16 * h;
    if (m < M) {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float* o = acc[j][h];
        uint2 pk;
        pk.x = pack_bf16x2(o[0] + __uint_as_float(bv[j].x << 16), o[1] + __uint_as_float(bv[j].x & 0xFFFF0000u));
        pk.y = pack_bf16x2(o[2] + __uint_as_float(bv[j].y << 16), o[3] + __uint_as_float(bv[j].y & 0xFFFF0000u));
        *(uint2*)(y + (size_t)m * N + n_lo + 16 * j) = pk;
      }
    }
  }
}

// Tile counts: x rows padded to 256 (the product's row tile), 32-row code tiles.
int w8a8_row_tiles(int M) { return (M + 255) / 256 * 8; }

hipError_t launch_w8a8_quant_act(const void* x, int M, int K, void* x8, void* sx, hipStream_t st) {
  const int MT = w8a8_row_tiles(M), KB = K / 128;
  hipLaunchKernelGGL(w8a8_quant_act_kernel, dim3(MT * KB), dim3(256), 0, st, (const uint16_t*)x, M, K, MT, MT * 32,
                     (int8_t*)x8, (float*)sx);
  return hipGetLastError();
}

hipError_t launch_w8a8_quant_weight(const void* w, int N, int K, void* w8, void* sw, hipStream_t st) {
  const int KB = K / 128;
  hipLaunchKernelGGL(w8a8_quant_weight_kernel, dim3((N / 128) * KB), dim3(256), 0, st, (const uint16_t*)w, K, N / 32, KB,
                     (int8_t*)w8, (float*)sw);
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const void* x8, const void* sx, const void* w8, const void* sw, const void* bias, int M,
                            int N, int K, void* y, hipStream_t st) {
  const int MT = w8a8_row_tiles(M), KB = K / 128, NT = N / 32;
  const int tiles_n = N / 256, tiles = (MT / 8) * tiles_n, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(w8a8_gemm_kernel, dim3(per_xcd * 8), dim3(512), 0, st, (const int8_t*)x8, (const float*)sx,
                     (const int8_t*)w8, (const float*)sw, (const uint16_t*)bias, M, N, KB, MT, NT, MT * 32, tiles_n,
                     tiles, per_xcd, (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace sagesla
