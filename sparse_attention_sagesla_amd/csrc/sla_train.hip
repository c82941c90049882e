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

// registers o .. o+7 of an accumulator as a bf16 operand
__device__ __forceinline__ v8bf pack8v(const v16f& x, int o) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; e++) t[e] = x[o + e];
  return pack8(t);
}

__device__ __forceinline__ v16f mfma(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Head-dim-reduction tiles store the 16-byte chunk of lane l of step s at position
// hd_swz(s, l) of its 64-chunk group (an involution: bits 2 and 3 of l flipped by the
// step's parity and by l / 32). A lane-contiguous operand read stays one permutation of
// a 1 KiB group; the transposing reads below (tokens as the reduction index, taken from
// the same tile) then hit every bank once per half-wave.
__device__ __forceinline__ int hd_swz(int s, int l) { return l ^ (((s & 1) << 2) | ((l >> 5) << 3)); }

// The operand of lane l for head-dim step s of key/query tile tt from an LDS copy of a
// head-dim-reduction tile.
__device__ __forceinline__ v8bf hd_op(const uint16_t* tile, int tt, int s, int l) {
  return *(const v8bf*)(tile + ((tt * 8 + s) * 64 + hd_swz(s, l)) * 8);
}

typedef short v4s_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_* lds_v4s_ptr;

// Byte offsets, within a head-dim-reduction tile in LDS, of the two transposing reads that
// give lane l the token-reduction operand of tile (tt, ct, t) = (0, 0, 0): within each
// 16 lanes (group G = l / 16), lanes 4a + b name channels 16(G % 2) + 4b .. +3 of token
// 4(G / 2) + a (+8 for the second read), and lane j of the group receives channel
// 16(G % 2) + j at those 4 tokens, which is the token-reduction lane order. Tile (tt, ct,
// t) adds tt * 8192 + ct * 2048 + t * 256 bytes.
__device__ __forceinline__ void tok_offsets(int l, uint32_t& o0, uint32_t& o1) {
  const int G = l >> 4, a = (l >> 2) & 3, b = l & 3, sp = G & 1, g = G >> 1, gch = b >> 1;
  const int i0 = 4 * g + a + 32 * gch, i1 = i0 + 8;
  o0 = (uint32_t)((sp * 64 + hd_swz(sp, i0)) * 16 + 8 * (b & 1));
  o1 = (uint32_t)((sp * 64 + hd_swz(sp, i1)) * 16 + 8 * (b & 1));
}

// The token-reduction operands of tiles (tt, ct = 0..3, t) in one block of 8 transposing
// reads, waited for inside it. Written out so that the compiler, which cannot tell which
// LDS object such a read depends on, adds no wait for DMAs still in flight: the caller
// has waited for this tile's copies.
typedef int v2i_ __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void tok_ops4(const uint16_t* tile, uint32_t o0, uint32_t o1, int tt, int t, v8bf (&out)[4]) {
  const uint32_t b = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)tile + tt * 8192 + t * 256;
  v2i_ x[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:6144\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(b + o0), "v"(b + o1)
      : "memory");
#pragma unroll
  for (int ct = 0; ct < 4; ct++) {
    const v4i v = {x[2 * ct][0], x[2 * ct][1], x[2 * ct + 1][0], x[2 * ct + 1][1]};
    out[ct] = __builtin_bit_cast(v8bf, v);
  }
}

__device__ __forceinline__ v8bf tok_op(const uint16_t* tile, uint32_t o0, uint32_t o1, int tt, int ct, int t) {
  const char* b = (const char*)tile + (tt * 8192 + ct * 2048 + t * 256);
  const v4s_ x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(b + o0));
  const v4s_ x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(b + o1));
  const v8s r = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  return __builtin_bit_cast(v8bf, r);
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

// X [BH][N][128] bf16 -> "head-dim-reduction tiles" [BH][Nb][kTrTile]: chunk
// (tt*8 + s)*64 + hd_swz(s, l) holds X[32tt + r][16s + 8g .. +7], the operand order of
// products that reduce over the head dimension, so that one operand is one 1 KiB read
// (tokens past N are 0).
__global__ __launch_bounds__(256) void sla_relayout_hd_kernel(const uint16_t* __restrict__ x, int N, int Nb,
                                                              uint16_t* __restrict__ xh) {
  const int bh = blockIdx.x / Nb, blk = blockIdx.x % Nb, t = threadIdx.x;
  const int n = block_len(blk, N);
  const uint16_t* src = x + ((size_t)bh * N + (size_t)blk * kBlk) * kD;
  uint16_t* dst = xh + ((size_t)bh * Nb + blk) * kTrTile;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int c = t + 256 * k;  // stored position (tt*8 + s)*64 + hd_swz(s, l)
    const int s = (c >> 6) & 7, l = hd_swz(s, c & 63), tt = c >> 9, row = 32 * tt + (l & 31), col = 16 * s + 8 * (l >> 5);
    v4i val = (v4i){0, 0, 0, 0};
    if (row < n) val = *(const v4i*)(src + (size_t)row * kD + col);
    *(v4i*)(dst + (size_t)c * 8) = val;
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
// One workgroup (4 waves) per (head, query block). Wave w = (kh, rg) owns query rows
// 32rg .. +31 (one per lane column) and keys 32kh .. +31 of every kept key block: the two
// key halves run separate online softmaxes, merged at the end. The kept blocks' K
// (head-dim-reduction tiles) and V (token-reduction tiles) arrive by DMA in a two-stage
// LDS ring, one block ahead; each wave copies a quarter of each tile. Per block and wave:
// S^T = K Q^T over its 32 keys, online softmax in the base-2 domain, O^T += V^T P^T.
// Epilogue: O_s (fp32, for the backward's D), lse, and out = O_s + y (bf16).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__global__ __launch_bounds__(256, 2) void sla_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ vt, const int* __restrict__ idx,
                                                         const uint16_t* __restrict__ y, int BH, int N, int Nb, int ksel,
                                                         int per_xcd, uint16_t* __restrict__ out,
                                                         float* __restrict__ os, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[kTrTile];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = w & 1, kh = w >> 1;
  const int l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int qi = kBlk * i + 32 * rg + r;
  const bool qvalid = qi < N;
  const uint16_t* Qh = q + (size_t)bh * N * kD;
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
  // each wave copies a quarter of each 16 KiB tile: 4 DMAs of 1 KiB (16 bytes per lane)
  auto issue = [&](uint16_t* dk_, uint16_t* dv_, int j) {
    const uint16_t* ks = k + ((size_t)bh * Nb + j) * kTrTile + (w * 4 * 64 + l) * 8;
    const uint16_t* vs = vt + ((size_t)bh * Nb + j) * kTrTile + (w * 4 * 64 + l) * 8;
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
      __builtin_amdgcn_global_load_lds((const void*)(ks + cc * 512), (lds_ptr_t)(dk_ + (w * 4 + cc) * 512), 16, 0, 0);
#pragma unroll
    for (int cc = 0; cc < 4; cc++)
      __builtin_amdgcn_global_load_lds((const void*)(vs + cc * 512), (lds_ptr_t)(dv_ + (w * 4 + cc) * 512), 16, 0, 0);
  };
  auto compute = [&](const uint16_t* ck, const uint16_t* cv, int j) {
    const int nj = block_len(j, N);
    if (nj <= 32 * kh) return;  // this wave's key half is past the sequence's end
    v16f acc = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) acc = mfma(hd_op(ck, kh, s, l), qop[s], acc);
    if (__builtin_expect(nj < 32 * kh + 32, 0)) {  // the partial last block: keys past its end drop out
      asm volatile("" ::: "memory");  // a real branch: the masking is not run on full blocks
#pragma unroll
      for (int v = 0; v < 16; v++)
        if (32 * kh + 8 * (v >> 2) + 4 * g + (v & 3) >= nj) acc[v] = -INFINITY;
    }
    // the maximum of the raw products; scaling by c > 0 commutes with it
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; v++) mx = fmaxf(mx, acc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx * c);
    // rescale only when some row of the wave has a new maximum (alpha = 1 exactly otherwise)
    if (__any(mn > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int ct = 0; ct < 4; ct++)
#pragma unroll
        for (int v = 0; v < 16; v++) o[ct][v] *= alpha;
    }
    m = mn;
    float sc[16];
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      sc[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], c, -mn));
      rs += sc[v];
    }
    rs += __shfl_xor(rs, 32);
    lsum += rs;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const v8bf pb = pack8(&sc[8 * t]);
#pragma unroll
      for (int ct = 0; ct < 4; ct++)
        o[ct] = mfma(*(const v8bf*)(cv + ((((kh * 4 + ct) * 2 + t) * 64) + l) * 8), pb, o[ct]);
    }
  };

  issue(sK0, sV0, irow[0]);
  for (int kk = 0; kk < ksel; kk += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMAs of block kk have landed
    __syncthreads();                // and the other waves'; all reads of the other stage are done
    if (kk + 1 < ksel) issue(sK1, sV1, irow[kk + 1]);
    compute(sK0, sV0, irow[kk]);
    if (kk + 1 < ksel) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kk + 2 < ksel) issue(sK0, sV0, irow[kk + 2]);
      compute(sK1, sV1, irow[kk + 1]);
    }
  }

  // merge the two key halves: the kh = 1 waves hand m, the row sum and O^T (in their
  // lane order) to the kh = 0 waves through the ring's memory
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* xo = reinterpret_cast<float*>(rg == 0 ? sK0 : sK1);  // 64 x 64 floats (one K tile)
  float* xm = reinterpret_cast<float*>(rg == 0 ? sV0 : sV1);  // 2 x 64 floats
  if (kh == 1) {
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v = 0; v < 16; v++) xo[(ct * 16 + v) * 64 + l] = o[ct][v];
    xm[l] = m;
    xm[64 + l] = lsum;
  }
  __syncthreads();
  if (kh == 1 || !qvalid) return;
  {
    const float m1 = xm[l], l1 = xm[64 + l];
    const float mt = fmaxf(m, m1);  // m is finite: key half 0 of every kept block has a key
    const float a0 = __builtin_amdgcn_exp2f(m - mt), a1 = __builtin_amdgcn_exp2f(m1 - mt);
    lsum = lsum * a0 + l1 * a1;
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v = 0; v < 16; v++) o[ct][v] = o[ct][v] * a0 + xo[(ct * 16 + v) * 64 + l] * a1;
    m = mt;
  }
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
      *(float4*)(os + rowoff + ch) = make_float4(a[0], a[1], a[2], a[3]);
      uint2 pk;
      pk.x = pack_bf16x2(a[0], a[1]);
      pk.y = pack_bf16x2(a[2], a[3]);
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
// One workgroup (4 waves) per (head, query block). Wave (kt, qh) takes query rows 32qh .. +31
// (one per lane column) against key tile kt (keys 32kt .. +31) of every kept block; P comes
// from the saved lse, so the two key tiles need no exchange until the end, where their dQ
// partial sums are added through LDS. D = rowsum(dO * O_s) first (stored for the dK/dV
// pass). The kept blocks' K and V (head-dim-reduction tiles) and K (token-reduction tiles)
// arrive by DMA in a two-stage LDS ring, one block ahead. Per block and wave:
// S^T = K Q^T, dP^T = V dO^T, dS^T = P^T * (dP^T - D), dQ^T += K^T dS^T.
__global__ __launch_bounds__(256, 2) void sla_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kh,
                                                            const uint16_t* __restrict__ vh,
                                                            const uint16_t* __restrict__ dout, const float* __restrict__ os,
                                                         const float* __restrict__ lse, const int* __restrict__ idx,
                                                         int BH, int N, int Nb, int ksel, int per_xcd,
                                                         float* __restrict__ dsum, float* __restrict__ dq) {
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[kTrTile];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[kTrTile];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int kt = w >> 1, qh = w & 1;
  const int qi = kBlk * i + 32 * qh + r;
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
      const float4 o0 = *(const float4*)(os + e), o1 = *(const float4*)(os + e + 4);
      const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
      for (int x = 0; x < 8; x++) dpart += (float)dop[s][x] * ov[x];
    }
  }
  const float D = dpart + __shfl_xor(dpart, 32);
  const float L = qvalid ? lse[(size_t)bh * N + qi] : 0.f;
  if (qvalid && g == 0 && kt == 0) dsum[(size_t)bh * N + qi] = D;

  v16f acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) acc[ct] = (v16f){};

  const int* irow = idx + ((size_t)bh * Nb + i) * ksel;
  // each wave copies a quarter of each 16 KiB tile: 4 DMAs of 1 KiB
  auto issue = [&](uint16_t* da, uint16_t* db, int j) {
    const size_t to = ((size_t)bh * Nb + j) * kTrTile + (w * 4 * 64 + l) * 8;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
      __builtin_amdgcn_global_load_lds((const void*)(kh + to + cc * 512), (lds_ptr_t)(da + (w * 4 + cc) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vh + to + cc * 512), (lds_ptr_t)(db + (w * 4 + cc) * 512), 16, 0, 0);
    }
  };
  uint32_t to0, to1;
  tok_offsets(l, to0, to1);
  // K^T for dQ comes from the same K tile through transposing reads
  auto compute = [&](const uint16_t* ca, const uint16_t* cb, int j) {
    const int nj = block_len(j, N);
    v16f s_ = (v16f){}, dp = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      s_ = mfma(hd_op(ca, kt, s, l), qop[s], s_);
      dp = mfma(hd_op(cb, kt, s, l), dop[s], dp);
    }
    // rows past the sequence's end have Q = dO = 0 and D = 0, so their dS is 0 without a
    // mask; keys past it (zero rows of the tiles) are masked in the partial last block
    float ds[16];
#pragma unroll
    for (int x = 0; x < 16; x++) ds[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_[x], c, -L)) * (dp[x] - D);
    if (__builtin_expect(nj < kBlk, 0)) {
      asm volatile("" ::: "memory");  // a real branch: the masking is not run on full blocks
#pragma unroll
      for (int x = 0; x < 16; x++)
        if (32 * kt + 8 * (x >> 2) + 4 * g + (x & 3) >= nj) ds[x] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const v8bf bq = pack8(&ds[8 * t]);
#pragma unroll
      for (int ct = 0; ct < 4; ct++) acc[ct] = mfma(tok_op(ca, to0, to1, kt, ct, t), bq, acc[ct]);
    }
  };

  issue(sA0, sB0, irow[0]);
  for (int kk = 0; kk < ksel; kk += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kk + 1 < ksel) issue(sA1, sB1, irow[kk + 1]);
    compute(sA0, sB0, irow[kk]);
    if (kk + 1 < ksel) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kk + 2 < ksel) issue(sA0, sB0, irow[kk + 2]);
      compute(sA1, sB1, irow[kk + 1]);
    }
  }

  // the key-tile-1 waves hand their partial sums to the key-tile-0 waves through LDS
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* red = qh ? (float*)sB0 : (float*)sA0;  // 16 KiB per query half
  if (kt == 1) {
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v = 0; v < 16; v++) red[(ct * 16 + v) * 64 + l] = acc[ct][v];
  }
  __syncthreads();
  if (kt == 1 || !qvalid) return;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v = 0; v < 16; v++) acc[ct][v] += red[(ct * 16 + v) * 64 + l];
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
// One workgroup (8 waves, 2 per SIMD) per (head, key block j). Wave (role, kh, qt) takes keys
// 32kh .. +31 (one per lane column) against query tile qt (rows 32qt .. +31) of every query
// block that keeps j, ascending (from the transposed mask); role 0 accumulates dV, role 1 dK
// (both form S; splitting them halves each wave's accumulators). The two query tiles'
// partial sums are added through LDS at the end. Per query block, its Q and dO
// (head-dim-reduction and token-reduction tiles), lse and D arrive by DMA in a two-stage LDS
// ring, one block ahead. Per block: S = Q K^T (lanes = keys, registers = queries), P from
// lse; role 0: dV^T += dO^T P; role 1: dP = dO V^T, dS = P * (dP - D), dK^T += Q^T dS.
// One ring slot of the dK/dV kernel: a query block's Q and dO head-dim-reduction tiles
// and its lse and D.
constexpr int kMaxMaskWords = 512;  // 32-bit words of a kept-by row: N <= 2^20 tokens

struct DkvSlot {
  uint16_t qh[kTrTile];
  uint16_t dh[kTrTile];
  float L[kBlk];
  float S[kBlk];
};

__device__ __forceinline__ int next_set(const uint32_t* row, int nw, int from) {
  for (int wi = from >> 5; wi < nw; wi++) {
    uint32_t b = row[wi];
    if (wi == (from >> 5)) b &= 0xFFFFFFFFu << (from & 31);
    if (b) return 32 * wi + __builtin_ctz(b);
  }
  return -1;
}

__global__ __launch_bounds__(512) void sla_bwd_dkdv_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                           const uint16_t* __restrict__ qh_, const uint16_t* __restrict__ doh,
                                                           const float* __restrict__ lse, const float* __restrict__ dsum,
                                                           const uint32_t* __restrict__ mask, int BH, int N, int Nb, int nw,
                                                           int per_xcd, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ __attribute__((aligned(1024))) DkvSlot z0, z1, z2, z3;
  __shared__ uint32_t s_mrow[kMaxMaskWords];  // this key block's kept-by row (Nb <= 32 * kMaxMaskWords)
  __shared__ float s_px[4 * 16 * 64];           // P of each (key half, query half), fp32
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, j = tile % Nb;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int role = w >> 2, kh = (w >> 1) & 1, qt = w & 1;
  const int kj = kBlk * j + 32 * kh + r;
  const bool kvalid = kj < N;
  const size_t hoff = (size_t)bh * N * kD;
  const float c = kLog2e * 0.08838834764831845f;

  v8bf kop[8], vop[8];
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const size_t e = hoff + (size_t)kj * kD + 16 * s + 8 * g;
    kop[s] = kvalid ? ld8(k + e) : (v8bf){};
    vop[s] = (kvalid && role == 1) ? ld8(v + e) : (v8bf){};
  }
  v16f acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) acc[ct] = (v16f){};

  const uint32_t* mrow = mask + ((size_t)bh * Nb + j) * nw;
  // per-lane byte offsets kept opaque, so that the DMAs use a scalar base + lane offset;
  // each wave copies an eighth of each 16 KiB tile (2 DMAs of 1 KiB) and the block's lse
  // and D (every wave the same 256 bytes, so that each issues six DMAs per step; rows
  // past N repeat the last row and are never used)
  int lo16 = (w * 2 * 64 + l) * 16, lo4 = l * 4;
  auto issue = [&](DkvSlot& z, int i) {
    asm volatile("" : "+v"(lo16), "+v"(lo4));
    const size_t tb = ((size_t)bh * Nb + i) * kTrTile * 2;  // bytes
    const char* s0 = (const char*)qh_ + tb;
    const char* s1 = (const char*)doh + tb;
#pragma unroll
    for (int cc = 0; cc < 2; cc++) {
      const int ld = (w * 2 + cc) * 512;
      __builtin_amdgcn_global_load_lds((const void*)(s0 + (uint32_t)lo16 + cc * 1024), (lds_ptr_t)(z.qh + ld), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(s1 + (uint32_t)lo16 + cc * 1024), (lds_ptr_t)(z.dh + ld), 16, 0, 0);
    }
    const size_t r0 = (size_t)bh * N + (size_t)kBlk * i;
    const int nrow = min(kBlk, N - kBlk * i);
    const uint32_t off4 = (uint32_t)min(lo4, 4 * (nrow - 1));
    __builtin_amdgcn_global_load_lds((const void*)((const char*)(lse + r0) + off4), (lds_ptr_t)z.L, 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)((const char*)(dsum + r0) + off4), (lds_ptr_t)z.S, 4, 0, 0);
  };
  uint32_t to0, to1;
  tok_offsets(l, to0, to1);
  // Q^T and dO^T (tokens as the reduction index) come from the same tiles through
  // transposing reads
  // The dV waves form S and P; P goes to the dK waves of the same (key half, query half)
  // through LDS (fp32, lane order), so that S is formed once per pair and each wave does
  // 16 products per step. A second barrier per step separates the write from the reads.
  auto compute = [&](const DkvSlot& z, int i) {
    const uint16_t *a = z.qh, *b = z.dh;
    const float *sl = z.L, *ss = z.S;
    const int ni = block_len(i, N);
    float* px = s_px + (kh * 2 + qt) * 16 * 64;
    float p[16];
    v16f dp = (v16f){};
    if (role == 0) {
      v16f s_ = (v16f){};
#pragma unroll
      for (int s = 0; s < 8; s++) s_ = mfma(hd_op(a, qt, s, l), kop[s], s_);
      // registers x hold query rows 32qt + 8(x/4) + 4g + x%4 of the block
#pragma unroll
      for (int x4 = 0; x4 < 4; x4++) {
        const float4 L4 = *(const float4*)(sl + 32 * qt + 8 * x4 + 4 * g);
        const float Lq[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) p[4 * x4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_[4 * x4 + e], c, -Lq[e]));
      }
      if (__builtin_expect(ni < kBlk, 0)) {  // the partial last query block: rows past its end drop out
        asm volatile("" ::: "memory");  // a real branch: the masking is not run on full blocks
#pragma unroll
        for (int x = 0; x < 16; x++)
          if (32 * qt + 8 * (x >> 2) + 4 * g + (x & 3) >= ni) p[x] = 0.f;
      }
#pragma unroll
      for (int x = 0; x < 16; x++) px[x * 64 + l] = p[x];
    } else {
#pragma unroll
      for (int s = 0; s < 8; s++) dp = mfma(hd_op(b, qt, s, l), vop[s], dp);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // P of this step written
    if (role == 1) {
#pragma unroll
      for (int x4 = 0; x4 < 4; x4++) {
        const float4 D4 = *(const float4*)(ss + 32 * qt + 8 * x4 + 4 * g);
        const float Dq[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int x = 4 * x4 + e;
          p[x] = px[x * 64 + l] * (dp[x] - Dq[e]);
        }
      }
    }
    const uint16_t* src = role == 0 ? b : a;  // dO^T for dV, Q^T for dK
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const v8bf pb = pack8(&p[8 * t]);
      v8bf op[4];
      tok_ops4(src, to0, to1, qt, t, op);
#pragma unroll
      for (int ct = 0; ct < 4; ct++) acc[ct] = mfma(op[ct], pb, acc[ct]);
    }
  };

  // Ring of four slots, one LDS object each: step n (the n-th query block that keeps
  // this key block) lives in slot n % 4; at the top of step n the DMAs of steps n + 1
  // and n + 2 (six each) may still be in flight. Past the last step the last block is
  // fetched again into the free slot, so that every step issues six DMAs.
  // the row goes to LDS first: a global load inside the loop would wait for every DMA
  // in flight (loads complete in order)
  for (int e = threadIdx.x; e < nw; e += 512) s_mrow[e] = mrow[e];
  __syncthreads();
  int cnt = 0;
  for (int wi = 0; wi < nw; wi++) cnt += __popc(s_mrow[wi]);
  auto next_blk = [&](int cur) {
    const int nx = next_set(s_mrow, nw, cur + 1);
    return nx < 0 ? cur : nx;
  };
  constexpr int kWaitImm = 12 | (7 << 4) | (15 << 8);  // vmcnt(12)
  int blk[4];
  int ia = 0;
  auto phase = [&](DkvSlot& cur, DkvSlot& prev, int k) {
    __builtin_amdgcn_s_waitcnt(kWaitImm);
    // step's slot complete from every wave; the previous step's slot free. A plain
    // barrier: a fence would wait for every DMA.
    asm volatile("s_barrier" ::: "memory");
    ia = next_blk(ia);
    issue(prev, ia);
    blk[(k + 3) & 3] = ia;
    compute(cur, blk[k]);
  };
  if (cnt > 0) {
    ia = next_set(s_mrow, nw, 0);
    blk[0] = ia;
    issue(z0, ia);
    ia = next_blk(ia);
    blk[1] = ia;
    issue(z1, ia);
    ia = next_blk(ia);
    blk[2] = ia;
    issue(z2, ia);
    int n = 0;
    for (; n + 4 <= cnt; n += 4) {
      phase(z0, z3, 0);
      phase(z1, z0, 1);
      phase(z2, z1, 2);
      phase(z3, z2, 3);
    }
    if (n < cnt) phase(z0, z3, 0);
    if (n + 1 < cnt) phase(z1, z0, 1);
    if (n + 2 < cnt) phase(z2, z1, 2);
  }

  // the query-tile-1 waves hand their partial sums to the query-tile-0 waves through LDS
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // 16 KiB per (role, key half)
  float* red = (float*)(role == 0 ? (kh == 0 ? z0.qh : z0.dh) : (kh == 0 ? z1.qh : z1.dh));
  if (qt == 1) {
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int x = 0; x < 16; x++) red[(ct * 16 + x) * 64 + l] = acc[ct][x];
  }
  __syncthreads();
  if (qt == 1 || !kvalid) return;
  const float sc = role == 1 ? 0.08838834764831845f : 1.f;  // dK carries the 1/sqrt(d) of the scores
  float* row = (role == 1 ? dk : dv) + hoff + (size_t)kj * kD;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * ct + 8 * v4 + 4 * g;
      float a4[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int x = 4 * v4 + e;
        a4[e] = (acc[ct][x] + red[(ct * 16 + x) * 64 + l]) * sc;
      }
      *(float4*)(row + ch) = make_float4(a4[0], a4[1], a4[2], a4[3]);
    }
}

// ------------------------------------------------------------------ backward: linear part
// With phi = softmax over the channels, per query row: u = phi(q) H^c, s = phi(q) . z^c,
// O_l = u / s, y = O_l W. Given dO:
//   dO_l = dO W^T;  du = dO_l / s;  ds = -(dO_l . O_l) / s;
//   dphi(q) = du H^c^T + ds z^c;  dq_l = phi (dphi - phi . dphi);
//   dH^c_i = sum_{rows of i} phi(q)^T du,  dz^c_i = sum phi(q) ds;
//   dH_j = sum of dH^c_i over the query blocks i that leave j out (likewise dz_j);
//   dphi(k_t) = dH_j v_t + dz_j,  dv_l = phi(k_t) dH_j,  dk_l = phi (dphi - phi . dphi);
//   dW = sum over rows of O_l^T dO.
// State layouts: the forward's S^c = [H^c^T ; z^c] (row c < 128 holds H^c[.][c], row 128
// z^c); the gradients dH^c_i and dH_j are stored as R = [dH ; dz] (row a < 128 holds
// dH[a][.], row 128 dz), which the masked complement product treats alike.

constexpr int kSp = 136;  // LDS row pitch (bf16) of a staged 129 x 128 state

__device__ __forceinline__ void stage_state(uint16_t (*dst)[kSp], const uint16_t* src, int t, int nthr) {
  for (int c = t; c < 129 * 16; c += nthr) {
    const int row = c >> 4, col = (c & 15) * 8;
    *(v4i*)&dst[row][col] = *(const v4i*)(src + row * kD + col);
  }
}

// 8 bf16 of column `col` at rows r(e) = base + 8(e/4) + e%4 (e = 0..7) of a staged tile:
// the token-reduction slot order of a 32x32 accumulator, with rows as the reduced index.
__device__ __forceinline__ v8bf lds_col8(const uint16_t (*tile)[kSp], int base, int col) {
  v8s x;
#pragma unroll
  for (int e = 0; e < 8; e++) x[e] = (short)tile[base + 8 * (e >> 2) + (e & 3)][col];
  return __builtin_bit_cast(v8bf, x);
}

// Per (head, query block), lanes = query rows (2 waves x 32). Adds dq_l into dq and writes
// phi(q), du, O_l (bf16, row-major) and ds (fp32) for the state gradients and dW.
// Two waves per SIMD (here and in sla_lin_bwd_k_kernel): left alone, the compiler adds
// accumulation registers beyond 256 per lane and the kernels run one wave per SIMD, 1.0 ms
// more for the two together at the Wan2.1-14B 720p shape.
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void sla_lin_bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ hc,
    const uint16_t* __restrict__ proj, int BH, int N, int Nb, int per_xcd, float* __restrict__ dq,
    uint16_t* __restrict__ phq_o, uint16_t* __restrict__ du_o, float* __restrict__ ds_o,
    uint16_t* __restrict__ ol_o) {
  __shared__ __attribute__((aligned(16))) uint16_t sS[129][kSp];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int qi = kBlk * i + 32 * w + r;
  const bool qvalid = qi < N;
  const size_t rowoff = ((size_t)bh * N + (qvalid ? qi : 0)) * kD;
  stage_state(sS, hc + ((size_t)bh * Nb + i) * kStateElems, threadIdx.x, 128);

  // phi(q) in the operand order (channels 16s + 8g .. +7), and the row's softmax stats
  float x[64];
#pragma unroll
  for (int s = 0; s < 8; s++) {
    const v8bf a = qvalid ? ld8(q + rowoff + 16 * s + 8 * g) : (v8bf){};
#pragma unroll
    for (int e = 0; e < 8; e++) x[8 * s + e] = (float)a[e];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 64; e++) mx = fmaxf(mx, x[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 64; e++) {
    x[e] = __expf(x[e] - mx);
    sum += x[e];
  }
  sum += __shfl_xor(sum, 32);
  const float isum = 1.f / sum;
  v8bf phb[8];
#pragma unroll
  for (int s = 0; s < 8; s++) {
    float t8[8];
#pragma unroll
    for (int e = 0; e < 8; e++) t8[e] = x[8 * s + e] * isum;
    phb[s] = pack8(t8);
    if (qvalid) *(v8bf*)(phq_o + rowoff + 16 * s + 8 * g) = phb[s];
  }
  __syncthreads();

  // u^T = S^c phi^T and dO_l^T = W dO^T (lanes = rows, registers = channels c)
  v16f u[4], dl[4];
  float zpart = 0.f;
#pragma unroll
  for (int s = 0; s < 8; s++) {
#pragma unroll
    for (int e = 0; e < 8; e++) zpart += bf16_to_f32(sS[128][16 * s + 8 * g + e]) * (float)phb[s][e];
  }
  const float sden = zpart + __shfl_xor(zpart, 32);
  v8bf dob[8];
#pragma unroll
  for (int s = 0; s < 8; s++) dob[s] = qvalid ? ld8(dout + rowoff + 16 * s + 8 * g) : (v8bf){};
#pragma unroll
  for (int ct = 0; ct < 4; ct++) {
    u[ct] = (v16f){};
    dl[ct] = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      u[ct] = mfma(*(const v8bf*)&sS[32 * ct + r][16 * s + 8 * g], phb[s], u[ct]);
      dl[ct] = mfma(ld8(proj + (32 * ct + r) * kD + 16 * s + 8 * g), dob[s], dl[ct]);
    }
  }
  const float is = 1.f / sden;
  float dpart = 0.f;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v = 0; v < 16; v++) {
      u[ct][v] *= is;  // O_l
      dpart += dl[ct][v] * u[ct][v];
    }
  const float dsv = -(dpart + __shfl_xor(dpart, 32)) * is;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v = 0; v < 16; v++) dl[ct][v] *= is;  // du
  if (qvalid) {
    if (g == 0) ds_o[(size_t)bh * N + qi] = dsv;
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int ch = 32 * ct + 8 * v4 + 4 * g;
        uint2 a, b;
        a.x = pack_bf16x2(u[ct][4 * v4], u[ct][4 * v4 + 1]);
        a.y = pack_bf16x2(u[ct][4 * v4 + 2], u[ct][4 * v4 + 3]);
        b.x = pack_bf16x2(dl[ct][4 * v4], dl[ct][4 * v4 + 1]);
        b.y = pack_bf16x2(dl[ct][4 * v4 + 2], dl[ct][4 * v4 + 3]);
        *(uint2*)(ol_o + rowoff + ch) = a;
        *(uint2*)(du_o + rowoff + ch) = b;
      }
  }

  // dphi^T[a][q] = sum_c H^c[a][c] du[q][c] + ds z^c[a]: A = S^c read down its columns,
  // B = du in the accumulator's own register order
  v16f dp[4];
#pragma unroll
  for (int at = 0; at < 4; at++) {
    dp[at] = (v16f){};
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int t = 0; t < 2; t++)
        dp[at] = mfma(lds_col8(sS, 32 * ct + 16 * t + 4 * g, 32 * at + r), pack8v(dl[ct], 8 * t), dp[at]);
  }
  // phi(q) at the accumulator's channels a = 32at + 8(v/4) + 4g + v%4, then dq_l
  float ph[4][16], dot = 0.f;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * at + 8 * v4 + 4 * g;
      const uint2 raw = qvalid ? *(const uint2*)(q + rowoff + ch) : make_uint2(0u, 0u);
      const float f[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                          __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u)};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int v = 4 * v4 + e;
        ph[at][v] = __expf(f[e] - mx) * isum;
        dp[at][v] += dsv * bf16_to_f32(sS[128][ch + e]);
        dot += ph[at][v] * dp[at][v];
      }
    }
  dot += __shfl_xor(dot, 32);
  if (!qvalid) return;
  float* drow = dq + rowoff;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * at + 8 * v4 + 4 * g;
      float4 o = *(float4*)(drow + ch);
      o.x += ph[at][4 * v4] * (dp[at][4 * v4] - dot);
      o.y += ph[at][4 * v4 + 1] * (dp[at][4 * v4 + 1] - dot);
      o.z += ph[at][4 * v4 + 2] * (dp[at][4 * v4 + 2] - dot);
      o.w += ph[at][4 * v4 + 3] * (dp[at][4 * v4 + 3] - dot);
      *(float4*)(drow + ch) = o;
    }
}

// Per (head, 16 consecutive query blocks): R_i = [dH^c_i ; dz^c_i] (bf16) for each block and
// their fp32 sum (the chunk's partial of the total). Wave w owns channels a = 32w .. +31:
// D[c][a] = sum_t du[t][c] phi[t][a] on the token-reduction tiles of du and phi; the ds
// row enters as a fifth tile whose only non-zero row is c = 0.
__global__ __launch_bounds__(256) void sla_lin_dhc_kernel(const uint16_t* __restrict__ phqt,
                                                          const uint16_t* __restrict__ dut,
                                                          const float* __restrict__ ds, int BH, int N, int Nb,
                                                          uint16_t* __restrict__ rs, float* __restrict__ rpart) {
  const int nc = (Nb + kChunk - 1) / kChunk;
  const int bh = blockIdx.x / nc, chunk = blockIdx.x % nc;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  v16f cs[5];
#pragma unroll
  for (int ct = 0; ct < 5; ct++) cs[ct] = (v16f){};
  const int i0 = chunk * kChunk, i1 = min(Nb, i0 + kChunk);
  for (int i = i0; i < i1; i++) {
    const size_t tb = ((size_t)bh * Nb + i) * kTrTile + l * 8;
    v16f acc[5];
#pragma unroll
    for (int ct = 0; ct < 5; ct++) acc[ct] = (v16f){};
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const v8bf b = ld8(phqt + tb + ((tt * 4 + w) * 2 + t) * 512);
#pragma unroll
        for (int ct = 0; ct < 4; ct++) acc[ct] = mfma(ld8(dut + tb + ((tt * 4 + ct) * 2 + t) * 512), b, acc[ct]);
        float dv8[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int tok = kBlk * i + 32 * tt + 16 * t + 8 * (e >> 2) + 4 * g + (e & 3);
          dv8[e] = (r == 0 && tok < N) ? ds[(size_t)bh * N + tok] : 0.f;
        }
        acc[4] = mfma(pack8(dv8), b, acc[4]);
      }
    // D[c][a]: lane = a (32w + r), registers = c rows 32ct + 8(v/4) + 4g + v%4: four
    // consecutive c per 8-byte store
    uint16_t* R = rs + ((size_t)bh * Nb + i) * kStateElems;
    const int a = 32 * w + r;
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int c = 32 * ct + 8 * v4 + 4 * g;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[ct][4 * v4]) | ((uint32_t)f32_to_bf16(acc[ct][4 * v4 + 1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[ct][4 * v4 + 2]) | ((uint32_t)f32_to_bf16(acc[ct][4 * v4 + 3]) << 16);
        *(uint2*)(R + a * kD + c) = pk;
#pragma unroll
        for (int e = 0; e < 4; e++) cs[ct][4 * v4 + e] += acc[ct][4 * v4 + e];
      }
    if (g == 0) R[kD * kD + a] = f32_to_bf16(acc[4][0]);
    cs[4][0] += acc[4][0];
  }
  float* P = rpart + ((size_t)bh * nc + chunk) * kStateElems;
  const int a = 32 * w + r;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++)
      *(float4*)(P + a * kD + 32 * ct + 8 * v4 + 4 * g) =
          make_float4(cs[ct][4 * v4], cs[ct][4 * v4 + 1], cs[ct][4 * v4 + 2], cs[ct][4 * v4 + 3]);
  if (g == 0) P[kD * kD + a] = cs[4][0];
}

// Per (bh, group of kGroup key blocks): the ascending union of the query blocks that keep
// any key block of the group (or, complement != 0, that leave it out), and one bit row per
// key block over the union positions, in the layout of the forward's union lists, from the
// transposed kept mask.
__global__ __launch_bounds__(256) void sla_union_t_kernel(const uint32_t* __restrict__ mask, int Nb, int nw, int ng,
                                                          int complement, int32_t* __restrict__ ulist,
                                                          uint32_t* __restrict__ umask, int32_t* __restrict__ ucount) {
  extern __shared__ uint32_t sh[];  // U[nw], base[nw + 1]
  uint32_t* U = sh;
  uint32_t* base = sh + nw;
  const int bh = blockIdx.x / ng, grp = blockIdx.x % ng;
  const int t = threadIdx.x, j = grp * kGroup + t;
  const bool jv = j < Nb;
  const uint32_t* row = mask + ((size_t)bh * Nb + (jv ? j : 0)) * nw;
  auto bits_of = [&](int wi) -> uint32_t {
    uint32_t b = jv ? row[wi] : 0u;
    if (complement && jv) {
      b = ~b;
      const int lo = 32 * wi;
      if (lo + 32 > Nb) b &= (Nb - lo) >= 32 ? 0xFFFFFFFFu : ((1u << (Nb - lo)) - 1u);
    }
    return b;
  };
  for (int wi = t; wi < nw; wi += 256) U[wi] = 0u;
  __syncthreads();
  for (int wi = 0; wi < nw; wi++) {
    const uint32_t b = bits_of(wi);
    if (b) atomicOr(&U[wi], b);
  }
  __syncthreads();
  if (t == 0) {
    uint32_t acc = 0;
    for (int wi = 0; wi < nw; wi++) {
      base[wi] = acc;
      acc += __popc(U[wi]);
    }
    base[nw] = acc;
    ucount[(size_t)bh * ng + grp] = (int32_t)acc;
  }
  __syncthreads();
  int32_t* ul = ulist + ((size_t)bh * ng + grp) * Nb;
  for (int wi = t; wi < nw; wi += 256) {
    uint32_t b = U[wi];
    int p = (int)base[wi];
    while (b) {
      ul[p++] = 32 * wi + __builtin_ctz(b);
      b &= b - 1;
    }
  }
  // this key block's bit row over the union positions, one 32-position word at a time
  uint32_t* um = umask + ((size_t)bh * ng + grp) * (size_t)nw * kGroup;
  const int total = (int)base[nw];
  uint32_t word = 0u;
  int p = 0;
  for (int wi = 0; wi < nw; wi++) {
    uint32_t b = U[wi];
    const uint32_t mine = bits_of(wi);
    while (b) {
      const uint32_t low = b & (0u - b);
      if (mine & low) word |= 1u << (p & 31);
      b &= b - 1;
      if ((++p & 31) == 0) {
        um[(size_t)((p >> 5) - 1) * kGroup + t] = word;
        word = 0u;
      }
    }
  }
  if (p & 31) um[(size_t)(p >> 5) * kGroup + t] = word;
  for (int pw = (total + 31) / 32; pw < nw; pw++) um[(size_t)pw * kGroup + t] = 0u;
}

// Per (head, key block), lanes = keys (2 waves x 32): adds dk_l and dv_l from R_j = [dH_j ; dz_j].
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void sla_lin_bwd_k_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const uint16_t* __restrict__ rj, int BH, int N,
    int Nb, int per_xcd, float* __restrict__ dk, float* __restrict__ dv) {
  __shared__ __attribute__((aligned(16))) uint16_t sR[129][kSp];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= BH * Nb) return;
  const int bh = tile / Nb, j = tile % Nb;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int kj = kBlk * j + 32 * w + r;
  const bool kvalid = kj < N;
  const size_t rowoff = ((size_t)bh * N + (kvalid ? kj : 0)) * kD;
  stage_state(sR, rj + ((size_t)bh * Nb + j) * kStateElems, threadIdx.x, 128);
  v8bf vb[8];
#pragma unroll
  for (int s = 0; s < 8; s++) vb[s] = kvalid ? ld8(v + rowoff + 16 * s + 8 * g) : (v8bf){};
  // phi(k) at the accumulator's channels a = 32at + 8(v/4) + 4g + v%4
  float ph[4][16];
  float mx = -INFINITY;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const uint2 raw = kvalid ? *(const uint2*)(k + rowoff + 32 * at + 8 * v4 + 4 * g) : make_uint2(0u, 0u);
      ph[at][4 * v4] = __uint_as_float(raw.x << 16);
      ph[at][4 * v4 + 1] = __uint_as_float(raw.x & 0xFFFF0000u);
      ph[at][4 * v4 + 2] = __uint_as_float(raw.y << 16);
      ph[at][4 * v4 + 3] = __uint_as_float(raw.y & 0xFFFF0000u);
#pragma unroll
      for (int e = 0; e < 4; e++) mx = fmaxf(mx, ph[at][4 * v4 + e]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sum = 0.f;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int x = 0; x < 16; x++) {
      ph[at][x] = __expf(ph[at][x] - mx);
      sum += ph[at][x];
    }
  sum += __shfl_xor(sum, 32);
  const float isum = 1.f / sum;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int x = 0; x < 16; x++) ph[at][x] *= isum;
  __syncthreads();

  // dphi^T[a][t] = sum_c dH[a][c] v[t][c] + dz[a]
  v16f dp[4];
  float dot = 0.f;
#pragma unroll
  for (int at = 0; at < 4; at++) {
    dp[at] = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) dp[at] = mfma(*(const v8bf*)&sR[32 * at + r][16 * s + 8 * g], vb[s], dp[at]);
#pragma unroll
    for (int x = 0; x < 16; x++) {
      dp[at][x] += bf16_to_f32(sR[128][32 * at + 8 * (x >> 2) + 4 * g + (x & 3)]);
      dot += ph[at][x] * dp[at][x];
    }
  }
  dot += __shfl_xor(dot, 32);
  // dv_l^T[c][t] = sum_a dH[a][c] phi[t][a]: A = R read down its columns, B = phi in the
  // accumulator's register order
  v16f dva[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) {
    dva[ct] = (v16f){};
#pragma unroll
    for (int at = 0; at < 4; at++)
#pragma unroll
      for (int t = 0; t < 2; t++)
        dva[ct] = mfma(lds_col8(sR, 32 * at + 16 * t + 4 * g, 32 * ct + r), pack8(&ph[at][8 * t]), dva[ct]);
  }
  if (!kvalid) return;
  float* krow = dk + rowoff;
  float* vrow = dv + rowoff;
#pragma unroll
  for (int at = 0; at < 4; at++)
#pragma unroll
    for (int v4 = 0; v4 < 4; v4++) {
      const int ch = 32 * at + 8 * v4 + 4 * g;
      float4 o = *(float4*)(krow + ch);
      o.x += ph[at][4 * v4] * (dp[at][4 * v4] - dot);
      o.y += ph[at][4 * v4 + 1] * (dp[at][4 * v4 + 1] - dot);
      o.z += ph[at][4 * v4 + 2] * (dp[at][4 * v4 + 2] - dot);
      o.w += ph[at][4 * v4 + 3] * (dp[at][4 * v4 + 3] - dot);
      *(float4*)(krow + ch) = o;
      float4 p = *(float4*)(vrow + ch);
      p.x += dva[at][4 * v4];
      p.y += dva[at][4 * v4 + 1];
      p.z += dva[at][4 * v4 + 2];
      p.w += dva[at][4 * v4 + 3];
      *(float4*)(vrow + ch) = p;
    }
}

// dW partial sums: workgroup p adds O_l^T dO over its share of the (head, block) pairs;
// wave w owns rows c = 32w .. +31 of dW. Then one pass adds the partials.
constexpr int kDwParts = 1024;

__global__ __launch_bounds__(256) void sla_dw_partial_kernel(const uint16_t* __restrict__ olt,
                                                             const uint16_t* __restrict__ dot_, int nblocks,
                                                             float* __restrict__ part) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int per = (nblocks + kDwParts - 1) / kDwParts;
  const int b0 = blockIdx.x * per, b1 = min(nblocks, b0 + per);
  v16f acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ct++) acc[ct] = (v16f){};
  for (int b = b0; b < b1; b++) {
    const size_t tb = (size_t)b * kTrTile + l * 8;
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const v8bf a = ld8(olt + tb + ((tt * 4 + w) * 2 + t) * 512);
#pragma unroll
        for (int ct = 0; ct < 4; ct++) acc[ct] = mfma(a, ld8(dot_ + tb + ((tt * 4 + ct) * 2 + t) * 512), acc[ct]);
      }
  }
  // D[c][c']: row c = 32w + 8(v/4) + 4g + v%4, column c' = 32ct + r
  float* P = part + (size_t)blockIdx.x * kD * kD;
#pragma unroll
  for (int ct = 0; ct < 4; ct++)
#pragma unroll
    for (int v = 0; v < 16; v++) P[(32 * w + 8 * (v >> 2) + 4 * g + (v & 3)) * kD + 32 * ct + r] = acc[ct][v];
}

__global__ __launch_bounds__(256) void sla_dw_reduce_kernel(const float* __restrict__ part, float* __restrict__ dw) {
  const int e = blockIdx.x * 256 + threadIdx.x;  // kD * kD elements
  float s = 0.f;
  for (int p = 0; p < kDwParts; p++) s += part[(size_t)p * kD * kD + e];
  dw[e] = s;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_sla_relayout(const void* x, int BH, int N, int Nb, void* xt, hipStream_t st) {
  hipLaunchKernelGGL(sla_relayout_kernel, dim3(BH * Nb), dim3(256), 0, st, (const uint16_t*)x, N, Nb, (uint16_t*)xt);
  return hipGetLastError();
}

hipError_t launch_sla_relayout_hd(const void* x, int BH, int N, int Nb, void* xh, hipStream_t st) {
  hipLaunchKernelGGL(sla_relayout_hd_kernel, dim3(BH * Nb), dim3(256), 0, st, (const uint16_t*)x, N, Nb,
                     (uint16_t*)xh);
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
  hipLaunchKernelGGL(sla_fwd_kernel, dim3(per_xcd * 8), dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)vt, (const int*)idx, (const uint16_t*)y, BH, N, Nb, ksel, per_xcd,
                     (uint16_t*)out, (float*)os, (float*)lse);
  return hipGetLastError();
}

hipError_t launch_sla_bwd_dq(const void* q, const void* kh, const void* vh, const void* dout,
                             const void* os, const void* lse, const void* idx, int BH, int N, int Nb, int ksel,
                             void* dsum, void* dq, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sla_bwd_dq_kernel, dim3(per_xcd * 8), dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)kh,
                     (const uint16_t*)vh, (const uint16_t*)dout, (const float*)os,
                     (const float*)lse, (const int*)idx, BH, N, Nb, ksel, per_xcd, (float*)dsum, (float*)dq);
  return hipGetLastError();
}

hipError_t launch_sla_bwd_dkdv(const void* k, const void* v, const void* qh, const void* doh,
                               const void* lse, const void* dsum, const void* mask, int BH, int N,
                               int Nb, void* dk, void* dv, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8, nw = (Nb + 31) / 32;
  hipLaunchKernelGGL(sla_bwd_dkdv_kernel, dim3(per_xcd * 8), dim3(512), 0, st, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)qh, (const uint16_t*)doh, (const float*)lse, (const float*)dsum, (const uint32_t*)mask, BH, N, Nb, nw,
                     per_xcd, (float*)dk, (float*)dv);
  return hipGetLastError();
}

hipError_t launch_sla_lin_bwd_q(const void* q, const void* dout, const void* hc, const void* proj, int BH, int N,
                                int Nb, void* dq, void* phq, void* du, void* ds, void* ol, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sla_lin_bwd_q_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const uint16_t*)q,
                     (const uint16_t*)dout, (const uint16_t*)hc, (const uint16_t*)proj, BH, N, Nb, per_xcd,
                     (float*)dq, (uint16_t*)phq, (uint16_t*)du, (float*)ds, (uint16_t*)ol);
  return hipGetLastError();
}

hipError_t launch_sla_lin_dhc(const void* phqt, const void* dut, const void* ds, int BH, int N, int Nb, void* rs,
                              void* rpart, hipStream_t st) {
  const int nc = (Nb + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(sla_lin_dhc_kernel, dim3(BH * nc), dim3(256), 0, st, (const uint16_t*)phqt,
                     (const uint16_t*)dut, (const float*)ds, BH, N, Nb, (uint16_t*)rs, (float*)rpart);
  return hipGetLastError();
}

hipError_t launch_sla_union_t(const void* mask, int BH, int Nb, int ksel, void* ulist, void* umask, void* ucount,
                              hipStream_t st) {
  const int nw = (Nb + 31) / 32, ng = (Nb + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(sla_union_t_kernel, dim3(BH * ng), dim3(256), (2 * nw + 1) * sizeof(uint32_t), st,
                     (const uint32_t*)mask, Nb, nw, ng, 2 * ksel > Nb ? 1 : 0, (int32_t*)ulist, (uint32_t*)umask,
                     (int32_t*)ucount);
  return hipGetLastError();
}

hipError_t launch_sla_lin_bwd_k(const void* k, const void* v, const void* rj, int BH, int N, int Nb, void* dk,
                                void* dv, hipStream_t st) {
  const int tiles = BH * Nb, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sla_lin_bwd_k_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const uint16_t*)k,
                     (const uint16_t*)v, (const uint16_t*)rj, BH, N, Nb, per_xcd, (float*)dk, (float*)dv);
  return hipGetLastError();
}

hipError_t launch_sla_dw(const void* olt, const void* dot, int nblocks, void* part, void* dw, hipStream_t st) {
  hipLaunchKernelGGL(sla_dw_partial_kernel, dim3(kDwParts), dim3(256), 0, st, (const uint16_t*)olt,
                     (const uint16_t*)dot, nblocks, (float*)part);
  hipLaunchKernelGGL(sla_dw_reduce_kernel, dim3(kD * kD / 256), dim3(256), 0, st, (const float*)part, (float*)dw);
  return hipGetLastError();
}

int sla_dw_parts() { return kDwParts; }

hipError_t launch_sla_zero(void* p, size_t words, hipStream_t st) {
  const int blocks = (int)((words + 255) / 256 < 65536 ? (words + 255) / 256 : 65536);
  hipLaunchKernelGGL(sla_fill_kernel, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, words);
  return hipGetLastError();
}

}  // namespace sagesla

