// Block-sparse quantized attention over the kept key blocks, with the fused epilogue
// out = O_s + y (y = O_l W_proj from the linear branch, optional).
//
// SLA computes only the top ~10 % of block pairs exactly and skips about 90 % of the
// work (TurboDiffusion explainer, news.qq.com, "First key: attention"); SageAttention
// runs that exact part on 8-bit data at the matrix cores' 8-bit peak (same section).
// Here QK^T is INT8 MFMA (v_mfma_i32_32x32x32_i8) and PV is FP8 e4m3 MFMA
// (v_mfma_f32_32x32x64_f8f6f4), with the online softmax in fp32 registers.
//
// Per query block i (64 rows) and kept key block j, for each row:
//   S = q8 . k8 (int32), a = (s_q[i] * s_k[j]) * c0 with c0 = fp32(log2(e)/sqrt(d)),
//   the reference m' = max(m, ceil(max float(S)*a)) (an integer, in log2 units: it moves
//   less often than the maximum itself, and each move is an exact power of two),
//   alpha = 2^(m - m'),
//   P8 = e4m3(2^x) with x = fma(F, a, c), F = 1.5*2^23 + S (exact in fp32) and
//        c = (log2(448) - m') - fp32(1.5*2^23 * a): 448 * 2^(S a - m') up to the fp32
//        roundings of c and of the fused product,
//   l = l*alpha + sum P8, acc = acc*alpha + P8 . V8   (l on the matrix cores too).
// Epilogue: O = acc * s_v / l (+ y), rounded to bf16: the average of the dequantized V
// rows weighted by the FP8 probabilities actually used. Kept blocks arrive best first.
//
// The integer products are accumulated on top of the bit pattern of 1.5*2^23, so the
// accumulator, read as fp32, already is 1.5*2^23 + S: the exponent needs no int->float
// conversion, and the row maximum is taken on the integers (the map is monotone).
//
// Work split: one workgroup of 2 waves per (bh, query block i); wave w owns query rows
// 32w..32w+31 (one query per lane pair l, l^32) and keeps everything in VGPRs, so two
// workgroups' waves share each SIMD. The K and V code tiles of the kept blocks go through
// a two-slot LDS ring, filled by direct global-to-LDS loads (wave 0 the K tiles, wave 1
// the V tiles) two blocks ahead for K and one for V, with one barrier per block.
// The loop is software pipelined: while the VALU computes the softmax of block u, the
// matrix cores run the PV product (and row sums) of block u - 1 and the QK^T product of
// block u + 1. These MFMAs are placed one or two at a time between groups of the
// softmax's exponentials, so that the VALU and the matrix cores work side by side.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace sagesla {

// Every rounding of the exponent's bias (c below) decides FP8 codes, so no multiply-add
// may be contracted into one rounding in this file.
#pragma clang fp contract(off)

constexpr float kLog2_448 = 8.807354922057604f;  // fp32(log2(448))
constexpr float kMagicF = 12582912.0f;           // 1.5 * 2^23
constexpr int kMagicI = 0x4B400000;              // its bit pattern

// c0 = fp32(log2(e) / sqrt(d)), rounded once from double; a compile-time constant, so that
// the loop holds no kernel argument it would have to reload (sqrt(128) as a double literal,
// checked against the library's sqrt at launch)
constexpr double kSqrtD = 11.313708498984760390;
constexpr float kC0 = (float)(1.4426950408889634 / kSqrtD);
static bool c0_matches() { return kC0 == (float)(1.4426950408889634 / sqrt((double)kD)) && kSqrtD == sqrt((double)kD); }

__device__ __forceinline__ int key_of_slot(int g, int t, int v) { return 32 * t + 8 * (v >> 2) + 4 * g + (v & 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format, no swizzle).
constexpr int kBufWord3 = 0x00020000;

// 1 KiB part n of an 8 KiB code tile (buffer offset soff + lane offset) into bytes
// n KiB .. of the LDS tile. The immediate offset stays 0: with LDS as the destination it
// would move the LDS address as well.
template <int N>
__device__ __forceinline__ void dma_part(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t lo, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + N * 1024), 16, lo, soff + N * 1024, 0, 0);
}

// Online-softmax state of the wave's 32 queries.
struct RowAcc {
  float m;      // reference: running max of S * a, rounded up to an integer
  v16f acc[4];  // O^T accumulators (4 tiles of 32 channels)
  v4f lacc;     // running row sums: lanes 0..15, element 0 (query l), 1 (query l + 16)
};

// LDS operand reads (lane-contiguous 16-byte rows: conflict-free)
__device__ __forceinline__ v4i k_op(const uint8_t* kt, int m, int l) {
  // QK^T product m of a block: key tile tt = m & 1, step s = m >> 1
  return *(const v4i*)(kt + (((m & 1) * 4 + (m >> 1)) * 64 + l) * 16);
}
__device__ __forceinline__ v8i v_op(const uint8_t* vt, int d, int l) {
  const v4i lo = *(const v4i*)(vt + ((2 * d) * 64 + l) * 16);
  const v4i hi = *(const v4i*)(vt + ((2 * d + 1) * 64 + l) * 16);
  return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The MFMA schedule of one block's softmax, as 13 slots issued between its 8 groups of
// exponentials: slots 0..3 the PV products of the previous block (channel tiles d), slot
// 4 its row sums (P8 as the B operand of a 16x16x128 product whose A operand selects, in
// rows 0 and 1, the key ranges that belong to queries 0..15 and 16..31), slots 5..12 the
// QK^T products of the next block (its two key tiles interleaved, so neighbouring
// products are independent). Group g is followed by the slots in kSlotBegin[g] ..
// kSlotBegin[g + 1] - 1.
constexpr int kSlotBegin[9] = {0, 1, 2, 3, 4, 6, 8, 10, 12};

struct Pipe {
  const uint8_t* vt;  // V tile of the previous block (LDS)
  const uint8_t* kt;  // K tile of the next block (LDS)
  v8i vop[4];         // V operands, all read at the start of the block
  v4i kop[8];         // K operands, likewise
};

template <int SLOT, bool PV>
__device__ __forceinline__ void slot(Pipe& pp, RowAcc& st, const v8i& pprev, const v8i& lsel, v16i (&Sn)[2],
                                     const v4i (&q)[4], const v16i& magic) {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SLOT < 4) {
    if constexpr (PV)
      st.acc[SLOT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pp.vop[SLOT], pprev, st.acc[SLOT], 0, 0, 0, 0, 0, 0);
  } else if constexpr (SLOT == 4) {
    if constexpr (PV) st.lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, pprev, st.lacc, 0, 0, 0, 0, 0, 0);
  } else {
    constexpr int m = SLOT - 5, tt = m & 1, s = m >> 1;
    if constexpr (s == 0)
      Sn[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(pp.kop[m], q[0], magic, 0, 0, 0);
    else
      Sn[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(pp.kop[m], q[s], Sn[tt], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int G, bool PV>
__device__ __forceinline__ void slots_after(Pipe& pp, RowAcc& st, const v8i& pprev, const v8i& lsel, v16i (&Sn)[2],
                                            const v4i (&q)[4], const v16i& magic) {
  if constexpr (kSlotBegin[G] + 0 < kSlotBegin[G + 1]) slot<kSlotBegin[G] + 0, PV>(pp, st, pprev, lsel, Sn, q, magic);
  if constexpr (kSlotBegin[G] + 1 < kSlotBegin[G + 1]) slot<kSlotBegin[G] + 1, PV>(pp, st, pprev, lsel, Sn, q, magic);
}

// One block: the online softmax of the wave's 32 rows (scores S, biased integers; keys
// masked out hold 0, below every biased score) -> the FP8 probabilities in the B-operand
// layout of O^T = V8^T P8^T, with the previous block's PV products and the next block's
// QK^T products issued between the exponential groups. The rescale of the accumulators
// by alpha comes last, after the previous block's PV products have been added: those
// products were taken against the previous maximum too.
template <bool PV>
__device__ __forceinline__ v8i block_step(v16i (&S)[2], RowAcc& st, float a, float ba, bool partial, int nlast, int g,
                                          int l, Pipe& pp, const v8i& pprev, const v8i& lsel, v16i (&Sn)[2],
                                          const v4i (&q)[4], const v16i& magic) {
  // every MFMA operand of the block, read from LDS before the row maximum: the LDS
  // latency is then covered by the maximum and the first exponential groups
  if constexpr (PV) {
#pragma unroll
    for (int d = 0; d < 4; d++) pp.vop[d] = v_op(pp.vt, d, l);
  }
#pragma unroll
  for (int m = 0; m < 8; m++) pp.kop[m] = k_op(pp.kt, m, l);
  // The partial last block: keys at or past nlast take no part. Their scores are set to
  // 0 before the maximum, and their FP8 weights to zero after the exponentials.
  if (partial) {
    // key_of_slot(g, ...) >= nlast against the lane's bound, formed here: hoisted out of
    // the loop, the 32 comparisons would hold 64 scalar registers for the whole kernel
    int thr = nlast - 4 * g;
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int v = 0; v < 16; v++)
        if (key_of_slot(0, tt, v) >= thr) S[tt][v] = 0;
  }
  int mx = 0;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int v = 0; v < 16; v++) mx = max(mx, S[tt][v]);
  {
    // the builtin returns unsigned lanes: compare as signed
    auto sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = max((int)sw[0], (int)sw[1]);
  }
  // float(S_max) = F_max - 1.5*2^23 exactly; the reference is its product with a rounded
  // up to an integer, never below the previous one
  const float mold = st.m;
  // (a plain v_max_f32: both operands are canonical, so fmaxf's quieting of mold, a loop
  // value the compiler cannot prove canonical, would only cost an instruction)
  float mn;
  asm("v_max_f32 %0, %1, %2" : "=v"(mn) : "v"(mold), "v"(__builtin_ceilf((__int_as_float(mx) - kMagicF) * a)));
  const bool moved = __builtin_amdgcn_ballot_w64(mn > mold) != 0;
  st.m = mn;
  // exponentials and FP8 packing, 4 scores per group. For the row maximum the fused
  // product may land a few ulps above log2(448); the FP8 conversion saturates
  // (448, 464] to 448.
  const float c = (kLog2_448 - mn) - ba;
  v8i pb;
#define SAGESLA_EXP(G)                                                                                   \
  {                                                                                                      \
    const int tt = (G) >> 2, v4 = (G) & 3;                                                               \
    float p[4];                                                                                          \
    _Pragma("unroll") for (int e = 0; e < 4; e++) p[e] =                                                 \
        __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(S[tt][4 * v4 + e]), a, c));                 \
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);                   \
    pb[G] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);                                       \
  }                                                                                                      \
  slots_after<G, PV>(pp, st, pprev, lsel, Sn, q, magic);
  SAGESLA_EXP(0)
  SAGESLA_EXP(1)
  SAGESLA_EXP(2)
  SAGESLA_EXP(3)
  SAGESLA_EXP(4)
  SAGESLA_EXP(5)
  SAGESLA_EXP(6)
  SAGESLA_EXP(7)
#undef SAGESLA_EXP
  slot<12, PV>(pp, st, pprev, lsel, Sn, q, magic);
  if (partial) {
    int thr = nlast - 4 * g;
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        uint32_t keep = 0u;
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (key_of_slot(0, tt, 4 * v4 + e) < thr) keep |= 0xFFu << (8 * e);
        pb[4 * tt + v4] &= (int)keep;
      }
  }
  // rescale only when some row's reference moved (alpha == 1 otherwise; a power of two)
  if (moved) {
    const float alpha = __builtin_amdgcn_exp2f(mold - mn);
#pragma unroll
    for (int d = 0; d < 4; d++) st.acc[d] *= alpha;
    // lane j < 16 holds the sums of queries j (element 0) and j + 16 (element 1)
    const float alpha_hi = __shfl(alpha, (__lane_id() & 15) + 16);
    st.lacc[0] *= alpha;
    st.lacc[1] *= alpha_hi;
  }
  return pb;
}

// One workgroup of 2 waves per (bh, query block i); wave w owns query rows 32w..32w+31.
// Block u of the kept list: at the top of its step (after the barrier) wave 0 starts the
// DMA of K(u + 2) into the slot K(u) has left and wave 1 that of V(u) into the slot of
// V(u - 2); then each wave runs block u's softmax with V(u - 1)'s PV and K(u + 1)'s
// QK^T products. Steps past the end of the list repeat its last block (their products
// are discarded).
__global__ __launch_bounds__(128, 2) void sparse_attn_kernel(
    const int8_t* __restrict__ q8, const float* __restrict__ sq, const int8_t* __restrict__ k8,
    const float* __restrict__ sk, const uint8_t* __restrict__ v8, const float* __restrict__ vamax,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ khead, const uint16_t* __restrict__ y, int N,
    int Nb, int ksel, int kstride, int tiles, int per_xcd, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_k0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_k1[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_v0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_v1[kBlkBytes];
  const int tile = xcd_tile(blockIdx.x, per_xcd);
  if (tile >= tiles) return;
  const int bh = tile / Nb, i = tile % Nb;
  const int t = threadIdx.x, l = t & 63, g = l >> 5, r = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index (uniform)
  const size_t hb = (size_t)bh * Nb;
  const int nk = khead ? khead[bh] : ksel;  // kept blocks of this head
  const int32_t* crit = idx + (hb + i) * kstride;
  const int last = nk - 1;
  const int nlast = block_len(Nb - 1, N);  // valid keys in the last block
  const bool has_partial = nlast < kBlk;
  // wave 0 streams K code tiles, wave 1 V code tiles, by buffer loads into LDS: the
  // resource holds the head's tiles (at most 16384 x 8 KiB), the block offset is a scalar
  // and the lane's 16 bytes the vector offset, so no address arithmetic runs on the VALU
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((w == 0 ? (const uint8_t*)k8 : v8) + hb * kBlkBytes), 0, Nb * kBlkBytes, kBufWord3);
  const uint32_t lo = (uint32_t)l * 16u;
  auto dma = [&](uint8_t* dst, int j) {
    const int s0 = j * kBlkBytes;
    dma_part<0>(rsrc, dst, lo, s0);
    dma_part<1>(rsrc, dst, lo, s0);
    dma_part<2>(rsrc, dst, lo, s0);
    dma_part<3>(rsrc, dst, lo, s0);
    dma_part<4>(rsrc, dst, lo, s0);
    dma_part<5>(rsrc, dst, lo, s0);
    dma_part<6>(rsrc, dst, lo, s0);
    dma_part<7>(rsrc, dst, lo, s0);
  };

  // kept-block indices: j(u), j(u + 1), j(u + 2) in scalar registers; j(u + 3) and the K
  // scale of block u + 1 arrive by vector loads one step ahead (a scalar load in the loop
  // would make every LDS wait a full wait)
  int ju = crit[0], ju1 = crit[min(1, last)], ju2 = crit[min(2, last)];
  float sku = sk[hb + ju];
  // Q8 B-operand for query tile w: 4 steps of 16 bytes
  v4i q[4];
  {
    const int8_t* qsrc = q8 + (hb + i) * kBlkBytes;
#pragma unroll
    for (int s = 0; s < 4; s++) q[s] = *(const v4i*)(qsrc + ((w * 4 + s) * 64 + l) * 16);
  }
  const float sqi = sq[hb + i];
  if (w == 0) {
    dma(s_k0, ju);
    dma(s_k1, ju1);
  }
  v16i magic = {kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI,
                kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI, kMagicI};
  // row-sum selector: e4m3 1.0 in row 0 over the key ranges of lanes 0..15 and 32..47
  // (queries 0..15), in row 1 over those of lanes 16..31 and 48..63
  const int lr = l & 15, lq = (l >> 4) & 1;
  const int one8 = ((lr == 0 && lq == 0) || (lr == 1 && lq == 1)) ? 0x38383838 : 0;
  const v8i lsel = {one8, one8, one8, one8, one8, one8, one8, one8};

  RowAcc st;
  st.m = -INFINITY;
  st.lacc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < 4; d++) st.acc[d] = (v16f){};

  v16i SA[2], SB[2];
  v8i PA = {}, PB = {};
  Pipe pp;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // QK^T of block 0
#pragma unroll
  for (int s = 0; s < 4; s++)
#pragma unroll
    for (int tt = 0; tt < 2; tt++)
      SA[tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(*(const v4i*)(s_k0 + ((tt * 4 + s) * 64 + l) * 16), q[s],
                                                     s == 0 ? magic : SA[tt], 0, 0, 0);

  // j(u + 3) and s_k of block u + 1, loaded during step u by vector loads (issued before
  // the step's DMA, and waited for at the next step's barrier). The lane offset lz is a
  // zero the compiler cannot see through: with a uniform address it would emit a scalar
  // load, and a pending scalar load turns every LDS wait of the step into a full wait.
  int lz;
  asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
  int jv3 = ju2;
  float skv1 = sku;

  // block u with K(u) in slot ks, K(u + 1) in slot kn, V(u - 1) in slot vp; V(u) goes to
  // slot vc. S: scores of block u; Sn: next block's; P: previous block's FP8 weights.
  auto step = [&](int u, uint8_t* ks, uint8_t* kn, uint8_t* vc, uint8_t* vp, v16i(&S)[2], v16i(&Sn)[2], v8i& Pprev,
                  v8i& Pcur, auto has_prev) {
    constexpr bool kPV = decltype(has_prev)::value;
    // K(u + 1) and V(u - 1) have landed (each wave waits for its own DMAs, the barrier for
    // the other's), and no wave reads K(u) or V(u - 2) any more
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the accumulator bias stays in VGPRs (rebuilding it from scalars costs 8 moves a block)
    asm volatile("" : "+v"(magic));
    if (u > 0) {
      ju = ju1;
      ju1 = ju2;
      ju2 = __builtin_amdgcn_readfirstlane(jv3);
      sku = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, skv1)));
    }
    jv3 = crit[min(u + 3, last) + lz];
    skv1 = sk[hb + ju1 + lz];
    if (w == 0)
      dma(ks, ju2);
    else
      dma(vc, ju);
    const float a = (sqi * sku) * kC0;
    const float ba = kMagicF * a;
    const bool partial = has_partial && ju == Nb - 1;
    pp.vt = vp;
    pp.kt = kn;
    Pcur = block_step<kPV>(S, st, a, ba, partial, nlast, g, l, pp, Pprev, lsel, Sn, q, magic);
  };

  // even steps: K(u) in s_k0, V(u) to s_v0; odd steps the other slots
  step(0, s_k0, s_k1, s_v0, s_v1, SA, SB, PB, PA, std::false_type{});
  int u = 1;
  for (; u + 1 < nk; u += 2) {
    step(u, s_k1, s_k0, s_v1, s_v0, SB, SA, PA, PB, std::true_type{});
    step(u + 1, s_k0, s_k1, s_v0, s_v1, SA, SB, PB, PA, std::true_type{});
  }
  if (u < nk) step(u, s_k1, s_k0, s_v1, s_v0, SB, SA, PA, PB, std::true_type{});
  // the last block's PV: V(last) and its weights (PA if last is even, PB if odd)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    const bool odd = (last & 1) != 0;
    const uint8_t* vt = odd ? s_v1 : s_v0;
    const v8i P = odd ? PB : PA;
#pragma unroll
    for (int d = 0; d < 4; d++)
      st.acc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v_op(vt, d, l), P, st.acc[d], 0, 0, 0, 0, 0, 0);
    st.lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lsel, P, st.lacc, 0, 0, 0, 0, 0, 0);
  }

  // V scales s_v[c] = amax_c / 448 once per channel, in the K slot no wave reads any more
  float* s_sv = (float*)s_k0;
  s_sv[t] = vamax[(size_t)bh * kD + t] / 448.0f;
  __syncthreads();
  const int qrow = i * kBlk + 32 * w + r;
  if (qrow < N) {
    // query r's sum: lane r & 15, element 0 for r < 16, element 1 otherwise
    const float l0 = __shfl(st.lacc[0], r & 15), l1 = __shfl(st.lacc[1], r & 15);
    const float inv_l = 1.0f / (r < 16 ? l0 : l1);
    uint16_t* orow = out + ((size_t)bh * N + qrow) * kD;
    const uint16_t* yrow = y ? y + ((size_t)bh * N + qrow) * kD : nullptr;
#pragma unroll
    for (int d = 0; d < 4; d++)
#pragma unroll
      for (int v4 = 0; v4 < 4; v4++) {
        const int c = 32 * d + 8 * v4 + 4 * g;
        const v4f sv = *(const v4f*)(s_sv + c);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = st.acc[d][4 * v4 + e] * (sv[e] * inv_l);
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

// khead: per-head counts (int32 [BH]) or NULL for ksel everywhere; idx rows are kstride apart.
hipError_t launch_sparse_attn(const void* q8, const void* sq, const void* k8, const void* sk,
                              const void* v8, const void* vamax, const void* idx, const void* khead, int kstride,
                              const void* y, int BH, int N, int Nb, int ksel, void* out, hipStream_t st) {
  if (!c0_matches()) return hipErrorInvalidValue;
  const int tiles = BH * Nb;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(per_xcd * 8), dim3(128), 0, st, (const int8_t*)q8,
                     (const float*)sq, (const int8_t*)k8, (const float*)sk, (const uint8_t*)v8,
                     (const float*)vamax, (const int32_t*)idx, (const int32_t*)khead, (const uint16_t*)y, N, Nb,
                     ksel, kstride, tiles, per_xcd, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const void* q8, const void* sq, const void* k8, const void* sk,
                              const void* v8, const void* vamax, const void* idx, const void* y, int BH,
                              int N, int Nb, int ksel, void* out, hipStream_t st) {
  return launch_sparse_attn(q8, sq, k8, sk, v8, vamax, idx, nullptr, ksel, y, BH, N, Nb, ksel, out, st);
}

}  // namespace sagesla
