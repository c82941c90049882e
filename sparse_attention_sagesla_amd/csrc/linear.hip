// Linear branch of SLA: complement state = total - kept blocks, then
// O_l = phi(q) H^c / (phi(q) . z^c) and y = O_l W_proj.
//
// SLA sends what it does not compute exactly to a linear-attention variant (bonega.ai
// blog, SLA paragraph; tiemojia.cn article, 2.2.1). With per-key-block states S_j
// (H_j^T and z_j, see quant_kv.hip) the complement of query block i is
//   S^c_i = S_total - sum_{j kept by i} S_j,
// so its cost does not depend on how many blocks are left to the linear branch.
// Neighbouring query blocks keep mostly the same key blocks, so the kept sums of a
// group of 256 consecutive query blocks are one matrix product on the matrix cores:
//   M[i][e] = sum_{u in union} C[i][u] * S_{union[u]}[e],  C = 0/1 kept mask,
// over the union of the group's kept sets (each state row is read once per group).
// phi is the softmax over the d channels of the raw bf16 row.
#include "common.h"

namespace sagesla {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_ __attribute__((ext_vector_type(4)));

constexpr int kUnionRange = 1024;  // key blocks per LDS pass of the union kernel

// ---------------------------------------------------------------- union of a group

// Per (bh, group): the ascending union of the kept key blocks of the group's kGroup
// query blocks, and which query blocks keep each entry, as one bit row per query block
// over the union positions. ulist: [BH][ng][Nb], ucount: [BH][ng],
// umask: [BH][ng][nw][kGroup] with nw = ceil(Nb / 32): bit p % 32 of umask[..][p / 32][qb]
// is set when query block qb keeps union entry p (one step's words are contiguous).
// complement != 0 (more than half the blocks kept): the same for the blocks NOT kept,
// so that the complement is summed directly instead of as total - kept (which would
// cancel almost all of the total and leave the bf16 rounding of the kept states).
// With khead the head keeps khead[bh] blocks (rows of idx kstride apart) and takes the
// complement form on its own count; else every head keeps ksel.
__global__ __launch_bounds__(256) void linear_union_kernel(const int32_t* __restrict__ idx, int Nb, int ksel,
                                                           const int32_t* __restrict__ khead, int kstride,
                                                           int ngroups, int complement_all,
                                                           int32_t* __restrict__ ulist,
                                                           uint32_t* __restrict__ umask,
                                                           int32_t* __restrict__ ucount) {
  __shared__ uint32_t s_flags[kUnionRange][kMaskWords];
  __shared__ int32_t s_pos[kUnionRange];  // key block (in the range) of each new union entry
  __shared__ int s_tmp[8];
  const int bh = blockIdx.x / ngroups, grp = blockIdx.x % ngroups, t = threadIdx.x;
  const int q0 = grp * kGroup, nq = min(kGroup, Nb - q0);
  const size_t gbase = (size_t)bh * ngroups + grp;
  const int nw = (Nb + 31) / 32;
  const int ks = khead ? khead[bh] : ksel;
  const int complement = khead ? (2 * ks > Nb) : complement_all;
  uint32_t* mrow = umask + gbase * kGroup * nw;
  for (int e = t; e < kGroup * nw; e += 256) mrow[e] = 0u;
  int count = 0;
  for (int r0 = 0; r0 < Nb; r0 += kUnionRange) {
    const int rl = min(kUnionRange, Nb - r0);
    for (int e = t; e < rl * kMaskWords; e += 256) (&s_flags[0][0])[e] = 0u;
    __syncthreads();
    const int32_t* src = idx + ((size_t)bh * Nb + q0) * kstride;
    for (int e = t; e < nq * ks; e += 256) {
      const int qb = e / ks;
      const int j = src[(size_t)qb * kstride + e % ks] - r0;
      if (j >= 0 && j < rl) atomicOr(&s_flags[j][qb >> 5], 1u << (qb & 31));
    }
    __syncthreads();
    // compact the non-empty entries in ascending order: thread t owns a contiguous range
    const int per = (rl + 255) / 256, j0 = t * per, j1 = min(rl, j0 + per);
    // membership bits of entry j for query-block word x: kept, or (complement) not kept
    // by one of the group's nq query blocks
    auto bits_of = [&](int j, int x) {
      const uint32_t f = s_flags[j][x];
      if (!complement) return f;
      const int lo = 32 * x;
      const uint32_t valid = nq >= lo + 32 ? 0xFFFFFFFFu : (nq <= lo ? 0u : (1u << (nq - lo)) - 1u);
      return ~f & valid;
    };
    auto any = [&](int j) {
      uint32_t o = 0u;
#pragma unroll
      for (int x = 0; x < kMaskWords; x++) o |= bits_of(j, x);
      return o != 0u;
    };
    int n = 0;
    for (int j = j0; j < j1; j++) n += any(j);
    // block exclusive scan of n
    const int lane = t & 63, w = t >> 6;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_tmp[w] = incl;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      if (k < w) off += s_tmp[k];
      tot += s_tmp[k];
    }
    int pos = off + incl - n;  // within this range
    for (int j = j0; j < j1; j++) {
      if (!any(j)) continue;
      ulist[gbase * Nb + count + pos] = r0 + j;
      s_pos[pos] = j;
      pos++;
    }
    __syncthreads();
    // bit rows: word wd of query block qb covers union positions 32 wd .. 32 wd + 31; the
    // words at the range's ends are shared with the neighbouring ranges (atomic OR).
    // Each half-wave takes one (wd, 32 query blocks) tile, a 32 x 32 bit transpose done
    // with ballots: lane i holds the query-block word of position 32 wd + i, and ballot b
    // gathers bit b (query block) over the 32 positions.
    if (tot > 0) {
      const int w0 = count >> 5, w1 = (count + tot - 1) >> 5, nwr = w1 - w0 + 1;
      const int ntile = nwr * kMaskWords, i = lane & 31, hw = lane >> 5;
      for (int base = 2 * w; base < ntile; base += 8) {  // 4 waves x 2 halves
        const int tile = base + hw;
        uint32_t word = 0u;
        int wd = 0, qw = 0;
        if (tile < ntile) {
          wd = w0 + tile / kMaskWords;
          qw = tile % kMaskWords;
          const int p = 32 * wd + i - count;
          if (p >= 0 && p < tot) word = bits_of(s_pos[p], qw);
        }
        uint32_t mine = 0u;
#pragma unroll
        for (int b = 0; b < 32; b++) {
          const unsigned long long m = __ballot((word >> b) & 1u);
          if (i == b) mine = hw ? (uint32_t)(m >> 32) : (uint32_t)m;
        }
        const int qb = 32 * qw + i;
        if (tile < ntile && mine && qb < nq) atomicOr(&mrow[(size_t)wd * kGroup + qb], mine);
      }
    }
    count += tot;
    __syncthreads();
  }
  if (t == 0) ucount[gbase] = count;
}

// ---------------------------------------------------------------- masked sum on MFMA

constexpr int kMgSlots = 4;  // ring depth: steps of 32 union entries in flight
typedef short v4s_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_* lds_v4s_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// gfx950 transposing LDS read: within each group of 16 lanes, lanes 4a..4a+3 each name
// 4 consecutive 16-bit elements of row a of a 4 x 16 tile, and lane j receives column j.
__device__ __forceinline__ v4s_ lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p));
}

// One ring slot: the step's 32 state rows x 128 columns (bf16, 256-byte rows of 16-byte
// chunks placed by mg_pos), the step's membership word of each of the group's query
// blocks (permuted, see issue), and the union entries of a later step (per wave: its 8
// rows in lanes 0..7 of a 64-word row). Each slot is its own LDS object, so that the
// compiler waits for a slot's own copies only.
struct MgSlot {
  uint16_t st[32 * 128];
  uint32_t mk[kGroup];
  int32_t ul[4 * 64];
};

// The 16 transposing reads of a step (rows r and r + 4 of each of the eight column tiles; a
// holds their LDS byte addresses), waited for in the same block. Written out so that the
// compiler, which cannot tell which ring slot's DMAs a read depends on, adds no wait of its
// own: the slot is complete by the explicit wait and barrier of the step.
typedef int v2i_ __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void mg_tr_reads16(const uint32_t (&a)[8], v2i_ (&x)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:1024\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:1024\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:1024\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:1024\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
        "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Chunk cc (0..15) of state row r sits at chunk position mg_pos(r, cc) of its 256-byte
// row (an involution). With it the two transposing reads of a half-wave (rows 8 kg + a,
// kg in {0, 1}, a in 0..3, four 8-byte column pieces each) cover all 64 banks once.
__device__ __forceinline__ int mg_pos(int r, int cc) { return cc ^ (2 * ((r & 3) | (((r >> 3) & 1) << 2))); }

// Per (bh, group, state row c in 0..128): for the group's kGroup query blocks i and the
// 128 columns a,
//   hc[i][c][a] = htot[c][a] - sum_u C[i][u] S_{union[u]}[c][a]
// (or the sum alone when the union lists the blocks NOT kept), taken transposed,
// M^T = S^T C^T, as [128 x U] x [U x kGroup] products on v_mfma_f32_16x16x32_bf16: the
// 0/1 mask is exact in bf16, the states are bf16, the sums fp32. Wave w owns query
// blocks 64w .. 64w+63 (4 column tiles) and the 8 row tiles of state columns; each lane
// ends with 4 consecutive columns of one query block per tile, stored as 8 bytes.
// Union entries stream in steps of 32 through a ring of kMgSlots LDS slots filled by
// global_load_lds DMA; the union entries that address a step's rows arrive kMgSlots
// steps before them. Tiles are ordered (bh, state row, group) and dealt to the XCDs in
// contiguous ranges (workgroup b runs on XCD b % 8), so the groups that read the same
// 256-byte row slice of the states run together on one XCD and share its L2.
__global__ __launch_bounds__(256, 2) void linear_mask_gemm_kernel(
    const uint16_t* __restrict__ hs, const float* __restrict__ htot, const int32_t* __restrict__ ulist,
    const uint32_t* __restrict__ umask, const int32_t* __restrict__ ucount, const int32_t* __restrict__ khead,
    int Nb, int ngroups, int complement_all, int ntiles, int per_xcd, uint16_t* __restrict__ hc) {
  __shared__ __attribute__((aligned(16))) MgSlot s0, s1, s2, s3;
  __shared__ __attribute__((aligned(8))) uint2 s_nib[16];  // nibble -> its 4 bits as bf16 0.0 / 1.0

  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= ntiles) return;
  const int per_bh = ngroups * 129;
  const int bh = tile / per_bh, rem = tile % per_bh;
  const int grp = rem % ngroups, c = rem / ngroups;
  const int complement = khead ? (2 * khead[bh] > Nb) : complement_all;
  const size_t gbase = (size_t)bh * ngroups + grp;
  const int U = ucount[gbase];
  const int32_t* ul = ulist + gbase * Nb;
  const int nw = (Nb + 31) / 32;
  const uint32_t* um = umask + gbase * kGroup * nw;
  const int t = threadIdx.x, lane = t & 63, l16 = lane & 15, kg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);

  if (t < 16) {
    uint2 e;
    e.x = ((t & 1) ? 0x3F80u : 0u) | ((t & 2) ? 0x3F800000u : 0u);  // bf16 1.0
    e.y = ((t & 4) ? 0x3F80u : 0u) | ((t & 8) ? 0x3F800000u : 0u);
    s_nib[t] = e;
  }

  v4f_ acc[4][8];
#pragma unroll
  for (int m = 0; m < 4; m++)
#pragma unroll
    for (int n = 0; n < 8; n++) acc[m][n] = (v4f_){0.f, 0.f, 0.f, 0.f};

  const int nsteps = (U + 31) / 32;
  // this lane's DMA rows: state rows 8w + 4k + lane/16 (k = 0, 1) of a step, chunk
  // position lane % 16
  const int dr0 = 8 * w + (lane >> 4), dr1 = dr0 + 4;
  const uint16_t* hs_row = hs + (size_t)bh * Nb * kStateElems + (size_t)c * kD;
  const uint32_t src0 = 8 * mg_pos(dr0, lane & 15), src1 = 8 * mg_pos(dr1, lane & 15);
  // Every DMA is issued, with step indices clamped to the last step, so that each wave
  // issues four per step (two of state rows, membership words, later union entries)
  // and the wait counts below are exact.
  auto issue_ul = [&](MgSlot& d, int step) {
    const int sb = min(step, nsteps - 1);
    const int u = min(32 * sb + 8 * w + (lane & 7), U - 1);
    __builtin_amdgcn_global_load_lds((const void*)(ul + u), (lds_void_ptr)(d.ul + 64 * w), 4, 0, 0);
  };
  auto issue = [&](MgSlot& d, int step) {
    const int sa = min(step, nsteps - 1);
    const int j0 = d.ul[64 * w + (lane >> 4)], j1 = d.ul[64 * w + 4 + (lane >> 4)];
    __builtin_amdgcn_global_load_lds((const void*)(hs_row + (size_t)j0 * kStateElems + src0),
                                     (lds_void_ptr)(d.st + 1024 * w), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(hs_row + (size_t)j1 * kStateElems + src1),
                                     (lds_void_ptr)(d.st + 1024 * w + 512), 16, 0, 0);
    // word position 64w + 4 p + m holds query block 64w + 16m + p: a lane's four words
    // (one per column tile) are one 16-byte read
    __builtin_amdgcn_global_load_lds((const void*)(um + (size_t)sa * kGroup + 64 * w + 16 * (lane & 3) + (lane >> 2)),
                                     (lds_void_ptr)(d.mk + 64 * w), 4, 0, 0);
    issue_ul(d, step + kMgSlots);
  };
  // lane (kg, l16) of the transposing reads: rows 8kg + ta (+4), columns 16n + 4tb .. +3
  const int ta = l16 >> 2, tb = l16 & 3, r0 = 8 * kg + ta;
  uint32_t toff[8];  // byte offsets in a slot's state tile
#pragma unroll
  for (int n = 0; n < 8; n++) toff[n] = 2 * (r0 * 128 + 8 * mg_pos(r0, 2 * n + (tb >> 1)) + 4 * (tb & 1));
  auto compute = [&](const MgSlot& d) {
    // B operand of column tile m: query block 64w + 16m + l16, union entries 8kg .. 8kg+7
    v8bf bop[4];
    const uint4 words = *(const uint4*)(d.mk + 64 * w + 4 * l16);
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const uint32_t word = m == 0 ? words.x : m == 1 ? words.y : m == 2 ? words.z : words.w;
      const uint32_t byte = (word >> (8 * kg)) & 255u;
      const uint2 lo = s_nib[byte & 15u], hi = s_nib[byte >> 4];
      bop[m] = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
    const uint32_t base = lds_addr(d.st);
    uint32_t ad[8];
#pragma unroll
    for (int n = 0; n < 8; n++) ad[n] = base + toff[n];
    v2i_ x[16];
    mg_tr_reads16(ad, x);
#pragma unroll
    for (int n = 0; n < 8; n++) {
      const v4i aop4 = {x[2 * n][0], x[2 * n][1], x[2 * n + 1][0], x[2 * n + 1][1]};
      const v8bf aop = __builtin_bit_cast(v8bf, aop4);
#pragma unroll
      for (int m = 0; m < 4; m++)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[m], acc[m][n], 0, 0, 0);
    }
  };
  // Ring: step s lives in slot s % 4. At the top of step s this wave has issued, after
  // the state rows and words of step s, the union entries of step s + 4 and the four
  // DMAs of each of steps s + 1 .. s + 2, all of which may still be in flight.
  static_assert(kMgSlots == 4, "the slot objects and the wait count assume a ring of 4");
  constexpr int kWait = 1 + 4 * (kMgSlots - 2);
  constexpr int kWaitImm = (kWait & 15) | ((kWait >> 4) << 14) | (7 << 4) | (15 << 8);  // vmcnt only
  auto phase = [&](MgSlot& cur, MgSlot& prev, int step) {
    __builtin_amdgcn_s_waitcnt(kWaitImm);
    // step's slot complete from every wave; step - 1's slot free (every wave has used
    // the operands it read from it). A plain barrier: a fence would wait for every DMA.
    asm volatile("s_barrier" ::: "memory");
    issue(prev, step + kMgSlots - 1);
    compute(cur);
  };
  if (nsteps > 0) {
    issue_ul(s0, 0);
    issue_ul(s1, 1);
    issue_ul(s2, 2);
    issue_ul(s3, 3);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's union entries of steps 0..3 (read by itself only)
    issue(s0, 0);
    issue(s1, 1);
    issue(s2, 2);
    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
      phase(s0, s3, s);
      phase(s1, s0, s + 1);
      phase(s2, s1, s + 2);
      phase(s3, s2, s + 3);
    }
    if (s < nsteps) phase(s0, s3, s);
    if (s + 1 < nsteps) phase(s1, s0, s + 1);
    if (s + 2 < nsteps) phase(s2, s1, s + 2);
    __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the workgroup ends
  }
  // hc = htot - M (kept sets) or M (complement sets): 4 consecutive columns of one query
  // block per lane and tile, one 8-byte store
  const int q0 = grp * kGroup;
  const float* ht = htot + (size_t)bh * kStateElems + c * kD;
  const float sgn = complement ? 1.f : -1.f;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const int qb = q0 + 64 * w + 16 * m + l16;
    if (qb < Nb) {
      uint16_t* dst = hc + ((size_t)bh * Nb + qb) * kStateElems + c * kD;
#pragma unroll
      for (int n = 0; n < 8; n++) {
        const int col = 16 * n + 4 * kg;
        const float4 tv = complement ? make_float4(0.f, 0.f, 0.f, 0.f) : *(const float4*)(ht + col);
        const v4f_ a = acc[m][n];
        uint2 o;
        o.x = pack_bf16x2(tv.x + sgn * a[0], tv.y + sgn * a[1]);
        o.y = pack_bf16x2(tv.z + sgn * a[2], tv.w + sgn * a[3]);
        *(uint2*)(dst + col) = o;
      }
    }
  }
}

// ---------------------------------------------------------------- output per query block

constexpr int kLs = 136;   // LDS row pitch (bf16) of the 128-wide tiles: 272 B
constexpr int kOutQB = 4;  // consecutive query blocks per workgroup (W_proj staged once)

// Rows a0..a0+7 of column c0 + lane%16 of a row-major [a][c] bf16 LDS tile (pitch kLs),
// through two transposing reads: the K=8 slice of a bf16 MFMA operand.
__device__ __forceinline__ v8bf tile_col8(const uint16_t* tile, int a0, int c0, int lane) {
  const int j = lane & 15, a = j >> 2, b = j & 3;
  const v4s_ r0 = lds_read_tr16(tile + (a0 + a) * kLs + c0 + 4 * b);
  const v4s_ r1 = lds_read_tr16(tile + (a0 + 4 + a) * kLs + c0 + 4 * b);
  const v8s v = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
  return __builtin_bit_cast(v8bf, v);
}

// Per-block inputs held in registers.
struct OutLoads {
  uint4 q[4];    // raw q: rows t/16 + 16 mm, channels 8 (t%16) .. +7
  v8bf sa[8];    // S^c rows 32 w + l%32, k-steps s: the A operands of num^T
  uint16_t zc;   // z^c[t % 128] (bf16; used by t < 128)
};

__device__ __forceinline__ void out_load(OutLoads& L, const uint16_t* q, const uint16_t* hc, int bh, int i, int N,
                                         int Nb, int t, int w, int lane) {
  // Every load is unconditional (rows past the block's end repeat its last row; their
  // results are never stored).
  const int n = block_len(i, N), rg = t >> 4, ch = t & 15;
#pragma unroll
  for (int mm = 0; mm < 4; mm++) {
    const int row = min(rg + 16 * mm, n - 1);
    L.q[mm] = *(const uint4*)(q + ((size_t)bh * N + (size_t)i * kBlk + row) * kD + ch * 8);
  }
  const uint16_t* S = hc + ((size_t)bh * Nb + i) * kStateElems;
  const int c = 32 * w + (lane & 31), g = lane >> 5;
#pragma unroll
  for (int s = 0; s < 8; s++) L.sa[s] = *(const v8bf*)(S + c * kD + 16 * s + 8 * g);
  L.zc = S[kD * kD + (t & (kD - 1))];
}

// One workgroup (256 threads, 4 waves) per kOutQB consecutive query blocks of one head:
//   O_l[r] = phi(q_r) H^c_i / (phi(q_r) . z^c_i),  y[r] = O_l[r] W_proj  (bf16).
// hc holds S^c_i = [H^c_i^T ; z^c_i] (129 x 128) in bf16. Both products are taken
// transposed, num^T = S^c phi^T and y^T = W^T O_l^T, so that every operand is a
// contiguous row (S^c from memory, phi and O_l from LDS) or a transposing LDS read of
// row-major W, and each lane ends with 4 consecutive channels of one row.
// Wave w owns channels 32 w .. 32 w + 31 of both products, for all 64 rows.
// A head that keeps every block (khead[bh] = Nb) has no complement: its y is zero.
__global__ __launch_bounds__(256, 3) void linear_out_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ hc,
                                                         const uint16_t* __restrict__ proj,
                                                         const int32_t* __restrict__ khead, int N, int Nb,
                                                         int groups, int per_xcd, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kD * kLs];    // W_proj [a][c]
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kBlk * kLs];  // phi(Q) [m][a], then O_l [m][c]
  __shared__ float s_zc[kD];
  __shared__ float s_den[kBlk];

  const int gid = xcd_tile(blockIdx.x, per_xcd);
  if (gid >= groups) return;
  const int nqb = (Nb + kOutQB - 1) / kOutQB;
  const int bh = gid / nqb, i0 = (gid % nqb) * kOutQB, i1 = min(Nb, i0 + kOutQB);
  const int t = threadIdx.x, lane = t & 63, g = lane >> 5, r = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  if (khead && khead[bh] >= Nb) {
    const size_t r0 = (size_t)i0 * kBlk, r1 = min((size_t)i1 * kBlk, (size_t)N);
    uint4* dst = (uint4*)(y + ((size_t)bh * N + r0) * kD);
    for (size_t e = t; e < (r1 - r0) * (kD / 8); e += 256) dst[e] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }

  OutLoads la;
  out_load(la, q, hc, bh, i0, N, Nb, t, w, lane);
  {
    // W_proj: all of this thread's loads in flight before its stores
    uint4 wv[kD * 16 / 256];
#pragma unroll
    for (int k = 0; k < kD * 16 / 256; k++) {
      const int e = t + 256 * k, a = e >> 4, c8 = (e & 15) * 8;
      wv[k] = *(const uint4*)(proj + a * kD + c8);
    }
#pragma unroll
    for (int k = 0; k < kD * 16 / 256; k++) {
      const int e = t + 256 * k, a = e >> 4, c8 = (e & 15) * 8;
      *(uint4*)(s_w + a * kLs + c8) = wv[k];
    }
  }
  auto process = [&](const OutLoads& cur, int i) {
    const int n = block_len(i, N);
    __syncthreads();  // the previous block is done with s_a, s_zc, s_den
    if (t < kD) s_zc[t] = bf16_to_f32(cur.zc);
    __syncthreads();
    // phi(q) rows (16 lanes per row) -> s_a; den = phi(q) . z^c in fp32
    {
      const int rg = t >> 4, ch = t & 15;
#pragma unroll
      for (int mm = 0; mm < 4; mm++) {
        const int row = rg + 16 * mm;
        const uint16_t* qh = (const uint16_t*)&cur.q[mm];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = bf16_to_f32(qh[e]);
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; e++) mx = fmaxf(mx, x[e]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) { x[e] = __expf(x[e] - mx); sum += x[e]; }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
        const float inv = 1.0f / sum;
        float den = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = x[e] * inv, p1 = x[e + 1] * inv;
          den += p0 * s_zc[ch * 8 + e] + p1 * s_zc[ch * 8 + e + 1];
          pk[e / 2] = f32_to_bf16(p0) | ((uint32_t)f32_to_bf16(p1) << 16);
        }
        *(uint4*)(s_a + row * kLs + ch * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) den += __shfl_xor(den, o);
        if (ch == 0) s_den[row] = den;
      }
    }
    __syncthreads();
    // num^T[c][m] = S^c[c][:] . phi[m][:]
    v16f num[2] = {(v16f){}, (v16f){}};
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        const v8bf b = *(const v8bf*)(s_a + (32 * mt + r) * kLs + 16 * s + 8 * g);
        num[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.sa[s], b, num[mt], 0, 0, 0);
      }
    __syncthreads();  // phi fully read
    // O_l[m][c] = num^T[c][m] / den[m] -> s_a row-major, 4 consecutive channels per store
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const float den = s_den[32 * mt + r];
      const float inv = den != 0.f ? 1.0f / den : 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int c = 32 * w + 8 * q4 + 4 * g;
        uint2 pk;
        pk.x = f32_to_bf16(num[mt][4 * q4] * inv) | ((uint32_t)f32_to_bf16(num[mt][4 * q4 + 1] * inv) << 16);
        pk.y = f32_to_bf16(num[mt][4 * q4 + 2] * inv) | ((uint32_t)f32_to_bf16(num[mt][4 * q4 + 3] * inv) << 16);
        *(uint2*)(s_a + (32 * mt + r) * kLs + c) = pk;
      }
    }
    __syncthreads();
    // y^T[c][m] = W[:][c] . O_l[m][:]
    v16f yo[2] = {(v16f){}, (v16f){}};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const v8bf a = tile_col8(s_w, 16 * s + 8 * g, 32 * w + 16 * ((lane >> 4) & 1), lane);
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        const v8bf b = *(const v8bf*)(s_a + (32 * mt + r) * kLs + 16 * s + 8 * g);
        yo[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, yo[mt], 0, 0, 0);
      }
    }
    uint16_t* ydst = y + ((size_t)bh * N + (size_t)i * kBlk) * kD;
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const int m = 32 * mt + r;
      if (m < n) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
          const int c = 32 * w + 8 * q4 + 4 * g;
          uint2 pk;
          pk.x = f32_to_bf16(yo[mt][4 * q4]) | ((uint32_t)f32_to_bf16(yo[mt][4 * q4 + 1]) << 16);
          pk.y = f32_to_bf16(yo[mt][4 * q4 + 2]) | ((uint32_t)f32_to_bf16(yo[mt][4 * q4 + 3]) << 16);
          *(uint2*)(ydst + (size_t)m * kD + c) = pk;
        }
      }
    }
  };
  // One load set: at 150 registers three workgroups share a CU (the LDS allows three as
  // well), and the other workgroups' work covers a block's load latency; that runs faster
  // than two workgroups with the next block's loads in flight in a second set.
  for (int i = i0; i < i1; i++) {
    if (i > i0) out_load(la, q, hc, bh, i, N, Nb, t, w, lane);
    process(la, i);
  }
}

int linear_groups(int Nb) { return (Nb + kGroup - 1) / kGroup; }

// The complement is summed directly over the blocks not kept when those are fewer than
// the kept ones (see linear_union_kernel).
static int use_complement_sets(int Nb, int ksel) { return 2 * ksel > Nb; }

static void launch_mask_gemm(const void* hs, const void* htot, const void* ulist, const void* umask,
                             const void* ucount, const void* khead, int BH, int Nb, int ksel, void* hc,
                             hipStream_t st) {
  const int ng = linear_groups(Nb);
  const int ntiles = BH * ng * 129, per_xcd = (ntiles + 7) / 8;
  hipLaunchKernelGGL(linear_mask_gemm_kernel, dim3(per_xcd * 8), dim3(256), 0, st, (const uint16_t*)hs,
                     (const float*)htot, (const int32_t*)ulist, (const uint32_t*)umask, (const int32_t*)ucount,
                     (const int32_t*)khead, Nb, ng, use_complement_sets(Nb, ksel), ntiles, per_xcd, (uint16_t*)hc);
}

static hipError_t launch_union(const void* idx, const void* khead, int kstride, int BH, int Nb, int ksel,
                               void* ulist, void* umask, void* ucount, hipStream_t st) {
  const int ng = linear_groups(Nb);
  hipLaunchKernelGGL(linear_union_kernel, dim3(BH * ng), dim3(256), 0, st, (const int32_t*)idx, Nb, ksel,
                     (const int32_t*)khead, kstride, ng, use_complement_sets(Nb, ksel), (int32_t*)ulist,
                     (uint32_t*)umask, (int32_t*)ucount);
  return hipGetLastError();
}

hipError_t launch_linear_union(const void* idx, int BH, int Nb, int ksel, void* ulist, void* umask, void* ucount,
                              hipStream_t st) {
  return launch_union(idx, nullptr, ksel, BH, Nb, ksel, ulist, umask, ucount, st);
}

static hipError_t launch_masked(const void* q, const void* hs, const void* htot, const void* proj,
                                const void* khead, int BH, int N, int Nb, int ksel, const void* ulist,
                                const void* umask, const void* ucount, void* hc, void* y, hipStream_t st) {
  launch_mask_gemm(hs, htot, ulist, umask, ucount, khead, BH, Nb, ksel, hc, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups = BH * ((Nb + kOutQB - 1) / kOutQB);
  const int per_xcd = (groups + 7) / 8;
  hipLaunchKernelGGL(linear_out_kernel, dim3(per_xcd * 8), dim3(256), 0, st, (const uint16_t*)q,
                     (const uint16_t*)hc, (const uint16_t*)proj, (const int32_t*)khead, N, Nb, groups, per_xcd,
                     (uint16_t*)y);
  return hipGetLastError();
}

hipError_t launch_linear_masked(const void* q, const void* hs, const void* htot, const void* proj, int BH, int N,
                                int Nb, int ksel, const void* ulist, const void* umask, const void* ucount, void* hc,
                                void* y, hipStream_t st) {
  return launch_masked(q, hs, htot, proj, nullptr, BH, N, Nb, ksel, ulist, umask, ucount, hc, y, st);
}

// The masked complement product alone, on lists built elsewhere (the backward passes
// state gradients through it with the kept relation transposed).
hipError_t launch_linear_mask_gemm(const void* hs, const void* htot, const void* ulist, const void* umask,
                                   const void* ucount, int BH, int Nb, int ksel, void* hc, hipStream_t st) {
  launch_mask_gemm(hs, htot, ulist, umask, ucount, nullptr, BH, Nb, ksel, hc, st);
  return hipGetLastError();
}

// khead: per-head counts (int32 [BH]) or NULL for ksel everywhere; idx rows are kstride apart.
hipError_t launch_linear_complement(const void* q, const void* idx, const void* khead, int kstride, const void* hs,
                                    const void* htot, const void* proj, int BH, int N, int Nb, int ksel, void* ulist,
                                    void* umask, void* ucount, void* hc, void* y, hipStream_t st) {
  hipError_t e = launch_union(idx, khead, kstride, BH, Nb, ksel, ulist, umask, ucount, st);
  if (e != hipSuccess) return e;
  return launch_masked(q, hs, htot, proj, khead, BH, N, Nb, ksel, ulist, umask, ucount, hc, y, st);
}

hipError_t launch_linear_complement(const void* q, const void* idx, const void* hs, const void* htot,
                                    const void* proj, int BH, int N, int Nb, int ksel, void* ulist,
                                    void* umask, void* ucount, void* hc, void* y, hipStream_t st) {
  return launch_linear_complement(q, idx, nullptr, ksel, hs, htot, proj, BH, N, Nb, ksel, ulist, umask, ucount, hc,
                                  y, st);
}

}  // namespace sagesla
