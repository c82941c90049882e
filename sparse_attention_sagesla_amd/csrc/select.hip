// Block scores and top-k key-block selection per query block.
//
// SLA keeps only the most strongly related pairs, a Top-K ratio of 0.1 (TurboDiffusion
// explainer, news.qq.com, "First key: attention"; 0.1-0.15 recommended in "From
// training to deployment"). Scores are s_ij = Qbar_i . Kbar_j / sqrt(d) in fp64, the
// selection key is that score rounded to fp32, and equal keys prefer the lower key
// index. The kept indices are written in processing order: the best block first
// (highest key, lowest index on ties), then the others ascending, so that the attention
// kernel's running maximum starts near its final value.
#include "common.h"

namespace sagesla {

constexpr int kSelThreads = 256;

// float -> uint32 with the same order (larger float -> larger integer)
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scores of up to 8 query-block rows (qbar in LDS, fp64) against key blocks j0 + 256 q,
// q < JT (JT <= 6): s = sum_c qbar[r][c] kbar[c][j] in channel order with fused multiply-adds,
// divided by sqrt(d) (one rounding), and stored as order-preserving fp32 keys.
template <int JT>
__device__ __forceinline__ void score_pass(const double* __restrict__ kb, const double (*s_qb)[kD],
                                           uint32_t* s_keys, int Nb, int nr, int j0) {
  const double inv_sqrt_d = 1.0 / sqrt((double)kD);
  double acc[JT][8];
#pragma unroll
  for (int q = 0; q < JT; q++)
#pragma unroll
    for (int r = 0; r < 8; r++) acc[q][r] = 0.0;
  // Key blocks past Nb read block Nb - 1 (their scores are not stored), so that every
  // load is unconditional.
  const double* kp[JT];
#pragma unroll
  for (int q = 0; q < JT; q++) kp[q] = kb + min(j0 + q * kSelThreads, Nb - 1);
  // Two channel pairs in flight, in register sets A and B used in turn (a register whose
  // load is in flight is never copied, which would make the compiler wait for it).
  double ka[JT][2], kc[JT][2];
#pragma unroll
  for (int q = 0; q < JT; q++) {
    ka[q][0] = kp[q][0];
    ka[q][1] = kp[q][(size_t)Nb];
    kc[q][0] = kp[q][(size_t)2 * Nb];
    kc[q][1] = kp[q][(size_t)3 * Nb];
  }
  auto fma_pair = [&](const double (&kv)[JT][2], int c) {
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const double2 qv = *(const double2*)&s_qb[r][c];  // one 16-byte broadcast read
#pragma unroll
      for (int q = 0; q < JT; q++) {
        acc[q][r] = __fma_rn(qv.x, kv[q][0], acc[q][r]);
        acc[q][r] = __fma_rn(qv.y, kv[q][1], acc[q][r]);
      }
    }
  };
  for (int c = 0; c < kD; c += 4) {
    fma_pair(ka, c);
    const int ca = c + 4 < kD ? c + 4 : c;  // (the last refills reload rows already read)
#pragma unroll
    for (int q = 0; q < JT; q++) {
      ka[q][0] = kp[q][(size_t)ca * Nb];
      ka[q][1] = kp[q][(size_t)(ca + 1) * Nb];
    }
    fma_pair(kc, c + 2);
    const int cc = c + 6 < kD ? c + 6 : c + 2;
#pragma unroll
    for (int q = 0; q < JT; q++) {
      kc[q][0] = kp[q][(size_t)cc * Nb];
      kc[q][1] = kp[q][(size_t)(cc + 1) * Nb];
    }
  }
#pragma unroll
  for (int q = 0; q < JT; q++) {
    const int j = j0 + q * kSelThreads;
    if (j < Nb) {
#pragma unroll
      for (int r = 0; r < 8; r++)
        if (r < nr) s_keys[r * Nb + j] = ord_key((float)(acc[q][r] * inv_sqrt_d));
    }
  }
}

// R query blocks of one head per workgroup (4 waves). Dynamic LDS: keys [R][Nb] uint32.
// Phase 1: all threads score the R rows against every key block (4 key blocks per
// thread in flight). Phase 2: one wave per row selects, with a wave-private histogram
// and ballots (no workgroup barriers).
__global__ __launch_bounds__(kSelThreads) void select_kernel(const double* __restrict__ qbar,
                                                             const double* __restrict__ kbart, int Nb,
                                                             int ksel, int R, int groups,
                                                             int32_t* __restrict__ idx) {
  extern __shared__ uint32_t s_keys[];  // [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  __shared__ uint32_t s_hist[4][256];

  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  for (int e = t; e < nr * kD; e += kSelThreads)
    s_qb[e / kD][e % kD] = qbar[((size_t)bh * Nb + g0 + e / kD) * kD + e % kD];
  __syncthreads();

  // ---- phase 1: scores (fp64, channel order fixed), keys = order-preserving fp32 bits.
  // Thread t scores key blocks t + 256 q; the ceil(Nb / 256) blocks per thread are taken
  // in the fewest balanced passes of at most 6.
  const double* kb = kbart + (size_t)bh * kD * Nb;
  const int kpt = (Nb + kSelThreads - 1) / kSelThreads;
  const int npass = (kpt + 5) / 6, jt = (kpt + npass - 1) / npass;
  for (int q0 = 0; q0 < kpt; q0 += jt) {
    const int n = min(jt, kpt - q0);
    switch (n) {
      case 1: score_pass<1>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
      case 2: score_pass<2>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
      case 3: score_pass<3>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
      case 4: score_pass<4>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
      case 5: score_pass<5>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
      default: score_pass<6>(kb, s_qb, s_keys, Nb, nr, t + q0 * kSelThreads); break;
    }
  }
  __syncthreads();

  // ---- phase 2: one wave per row
  const int lane = t & 63, w = t >> 6;
  uint32_t* hist = s_hist[w];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = w; r < nr; r += 4) {
    const uint32_t* keys = s_keys + r * Nb;
    // radix select (4 x 8 bits, most significant first) of the ksel-th largest key
    uint32_t prefix = 0, mask = 0;
    int kk = ksel;
    for (int pass = 0; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
#pragma unroll
      for (int b = 0; b < 4; b++) hist[4 * lane + b] = 0u;
      // the wave's LDS operations execute in order; keep the compiler from moving them
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < Nb; j += 64) {
        const uint32_t u = keys[j];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      // lane owns bins 4*lane .. 4*lane+3; suffix counts from the top bin down
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int loc = h0 + h1 + h2 + h3;
      int suf = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
      }
      int above = suf - loc;
      const int hs[4] = {h0, h1, h2, h3};
      int sel_bin = -1, sel_k = 0;
#pragma unroll
      for (int b = 3; b >= 0; b--) {
        if (above < kk && above + hs[b] >= kk) {
          sel_bin = 4 * lane + b;
          sel_k = kk - above;
        }
        above += hs[b];
      }
      const unsigned long long who = __ballot(sel_bin >= 0);
      const int src = __ffsll((long long)who) - 1;
      sel_bin = __shfl(sel_bin, src);
      sel_k = __shfl(sel_k, src);
      prefix |= (uint32_t)sel_bin << shift;
      mask |= 255u << shift;
      kk = sel_k;
      __builtin_amdgcn_wave_barrier();
    }
    // best block: highest key, lowest index
    uint32_t kmax = 0u;
    for (int j = lane; j < Nb; j += 64) kmax = max(kmax, keys[j]);
    for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    int jb = INT_MAX;
    for (int j0 = 0; j0 < Nb && jb == INT_MAX; j0 += 64) {
      const int j = j0 + lane;
      const unsigned long long hit = __ballot(j < Nb && keys[j] == kmax);
      if (hit) jb = j0 + __ffsll((long long)hit) - 1;
    }
    // keys > prefix are kept; of the keys == prefix the kk lowest indices; ascending
    // after the best block
    int32_t* out = idx + ((size_t)bh * Nb + g0 + r) * ksel;
    if (lane == 0) out[0] = jb;
    int pos = 1, eq_seen = 0;
    for (int j0 = 0; j0 < Nb; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t u = j < Nb ? keys[j] : 0u;
      const bool eq = j < Nb && u == prefix;
      const unsigned long long eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & below);
      const bool keep = j < Nb && (u > prefix || (eq && eq_rank < kk)) && j != jb;
      const unsigned long long km = __ballot(keep);
      if (keep) out[pos + __popcll(km & below)] = j;
      pos += __popcll(km);
      eq_seen += __popcll(eqm);
    }
  }
}

int select_rows_per_group(int Nb) {
  int R = 16384 / Nb;  // keys of R rows in at most 64 KiB of LDS
  return R < 1 ? 1 : (R > 8 ? 8 : R);
}

hipError_t launch_select(const void* qbar, const void* kbart, int BH, int Nb, int ksel, void* idx,
                         hipStream_t st) {
  const int R = select_rows_per_group(Nb);
  const int groups = (Nb + R - 1) / R;
  size_t lds = (size_t)R * Nb * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kernel, dim3(BH * groups), dim3(kSelThreads), lds, st,
                     (const double*)qbar, (const double*)kbart, Nb, ksel, R, groups, (int32_t*)idx);
  return hipGetLastError();
}

}  // namespace sagesla
