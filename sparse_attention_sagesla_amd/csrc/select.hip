// Block scores and top-k key-block selection per query block.
//
// SLA keeps only the most strongly related pairs, a Top-K ratio of 0.1 (TurboDiffusion
// explainer, news.qq.com, "First key: attention"; 0.1-0.15 recommended in "From
// training to deployment"). Scores are s_ij = Qbar_i . Kbar_j / sqrt(d) in fp64, and the
// selection compares those fp64 scores exactly (order-preserving 64-bit keys); equal
// scores prefer the lower key index. The kept indices are written in processing order:
// the best block first (highest score, lowest index on ties), then the others ascending,
// so that the attention kernel's running maximum starts near its final value.
#include "common.h"

namespace sagesla {

constexpr int kSelThreads = 256;

// double -> uint64 with the same order (larger double -> larger integer); -0 is taken
// as +0 (adding +0 does that), so that equal scores give equal keys
__device__ __forceinline__ uint64_t ord_key(double f) {
  const uint64_t u = (uint64_t)__double_as_longlong(f + 0.0);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// the fp64 score of a key (the inverse of ord_key)
__device__ __forceinline__ double key_value(uint64_t u) {
  const uint64_t b = (u & 0x8000000000000000ull) ? (u & 0x7FFFFFFFFFFFFFFFull) : ~u;
  return __longlong_as_double((long long)b);
}

// The k largest keys of a row are those whose bits under mask exceed prefix, and the kk
// lowest-indexed of those equal to it.
struct Threshold {
  uint64_t prefix, mask;
  int kk;
};

// Radix select of the k-th largest key of a row (one wave, hist: its 256-bin LDS
// histogram), 8 bits per pass from the top. After a pass the keys whose selected bits
// exceed the prefix are kept, and kk more are wanted from those equal to it; when that
// whole bin is wanted the selection is complete (for distinct fp64 scores this happens
// after a few passes).
__device__ Threshold radix_threshold(const uint64_t* keys, int Nb, int k, uint32_t* hist, int lane) {
  Threshold th = {0u, 0u, k};
  for (int pass = 0; pass < 8; pass++) {
    const int shift = 56 - 8 * pass;
#pragma unroll
    for (int b = 0; b < 4; b++) hist[4 * lane + b] = 0u;
    // the wave's LDS operations execute in order; keep the compiler from moving them
    __builtin_amdgcn_wave_barrier();
    for (int j = lane; j < Nb; j += 64) {
      const uint64_t u = keys[j];
      if ((u & th.mask) == th.prefix) atomicAdd(&hist[(uint32_t)(u >> shift) & 255u], 1u);
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
    int sel_bin = -1, sel_k = 0, sel_n = 0;
#pragma unroll
    for (int b = 3; b >= 0; b--) {
      if (above < th.kk && above + hs[b] >= th.kk) {
        sel_bin = 4 * lane + b;
        sel_k = th.kk - above;
        sel_n = hs[b];
      }
      above += hs[b];
    }
    const unsigned long long who = __ballot(sel_bin >= 0);
    const int src = __ffsll((long long)who) - 1;
    sel_bin = __shfl(sel_bin, src);
    sel_k = __shfl(sel_k, src);
    sel_n = __shfl(sel_n, src);
    th.prefix |= (uint64_t)sel_bin << shift;
    th.mask |= (uint64_t)255u << shift;
    th.kk = sel_k;
    __builtin_amdgcn_wave_barrier();
    if (sel_n == sel_k) break;  // every key of the bin is kept
  }
  return th;
}

// Sum of a wave's values, the same butterfly on every lane (every lane ends with the
// same bits: each step adds the same two values)
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Scores of up to 8 query-block rows (qbar in LDS, fp64) against key blocks j0 + 256 q,
// q < JT (JT <= 6): s = sum_c qbar[r][c] kbar[c][j] in channel order with fused multiply-adds,
// divided by sqrt(d) (one rounding), and stored as order-preserving 64-bit keys.
template <int JT>
__device__ __forceinline__ void score_pass(const double* __restrict__ kb, const double (*s_qb)[kD],
                                           uint64_t* s_keys, int Nb, int nr, int j0) {
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
        if (r < nr) s_keys[r * Nb + j] = ord_key(acc[q][r] * inv_sqrt_d);
    }
  }
}

// R query blocks of one head per workgroup (4 waves). Dynamic LDS: keys [R][Nb] uint64.
// Phase 1: all threads score the R rows against every key block (4 key blocks per
// thread in flight). Phase 2: one wave per row selects, with a wave-private histogram
// and ballots (no workgroup barriers).
// Phase 1 of both selection kernels: the scores of the workgroup's rows as keys in LDS.
__device__ __forceinline__ void score_rows(const double* __restrict__ qbar, const double* __restrict__ kbart,
                                           int Nb, int bh, int g0, int nr, double (*s_qb)[kD], uint64_t* s_keys) {
  const int t = threadIdx.x;
  for (int e = t; e < nr * kD; e += kSelThreads)
    s_qb[e / kD][e % kD] = qbar[((size_t)bh * Nb + g0 + e / kD) * kD + e % kD];
  __syncthreads();
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
}

// R query blocks of one head per workgroup (4 waves). Dynamic LDS: keys [R][Nb] uint64.
// Phase 1: all threads score the R rows against every key block (4 key blocks per
// thread in flight). Phase 2: one wave per row selects, with a wave-private histogram
// and ballots (no workgroup barriers). The head keeps khead[bh] blocks when khead is
// given, else ksel; rows are kstride apart, positions past the count are set to -1.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const double* __restrict__ qbar,
                                                             const double* __restrict__ kbart, int Nb,
                                                             int ksel, const int32_t* __restrict__ khead,
                                                             int kstride, int R, int groups,
                                                             int32_t* __restrict__ idx) {
  extern __shared__ uint64_t s_keys[];  // [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  __shared__ uint32_t s_hist[4][256];

  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  const int ks = khead ? khead[bh] : ksel;
  score_rows(qbar, kbart, Nb, bh, g0, nr, s_qb, s_keys);

  // ---- phase 2: one wave per row
  const int lane = t & 63, w = t >> 6;
  uint32_t* hist = s_hist[w];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = w; r < nr; r += 4) {
    const uint64_t* keys = s_keys + r * Nb;
    const Threshold th = radix_threshold(keys, Nb, ks, hist, lane);
    const uint64_t prefix = th.prefix, mask = th.mask;
    const int kk = th.kk;
    // best block: highest key, lowest index
    uint64_t kmax = 0u;
    for (int j = lane; j < Nb; j += 64) kmax = max(kmax, keys[j]);
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t y = (uint64_t)__shfl_xor((long long)kmax, o);
      kmax = max(kmax, y);
    }
    int jb = INT_MAX;
    for (int j0 = 0; j0 < Nb && jb == INT_MAX; j0 += 64) {
      const int j = j0 + lane;
      const unsigned long long hit = __ballot(j < Nb && keys[j] == kmax);
      if (hit) jb = j0 + __ffsll((long long)hit) - 1;
    }
    // keys whose selected bits exceed the prefix are kept; of those equal to it the kk
    // lowest indices; ascending after the best block
    int32_t* out = idx + ((size_t)bh * Nb + g0 + r) * kstride;
    if (lane == 0) out[0] = jb;
    for (int p = ks + lane; p < kstride; p += 64) out[p] = -1;
    int pos = 1, eq_seen = 0;
    for (int j0 = 0; j0 < Nb; j0 += 64) {
      const int j = j0 + lane;
      const uint64_t um = j < Nb ? (keys[j] & mask) : 0u;
      const bool eq = j < Nb && um == prefix;
      const unsigned long long eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & below);
      const bool keep = j < Nb && (um > prefix || (eq && eq_rank < kk)) && j != jb;
      const unsigned long long km = __ballot(keep);
      if (keep) out[pos + __popcll(km & below)] = j;
      pos += __popcll(km);
      eq_seen += __popcll(eqm);
    }
  }
}

// Content-adaptive count, per row: the fewest blocks, in selection order, whose pooled
// mass n_j exp(s_j - max s) reaches tau of the row's total. R rows per workgroup as in
// select_kernel; dynamic LDS: keys [R][Nb] uint64, then the masses [R][Nb] fp64. Each
// wave finds its row's count by bisection on k: the mass of the k largest keys is a sum
// over the lanes' kept blocks in index order (the same order for every k, so it never
// decreases as k grows, and at k = Nb it is the row total bit for bit).
__global__ __launch_bounds__(kSelThreads) void adaptive_k_kernel(const double* __restrict__ qbar,
                                                                 const double* __restrict__ kbart, int N, int Nb,
                                                                 double tau, int R, int groups,
                                                                 int32_t* __restrict__ k_rows) {
  extern __shared__ uint64_t s_keys[];  // [R][Nb], then masses [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  __shared__ uint32_t s_hist[4][256];

  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  score_rows(qbar, kbart, Nb, bh, g0, nr, s_qb, s_keys);

  const int lane = t & 63, w = t >> 6;
  uint32_t* hist = s_hist[w];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = w; r < nr; r += 4) {
    const uint64_t* keys = s_keys + r * Nb;
    double* mass = (double*)(s_keys + (size_t)R * Nb) + (size_t)r * Nb;
    uint64_t kmax = 0u;
    for (int j = lane; j < Nb; j += 64) kmax = max(kmax, keys[j]);
    for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint64_t)__shfl_xor((long long)kmax, o));
    const double mx = key_value(kmax);
    double part = 0.0;
    for (int j = lane; j < Nb; j += 64) {
      const double m = (double)block_len(j, N) * exp(key_value(keys[j]) - mx);
      mass[j] = m;
      part += m;
    }
    const double T = tau * wave_sum(part);
    // mass of the k largest keys (ties: the lower indices)
    auto top_mass = [&](int k) {
      const Threshold th = radix_threshold(keys, Nb, k, hist, lane);
      double acc = 0.0;
      int eq_seen = 0;
      for (int j0 = 0; j0 < Nb; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t um = j < Nb ? (keys[j] & th.mask) : 0u;
        const bool eq = j < Nb && um == th.prefix;
        const unsigned long long eqm = __ballot(eq);
        const int eq_rank = eq_seen + __popcll(eqm & below);
        if (j < Nb && (um > th.prefix || (eq && eq_rank < th.kk))) acc += mass[j];
        eq_seen += __popcll(eqm);
      }
      return wave_sum(acc);
    };
    int lo = 1, hi = Nb;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (top_mass(mid) >= T)
        hi = mid;
      else
        lo = mid + 1;
    }
    if (lane == 0) k_rows[(size_t)bh * Nb + g0 + r] = lo;
  }
}

// A head's count from its rows' counts: clamp(ceil(sum / Nb), kmin, kmax) on integers.
__global__ __launch_bounds__(256) void adaptive_head_kernel(const int32_t* __restrict__ k_rows, int Nb, int kmin,
                                                            int kmax, int32_t* __restrict__ khead) {
  __shared__ long long s_part[4];
  const int bh = blockIdx.x, t = threadIdx.x;
  long long sum = 0;
  for (int i = t; i < Nb; i += 256) sum += k_rows[(size_t)bh * Nb + i];
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if ((t & 63) == 0) s_part[t >> 6] = sum;
  __syncthreads();
  if (t == 0) {
    const long long tot = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    long long k = (tot + Nb - 1) / Nb;
    k = k < kmin ? kmin : (k > kmax ? kmax : k);
    khead[bh] = (int32_t)k;
  }
}

int select_rows_per_group(int Nb) {
  int R = 8192 / Nb;  // keys of R rows in at most 64 KiB of LDS (one row up to 128 KiB)
  return R < 1 ? 1 : (R > 8 ? 8 : R);
}

// khead: per-head counts (int32 [BH]) or NULL for ksel everywhere; kstride >= every count.
hipError_t launch_select(const void* qbar, const void* kbart, int BH, int Nb, int ksel, const void* khead,
                         int kstride, void* idx, hipStream_t st) {
  const int R = select_rows_per_group(Nb);
  const int groups = (Nb + R - 1) / R;
  size_t lds = (size_t)R * Nb * sizeof(uint64_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3(BH * groups), dim3(kSelThreads), lds, st, (const double*)qbar,
                     (const double*)kbart, Nb, ksel, (const int32_t*)khead, kstride, R, groups, (int32_t*)idx);
  return hipGetLastError();
}

hipError_t launch_select(const void* qbar, const void* kbart, int BH, int Nb, int ksel, void* idx,
                         hipStream_t st) {
  return launch_select(qbar, kbart, BH, Nb, ksel, nullptr, ksel, idx, st);
}

// The largest Nb the adaptive count supports: one row's keys and masses in 128 KiB of LDS.
int adaptive_max_blocks() { return 8192; }

hipError_t launch_adaptive_ksel(const void* qbar, const void* kbart, int BH, int N, int Nb, double tau, int kmin,
                                int kmax, void* k_rows, void* khead, hipStream_t st) {
  int R = 4096 / Nb;
  R = R < 1 ? 1 : (R > 8 ? 8 : R);
  const int groups = (Nb + R - 1) / R;
  const size_t lds = (size_t)R * Nb * 16;
  if (lds > 65536) {
    hipError_t e =
        hipFuncSetAttribute((const void*)adaptive_k_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(adaptive_k_kernel, dim3(BH * groups), dim3(kSelThreads), lds, st, (const double*)qbar,
                     (const double*)kbart, N, Nb, tau, R, groups, (int32_t*)k_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adaptive_head_kernel, dim3(BH), dim3(256), 0, st, (const int32_t*)k_rows, Nb, kmin, kmax,
                     (int32_t*)khead);
  return hipGetLastError();
}

}  // namespace sagesla
