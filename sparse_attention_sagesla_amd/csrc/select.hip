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

// The second half of a radix pass, from the wave's 256-bin histogram of the keys still
// matching th: the bin (digits at shift) that holds the kk-th largest, counted from the top
// bin down. Returns whether that whole bin is kept (the selection is then complete).
__device__ __forceinline__ bool radix_pick(const uint32_t* hist, int lane, int shift, Threshold& th) {
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
  return sel_n == sel_k;  // every key of the bin is kept
}

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
    if (radix_pick(hist, lane, shift, th)) break;
  }
  return th;
}

// The same selection with a row's keys in registers: lane l holds keys l + 64 m (m < M;
// entries at or past Nb are excluded), so no pass waits on an LDS read of the keys.
template <int M>
__device__ Threshold radix_threshold_regs(const uint64_t (&key)[M], int Nb, int k, uint32_t* hist, int lane) {
  Threshold th = {0u, 0u, k};
  for (int pass = 0; pass < 8; pass++) {
    const int shift = 56 - 8 * pass;
#pragma unroll
    for (int b = 0; b < 4; b++) hist[4 * lane + b] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < M; m++) {
      if (64 * m >= Nb) break;  // uniform: the row's last key slot
      if (lane + 64 * m < Nb && (key[m] & th.mask) == th.prefix)
        atomicAdd(&hist[(uint32_t)(key[m] >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    if (radix_pick(hist, lane, shift, th)) break;
  }
  return th;
}

// One row's selection by one wave, its keys in registers (Nb <= 64 M): the kept indices
// best first, then ascending; positions from ks to kstride are set to -1.
template <int M>
__device__ void select_row_regs(const uint64_t* keys, int Nb, int ks, int kstride, uint32_t* hist, int lane,
                                int32_t* out) {
  const unsigned long long below = (1ull << lane) - 1ull;
  uint64_t key[M];
#pragma unroll
  for (int m = 0; m < M; m++) key[m] = lane + 64 * m < Nb ? keys[lane + 64 * m] : 0u;
  const Threshold th = radix_threshold_regs<M>(key, Nb, ks, hist, lane);
  const uint64_t prefix = th.prefix, mask = th.mask;
  const int kk = th.kk;
  // best block: highest key, lowest index (each lane's candidate, then the wave's)
  uint64_t kbest = 0u;
  int jb = INT_MAX;
#pragma unroll
  for (int m = 0; m < M; m++) {
    if (64 * m >= Nb) break;
    if (lane + 64 * m < Nb && key[m] > kbest) {
      kbest = key[m];
      jb = lane + 64 * m;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t ko = (uint64_t)__shfl_xor((long long)kbest, o);
    const int jo = __shfl_xor(jb, o);
    if (ko > kbest || (ko == kbest && jo < jb)) {
      kbest = ko;
      jb = jo;
    }
  }
  if (lane == 0) out[0] = jb;
  for (int p = ks + lane; p < kstride; p += 64) out[p] = -1;
  int pos = 1, eq_seen = 0;
#pragma unroll
  for (int m = 0; m < M; m++) {
    if (64 * m >= Nb) break;
    const int j = 64 * m + lane;
    const uint64_t um = j < Nb ? (key[m] & mask) : 0u;
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
                                                             int kstride, const uint64_t* __restrict__ keys_in,
                                                             int R, int groups, int32_t* __restrict__ idx) {
  extern __shared__ uint64_t s_keys[];  // [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  __shared__ uint32_t s_hist[4][256];

  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  const int ks = khead ? khead[bh] : ksel;
  if (keys_in) {  // the scores' keys, already computed for these rows
    const uint64_t* src = keys_in + ((size_t)bh * Nb + g0) * Nb;
    for (int e = t; e < nr * Nb; e += kSelThreads) s_keys[e] = src[e];
    __syncthreads();
  } else {
    score_rows(qbar, kbart, Nb, bh, g0, nr, s_qb, s_keys);
  }

  // ---- phase 2: one wave per row
  const int lane = t & 63, w = t >> 6;
  uint32_t* hist = s_hist[w];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = w; r < nr; r += 4) {
    const uint64_t* keys = s_keys + r * Nb;
    int32_t* orow = idx + ((size_t)bh * Nb + g0 + r) * kstride;
    if (Nb <= 64 * 32) {  // keys in registers (the branch is uniform)
      if (Nb <= 64 * 8)
        select_row_regs<8>(keys, Nb, ks, kstride, hist, lane, orow);
      else if (Nb <= 64 * 16)
        select_row_regs<16>(keys, Nb, ks, kstride, hist, lane, orow);
      else
        select_row_regs<32>(keys, Nb, ks, kstride, hist, lane, orow);
      continue;
    }
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
// mass n_j exp(s_j - max s) reaches T = tau * (row total). The row's keys and masses sit
// in registers of a team of threads (one wave, or the whole workgroup for long rows):
// team member p holds key blocks p + P m (m < M, P the team size).
// With mass_ge(x) = the mass of the keys >= x (each member's sum in m order, then the
// team's fixed reduction tree: every member gets the same bits, and the sum never grows
// as x grows), the last block taken has the largest key x* with mass_ge(x*) >= T.
// Bisection on the 64-bit key space finds it: the interval [lo, hi] holds x*,
// mass_ge(lo) >= T and mass_ge(hi + 1) < T, and the search stops as soon as one key is
// left in it. Then k = #(keys > x*) + r, where r counts the blocks with key x* that are
// needed, in index order (1 unless scores are exactly equal).

// Reductions over one wave.
struct WaveTeam {
  static constexpr int P = 64;
  int lane;
  __device__ int member() const { return lane; }
  __device__ void sum(double& a, int& c) {
    a = wave_sum(a);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  }
  __device__ void max2(uint64_t& x, uint64_t& y) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      x = max(x, (uint64_t)__shfl_xor((long long)x, o));
      y = max(y, (uint64_t)__shfl_xor((long long)y, o));
    }
  }
  __device__ int from_leader(int v) { return __shfl(v, 0); }
};

// Reductions over the workgroup's four waves: the waves' butterflies, then the four
// partial results in wave order from LDS. Two sets of slots used in turn, so one barrier
// per reduction suffices.
struct GroupTeam {
  static constexpr int P = kSelThreads;
  int t, lane, w, par;
  double (*rd)[4];
  int (*ri)[4];
  uint64_t (*ru)[4][2];
  __device__ int member() const { return t; }
  __device__ void sum(double& a, int& c) {
    a = wave_sum(a);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) {
      rd[par][w] = a;
      ri[par][w] = c;
    }
    __syncthreads();
    a = ((rd[par][0] + rd[par][1]) + rd[par][2]) + rd[par][3];
    c = ri[par][0] + ri[par][1] + ri[par][2] + ri[par][3];
    par ^= 1;
  }
  __device__ void max2(uint64_t& x, uint64_t& y) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      x = max(x, (uint64_t)__shfl_xor((long long)x, o));
      y = max(y, (uint64_t)__shfl_xor((long long)y, o));
    }
    if (lane == 0) {
      ru[par][w][0] = x;
      ru[par][w][1] = y;
    }
    __syncthreads();
    x = max(max(ru[par][0][0], ru[par][1][0]), max(ru[par][2][0], ru[par][3][0]));
    y = max(max(ru[par][0][1], ru[par][1][1]), max(ru[par][2][1], ru[par][3][1]));
    par ^= 1;
  }
  __device__ int from_leader(int v) {
    if (t == 0) ri[par][0] = v;
    __syncthreads();
    v = ri[par][0];
    par ^= 1;
    return v;
  }
};

// The count of one row (keys in LDS), the same value on every team member.
template <int M, class Team>
__device__ int row_count(const uint64_t* keys, int Nb, int N, double tau, Team& tm) {
  const int p = tm.member();
  // keys of absent blocks are 0, below the key of every finite score, with mass 0
  uint64_t kv[M];
  double mv[M];
  uint64_t kmax = 0u, nmin = 0u;  // nmin: the largest ~key, i.e. ~(smallest key)
#pragma unroll
  for (int m = 0; m < M; m++) {
    const int j = p + Team::P * m;
    kv[m] = j < Nb ? keys[j] : 0u;
    kmax = max(kmax, kv[m]);
    if (j < Nb) nmin = max(nmin, ~kv[m]);
  }
  tm.max2(kmax, nmin);
  const double mx = key_value(kmax);
  double W = 0.0;
  int cnt = 0;
#pragma unroll
  for (int m = 0; m < M; m++) {
    const int j = p + Team::P * m;
    mv[m] = j < Nb ? (double)block_len(j, N) * exp(key_value(kv[m]) - mx) : 0.0;
    W += mv[m];
  }
  tm.sum(W, cnt);
  const double T = tau * W;
  uint64_t lo = ~nmin, hi = kmax;
  cnt = Nb;  // keys in [lo, hi]
  while (cnt > 1 && lo < hi) {
    const uint64_t mid = hi - ((hi - lo) >> 1);  // in (lo, hi]
    double a = 0.0;
    int c = 0;
#pragma unroll
    for (int m = 0; m < M; m++) {
      const bool ge = kv[m] >= mid;
      a += ge ? mv[m] : 0.0;
      c += (ge && kv[m] <= hi) ? 1 : 0;
    }
    tm.sum(a, c);
    if (a >= T) {
      lo = mid;
      cnt = c;
    } else {
      hi = mid - 1;
      cnt -= c;
    }
  }
  // x*: the key in [lo, hi] (the only one, or lo == hi)
  uint64_t xs = 0u, unused = 0u;
#pragma unroll
  for (int m = 0; m < M; m++)
    if (kv[m] >= lo && kv[m] <= hi) xs = max(xs, kv[m]);
  tm.max2(xs, unused);
  double mgt = 0.0;
  int cpk = 0;
#pragma unroll
  for (int m = 0; m < M; m++) {
    mgt += kv[m] > xs ? mv[m] : 0.0;
    cpk += (kv[m] > xs ? 1 : 0) + (kv[m] == xs ? 65536 : 0);
  }
  tm.sum(mgt, cpk);
  const int cgt = cpk & 0xFFFF, neq = cpk >> 16;
  int r = 1;
  if (neq > 1) {
    // equal scores at the boundary: taken in index order until the mass reaches T
    if (p == 0) {
      double run = mgt;
      r = 0;
      for (int j = 0; j < Nb && r < neq; j++) {
        if (keys[j] != xs) continue;
        r++;
        run += (double)block_len(j, N) * exp(key_value(keys[j]) - mx);
        if (run >= T) break;
      }
    }
    r = tm.from_leader(r);
  }
  return cgt + r;
}

// One wave per row (rows of up to 64 M key blocks). R rows per workgroup as in
// select_kernel; dynamic LDS: keys [R][Nb]. keys_out (may be NULL): the rows' keys
// [BH][Nb][Nb], for the selection that follows.
template <int M>
__global__ __launch_bounds__(kSelThreads) void adaptive_k_wave_kernel(const double* __restrict__ qbar,
                                                                      const double* __restrict__ kbart, int N,
                                                                      int Nb, double tau, int R, int groups,
                                                                      int32_t* __restrict__ k_rows,
                                                                      uint64_t* __restrict__ keys_out) {
  extern __shared__ uint64_t s_keys[];  // [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  score_rows(qbar, kbart, Nb, bh, g0, nr, s_qb, s_keys);
  if (keys_out) {
    uint64_t* dst = keys_out + ((size_t)bh * Nb + g0) * Nb;
    for (int e = t; e < nr * Nb; e += kSelThreads) dst[e] = s_keys[e];
  }
  WaveTeam tm{t & 63};
  for (int r = t >> 6; r < nr; r += 4) {
    const int k = row_count<M>(s_keys + r * Nb, Nb, N, tau, tm);
    if (tm.lane == 0) k_rows[(size_t)bh * Nb + g0 + r] = k;
  }
}

// The whole workgroup per row (rows of up to 256 M key blocks), rows one after another.
template <int M>
__global__ __launch_bounds__(kSelThreads) void adaptive_k_group_kernel(const double* __restrict__ qbar,
                                                                       const double* __restrict__ kbart, int N,
                                                                       int Nb, double tau, int R, int groups,
                                                                       int32_t* __restrict__ k_rows,
                                                                       uint64_t* __restrict__ keys_out) {
  extern __shared__ uint64_t s_keys[];  // [R][Nb]
  __shared__ __attribute__((aligned(16))) double s_qb[8][kD];
  __shared__ double s_rd[2][4];
  __shared__ int s_ri[2][4];
  __shared__ uint64_t s_ru[2][4][2];
  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  score_rows(qbar, kbart, Nb, bh, g0, nr, s_qb, s_keys);
  if (keys_out) {
    uint64_t* dst = keys_out + ((size_t)bh * Nb + g0) * Nb;
    for (int e = t; e < nr * Nb; e += kSelThreads) dst[e] = s_keys[e];
  }
  GroupTeam tm{t, t & 63, t >> 6, 0, s_rd, s_ri, s_ru};
  for (int r = 0; r < nr; r++) {
    const int k = row_count<M>(s_keys + r * Nb, Nb, N, tau, tm);
    if (t == 0) k_rows[(size_t)bh * Nb + g0 + r] = k;
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
// keys_in: the rows' score keys (uint64 [BH][Nb][Nb], from the adaptive count) or NULL.
hipError_t launch_select(const void* qbar, const void* kbart, int BH, int Nb, int ksel, const void* khead,
                         int kstride, const void* keys_in, void* idx, hipStream_t st) {
  const int R = select_rows_per_group(Nb);
  const int groups = (Nb + R - 1) / R;
  size_t lds = (size_t)R * Nb * sizeof(uint64_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3(BH * groups), dim3(kSelThreads), lds, st, (const double*)qbar,
                     (const double*)kbart, Nb, ksel, (const int32_t*)khead, kstride, (const uint64_t*)keys_in, R,
                     groups, (int32_t*)idx);
  return hipGetLastError();
}

hipError_t launch_select(const void* qbar, const void* kbart, int BH, int Nb, int ksel, void* idx,
                         hipStream_t st) {
  return launch_select(qbar, kbart, BH, Nb, ksel, nullptr, ksel, nullptr, idx, st);
}

// The largest Nb the adaptive count supports: 32 key blocks per thread.
int adaptive_max_blocks() { return 32 * kSelThreads; }

template <class K>
static hipError_t launch_adaptive_k(K kernel, const void* qbar, const void* kbart, int BH, int N, int Nb, double tau,
                                    void* k_rows, void* keys_out, hipStream_t st) {
  const int R = select_rows_per_group(Nb);
  const int groups = (Nb + R - 1) / R;
  const size_t lds = (size_t)R * Nb * sizeof(uint64_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(BH * groups), dim3(kSelThreads), lds, st, (const double*)qbar,
                     (const double*)kbart, N, Nb, tau, R, groups, (int32_t*)k_rows, (uint64_t*)keys_out);
  return hipGetLastError();
}

// keys_out: uint64 [BH][Nb][Nb] or NULL
hipError_t launch_adaptive_ksel(const void* qbar, const void* kbart, int BH, int N, int Nb, double tau, int kmin,
                                int kmax, void* k_rows, void* khead, void* keys_out, hipStream_t st) {
  hipError_t e;
#define SAGESLA_ADAPTIVE_K(KER) e = launch_adaptive_k(KER, qbar, kbart, BH, N, Nb, tau, k_rows, keys_out, st)
  if (Nb <= 64 * 4)
    SAGESLA_ADAPTIVE_K(adaptive_k_wave_kernel<4>);
  else if (Nb <= 64 * 8)
    SAGESLA_ADAPTIVE_K(adaptive_k_wave_kernel<8>);
  else if (Nb <= 64 * 16)
    SAGESLA_ADAPTIVE_K(adaptive_k_wave_kernel<16>);
  else if (Nb <= 64 * 32)
    SAGESLA_ADAPTIVE_K(adaptive_k_wave_kernel<32>);
  else if (Nb <= kSelThreads * 16)
    SAGESLA_ADAPTIVE_K(adaptive_k_group_kernel<16>);
  else
    SAGESLA_ADAPTIVE_K(adaptive_k_group_kernel<32>);
#undef SAGESLA_ADAPTIVE_K
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(adaptive_head_kernel, dim3(BH), dim3(256), 0, st, (const int32_t*)k_rows, Nb, kmin, kmax,
                     (int32_t*)khead);
  return hipGetLastError();
}

}  // namespace sagesla
