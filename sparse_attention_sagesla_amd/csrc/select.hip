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

__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* s_u) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  if ((threadIdx.x & 63) == 0) s_u[threadIdx.x >> 6] = x;
  __syncthreads();
  x = max(max(s_u[0], s_u[1]), max(s_u[2], s_u[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ int block_min_i32(int x, uint32_t* s_u) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) s_u[threadIdx.x >> 6] = (uint32_t)x;
  __syncthreads();
  x = min(min((int)s_u[0], (int)s_u[1]), min((int)s_u[2], (int)s_u[3]));
  __syncthreads();
  return x;
}

// exclusive prefix sum over the 256 threads of the block; returns this thread's prefix,
// *total receives the block total. Uses s_tmp[4 + 1].
__device__ __forceinline__ int block_excl_scan(int x, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
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
    int c = s_tmp[k];
    if (k < w) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + incl - x;
}

// R query blocks of one head per workgroup. Dynamic LDS: keys [R][Nb] uint32.
__global__ __launch_bounds__(kSelThreads) void select_kernel(const double* __restrict__ qbar,
                                                             const double* __restrict__ kbart, int Nb,
                                                             int ksel, int R, int groups,
                                                             int32_t* __restrict__ idx) {
  extern __shared__ uint32_t s_keys[];  // [R][Nb]
  __shared__ double s_qb[8][kD];
  __shared__ int s_hist[256];
  __shared__ int s_tmp[8];
  __shared__ int s_sel[2];
  __shared__ uint32_t s_red[4];

  const int bh = blockIdx.x / groups, g0 = (blockIdx.x % groups) * R;
  const int nr = min(R, Nb - g0);
  const int t = threadIdx.x;
  for (int e = t; e < nr * kD; e += kSelThreads)
    s_qb[e / kD][e % kD] = qbar[((size_t)bh * Nb + g0 + e / kD) * kD + e % kD];
  __syncthreads();

  // scores: thread per key block j, R rows at once; kbart is channel-major so the
  // loads of consecutive threads are contiguous.
  const double inv_sqrt_d = 1.0 / sqrt((double)kD);
  const double* kb = kbart + (size_t)bh * kD * Nb;
  for (int j = t; j < Nb; j += kSelThreads) {
    double acc[8];
#pragma unroll
    for (int r = 0; r < 8; r++) acc[r] = 0.0;
    for (int c = 0; c < kD; c++) {
      double kv = kb[(size_t)c * Nb + j];
#pragma unroll
      for (int r = 0; r < 8; r++)
        if (r < nr) acc[r] = __fma_rn(s_qb[r][c], kv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < 8; r++)
      if (r < nr) s_keys[r * Nb + j] = ord_key((float)(acc[r] * inv_sqrt_d));
  }
  __syncthreads();

  const int per = (Nb + kSelThreads - 1) / kSelThreads;  // contiguous range per thread
  for (int r = 0; r < nr; r++) {
    const uint32_t* keys = s_keys + r * Nb;
    // radix select (4 x 8 bits, most significant first) of the ksel-th largest key
    uint32_t prefix = 0, mask = 0;
    int kk = ksel;
    for (int pass = 0; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
      s_hist[t] = 0;
      __syncthreads();
      for (int j = t; j < Nb; j += kSelThreads) {
        uint32_t u = keys[j];
        if ((u & mask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (t < 64) {
        // lane t owns bins 4t..4t+3; suffix sums from the top bin down
        int h0 = s_hist[4 * t], h1 = s_hist[4 * t + 1], h2 = s_hist[4 * t + 2], h3 = s_hist[4 * t + 3];
        int loc = h0 + h1 + h2 + h3;
        int suf = loc;  // inclusive suffix over lanes >= t
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          int y = __shfl_down(suf, o);
          if (t + o < 64) suf += y;
        }
        int above = suf - loc;  // keys in bins above this lane's four
        int hs[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int b = 3; b >= 0; b--) {
          if (above < kk && above + hs[b] >= kk) {
            s_sel[0] = 4 * t + b;
            s_sel[1] = kk - above;
          }
          above += hs[b];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_sel[0] << shift;
      mask |= 255u << shift;
      kk = s_sel[1];
      __syncthreads();
    }
    // the best block (highest key, lowest index) goes first
    const int j0 = t * per, j1 = min(Nb, j0 + per);
    uint32_t kmax = 0u;
    for (int j = j0; j < j1; j++) kmax = max(kmax, keys[j]);
    kmax = block_max_u32(kmax, s_red);
    int jb = INT_MAX;
    for (int j = j0; j < j1; j++)
      if (keys[j] == kmax) { jb = j; break; }
    jb = block_min_i32(jb, s_red);
    // keys > prefix are all kept; of the keys == prefix keep the kk lowest indices
    int n_eq = 0;
    for (int j = j0; j < j1; j++) n_eq += (keys[j] == prefix);
    int tot;
    int eq_before = block_excl_scan(n_eq, s_tmp, &tot);
    int n_keep = 0;
    {
      int e = eq_before;
      for (int j = j0; j < j1; j++) {
        uint32_t u = keys[j];
        bool keep = false;
        if (u > prefix) keep = true;
        else if (u == prefix) { keep = (e < kk); e++; }
        n_keep += keep && j != jb;
      }
    }
    int pos = 1 + block_excl_scan(n_keep, s_tmp, &tot);
    int32_t* out = idx + ((size_t)bh * Nb + g0 + r) * ksel;
    if (t == 0) out[0] = jb;
    {
      int e = eq_before;
      for (int j = j0; j < j1; j++) {
        uint32_t u = keys[j];
        bool keep = false;
        if (u > prefix) keep = true;
        else if (u == prefix) { keep = (e < kk); e++; }
        if (keep && j != jb) out[pos++] = j;
      }
    }
    __syncthreads();
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
