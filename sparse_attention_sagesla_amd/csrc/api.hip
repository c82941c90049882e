// C ABI of the SageSLA forward: argument validation, workspace layout and the launch
// sequence pool -> head stats -> select -> quantize K/V (+ linear states) -> linear
// totals -> linear complement -> sparse attention with the fused epilogue.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/sagesla.h"
#include "common.h"

namespace sagesla {
hipError_t launch_pool(const void*, const void*, const void*, int, int, int, void*, void*, void*, void*,
                       void*, void*, hipStream_t);
hipError_t launch_head_stats(const void*, const void*, int, int, int, void*, void*, hipStream_t);
hipError_t launch_select(const void*, const void*, int, int, int, void*, hipStream_t);
hipError_t launch_select(const void*, const void*, int, int, int, const void*, int, const void*, void*, hipStream_t);
int adaptive_max_blocks();
hipError_t launch_adaptive_ksel(const void*, const void*, int, int, int, double, int, int, void*, void*, void*,
                                hipStream_t);
hipError_t launch_quant_kv(const void*, const void*, const void*, const void*, int, int, int, void*, void*,
                           void*, void*, void*, hipStream_t);
hipError_t launch_linear_total(const void*, int, int, void*, hipStream_t);
hipError_t launch_linear_complement(const void*, const void*, const void*, const void*, const void*, int, int,
                                    int, int, void*, void*, void*, void*, void*, hipStream_t);
hipError_t launch_linear_union(const void*, int, int, int, void*, void*, void*, hipStream_t);
hipError_t launch_linear_masked(const void*, const void*, const void*, const void*, int, int, int, int, const void*,
                                const void*, const void*, void*, void*, hipStream_t);
hipError_t launch_linear_complement(const void*, const void*, const void*, int, const void*, const void*, const void*,
                                    int, int, int, int, void*, void*, void*, void*, void*, hipStream_t);
hipError_t launch_sparse_attn(const void*, const void*, const void*, const void*, const void*, const void*,
                              const void*, const void*, int, int, int, int, void*, hipStream_t);
hipError_t launch_sparse_attn(const void*, const void*, const void*, const void*, const void*, const void*,
                              const void*, const void*, int, const void*, int, int, int, int, void*, hipStream_t);
hipError_t launch_sla_relayout(const void*, int, int, int, void*, hipStream_t);
hipError_t launch_sla_kept_mask(const void*, int, int, int, void*, hipStream_t);
hipError_t launch_sla_relayout_hd(const void*, int, int, int, void*, hipStream_t);
hipError_t launch_sla_fwd(const void*, const void*, const void*, const void*, const void*, int, int, int, int, void*,
                          void*, void*, hipStream_t);
hipError_t launch_sla_bwd_dq(const void*, const void*, const void*, const void*, const void*, const void*, const void*,
                             int, int, int, int, void*, void*, hipStream_t);
hipError_t launch_sla_bwd_dkdv(const void*, const void*, const void*, const void*, const void*, const void*,
                               const void*, int, int, int, void*, void*, hipStream_t);
hipError_t launch_sla_lin_bwd_q(const void*, const void*, const void*, const void*, int, int, int, void*, void*, void*,
                                void*, void*, hipStream_t);
hipError_t launch_sla_lin_dhc(const void*, const void*, const void*, int, int, int, void*, void*, hipStream_t);
hipError_t launch_sla_union_t(const void*, int, int, int, void*, void*, void*, hipStream_t);
hipError_t launch_linear_mask_gemm(const void*, const void*, const void*, const void*, const void*, int, int, int,
                                   void*, hipStream_t);
hipError_t launch_sla_lin_bwd_k(const void*, const void*, const void*, int, int, int, void*, void*, hipStream_t);
hipError_t launch_sla_dw(const void*, const void*, int, void*, void*, hipStream_t);
int sla_dw_parts();
hipError_t launch_sla_zero(void*, size_t, hipStream_t);
hipError_t launch_prepare(const void*, const void*, const void*, double, int, int, int, int, void*, void*, void*,
                          void*, void*, void*, void*, void*, void*, void*, hipStream_t);
int w8a8_row_tiles(int M);
hipError_t launch_w8a8_quant_act(const void*, int, int, void*, void*, hipStream_t);
hipError_t launch_w8a8_quant_weight(const void*, int, int, void*, void*, hipStream_t);
hipError_t launch_w8a8_gemm(const void*, const void*, const void*, const void*, const void*, int, int, int, void*,
                            hipStream_t);
}  // namespace sagesla

using namespace sagesla;

namespace {

constexpr int kMaxN = 1 << 20;

struct Geom {
  int BH, N, Nb, ksel, Nc, Ng;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int ksel_of(int Nb, double topk) {
  double x = ceil(topk * (double)Nb - 1e-9);
  int k = (int)x;
  if (k < 1) k = 1;
  if (k > Nb) k = Nb;
  return k;
}

// Host-only validation of the sizes shared by every entry point.
sagesla_status check_sizes(int B, int H, int N, int d, int block, Geom* gm) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return SAGESLA_ERR_INVALID_ARGUMENT;
  if (d != kD || block != kBlk) return SAGESLA_ERR_UNSUPPORTED;
  long long BH = (long long)B * H;
  int Nb = (N + kBlk - 1) / kBlk;
  if (BH * Nb >= (1LL << 31) || BH * N >= (1LL << 40)) return SAGESLA_ERR_INVALID_ARGUMENT;
  gm->BH = (int)BH;
  gm->N = N;
  gm->Nb = Nb;
  gm->Nc = (Nb + kChunk - 1) / kChunk;
  gm->Ng = (Nb + kGroup - 1) / kGroup;
  gm->ksel = Nb;
  return SAGESLA_OK;
}

sagesla_status check_topk(double topk, Geom* gm) {
  if (!(topk > 0.0 && topk <= 1.0)) return SAGESLA_ERR_INVALID_ARGUMENT;
  gm->ksel = ksel_of(gm->Nb, topk);
  return SAGESLA_OK;
}

// Content-adaptive counts: 0 < topk_min <= topk_max <= 1, 0 < tau <= 1, and at most
// adaptive_max_blocks() key blocks. gm->ksel becomes the largest count (the row stride of
// the kept lists); *kmin the smallest.
sagesla_status check_adaptive(double topk_min, double topk_max, double tau, Geom* gm, int* kmin) {
  if (!(topk_min > 0.0 && topk_min <= topk_max && topk_max <= 1.0) || !(tau > 0.0 && tau <= 1.0))
    return SAGESLA_ERR_INVALID_ARGUMENT;
  if (gm->Nb > adaptive_max_blocks()) return SAGESLA_ERR_UNSUPPORTED;
  *kmin = ksel_of(gm->Nb, topk_min);
  gm->ksel = ksel_of(gm->Nb, topk_max);
  return SAGESLA_OK;
}

sagesla_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return SAGESLA_ERR_INVALID_ARGUMENT;
  return SAGESLA_OK;
}

sagesla_status check_opt_ptr(const void* p) {
  return (p != nullptr && !aligned16(p)) ? SAGESLA_ERR_INVALID_ARGUMENT : SAGESLA_OK;
}

// The current device must be gfx950 (checked once per device).
sagesla_status check_device() {
  static std::mutex mu;
  static int state[64];  // 0 unknown, 1 ok, 2 unsupported
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGESLA_ERR_HIP;
  if (dev < 0 || dev >= 64) return SAGESLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SAGESLA_ERR_HIP;
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  return state[dev] == 1 ? SAGESLA_OK : SAGESLA_ERR_UNSUPPORTED;
}

sagesla_status from_hip(hipError_t e) { return e == hipSuccess ? SAGESLA_OK : SAGESLA_ERR_HIP; }

// A second stream per device on which the forward runs the key-block selection (and the
// union of the kept lists) beside the K/V quantization and the linear-state totals: both
// need only the pooling and the head statistics, and the selection is bound by fp64 and
// LDS work where the quantization is bound by HBM. The stream and its two events are created on first use (not while the
// caller's stream is being captured) and kept until the process ends; the stream has the
// default priority. fork_mu is held from the fork to the join, so that concurrent callers
// never interleave their uses of the two events.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ready = false, failed = false;
};
static std::mutex side_mu, fork_mu;
static SideStream side_streams[64];

static SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(side_mu);
  SideStream& ss = side_streams[dev];
  if (ss.ready) return &ss;
  if (ss.failed) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
    ss.failed = true;  // the forward then runs on the caller's stream alone
    return nullptr;
  }
  ss.ready = true;
  return &ss;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// keys: the score-key region of the adaptive forward
void layout(const Geom& gm, bool linear, size_t off[SAGESLA_WS_COUNT], size_t* total, bool keys = false) {
  const size_t BH = gm.BH, Nb = gm.Nb, N = gm.N, D = kD, Nc = gm.Nc, Ng = gm.Ng, ks = gm.ksel;
  const size_t SE = kStateElems;
  size_t sz[SAGESLA_WS_COUNT] = {};
  sz[SAGESLA_WS_QBAR] = BH * Nb * D * 8;
  sz[SAGESLA_WS_KBART] = BH * Nb * D * 8;
  sz[SAGESLA_WS_KSUM] = BH * Nb * D * 8;
  sz[SAGESLA_WS_VAMAXB] = BH * Nb * D * 4;
  sz[SAGESLA_WS_KMEAN] = BH * D * 4;
  sz[SAGESLA_WS_VAMAX] = BH * D * 4;
  sz[SAGESLA_WS_Q8] = BH * Nb * kBlkBytes;
  sz[SAGESLA_WS_SQ] = BH * Nb * 4;
  sz[SAGESLA_WS_K8] = BH * Nb * kBlkBytes;
  sz[SAGESLA_WS_SK] = BH * Nb * 4;
  sz[SAGESLA_WS_V8] = BH * Nb * kBlkBytes;
  sz[SAGESLA_WS_IDX] = BH * Nb * ks * 4;
  if (linear) {
    sz[SAGESLA_WS_HS] = BH * Nb * SE * 2;
    sz[SAGESLA_WS_HPART] = BH * Nc * SE * 4;
    sz[SAGESLA_WS_HTOT] = BH * SE * 4;
    sz[SAGESLA_WS_ULIST] = BH * Ng * Nb * 4;
    sz[SAGESLA_WS_UMASK] = BH * Ng * kGroup * ((Nb + 31) / 32) * 4;
    sz[SAGESLA_WS_UCOUNT] = BH * Ng * 4;
    sz[SAGESLA_WS_HC] = BH * Nb * SE * 2;
    sz[SAGESLA_WS_Y] = BH * N * D * 2;
  }
  if (keys) sz[SAGESLA_WS_KEYS] = BH * Nb * Nb * 8;
  size_t o = 0;
  for (int r = 0; r < SAGESLA_WS_COUNT; r++) {
    if (sz[r] == 0) continue;
    off[r] = o;
    o += align256(sz[r]);
  }
  for (int r = 0; r < SAGESLA_WS_COUNT; r++)
    if (sz[r] == 0) off[r] = o;
  *total = o;
}

}  // namespace

extern "C" {

int sagesla_version(void) { return 100; }

const char* sagesla_status_string(sagesla_status s) {
  switch (s) {
    case SAGESLA_OK: return "ok";
    case SAGESLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SAGESLA_ERR_UNSUPPORTED:
      return "unsupported (d must be 128, block 64, device gfx950; the adaptive count takes at most 8192 blocks)";
    case SAGESLA_ERR_WORKSPACE: return "workspace too small";
    case SAGESLA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

sagesla_status sagesla_ksel(int N, int block, double topk, int* ksel) {
  Geom gm;
  if (!ksel) return SAGESLA_ERR_INVALID_ARGUMENT;
  sagesla_status s = check_sizes(1, 1, N, kD, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  *ksel = gm.ksel;
  return SAGESLA_OK;
}

sagesla_status sagesla_workspace_layout(int B, int H, int N, int d, int block, double topk, int linear,
                                        size_t offsets[SAGESLA_WS_COUNT]) {
  Geom gm;
  if (!offsets) return SAGESLA_ERR_INVALID_ARGUMENT;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  size_t total;
  layout(gm, linear != 0 && gm.ksel < gm.Nb, offsets, &total);
  return SAGESLA_OK;
}

sagesla_status sagesla_workspace_size(int B, int H, int N, int d, int block, double topk, int linear,
                                      size_t* bytes) {
  Geom gm;
  if (!bytes) return SAGESLA_ERR_INVALID_ARGUMENT;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  size_t off[SAGESLA_WS_COUNT];
  layout(gm, linear != 0 && gm.ksel < gm.Nb, off, bytes);
  return SAGESLA_OK;
}

static sagesla_status run_fwd(const void* q, const void* k, const void* v, const void* proj, int B, int H, int N,
                              int d, double topk, int block, void* out, void* workspace, size_t workspace_bytes,
                              sagesla_stream_t stream, bool pooled, bool fork = true);

sagesla_status sagesla_fwd(const void* q, const void* k, const void* v, const void* proj, int B, int H, int N,
                           int d, double topk, int block, void* out, void* workspace, size_t workspace_bytes,
                           sagesla_stream_t stream) {
  return run_fwd(q, k, v, proj, B, H, N, d, topk, block, out, workspace, workspace_bytes, stream, false);
}

sagesla_status sagesla_fwd_prepared(const void* q, const void* k, const void* v, const void* proj, int B, int H,
                                    int N, int d, double topk, int block, void* out, void* workspace,
                                    size_t workspace_bytes, sagesla_stream_t stream) {
  return run_fwd(q, k, v, proj, B, H, N, d, topk, block, out, workspace, workspace_bytes, stream, true);
}

sagesla_status sagesla_prepare(const void* qkv, const void* gq, const void* gk, double eps, int B, int H, int N,
                               int d, double topk, int block, int linear, void* q, void* k, void* v, void* workspace,
                               size_t workspace_bytes, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if (!(eps >= 0.0 && eps < 1e30)) return SAGESLA_ERR_INVALID_ARGUMENT;
  if ((s = check_ptrs({qkv, gq, gk, q, k, v, workspace})) != SAGESLA_OK) return s;
  size_t off[SAGESLA_WS_COUNT], total;
  layout(gm, linear != 0 && gm.ksel < gm.Nb, off, &total);
  if (workspace_bytes < total) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;
  char* ws = (char*)workspace;
  auto P = [&](int r) { return (void*)(ws + off[r]); };
  // the per-token scales live in the K8 region until the forward's K quantization overwrites it
  return from_hip(launch_prepare(qkv, gq, gk, eps, B, H, N, gm.Nb, P(SAGESLA_WS_K8), q, k, v, P(SAGESLA_WS_QBAR),
                                 P(SAGESLA_WS_KBART), P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), P(SAGESLA_WS_Q8),
                                 P(SAGESLA_WS_SQ), (hipStream_t)stream));
}

}  // extern "C"

static sagesla_status run_fwd(const void* q, const void* k, const void* v, const void* proj, int B, int H, int N,
                              int d, double topk, int block, void* out, void* workspace, size_t workspace_bytes,
                              sagesla_stream_t stream, bool pooled, bool fork) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, out, workspace})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(proj)) != SAGESLA_OK) return s;
  const bool linear = proj != nullptr && gm.ksel < gm.Nb;
  size_t off[SAGESLA_WS_COUNT], total;
  layout(gm, linear, off, &total);
  if (workspace_bytes < total) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto P = [&](int r) { return (void*)(ws + off[r]); };
  hipError_t e;
  if (!pooled && (e = launch_pool(q, k, v, gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART),
                                  P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), P(SAGESLA_WS_Q8), P(SAGESLA_WS_SQ),
                                  st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_head_stats(P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), gm.BH, gm.N, gm.Nb,
                             P(SAGESLA_WS_KMEAN), P(SAGESLA_WS_VAMAX), st)) != hipSuccess)
    return from_hip(e);
  // the selection (and the union of the kept lists, which needs nothing else) on the side
  // stream when there is one, beside the quantization and the totals; every later stage
  // waits for both
  SideStream* side = fork ? side_stream(st) : nullptr;
  std::unique_lock<std::mutex> fork_lk(fork_mu, std::defer_lock);
  if (side) {
    fork_lk.lock();
    if (hipEventRecord(side->fork, st) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
      return SAGESLA_ERR_HIP;
  }
  hipStream_t sel_st = side ? side->s : st;
  hipError_t es = launch_select(P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_WS_IDX),
                                sel_st);
  if (es == hipSuccess && linear)
    es = launch_linear_union(P(SAGESLA_WS_IDX), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_WS_ULIST), P(SAGESLA_WS_UMASK),
                             P(SAGESLA_WS_UCOUNT), sel_st);
  if (es == hipSuccess)
    es = launch_quant_kv(k, v, P(SAGESLA_WS_KMEAN), P(SAGESLA_WS_VAMAX), gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_K8),
                         P(SAGESLA_WS_SK), P(SAGESLA_WS_V8), linear ? P(SAGESLA_WS_HS) : nullptr,
                         linear ? P(SAGESLA_WS_HPART) : nullptr, st);
  if (es == hipSuccess && linear)
    es = launch_linear_total(P(SAGESLA_WS_HPART), gm.BH, gm.Nb, P(SAGESLA_WS_HTOT), st);
  if (side) {  // the join, also after a failed launch: the caller's stream never runs ahead
    if (hipEventRecord(side->join, side->s) != hipSuccess || hipStreamWaitEvent(st, side->join, 0) != hipSuccess)
      return SAGESLA_ERR_HIP;
    fork_lk.unlock();
  }
  if (es != hipSuccess) return from_hip(es);
  if (linear) {
    if ((e = launch_linear_masked(q, P(SAGESLA_WS_HS), P(SAGESLA_WS_HTOT), proj, gm.BH, gm.N, gm.Nb, gm.ksel,
                                  P(SAGESLA_WS_ULIST), P(SAGESLA_WS_UMASK), P(SAGESLA_WS_UCOUNT),
                                  P(SAGESLA_WS_HC), P(SAGESLA_WS_Y), st)) != hipSuccess)
      return from_hip(e);
  }
  e = launch_sparse_attn(P(SAGESLA_WS_Q8), P(SAGESLA_WS_SQ), P(SAGESLA_WS_K8), P(SAGESLA_WS_SK),
                         P(SAGESLA_WS_V8), P(SAGESLA_WS_VAMAX), P(SAGESLA_WS_IDX),
                         linear ? P(SAGESLA_WS_Y) : nullptr, gm.BH, gm.N, gm.Nb, gm.ksel, out, st);
  return from_hip(e);
}

extern "C" {

// ---------------------------------------------------------------- tensor descriptors

static bool t_contiguous(const sagesla_tensor* t) {
  int64_t want = 1;
  for (int a = t->ndim - 1; a >= 0; a--) {
    if (t->shape[a] < 1) return false;
    if (t->shape[a] > 1 && t->stride[a] != want) return false;
    want *= t->shape[a];
  }
  return true;
}

static sagesla_status t_check(const sagesla_tensor* t, sagesla_dtype dtype, int ndim) {
  if (!t || !t->data || t->dtype != dtype || t->ndim != ndim || !t_contiguous(t)) return SAGESLA_ERR_INVALID_ARGUMENT;
  return SAGESLA_OK;
}

sagesla_status sagesla_fwd_tensors(const sagesla_tensor* q, const sagesla_tensor* k, const sagesla_tensor* v,
                                   const sagesla_tensor* proj, double topk, int block, sagesla_tensor* out,
                                   const sagesla_tensor* workspace, sagesla_stream_t stream) {
  sagesla_status s;
  if ((s = t_check(q, SAGESLA_BF16, 4)) != SAGESLA_OK || (s = t_check(k, SAGESLA_BF16, 4)) != SAGESLA_OK ||
      (s = t_check(v, SAGESLA_BF16, 4)) != SAGESLA_OK || (s = t_check(out, SAGESLA_BF16, 4)) != SAGESLA_OK ||
      (s = t_check(workspace, SAGESLA_U8, 1)) != SAGESLA_OK)
    return s;
  for (int a = 0; a < 4; a++)
    if (k->shape[a] != q->shape[a] || v->shape[a] != q->shape[a] || out->shape[a] != q->shape[a])
      return SAGESLA_ERR_INVALID_ARGUMENT;
  for (int a = 0; a < 4; a++)
    if (q->shape[a] > INT32_MAX) return SAGESLA_ERR_INVALID_ARGUMENT;
  const int B = (int)q->shape[0], H = (int)q->shape[1], N = (int)q->shape[2], d = (int)q->shape[3];
  if (proj) {
    if ((s = t_check(proj, SAGESLA_BF16, 2)) != SAGESLA_OK) return s;
    if (proj->shape[0] != d || proj->shape[1] != d) return SAGESLA_ERR_INVALID_ARGUMENT;
  }
  return run_fwd(q->data, k->data, v->data, proj ? proj->data : nullptr, B, H, N, d, topk, block, out->data,
                 workspace->data, (size_t)workspace->shape[0], stream, false);
}

// ---------------------------------------------------------------- forward without allocation

// The workspace of sagesla_fwd_noalloc: one fixed-size device array, which every GPU the
// library runs on holds (its own copy) until the process ends. In host code the name is
// only a stand-in for the symbol; the device address comes from hipGetSymbolAddress, once
// per device, and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[SAGESLA_NOALLOC_SCRATCH_BYTES];

static sagesla_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGESLA_ERR_HIP;
  if (dev < 0 || dev >= 64) return SAGESLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SAGESLA_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return SAGESLA_OK;
}

sagesla_status sagesla_fwd_noalloc(const void* q, const void* k, const void* v, const void* proj, int B, int H,
                                   int N, int d, double topk, int block, void* out, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, out})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(proj)) != SAGESLA_OK) return s;
  size_t off[SAGESLA_WS_COUNT], total;
  layout(gm, proj != nullptr && gm.ksel < gm.Nb, off, &total);
  if (total > (size_t)SAGESLA_NOALLOC_SCRATCH_BYTES) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != SAGESLA_OK) return s;
  return run_fwd(q, k, v, proj, B, H, N, d, topk, block, out, ws, (size_t)SAGESLA_NOALLOC_SCRATCH_BYTES, stream,
                 false, false);
}

// ---------------------------------------------------------------- content-adaptive count

// The adaptive forward's workspace: the fixed-count layout at the largest count, with the
// linear regions whenever some head may leave blocks out (kmin < Nb).
static sagesla_status adaptive_layout(int B, int H, int N, int d, int block, double topk_min, double topk_max,
                                      double tau, int linear, Geom* gm, int* kmin, size_t off[SAGESLA_WS_COUNT],
                                      size_t* total) {
  sagesla_status s = check_sizes(B, H, N, d, block, gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_adaptive(topk_min, topk_max, tau, gm, kmin)) != SAGESLA_OK) return s;
  layout(*gm, linear != 0 && *kmin < gm->Nb, off, total, true);
  return SAGESLA_OK;
}

sagesla_status sagesla_adaptive_workspace_size(int B, int H, int N, int d, int block, double topk_min,
                                               double topk_max, int linear, size_t* bytes) {
  Geom gm;
  int kmin;
  size_t off[SAGESLA_WS_COUNT];
  if (!bytes) return SAGESLA_ERR_INVALID_ARGUMENT;
  return adaptive_layout(B, H, N, d, block, topk_min, topk_max, 1.0, linear, &gm, &kmin, off, bytes);
}

sagesla_status sagesla_adaptive_workspace_layout(int B, int H, int N, int d, int block, double topk_min,
                                                 double topk_max, int linear, size_t offsets[SAGESLA_WS_COUNT]) {
  Geom gm;
  int kmin;
  size_t total;
  if (!offsets) return SAGESLA_ERR_INVALID_ARGUMENT;
  return adaptive_layout(B, H, N, d, block, topk_min, topk_max, 1.0, linear, &gm, &kmin, offsets, &total);
}

sagesla_status sagesla_adaptive_ksel(const void* qbar, const void* kbart, int B, int H, int N, int d, int block,
                                     double topk_min, double topk_max, double tau, void* k_rows, void* k_head,
                                     sagesla_stream_t stream) {
  Geom gm;
  int kmin;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_adaptive(topk_min, topk_max, tau, &gm, &kmin)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({qbar, kbart, k_rows, k_head})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_adaptive_ksel(qbar, kbart, gm.BH, gm.N, gm.Nb, tau, kmin, gm.ksel, k_rows, k_head, nullptr,
                                       (hipStream_t)stream));
}

sagesla_status sagesla_fwd_adaptive(const void* q, const void* k, const void* v, const void* proj, int B, int H,
                                    int N, int d, double topk_min, double topk_max, double tau, int block, void* out,
                                    void* k_rows, void* k_head, void* workspace, size_t workspace_bytes,
                                    sagesla_stream_t stream) {
  Geom gm;
  int kmin;
  size_t off[SAGESLA_WS_COUNT], total;
  sagesla_status s =
      adaptive_layout(B, H, N, d, block, topk_min, topk_max, tau, proj != nullptr, &gm, &kmin, off, &total);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, out, k_rows, k_head, workspace})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(proj)) != SAGESLA_OK) return s;
  if (workspace_bytes < total) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;
  const bool linear = proj != nullptr && kmin < gm.Nb;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto P = [&](int r) { return (void*)(ws + off[r]); };
  const int kmax = gm.ksel;
  hipError_t e;
  if ((e = launch_pool(q, k, v, gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART), P(SAGESLA_WS_KSUM),
                       P(SAGESLA_WS_VAMAXB), P(SAGESLA_WS_Q8), P(SAGESLA_WS_SQ), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_head_stats(P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_KMEAN),
                             P(SAGESLA_WS_VAMAX), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_adaptive_ksel(P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART), gm.BH, gm.N, gm.Nb, tau, kmin, kmax, k_rows,
                                k_head, P(SAGESLA_WS_KEYS), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_select(P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART), gm.BH, gm.Nb, kmax, k_head, kmax,
                         P(SAGESLA_WS_KEYS), P(SAGESLA_WS_IDX), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_quant_kv(k, v, P(SAGESLA_WS_KMEAN), P(SAGESLA_WS_VAMAX), gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_K8),
                           P(SAGESLA_WS_SK), P(SAGESLA_WS_V8), linear ? P(SAGESLA_WS_HS) : nullptr,
                           linear ? P(SAGESLA_WS_HPART) : nullptr, st)) != hipSuccess)
    return from_hip(e);
  if (linear) {
    if ((e = launch_linear_total(P(SAGESLA_WS_HPART), gm.BH, gm.Nb, P(SAGESLA_WS_HTOT), st)) != hipSuccess)
      return from_hip(e);
    if ((e = launch_linear_complement(q, P(SAGESLA_WS_IDX), k_head, kmax, P(SAGESLA_WS_HS), P(SAGESLA_WS_HTOT), proj,
                                      gm.BH, gm.N, gm.Nb, kmax, P(SAGESLA_WS_ULIST), P(SAGESLA_WS_UMASK),
                                      P(SAGESLA_WS_UCOUNT), P(SAGESLA_WS_HC), P(SAGESLA_WS_Y), st)) != hipSuccess)
      return from_hip(e);
  }
  return from_hip(launch_sparse_attn(P(SAGESLA_WS_Q8), P(SAGESLA_WS_SQ), P(SAGESLA_WS_K8), P(SAGESLA_WS_SK),
                                     P(SAGESLA_WS_V8), P(SAGESLA_WS_VAMAX), P(SAGESLA_WS_IDX), k_head, kmax,
                                     linear ? P(SAGESLA_WS_Y) : nullptr, gm.BH, gm.N, gm.Nb, kmax, out, st));
}

// ---------------------------------------------------------------- grouped stages

sagesla_status sagesla_pool_select(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                                   int block, double topk, void* qbar, void* kbart, void* ksum, void* vamax_blk,
                                   void* q8, void* sq, void* kmean, void* vamax, void* idx,
                                   sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, qbar, kbart, ksum, vamax_blk, q8, sq, kmean, vamax, idx})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_pool(q, k, v, gm.BH, gm.N, gm.Nb, qbar, kbart, ksum, vamax_blk, q8, sq, st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_head_stats(ksum, vamax_blk, gm.BH, gm.N, gm.Nb, kmean, vamax, st)) != hipSuccess)
    return from_hip(e);
  return from_hip(launch_select(qbar, kbart, gm.BH, gm.Nb, gm.ksel, idx, st));
}

sagesla_status sagesla_quantize(const void* k, const void* v, const void* kmean, const void* vamax, int B, int H,
                                int N, int d, int block, void* k8, void* sk, void* v8, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({k, v, kmean, vamax, k8, sk, v8})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_quant_kv(k, v, kmean, vamax, gm.BH, gm.N, gm.Nb, k8, sk, v8, nullptr, nullptr,
                                  (hipStream_t)stream));
}

sagesla_status sagesla_linear_states(const void* k, const void* v, const void* kmean, const void* vamax, int B,
                                     int H, int N, int d, int block, void* k8, void* sk, void* v8, void* hs,
                                     void* hpart, void* htot, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({k, v, kmean, vamax, k8, sk, v8, hs, hpart, htot})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if ((e = launch_quant_kv(k, v, kmean, vamax, gm.BH, gm.N, gm.Nb, k8, sk, v8, hs, hpart, st)) != hipSuccess)
    return from_hip(e);
  return from_hip(launch_linear_total(hpart, gm.BH, gm.Nb, htot, st));
}

// ---------------------------------------------------------------- single stages

sagesla_status sagesla_pool(const void* q, const void* k, const void* v, int B, int H, int N, int d, int block,
                            void* qbar, void* kbart, void* ksum, void* vamax_blk, void* q8, void* sq,
                            sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, qbar, kbart, ksum, vamax_blk, q8, sq})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_pool(q, k, v, gm.BH, gm.N, gm.Nb, qbar, kbart, ksum, vamax_blk, q8, sq,
                              (hipStream_t)stream));
}

sagesla_status sagesla_head_stats(const void* ksum, const void* vamax_blk, int B, int H, int N, int d, int block,
                                  void* kmean, void* vamax, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({ksum, vamax_blk, kmean, vamax})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_head_stats(ksum, vamax_blk, gm.BH, gm.N, gm.Nb, kmean, vamax, (hipStream_t)stream));
}

sagesla_status sagesla_select(const void* qbar, const void* kbart, int B, int H, int N, int d, int block,
                              double topk, void* idx, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({qbar, kbart, idx})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_select(qbar, kbart, gm.BH, gm.Nb, gm.ksel, idx, (hipStream_t)stream));
}

sagesla_status sagesla_quant_kv(const void* k, const void* v, const void* kmean, const void* vamax, int B, int H,
                                int N, int d, int block, void* k8, void* sk, void* v8, void* hs, void* hpart,
                                sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({k, v, kmean, vamax, k8, sk, v8})) != SAGESLA_OK) return s;
  const bool st = hs != nullptr;
  if (st && (s = check_ptrs({hs, hpart})) != SAGESLA_OK) return s;
  if (!st && hpart) return SAGESLA_ERR_INVALID_ARGUMENT;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_quant_kv(k, v, kmean, vamax, gm.BH, gm.N, gm.Nb, k8, sk, v8, hs, hpart,
                                  (hipStream_t)stream));
}

sagesla_status sagesla_linear_total(const void* hpart, int B, int H, int N, int d, int block, void* htot,
                                    sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({hpart, htot})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_linear_total(hpart, gm.BH, gm.Nb, htot, (hipStream_t)stream));
}

sagesla_status sagesla_linear_complement(const void* q, const void* idx, const void* hs, const void* htot,
                                         const void* proj, int B, int H, int N, int d, int block, double topk,
                                         void* ulist, void* umask, void* ucount, void* hc, void* y,
                                         sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, idx, hs, htot, proj, ulist, umask, ucount, hc, y})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_linear_complement(q, idx, hs, htot, proj, gm.BH, gm.N, gm.Nb, gm.ksel, ulist, umask,
                                           ucount, hc, y, (hipStream_t)stream));
}

sagesla_status sagesla_sparse_attn(const void* q8, const void* sq, const void* k8, const void* sk, const void* v8,
                                   const void* vamax, const void* idx, const void* y, int B, int H, int N, int d,
                                   int block, double topk, void* out, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q8, sq, k8, sk, v8, vamax, idx, out})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(y)) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_sparse_attn(q8, sq, k8, sk, v8, vamax, idx, y, gm.BH, gm.N, gm.Nb, gm.ksel, out,
                                     (hipStream_t)stream));
}

// ---------------------------------------------------------------- W8A8 linear layer

static sagesla_status w8a8_check(int M, int N, int K) {
  if (M < 1 || M > (1 << 24) || K < 128 || K % 128 != 0 || K > (1 << 16) || N < 256 || N % 256 != 0 ||
      N > (1 << 16))
    return SAGESLA_ERR_INVALID_ARGUMENT;
  return SAGESLA_OK;
}

sagesla_status sagesla_w8a8_sizes(int M, int N, int K, size_t* x8_bytes, size_t* sx_bytes, size_t* w8_bytes,
                                  size_t* sw_bytes) {
  sagesla_status s = w8a8_check(M, N, K);
  if (s != SAGESLA_OK) return s;
  const size_t Mp = (size_t)w8a8_row_tiles(M) * 32, KB = K / 128;
  if (x8_bytes) *x8_bytes = Mp * K;
  if (sx_bytes) *sx_bytes = KB * Mp * 4;
  if (w8_bytes) *w8_bytes = (size_t)N * K;
  if (sw_bytes) *sw_bytes = (size_t)(N / 128) * KB * 4;
  return SAGESLA_OK;
}

sagesla_status sagesla_w8a8_quant_weight(const void* w, int N, int K, void* w8, void* sw, sagesla_stream_t stream) {
  sagesla_status s = w8a8_check(1, N, K);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({w, w8, sw})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_w8a8_quant_weight(w, N, K, w8, sw, (hipStream_t)stream));
}

sagesla_status sagesla_w8a8_quant_act(const void* x, int M, int K, void* x8, void* sx, sagesla_stream_t stream) {
  sagesla_status s = w8a8_check(M, 256, K);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({x, x8, sx})) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_w8a8_quant_act(x, M, K, x8, sx, (hipStream_t)stream));
}

sagesla_status sagesla_w8a8_gemm(const void* x8, const void* sx, const void* w8, const void* sw, const void* bias,
                                 int M, int N, int K, void* y, sagesla_stream_t stream) {
  sagesla_status s = w8a8_check(M, N, K);
  if (s != SAGESLA_OK) return s;
  if ((s = check_ptrs({x8, sx, w8, sw, y})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(bias)) != SAGESLA_OK) return s;
  if ((s = check_device()) != SAGESLA_OK) return s;
  return from_hip(launch_w8a8_gemm(x8, sx, w8, sw, bias, M, N, K, y, (hipStream_t)stream));
}

// ---------------------------------------------------------------- SLA training path

}  // extern "C"

namespace {

// The forward regions, then the training regions, each 256-byte aligned.
void sla_layout(const Geom& gm, bool linear, size_t off[SAGESLA_SLA_WS_COUNT], size_t* total) {
  size_t base;
  layout(gm, linear, off, &base);
  const size_t BH = gm.BH, N = gm.N, Nb = gm.Nb, D = kD, nw = (gm.Nb + 31) / 32;
  const size_t tiles = BH * Nb * (size_t)kBlk * kD * 2;
  size_t sz[SAGESLA_SLA_WS_COUNT] = {};
  sz[SAGESLA_SLA_WS_LSE] = BH * N * 4;
  sz[SAGESLA_SLA_WS_OS] = BH * N * D * 4;
  sz[SAGESLA_SLA_WS_KT] = tiles;
  sz[SAGESLA_SLA_WS_VT] = tiles;
  sz[SAGESLA_SLA_WS_QT] = tiles;
  sz[SAGESLA_SLA_WS_DOT] = tiles;
  sz[SAGESLA_SLA_WS_DSUM] = BH * N * 4;
  sz[SAGESLA_SLA_WS_MASK] = BH * Nb * nw * 4;
  sz[SAGESLA_SLA_WS_H0] = tiles;
  sz[SAGESLA_SLA_WS_H1] = tiles;
  if (linear) {
    sz[SAGESLA_SLA_WS_PHQ] = BH * N * D * 2;
    sz[SAGESLA_SLA_WS_DU] = BH * N * D * 2;
    sz[SAGESLA_SLA_WS_OL] = BH * N * D * 2;
    sz[SAGESLA_SLA_WS_DS] = BH * N * 4;
    sz[SAGESLA_SLA_WS_DWP] = (size_t)sla_dw_parts() * D * D * 4;
  }
  size_t o = align256(base);
  for (int r = SAGESLA_WS_COUNT; r < SAGESLA_SLA_WS_COUNT; r++) {
    off[r] = o;
    o += align256(sz[r]);
  }
  *total = o;
}

}  // namespace

extern "C" {

sagesla_status sagesla_sla_workspace_size(int B, int H, int N, int d, int block, double topk, int linear,
                                          size_t* bytes) {
  Geom gm;
  if (!bytes) return SAGESLA_ERR_INVALID_ARGUMENT;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  size_t off[SAGESLA_SLA_WS_COUNT];
  sla_layout(gm, linear != 0 && gm.ksel < gm.Nb, off, bytes);
  return SAGESLA_OK;
}

sagesla_status sagesla_sla_workspace_layout(int B, int H, int N, int d, int block, double topk, int linear,
                                            size_t offsets[SAGESLA_SLA_WS_COUNT]) {
  Geom gm;
  if (!offsets) return SAGESLA_ERR_INVALID_ARGUMENT;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  size_t total;
  sla_layout(gm, linear != 0 && gm.ksel < gm.Nb, offsets, &total);
  return SAGESLA_OK;
}

sagesla_status sagesla_sla_fwd(const void* q, const void* k, const void* v, const void* proj, int B, int H, int N,
                               int d, double topk, int block, void* out, void* workspace, size_t workspace_bytes,
                               sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, out, workspace})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(proj)) != SAGESLA_OK) return s;
  const bool linear = proj != nullptr && gm.ksel < gm.Nb;
  size_t off[SAGESLA_SLA_WS_COUNT], total;
  sla_layout(gm, linear, off, &total);
  if (workspace_bytes < total) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto P = [&](int r) { return (void*)(ws + off[r]); };
  hipError_t e;
  if ((e = launch_pool(q, k, v, gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART),
                       P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), P(SAGESLA_WS_Q8), P(SAGESLA_WS_SQ), st)) !=
      hipSuccess)
    return from_hip(e);
  if ((e = launch_select(P(SAGESLA_WS_QBAR), P(SAGESLA_WS_KBART), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_WS_IDX),
                         st)) != hipSuccess)
    return from_hip(e);
  if (linear) {
    // the linear states come with the K/V quantization pass (its codes go unused here)
    if ((e = launch_head_stats(P(SAGESLA_WS_KSUM), P(SAGESLA_WS_VAMAXB), gm.BH, gm.N, gm.Nb,
                               P(SAGESLA_WS_KMEAN), P(SAGESLA_WS_VAMAX), st)) != hipSuccess)
      return from_hip(e);
    if ((e = launch_quant_kv(k, v, P(SAGESLA_WS_KMEAN), P(SAGESLA_WS_VAMAX), gm.BH, gm.N, gm.Nb, P(SAGESLA_WS_K8),
                             P(SAGESLA_WS_SK), P(SAGESLA_WS_V8), P(SAGESLA_WS_HS), P(SAGESLA_WS_HPART), st)) !=
        hipSuccess)
      return from_hip(e);
    if ((e = launch_linear_total(P(SAGESLA_WS_HPART), gm.BH, gm.Nb, P(SAGESLA_WS_HTOT), st)) != hipSuccess)
      return from_hip(e);
    if ((e = launch_linear_complement(q, P(SAGESLA_WS_IDX), P(SAGESLA_WS_HS), P(SAGESLA_WS_HTOT), proj, gm.BH,
                                      gm.N, gm.Nb, gm.ksel, P(SAGESLA_WS_ULIST), P(SAGESLA_WS_UMASK),
                                      P(SAGESLA_WS_UCOUNT), P(SAGESLA_WS_HC), P(SAGESLA_WS_Y), st)) != hipSuccess)
      return from_hip(e);
  }
  if ((e = launch_sla_relayout(v, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_VT), st)) != hipSuccess) return from_hip(e);
  // K in head-dim-reduction tiles (in the K tile region, which the backward rewrites)
  if ((e = launch_sla_relayout_hd(k, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_KT), st)) != hipSuccess)
    return from_hip(e);
  e = launch_sla_fwd(q, P(SAGESLA_SLA_WS_KT), P(SAGESLA_SLA_WS_VT), P(SAGESLA_WS_IDX), linear ? P(SAGESLA_WS_Y) : nullptr, gm.BH,
                     gm.N, gm.Nb, gm.ksel, out, P(SAGESLA_SLA_WS_OS), P(SAGESLA_SLA_WS_LSE), st);
  return from_hip(e);
}

sagesla_status sagesla_sla_bwd(const void* q, const void* k, const void* v, const void* proj, const void* dout,
                               int B, int H, int N, int d, double topk, int block, void* dq, void* dk, void* dv,
                               void* dproj, void* workspace, size_t workspace_bytes, sagesla_stream_t stream) {
  Geom gm;
  sagesla_status s = check_sizes(B, H, N, d, block, &gm);
  if (s != SAGESLA_OK) return s;
  if ((s = check_topk(topk, &gm)) != SAGESLA_OK) return s;
  if ((s = check_ptrs({q, k, v, dout, dq, dk, dv, workspace})) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(proj)) != SAGESLA_OK) return s;
  if ((s = check_opt_ptr(dproj)) != SAGESLA_OK) return s;
  if ((proj == nullptr) != (dproj == nullptr)) return SAGESLA_ERR_INVALID_ARGUMENT;
  const bool linear = proj != nullptr && gm.ksel < gm.Nb;
  size_t off[SAGESLA_SLA_WS_COUNT], total;
  sla_layout(gm, linear, off, &total);
  if (workspace_bytes < total) return SAGESLA_ERR_WORKSPACE;
  if ((s = check_device()) != SAGESLA_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto P = [&](int r) { return (void*)(ws + off[r]); };
  hipError_t e;
  // sparse part: dq, dk, dv written
  if ((e = launch_sla_kept_mask(P(SAGESLA_WS_IDX), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_SLA_WS_MASK), st)) != hipSuccess)
    return from_hip(e);
  // dQ: K and V in head-dim-reduction tiles (V's in the V tile region); the kernel reads K
  // with tokens as the reduction index from the same tile
  if ((e = launch_sla_relayout_hd(k, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_H0), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_relayout_hd(v, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_VT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_bwd_dq(q, P(SAGESLA_SLA_WS_H0), P(SAGESLA_SLA_WS_VT), dout,
                             P(SAGESLA_SLA_WS_OS), P(SAGESLA_SLA_WS_LSE),
                             P(SAGESLA_WS_IDX), gm.BH, gm.N, gm.Nb, gm.ksel, P(SAGESLA_SLA_WS_DSUM), dq, st)) !=
      hipSuccess)
    return from_hip(e);
  // dK, dV: Q and dO in head-dim-reduction tiles (Q's in H0, which K's no longer need),
  // read with either index reduced
  if ((e = launch_sla_relayout_hd(q, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_H0), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_relayout_hd(dout, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_H1), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_bwd_dkdv(k, v, P(SAGESLA_SLA_WS_H0), P(SAGESLA_SLA_WS_H1), P(SAGESLA_SLA_WS_LSE),
                               P(SAGESLA_SLA_WS_DSUM),
                               P(SAGESLA_SLA_WS_MASK), gm.BH, gm.N, gm.Nb, dk, dv, st)) != hipSuccess)
    return from_hip(e);
  if (proj == nullptr) return SAGESLA_OK;
  if (!linear) {  // every block kept: no linear part, dW = 0
    return from_hip(launch_sla_zero(dproj, (size_t)kD * kD, st));
  }
  // linear part: added into dq, dk, dv; the token-reduction tiles of phi(q), du and O_l
  // reuse the K, Q and V tile regions, the state gradients the forward's state regions
  if ((e = launch_sla_lin_bwd_q(q, dout, P(SAGESLA_WS_HC), proj, gm.BH, gm.N, gm.Nb, dq, P(SAGESLA_SLA_WS_PHQ),
                                P(SAGESLA_SLA_WS_DU), P(SAGESLA_SLA_WS_DS), P(SAGESLA_SLA_WS_OL), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_relayout(P(SAGESLA_SLA_WS_PHQ), gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_KT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_relayout(P(SAGESLA_SLA_WS_DU), gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_QT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_relayout(P(SAGESLA_SLA_WS_OL), gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_VT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_lin_dhc(P(SAGESLA_SLA_WS_KT), P(SAGESLA_SLA_WS_QT), P(SAGESLA_SLA_WS_DS), gm.BH, gm.N, gm.Nb,
                              P(SAGESLA_WS_HS), P(SAGESLA_WS_HPART), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_linear_total(P(SAGESLA_WS_HPART), gm.BH, gm.Nb, P(SAGESLA_WS_HTOT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_union_t(P(SAGESLA_SLA_WS_MASK), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_WS_ULIST),
                              P(SAGESLA_WS_UMASK), P(SAGESLA_WS_UCOUNT), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_linear_mask_gemm(P(SAGESLA_WS_HS), P(SAGESLA_WS_HTOT), P(SAGESLA_WS_ULIST), P(SAGESLA_WS_UMASK),
                                   P(SAGESLA_WS_UCOUNT), gm.BH, gm.Nb, gm.ksel, P(SAGESLA_WS_HC), st)) != hipSuccess)
    return from_hip(e);
  if ((e = launch_sla_lin_bwd_k(k, v, P(SAGESLA_WS_HC), gm.BH, gm.N, gm.Nb, dk, dv, st)) != hipSuccess)
    return from_hip(e);
  // dW = O_l^T dO: both in token-reduction tiles
  if ((e = launch_sla_relayout(dout, gm.BH, gm.N, gm.Nb, P(SAGESLA_SLA_WS_DOT), st)) != hipSuccess)
    return from_hip(e);
  e = launch_sla_dw(P(SAGESLA_SLA_WS_VT), P(SAGESLA_SLA_WS_DOT), gm.BH * gm.Nb, P(SAGESLA_SLA_WS_DWP), dproj, st);
  return from_hip(e);
}

}  // extern "C"
