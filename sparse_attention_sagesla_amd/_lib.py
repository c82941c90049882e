"""ctypes binding of libsagesla.so (the C ABI declared in include/sagesla.h).

Argument marshalling only: torch tensors provide device memory and the stream; every
step of the computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or the device is not gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsagesla.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)

WS_REGIONS = ["qbar", "kbart", "ksum", "vamax_blk", "kmean", "vamax", "q8", "sq", "k8", "sk", "v8", "idx",
              "hs", "hpart", "htot", "ulist", "umask", "ucount", "hc", "y", "keys"]
WS_COUNT = len(WS_REGIONS)
GROUP = 256  # query blocks per group of the linear-branch complement (union lists, masks)

EXPORTS = ["sagesla_version", "sagesla_status_string", "sagesla_ksel", "sagesla_workspace_size",
           "sagesla_workspace_layout", "sagesla_fwd", "sagesla_pool", "sagesla_head_stats", "sagesla_select",
           "sagesla_quant_kv", "sagesla_linear_total", "sagesla_linear_complement", "sagesla_sparse_attn",
           "sagesla_w8a8_sizes", "sagesla_w8a8_quant_weight", "sagesla_w8a8_quant_act", "sagesla_w8a8_gemm",
           "sagesla_sla_workspace_size", "sagesla_sla_workspace_layout", "sagesla_sla_fwd", "sagesla_sla_bwd",
           "sagesla_prepare", "sagesla_fwd_prepared", "sagesla_fwd_tensors", "sagesla_pool_select",
           "sagesla_quantize", "sagesla_linear_states", "sagesla_fwd_noalloc", "sagesla_adaptive_workspace_size",
           "sagesla_adaptive_workspace_layout", "sagesla_adaptive_ksel", "sagesla_fwd_adaptive"]

# sagesla_dtype values and the sagesla_tensor descriptor
DT_BF16, DT_F32, DT_I8, DT_FP8E4M3, DT_I32, DT_U8 = range(6)


class Tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int), ("ndim", C.c_int),
                ("shape", C.c_int64 * 4), ("stride", C.c_int64 * 4)]


_TORCH_DT = {torch.bfloat16: DT_BF16, torch.float32: DT_F32, torch.int8: DT_I8, torch.int32: DT_I32,
             torch.uint8: DT_U8}


def tensor_desc(t) -> Tensor:
    """The sagesla_tensor descriptor of a torch tensor (element strides as torch has them)."""
    d = Tensor()
    d.data = t.data_ptr()
    d.dtype = _TORCH_DT.get(t.dtype, DT_FP8E4M3 if t.dtype == getattr(torch, "float8_e4m3fn", None) else -1)
    d.ndim = t.dim()
    for a in range(t.dim()):
        d.shape[a] = t.shape[a]
        d.stride[a] = t.stride(a)
    return d
SLA_WS_REGIONS = WS_REGIONS + ["lse", "os", "kt", "vt", "qt", "dot", "dsum", "mask", "h0", "h1", "phq", "du", "ol", "ds", "dwp"]
SLA_WS_COUNT = len(SLA_WS_REGIONS)

_lib = None


class SageSLAError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libsagesla.so is not built (run sparse_attention_sagesla_amd/build.py); "
                              "there is no fallback path")
        L = C.CDLL(LIB_PATH)
        P, i32, f64, sz = C.c_void_p, C.c_int, C.c_double, C.c_size_t
        dims = [i32, i32, i32, i32]
        sigs = {
            "sagesla_version": (i32, []),
            "sagesla_status_string": (C.c_char_p, [i32]),
            "sagesla_ksel": (i32, [i32, i32, f64, C.POINTER(i32)]),
            "sagesla_workspace_size": (i32, dims + [i32, f64, i32, C.POINTER(sz)]),
            "sagesla_workspace_layout": (i32, dims + [i32, f64, i32, C.POINTER(sz * WS_COUNT)]),
            "sagesla_fwd": (i32, [P, P, P, P] + dims + [f64, i32, P, P, sz, P]),
            "sagesla_pool": (i32, [P, P, P] + dims + [i32] + [P] * 6 + [P]),
            "sagesla_head_stats": (i32, [P, P] + dims + [i32, P, P, P]),
            "sagesla_select": (i32, [P, P] + dims + [i32, f64, P, P]),
            "sagesla_quant_kv": (i32, [P, P, P, P] + dims + [i32] + [P] * 5 + [P]),
            "sagesla_linear_total": (i32, [P] + dims + [i32, P, P]),
            "sagesla_linear_complement": (i32, [P] * 5 + dims + [i32, f64] + [P] * 5 + [P]),
            "sagesla_sparse_attn": (i32, [P] * 8 + dims + [i32, f64, P, P]),
            "sagesla_w8a8_sizes": (i32, [i32, i32, i32] + [C.POINTER(sz)] * 4),
            "sagesla_w8a8_quant_weight": (i32, [P, i32, i32, P, P, P]),
            "sagesla_w8a8_quant_act": (i32, [P, i32, i32, P, P, P]),
            "sagesla_w8a8_gemm": (i32, [P] * 5 + [i32, i32, i32, P, P]),
            "sagesla_sla_workspace_size": (i32, dims + [i32, f64, i32, C.POINTER(sz)]),
            "sagesla_sla_workspace_layout": (i32, dims + [i32, f64, i32, C.POINTER(sz * SLA_WS_COUNT)]),
            "sagesla_sla_fwd": (i32, [P, P, P, P] + dims + [f64, i32, P, P, sz, P]),
            "sagesla_sla_bwd": (i32, [P] * 5 + dims + [f64, i32] + [P] * 5 + [sz, P]),
            "sagesla_prepare": (i32, [P, P, P, f64] + dims + [f64, i32, i32, P, P, P, P, sz, P]),
            "sagesla_fwd_prepared": (i32, [P, P, P, P] + dims + [f64, i32, P, P, sz, P]),
            "sagesla_fwd_tensors": (i32, [C.POINTER(Tensor)] * 4 + [f64, i32, C.POINTER(Tensor),
                                                                    C.POINTER(Tensor), P]),
            "sagesla_pool_select": (i32, [P, P, P] + dims + [i32, f64] + [P] * 9 + [P]),
            "sagesla_quantize": (i32, [P, P, P, P] + dims + [i32, P, P, P, P]),
            "sagesla_linear_states": (i32, [P, P, P, P] + dims + [i32] + [P] * 6 + [P]),
            "sagesla_fwd_noalloc": (i32, [P, P, P, P] + dims + [f64, i32, P, P]),
            "sagesla_adaptive_workspace_size": (i32, dims + [i32, f64, f64, i32, C.POINTER(sz)]),
            "sagesla_adaptive_workspace_layout": (i32, dims + [i32, f64, f64, i32, C.POINTER(sz * WS_COUNT)]),
            "sagesla_adaptive_ksel": (i32, [P, P] + dims + [i32, f64, f64, f64, P, P, P]),
            "sagesla_fwd_adaptive": (i32, [P, P, P, P] + dims + [f64, f64, f64, i32, P, P, P, P, sz, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().sagesla_status_string(int(s)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, what):
    if status != OK:
        raise SageSLAError(status, what)


def ksel(N: int, topk: float, block: int = 64) -> int:
    out = C.c_int()
    _check(lib().sagesla_ksel(N, block, float(topk), C.byref(out)), "sagesla_ksel")
    return out.value


def workspace_size(B, H, N, d=128, block=64, topk=0.1, linear=True) -> int:
    out = C.c_size_t()
    _check(lib().sagesla_workspace_size(B, H, N, d, block, float(topk), int(bool(linear)), C.byref(out)),
           "sagesla_workspace_size")
    return out.value


def workspace_layout(B, H, N, d=128, block=64, topk=0.1, linear=True) -> dict:
    arr = (C.c_size_t * WS_COUNT)()
    _check(lib().sagesla_workspace_layout(B, H, N, d, block, float(topk), int(bool(linear)), C.byref(arr)),
           "sagesla_workspace_layout")
    return {name: arr[i] for i, name in enumerate(WS_REGIONS)}


def _shape(q):
    if q.dim() != 4 or q.dtype != torch.bfloat16 or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q/k/v must be contiguous bf16 CUDA tensors of shape [B, H, N, d]")
    return q.shape


def alloc_workspace(q, topk=0.1, linear=True, block=64):
    B, H, N, d = _shape(q)
    n = workspace_size(B, H, N, d, block, topk, linear)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def fwd(q, k, v, proj=None, topk=0.1, block=64, out=None, workspace=None, stream=None):
    """out = SageSLA(q, k, v) [+ linear branch through proj]. Returns out (bf16 [B, H, N, d])."""
    B, H, N, d = _shape(q)
    for x in (k, v):
        if _shape(x) != q.shape:
            raise ValueError("q, k, v shapes differ")
    if proj is not None and (proj.shape != (d, d) or proj.dtype != torch.bfloat16 or not proj.is_contiguous()):
        raise ValueError("proj must be a contiguous bf16 [d, d] tensor")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(q, topk, proj is not None, block)
    st = lib().sagesla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(proj), B, H, N, d, float(topk), block, _ptr(out),
                           _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sagesla_fwd")
    return out


def workspace_views(ws, B, H, N, d=128, block=64, topk=0.1, linear=True) -> dict:
    """Typed torch views of the intermediates left in a workspace by fwd()."""
    lay = workspace_layout(B, H, N, d, block, topk, linear)
    return _views(ws, lay, B * H, N, d, block, ksel(N, topk, block))


def _views(ws, lay, BH, N, d, block, k):
    Nb = (N + block - 1) // block
    Nc = (Nb + 15) // 16
    Ng = (Nb + GROUP - 1) // GROUP
    SE = 129 * d
    spec = {
        "qbar": (torch.float64, (BH, Nb, d)), "kbart": (torch.float64, (BH, d, Nb)),
        "ksum": (torch.float64, (BH, Nb, d)), "vamax_blk": (torch.float32, (BH, Nb, d)),
        "kmean": (torch.float32, (BH, d)), "vamax": (torch.float32, (BH, d)),
        "q8": (torch.int8, (BH, Nb, 8192)), "sq": (torch.float32, (BH, Nb)),
        "k8": (torch.int8, (BH, Nb, 8192)), "sk": (torch.float32, (BH, Nb)),
        "v8": (torch.uint8, (BH, Nb, 8192)), "idx": (torch.int32, (BH, Nb, k)),
        "hs": (torch.bfloat16, (BH, Nb, 129, d)), "hpart": (torch.float32, (BH, Nc, 129, d)),
        "htot": (torch.float32, (BH, 129, d)), "ulist": (torch.int32, (BH, Ng, Nb)),
        "umask": (torch.int32, (BH, Ng, (Nb + 31) // 32, GROUP)), "ucount": (torch.int32, (BH, Ng)),
        "hc": (torch.bfloat16, (BH, Nb, 129, d)), "y": (torch.bfloat16, (BH, N, d)),
        "keys": (torch.int64, (BH, Nb, Nb)),
    }
    total = ws.numel()
    out = {}
    for name, (dt, shape) in spec.items():
        off = lay[name]
        nbytes = torch.Size(shape).numel() * torch.empty((), dtype=dt).element_size()
        if off >= total or off + nbytes > total:
            continue
        out[name] = ws[off:off + nbytes].view(dt).view(shape)
    return out


# ---------------------------------------------------------------- content-adaptive count

def adaptive_workspace_size(B, H, N, d=128, block=64, topk_min=0.05, topk_max=0.25, linear=True) -> int:
    out = C.c_size_t()
    _check(lib().sagesla_adaptive_workspace_size(B, H, N, d, block, float(topk_min), float(topk_max),
                                                 int(bool(linear)), C.byref(out)), "sagesla_adaptive_workspace_size")
    return out.value


def adaptive_workspace_layout(B, H, N, d=128, block=64, topk_min=0.05, topk_max=0.25, linear=True) -> dict:
    arr = (C.c_size_t * WS_COUNT)()
    _check(lib().sagesla_adaptive_workspace_layout(B, H, N, d, block, float(topk_min), float(topk_max),
                                                   int(bool(linear)), C.byref(arr)),
           "sagesla_adaptive_workspace_layout")
    return {name: arr[i] for i, name in enumerate(WS_REGIONS)}


def adaptive_workspace_views(ws, B, H, N, d=128, block=64, topk_min=0.05, topk_max=0.25, linear=True) -> dict:
    """Typed views of what fwd_adaptive() leaves in its workspace; idx is [BH, Nb, kmax]."""
    lay = adaptive_workspace_layout(B, H, N, d, block, topk_min, topk_max, linear)
    return _views(ws, lay, B * H, N, d, block, ksel(N, topk_max, block))


def adaptive_ksel(qbar, kbart, B, H, N, topk_min=0.05, topk_max=0.25, tau=0.9, d=128, block=64, k_rows=None,
                  k_head=None, stream=None):
    """Per-row and per-head content-adaptive counts from the pooled means. Returns (k_rows
    int32 [B*H, Nb], k_head int32 [B*H])."""
    Nb = (N + block - 1) // block
    if k_rows is None:
        k_rows = torch.empty(B * H, Nb, dtype=torch.int32, device=qbar.device)
    if k_head is None:
        k_head = torch.empty(B * H, dtype=torch.int32, device=qbar.device)
    _check(lib().sagesla_adaptive_ksel(_ptr(qbar), _ptr(kbart), B, H, N, d, block, float(topk_min),
                                       float(topk_max), float(tau), _ptr(k_rows), _ptr(k_head), _stream(stream)),
           "sagesla_adaptive_ksel")
    return k_rows, k_head


def fwd_adaptive(q, k, v, proj=None, topk_min=0.05, topk_max=0.25, tau=0.9, block=64, out=None, k_rows=None,
                 k_head=None, workspace=None, stream=None):
    """The forward with a content-adaptive count per head. Returns (out, k_rows, k_head)."""
    B, H, N, d = _shape(q)
    for x in (k, v):
        if _shape(x) != q.shape:
            raise ValueError("q, k, v shapes differ")
    if proj is not None and (proj.shape != (d, d) or proj.dtype != torch.bfloat16 or not proj.is_contiguous()):
        raise ValueError("proj must be a contiguous bf16 [d, d] tensor")
    Nb = (N + block - 1) // block
    if out is None:
        out = torch.empty_like(q)
    if k_rows is None:
        k_rows = torch.empty(B * H, Nb, dtype=torch.int32, device=q.device)
    if k_head is None:
        k_head = torch.empty(B * H, dtype=torch.int32, device=q.device)
    if workspace is None:
        n = adaptive_workspace_size(B, H, N, d, block, topk_min, topk_max, proj is not None)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    st = lib().sagesla_fwd_adaptive(_ptr(q), _ptr(k), _ptr(v), _ptr(proj), B, H, N, d, float(topk_min),
                                    float(topk_max), float(tau), block, _ptr(out), _ptr(k_rows), _ptr(k_head),
                                    _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "sagesla_fwd_adaptive")
    return out, k_rows, k_head


# ---------------------------------------------------------------- W8A8 linear layer

def w8a8_sizes(M: int, N: int, K: int) -> dict:
    """Bytes of the activation codes/scales and weight codes/scales (see include/sagesla.h)."""
    out = [C.c_size_t() for _ in range(4)]
    _check(lib().sagesla_w8a8_sizes(M, N, K, *[C.byref(o) for o in out]), "sagesla_w8a8_sizes")
    return dict(zip(["x8", "sx", "w8", "sw"], [o.value for o in out]))


def w8a8_quant_weight(w, stream=None):
    """bf16 [N][K] weight -> (w8 uint8 codes, sw fp32 [N/128][K/128])."""
    N, K = w.shape
    sz = w8a8_sizes(1, N, K)
    w8 = torch.empty(sz["w8"], dtype=torch.uint8, device=w.device)
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    _check(lib().sagesla_w8a8_quant_weight(_ptr(w), N, K, _ptr(w8), _ptr(sw), _stream(stream)),
           "sagesla_w8a8_quant_weight")
    return w8, sw


def w8a8_quant_act(x, stream=None):
    """bf16 [M][K] activations -> (x8 uint8 codes, sx fp32 [K/128][Mp])."""
    M, K = x.shape
    sz = w8a8_sizes(M, 256, K)
    x8 = torch.empty(sz["x8"], dtype=torch.uint8, device=x.device)
    sx = torch.empty((K // 128, sz["sx"] // (4 * (K // 128))), dtype=torch.float32, device=x.device)
    _check(lib().sagesla_w8a8_quant_act(_ptr(x), M, K, _ptr(x8), _ptr(sx), _stream(stream)),
           "sagesla_w8a8_quant_act")
    return x8, sx


def w8a8_gemm(x8, sx, w8, sw, M, N, K, bias=None, out=None, stream=None):
    """y bf16 [M][N] from the codes and scales."""
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x8.device)
    _check(lib().sagesla_w8a8_gemm(_ptr(x8), _ptr(sx), _ptr(w8), _ptr(sw), _ptr(bias), M, N, K, _ptr(out),
                                   _stream(stream)), "sagesla_w8a8_gemm")
    return out


def w8a8_linear(x, w8, sw, N, bias=None, stream=None):
    """The layer: quantize x, then the block-scaled INT8 product with the quantized weight."""
    M, K = x.shape
    x8, sx = w8a8_quant_act(x, stream)
    return w8a8_gemm(x8, sx, w8, sw, M, N, K, bias=bias, stream=stream)


# ---------------------------------------------------------------- SLA training path

def sla_workspace_size(B, H, N, d=128, block=64, topk=0.1, linear=True) -> int:
    out = C.c_size_t()
    _check(lib().sagesla_sla_workspace_size(B, H, N, d, block, float(topk), int(bool(linear)), C.byref(out)),
           "sagesla_sla_workspace_size")
    return out.value


def sla_workspace_layout(B, H, N, d=128, block=64, topk=0.1, linear=True) -> dict:
    arr = (C.c_size_t * SLA_WS_COUNT)()
    _check(lib().sagesla_sla_workspace_layout(B, H, N, d, block, float(topk), int(bool(linear)), C.byref(arr)),
           "sagesla_sla_workspace_layout")
    return {name: arr[i] for i, name in enumerate(SLA_WS_REGIONS)}


def sla_fwd(q, k, v, proj=None, topk=0.1, block=64, out=None, workspace=None, stream=None):
    """Unquantized SLA forward. Returns (out bf16 [B, H, N, d], workspace); the workspace
    holds what sla_bwd needs."""
    B, H, N, d = _shape(q)
    for x in (k, v):
        if _shape(x) != q.shape:
            raise ValueError("q, k, v shapes differ")
    if proj is not None and (proj.shape != (d, d) or proj.dtype != torch.bfloat16 or not proj.is_contiguous()):
        raise ValueError("proj must be a contiguous bf16 [d, d] tensor")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(sla_workspace_size(B, H, N, d, block, topk, proj is not None), dtype=torch.uint8,
                                device=q.device)
    _check(lib().sagesla_sla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(proj), B, H, N, d, float(topk), block, _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream)), "sagesla_sla_fwd")
    return out, workspace


def sla_bwd(q, k, v, dout, workspace, proj=None, topk=0.1, block=64, dq=None, dk=None, dv=None, dproj=None,
            stream=None):
    """SLA backward from the workspace of sla_fwd on the same inputs. Returns (dq, dk, dv)
    fp32 [B, H, N, d] (and dproj fp32 [d, d] when proj is given)."""
    B, H, N, d = _shape(q)
    if _shape(dout) != q.shape:
        raise ValueError("dout shape differs")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    if proj is not None and dproj is None:
        dproj = torch.empty((d, d), dtype=torch.float32, device=q.device)
    _check(lib().sagesla_sla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(proj), _ptr(dout), B, H, N, d, float(topk), block,
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dproj), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "sagesla_sla_bwd")
    return (dq, dk, dv) if proj is None else (dq, dk, dv, dproj)


def sla_workspace_views(ws, B, H, N, d=128, block=64, topk=0.1, linear=True) -> dict:
    """Typed views of the training intermediates (idx, lse, os, dsum, mask, y)."""
    lay = sla_workspace_layout(B, H, N, d, block, topk, linear)
    BH, Nb = B * H, (N + block - 1) // block
    spec = {"idx": (torch.int32, (BH, Nb, ksel(N, topk, block))), "lse": (torch.float32, (BH, N)),
            "os": (torch.float32, (BH, N, d)), "dsum": (torch.float32, (BH, N)),
            "mask": (torch.int32, (BH, Nb, (Nb + 31) // 32)), "y": (torch.bfloat16, (BH, N, d))}
    out = {}
    for name, (dt, shape) in spec.items():
        off = lay[name]
        nbytes = torch.Size(shape).numel() * torch.empty((), dtype=dt).element_size()
        if off + nbytes <= ws.numel():
            out[name] = ws[off:off + nbytes].view(dt).view(shape)
    return out


# ---------------------------------------------------------------- producer-side fusion

def prepare(qkv, gq, gk, H, eps=1e-6, topk=0.1, linear=True, block=64, q=None, k=None, v=None, workspace=None,
            stream=None):
    """RMSNorm of q and k + attention layout + the pool stage, from the QKV projection
    output qkv bf16 [B, N, 3*H*d]. Returns (q, k, v, workspace) for fwd_prepared."""
    B, N, C = qkv.shape
    d = C // (3 * H)
    shape = (B, H, N, d)
    q = torch.empty(shape, dtype=torch.bfloat16, device=qkv.device) if q is None else q
    k = torch.empty(shape, dtype=torch.bfloat16, device=qkv.device) if k is None else k
    v = torch.empty(shape, dtype=torch.bfloat16, device=qkv.device) if v is None else v
    if workspace is None:
        workspace = torch.empty(workspace_size(B, H, N, d, block, topk, linear), dtype=torch.uint8,
                                device=qkv.device)
    _check(lib().sagesla_prepare(_ptr(qkv), _ptr(gq), _ptr(gk), float(eps), B, H, N, d, float(topk), block,
                                 int(bool(linear)), _ptr(q), _ptr(k), _ptr(v), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "sagesla_prepare")
    return q, k, v, workspace


def fwd_prepared(q, k, v, workspace, proj=None, topk=0.1, block=64, out=None, stream=None):
    """The forward from the stage after pooling, on the workspace prepare() filled."""
    B, H, N, d = _shape(q)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().sagesla_fwd_prepared(_ptr(q), _ptr(k), _ptr(v), _ptr(proj), B, H, N, d, float(topk), block,
                                      _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "sagesla_fwd_prepared")
    return out

