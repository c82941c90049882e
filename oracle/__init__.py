"""CPU oracle for the SageSLA attention forward (test infrastructure only).

Plain C in ``sagesla_oracle.c`` (fp64, scalar, no FMA contraction), loaded with ctypes.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use this package;
the GPU library never imports or links it, and it never imports the GPU library.

All functions work on numpy arrays. bf16 tensors are passed as their uint16 bit
patterns, one head at a time, [N, d] row-major.
"""
from __future__ import annotations

import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        i32, f64, sz = C.c_int, C.c_double, C.c_size_t
        sigs = {
            "oracle_bf16_to_double": (f64, [C.c_uint16]),
            "oracle_double_to_bf16": (C.c_uint16, [f64]),
            "oracle_e4m3_decode": (f64, [C.c_uint8]),
            "oracle_e4m3_encode": (C.c_uint8, [C.c_float]),
            "oracle_e4m3_encode_n": (None, [P, P, sz]),
            "oracle_e4m3_decode_n": (None, [P, P, sz]),
            "oracle_num_blocks": (i32, [i32, i32]),
            "oracle_ksel": (i32, [f64, i32]),
            "oracle_pool": (None, [P, i32, i32, i32, P]),
            "oracle_scores": (None, [P, P, i32, i32, i32, P]),
            "oracle_select": (None, [P, i32, i32, i32, P]),
            "oracle_order_best_first": (None, [P, i32, P]),
            "oracle_k_mean": (None, [P, i32, i32, P]),
            "oracle_quant_blocks": (None, [P, i32, i32, i32, P, P]),
            "oracle_quant_v": (None, [P, i32, i32, P, P]),
            "oracle_dot_i8": (C.c_int32, [P, P, i32]),
            "oracle_sparse_block": (None, [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P]),
            "oracle_sparse_block_fp64": (None, [P, P, P, P, i32, i32, i32, i32, i32, P]),
            "oracle_phi": (None, [P, i32, P]),
            "oracle_linear_states": (None, [P, P, i32, i32, i32, P, P]),
            "oracle_linear_block": (None, [P, P, P, P, i32, i32, i32, i32, i32, P]),
            "oracle_project": (None, [P, P, i32, i32, P]),
            "oracle_sagesla_head": (i32, [P, P, P, P, i32, i32, i32, f64, i32, P, i32, P, P, P, P]),
            "oracle_adaptive_k": (None, [P, i32, i32, i32, i32, f64, P, P]),
            "oracle_adaptive_ksel": (i32, [P, i32, i32, i32]),
            "oracle_sagesla_head_adaptive": (i32, [P, P, P, P, i32, i32, i32, f64, f64, f64, i32, P, i32, P, P, P,
                                                   P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ number formats

def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_p(x), _p(out), x.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_n(_p(c), _p(out), c.size)
    return out


def bf16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_blocks(N: int, blk: int = 64) -> int:
    return lib().oracle_num_blocks(N, blk)


def ksel(topk: float, Nb: int) -> int:
    return lib().oracle_ksel(topk, Nb)


# ------------------------------------------------------------------ stages (one head)

def pool(x_bits, blk=64):
    x = _c(x_bits, np.uint16)
    N, d = x.shape
    out = np.empty((num_blocks(N, blk), d), np.float64)
    lib().oracle_pool(_p(x), N, d, blk, _p(out))
    return out


def scores(qbar, kbar):
    """[nq, nk] block scores qbar_i . kbar_j / sqrt(d)."""
    qbar, kbar = _c(qbar, np.float64), _c(kbar, np.float64)
    nq, d = qbar.shape
    nk = kbar.shape[0]
    out = np.empty((nq, nk), np.float64)
    lib().oracle_scores(_p(qbar), _p(kbar), nq, nk, d, _p(out))
    return out


def select(score_mat, k: int):
    """Top-k columns of every row (score desc, index asc), ascending. [nq, k] int32."""
    s = _c(score_mat, np.float64)
    nq, nk = s.shape
    idx = np.empty((nq, k), np.int32)
    lib().oracle_select(_p(s), nq, nk, k, _p(idx))
    return idx


def adaptive_k(score_mat, N, tau, blk=64):
    """Per query block: the fewest blocks (selection order) whose pooled attention mass
    n_j exp(s_ij - max) reaches tau of the row's total. Returns (k [nq] int32, margin [nq])
    where margin is the distance of tau from the nearer prefix mass around the decision,
    relative to the row's total."""
    s = _c(score_mat, np.float64)
    nq, Nb = s.shape
    k = np.empty(nq, np.int32)
    margin = np.empty(nq, np.float64)
    lib().oracle_adaptive_k(_p(s), nq, Nb, N, blk, float(tau), _p(k), _p(margin))
    return k, margin


def adaptive_ksel(k_rows, kmin, kmax):
    """A head's count: clamp(ceil(mean k_i - 1e-9), kmin, kmax)."""
    k = _c(k_rows, np.int32)
    return lib().oracle_adaptive_ksel(_p(k), len(k), int(kmin), int(kmax))


def order_best_first(score_row, kept):
    """Processing order of one row's kept blocks: best score first, then ascending."""
    row = _c(score_row, np.float64)
    out = np.array(kept, np.int32, copy=True)
    lib().oracle_order_best_first(_p(row), len(out), _p(out))
    return out


def k_mean(k_bits):
    k = _c(k_bits, np.uint16)
    N, d = k.shape
    mu = np.empty(d, np.float32)
    lib().oracle_k_mean(_p(k), N, d, _p(mu))
    return mu


def quant_blocks(x_f32, blk=64):
    x = _c(x_f32, np.float32)
    N, d = x.shape
    Nb = num_blocks(N, blk)
    q8 = np.empty((Nb * blk, d), np.int8)
    s = np.empty(Nb, np.float32)
    lib().oracle_quant_blocks(_p(x), N, d, blk, _p(q8), _p(s))
    return q8, s


def quant_v(v_bits):
    v = _c(v_bits, np.uint16)
    N, d = v.shape
    v8 = np.empty((N, d), np.uint8)
    sv = np.empty(d, np.float32)
    lib().oracle_quant_v(_p(v), N, d, _p(v8), _p(sv))
    return v8, sv


def dot_i8(a, b) -> int:
    a, b = _c(a, np.int8), _c(b, np.int8)
    return int(lib().oracle_dot_i8(_p(a), _p(b), a.size))


def quantize_head(q_bits, k_bits, v_bits, blk=64):
    """Q8/K8/V8 and scales of one head, as the quantized path computes them."""
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    qf = bf16_to_f64(q).astype(np.float32)
    q8, sq = quant_blocks(qf, blk)
    mu = k_mean(k)
    kf = bf16_to_f64(k).astype(np.float32) - mu[None, :]
    k8, sk = quant_blocks(kf.astype(np.float32), blk)
    v8, sv = quant_v(v_bits)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv, kmean=mu)


def sparse_block(qz, idx, N, blk, qb, stats=False):
    """O_s rows of query block qb from the quantized tensors in qz (quantize_head). With
    stats, also each row's final FP8 row sum l and reference m: (out, l, m)."""
    d = qz["q8"].shape[1]
    k = idx.shape[1]
    out = np.zeros((blk, d), np.float64)
    idx = _c(idx, np.int32)
    l = np.zeros(blk, np.float64) if stats else None
    m = np.zeros(blk, np.float32) if stats else None
    lib().oracle_sparse_block(_p(qz["q8"]), _p(qz["k8"]), _p(qz["v8"]), _p(qz["sq"]), _p(qz["sk"]),
                              _p(qz["sv"]), _p(idx), k, N, d, blk, qb, _p(out), _p(l), _p(m))
    return (out, l, m) if stats else out


def phi(x_bits):
    x = _c(x_bits, np.uint16)
    out = np.empty(x.shape, np.float64)
    d = x.shape[-1]
    for r in range(x.size // d):
        lib().oracle_phi(_p(x.reshape(-1, d)[r]), d, _p(out.reshape(-1, d)[r]))
    return out


def linear_states(k_bits, v_bits, blk=64):
    k, v = _c(k_bits, np.uint16), _c(v_bits, np.uint16)
    N, d = k.shape
    Nb = num_blocks(N, blk)
    H = np.empty((Nb, d, d), np.float64)
    z = np.empty((Nb, d), np.float64)
    lib().oracle_linear_states(_p(k), _p(v), N, d, blk, _p(H), _p(z))
    return H, z


def linear_block(q_bits, H, z, idx, blk, qb):
    q = _c(q_bits, np.uint16)
    N, d = q.shape
    out = np.zeros((blk, d), np.float64)
    idx = _c(idx, np.int32)
    lib().oracle_linear_block(_p(q), _p(_c(H, np.float64)), _p(_c(z, np.float64)), _p(idx),
                              idx.shape[1], N, d, blk, qb, _p(out))
    return out


def project(ol, w_bits):
    ol = _c(ol, np.float64)
    w = _c(w_bits, np.uint16)
    rows, d = ol.shape
    y = np.empty((rows, d), np.float64)
    lib().oracle_project(_p(ol), _p(w), rows, d, _p(y))
    return y


# ------------------------------------------------------------------ whole head / all heads

def sagesla_head(q_bits, k_bits, v_bits, w_bits, topk, quant=True, qblocks=None, blk=64):
    """SageSLA forward of one head. Returns dict(out, out_s, out_l, idx, ksel, qblocks).

    out/out_s/out_l are [len(qblocks)*blk, d] fp64; rows past N in the last block are 0.
    idx is [Nb, ksel] in processing order (best first, then ascending); rows of query
    blocks not listed in qblocks are -1.
    """
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    w = None if w_bits is None else _c(w_bits, np.uint16)
    N, d = q.shape
    Nb = num_blocks(N, blk)
    qbl = np.arange(Nb, dtype=np.int32) if qblocks is None else _c(qblocks, np.int32)
    ks = ksel(topk, Nb)
    out = np.zeros((len(qbl) * blk, d), np.float64)
    os_ = np.zeros_like(out)
    ol = np.zeros_like(out)
    idx = np.empty((Nb, ks), np.int32)
    r = lib().oracle_sagesla_head(_p(q), _p(k), _p(v), _p(w), N, d, blk, float(topk), int(bool(quant)),
                                  _p(qbl), len(qbl), _p(out), _p(os_), _p(ol), _p(idx))
    if r < 0:
        raise ValueError("oracle_sagesla_head: bad arguments")
    return dict(out=out, out_s=os_, out_l=ol, idx=idx, ksel=ks, qblocks=qbl)


def sagesla_head_adaptive(q_bits, k_bits, v_bits, w_bits, topk_min, topk_max, tau, quant=True, qblocks=None,
                          blk=64):
    """SageSLA forward of one head with its content-adaptive count. Returns dict(out, out_s,
    out_l, idx, ksel, k_rows, qblocks); idx is [Nb, kmax] (kmax = ksel(topk_max)), -1 past
    the head's ksel."""
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    v = _c(v_bits, np.uint16)
    w = None if w_bits is None else _c(w_bits, np.uint16)
    N, d = q.shape
    Nb = num_blocks(N, blk)
    qbl = np.arange(Nb, dtype=np.int32) if qblocks is None else _c(qblocks, np.int32)
    kmax = ksel(topk_max, Nb)
    out = np.zeros((len(qbl) * blk, d), np.float64)
    os_ = np.zeros_like(out)
    ol = np.zeros_like(out)
    idx = np.empty((Nb, kmax), np.int32)
    k_rows = np.empty(Nb, np.int32)
    r = lib().oracle_sagesla_head_adaptive(_p(q), _p(k), _p(v), _p(w), N, d, blk, float(topk_min),
                                           float(topk_max), float(tau), int(bool(quant)), _p(qbl), len(qbl),
                                           _p(out), _p(os_), _p(ol), _p(idx), _p(k_rows))
    if r < 0:
        raise ValueError("oracle_sagesla_head_adaptive: bad arguments")
    return dict(out=out, out_s=os_, out_l=ol, idx=idx, ksel=r, k_rows=k_rows, qblocks=qbl)


def sagesla(q_bits, k_bits, v_bits, w_bits, topk, quant=True, heads=None, qblocks=None, blk=64,
            threads=None):
    """All (or the listed) heads of [B, H, N, d] inputs; heads run in parallel threads.

    heads: list of (b, h); qblocks: list of query blocks per head (or None = all).
    Returns {(b, h): sagesla_head(...)}.
    """
    B, H = q_bits.shape[:2]
    hs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    threads = threads or min(len(hs), os.cpu_count() or 1)

    def run(bh):
        b, h = bh
        return bh, sagesla_head(q_bits[b, h], k_bits[b, h], v_bits[b, h], w_bits, topk, quant,
                                qblocks, blk)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(run, hs))
