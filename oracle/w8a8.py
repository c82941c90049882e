"""CPU oracle for the W8A8 linear layer (test infrastructure only; see w8a8_oracle.c).

INT8 weights in 128 x 128 blocks with one scale each, INT8 activations with one scale per
token and 128-channel block, integer products summed per block, scaled and summed in fp64
(TurboDiffusion explainer, news.qq.com, "Third key"). Arrays are numpy; bf16 tensors are
passed as uint16 bit patterns, row-major.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import lib as _oracle_lib

_ready = False


def _lib():
    global _ready
    L = _oracle_lib()
    if not _ready:
        P, i32 = C.c_void_p, C.c_int
        for name, args in {
            "oracle_w8a8_quant_act": [P, i32, i32, P, P],
            "oracle_w8a8_quant_weight": [P, i32, i32, P, P],
            "oracle_w8a8_gemm": [P, P, P, P, P, i32, i32, i32, i32, i32, P],
        }.items():
            fn = getattr(L, name)
            fn.restype = None
            fn.argtypes = args
        _ready = True
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def quant_act(x_bits):
    """x [M][K] bf16 bits -> (q [M][K] int8, s [M][K/128] fp32)."""
    x = np.ascontiguousarray(x_bits, np.uint16)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.int8)
    s = np.empty((M, K // 128), np.float32)
    _lib().oracle_w8a8_quant_act(_p(x), M, K, _p(q), _p(s))
    return q, s


def quant_weight(w_bits):
    """w [N][K] bf16 bits -> (q [N][K] int8, s [N/128][K/128] fp32)."""
    w = np.ascontiguousarray(w_bits, np.uint16)
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    q = np.empty((N, K), np.int8)
    s = np.empty((N // 128, K // 128), np.float32)
    _lib().oracle_w8a8_quant_weight(_p(w), N, K, _p(q), _p(s))
    return q, s


def gemm(qx, sx, qw, sw, bias_bits=None, rows=None):
    """y [M][N] fp64 from the codes and scales; rows = (m0, m1) limits the rows computed
    (the others are NaN)."""
    qx = np.ascontiguousarray(qx, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    sx = np.ascontiguousarray(sx, np.float32)
    sw = np.ascontiguousarray(sw, np.float32)
    M, K = qx.shape
    N = qw.shape[0]
    b = None if bias_bits is None else np.ascontiguousarray(bias_bits, np.uint16)
    m0, m1 = rows if rows is not None else (0, M)
    y = np.full((M, N), np.nan)
    _lib().oracle_w8a8_gemm(_p(qx), _p(sx), _p(qw), _p(sw), _p(b), M, N, K, m0, m1, _p(y))
    return y


def linear(x_bits, w_bits, bias_bits=None, rows=None):
    """The whole W8A8 layer: quantize both operands, then the block-scaled product."""
    qx, sx = quant_act(x_bits)
    qw, sw = quant_weight(w_bits)
    return gemm(qx, sx, qw, sw, bias_bits, rows)
