"""CPU oracle for the producer-side step before SageSLA (test infrastructure only).

The pages credit rewritten LayerNorm/RMSNorm kernels fused with their neighbours, and
operator fusion in general, with part of the end-to-end speedup (news.qq.com explainer,
"Fourth key"). Here the neighbour is the attention's first pass: the QKV projection's
output [B, N, 3, H, d] (token-major, as a linear layer writes it) is normalized, laid out as
[B, H, N, d], and pooled / Q-quantized (the pool stage) in one pass.

RMSNorm over the model width D = H*d (as in the Wan models' q/k norms), per token:
    ss = sum x^2 (fp64; the squares of bf16 values are exact), r = fp32(1 / sqrt(ss / D + eps))
    n  = bf16_rne(fp32(x) * r),   out = bf16_rne(fp32(n) * fp32(g))
(normalize in fp32, round to the activation type, then scale by the learned weight g);
V is copied. The pool-stage outputs then follow from these bf16 tensors by the attention
oracle's own pooling and quantization functions. Arrays are numpy; bf16 as uint16 bits.
"""
from __future__ import annotations

import numpy as np


def _f32_of_bf16(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_rne(f32):
    u = np.asarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rms_scale(x_bits, eps):
    """Per-row r = fp32(1 / sqrt(mean(x^2) + eps)) of bf16 rows [n][D] (fp64 up to the
    final rounding)."""
    x = _f32_of_bf16(x_bits).astype(np.float64)
    D = x.shape[-1]
    ss = (x * x).sum(axis=-1)
    return (1.0 / np.sqrt(ss / D + eps)).astype(np.float32)


def rmsnorm(x_bits, g_bits, eps):
    """bf16 rows [n][D] -> bf16 rows: bf16(bf16(x * r) * g)."""
    r = rms_scale(x_bits, eps)
    n = _bf16_rne(_f32_of_bf16(x_bits) * r[..., None])
    return _bf16_rne(_f32_of_bf16(n) * _f32_of_bf16(g_bits))


def prepare(qkv_bits, gq_bits, gk_bits, H, d, eps):
    """One batch element: qkv [N][3*H*d] bf16 -> (q, k, v) [H][N][d] bf16 (q, k normalized)."""
    x = np.asarray(qkv_bits, np.uint16)
    N = x.shape[0]
    D = H * d
    q = rmsnorm(x[:, :D], gq_bits, eps)
    k = rmsnorm(x[:, D:2 * D], gk_bits, eps)
    v = x[:, 2 * D:3 * D]
    heads = lambda t: np.ascontiguousarray(t.reshape(N, H, d).transpose(1, 0, 2))
    return heads(q), heads(k), heads(v)
