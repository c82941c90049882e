"""Seeded synthetic attention inputs with the shapes of the Wan2.x video DiT layers.

The pages measure SageSLA inside Wan2.1/Wan2.2 video models on real prompts
(TurboDiffusion explainer on news.qq.com, sections "Why video generation is so slow"
and "From training to deployment"; dgmzs.com.cn summary, section "Evaluation").
Those weights and prompts are not available, so these tensors stand in for the
attention inputs of one layer: bf16 Q, K, V of shape [B, H, N, d] over a latent
video grid of T x Hh x W tokens in (t, y, x) row-major order, plus a d x d bf16
projection matrix for the linear branch.

This module holds only the input recipe. It computes nothing of the attention
method itself and is shared by the oracle tests and the GPU path.

Recipe (all draws are seeded):
  * scalar parameters (field frequencies, phases, amplitudes, per-channel K offsets,
    W_proj, long-range pairs) come from numpy ``default_rng(seed)`` in a fixed order,
    so they are identical on every device;
  * bulk noise (Q, K, V noise) comes from ``torch.Generator(device).manual_seed(seed)``
    on the device that holds the tensors. The same seed therefore gives different
    noise on CPU and on GPU; every comparison feeds one generated set of bf16 bytes
    to both sides.
  * field F[h, n, c] = sum_{k<8} a * sin(2*pi*(ft*t/T + fy*y/Hh + fx*x/W) + phase),
    ft, fy, fx ~ U[0, 2) cycles per axis extent, phase ~ U[0, 2*pi), a ~ N(0, 1/4),
    which has unit variance per channel. Q and K share F (the source of locality).
  * Q = F + s*eps, K = F + s*eps' + m_c with m_c ~ N(0, 4) per (h, c), V ~ N(0, 1).
  * "iid" kind (the tiny case): Q, K, V ~ N(0, 1) and K += m_c.
  * "longrange" kind adds M = round(0.05*N) token pairs (r, s) at grid Manhattan
    distance >= 16; each gets u = (sqrt(d)/2) * g_hat (a random unit direction)
    added to Q_r, K_r, Q_s and K_s.
  * W_proj ~ N(0, 1/d). Everything is rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    grid: tuple  # (T, Hh, W) latent token grid; N = T*Hh*W
    d: int
    topk: float
    kind: str  # "iid", "field", "longrange"
    noise: float
    seed: int
    linear: bool = True  # False: the linear branch is off (proj is not passed)
    block: int = 64
    note: str = ""

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w


# The five workloads: a tiny case, three Wan2.1 layer shapes and the I2V-A14B-720P
# variant (plus its dense SageAttention run at the same shape).
CONFIGS = {
    "tiny": Config("tiny", 1, 2, (2, 32, 32), 128, 0.1, "iid", 0.0, 0,
                   note="B=1 H=2 N=2048, iid N(0,1) with per-channel K offset"),
    "wan1.3b-480p": Config("wan1.3b-480p", 1, 12, (21, 30, 52), 128, 0.1, "field", 0.5, 1,
                           note="Wan2.1-1.3B-480P attention layer"),
    "wan14b-480p": Config("wan14b-480p", 1, 40, (21, 30, 52), 128, 0.1, "field", 0.5, 2,
                          note="Wan2.1-14B-480P attention layer"),
    "wan14b-720p": Config("wan14b-720p", 1, 40, (21, 45, 80), 128, 0.1, "field", 0.5, 3,
                          note="Wan2.1-14B-720P attention layer (headline)"),
    "i2v-a14b-720p": Config("i2v-a14b-720p", 1, 40, (21, 45, 80), 128, 0.15, "longrange", 0.2, 4,
                            note="Wan2.2-I2V-A14B-720P attention layer"),
    "i2v-a14b-720p-dense": Config("i2v-a14b-720p-dense", 1, 40, (21, 45, 80), 128, 1.0,
                                  "longrange", 0.2, 4, linear=False,
                                  note="dense SageAttention at the I2V shape (topk=1, no linear branch)"),
}


def scaled(cfg: Config, H: int | None = None, grid: tuple | None = None, seed: int | None = None,
           topk: float | None = None, name: str | None = None, linear: bool | None = None,
           B: int | None = None) -> Config:
    """A copy of ``cfg`` with fewer heads / a smaller grid (same recipe), for quick tests."""
    from dataclasses import replace
    kw = {}
    if B is not None:
        kw["B"] = B
    if H is not None:
        kw["H"] = H
    if grid is not None:
        kw["grid"] = tuple(grid)
    if seed is not None:
        kw["seed"] = seed
    if topk is not None:
        kw["topk"] = topk
    if linear is not None:
        kw["linear"] = linear
    kw["name"] = name or (cfg.name + "-scaled")
    return replace(cfg, **kw)


def _grid_coords(grid, device):
    T, Hh, W = grid
    n = torch.arange(T * Hh * W, device=device, dtype=torch.int64)
    t = n // (Hh * W)
    y = (n // W) % Hh
    x = n % W
    return t, y, x


def _field_head(params, grid, device):
    """F[n, c] for one head; params = (ft, fy, fx, phase, amp), each [d, 8] float64."""
    T, Hh, W = grid
    t, y, x = _grid_coords(grid, device)
    ft, fy, fx, ph, amp = (torch.as_tensor(p, device=device, dtype=torch.float32) for p in params)
    tt = (t.to(torch.float32) / T)[:, None, None]
    yy = (y.to(torch.float32) / Hh)[:, None, None]
    xx = (x.to(torch.float32) / W)[:, None, None]
    ang = (2.0 * math.pi) * (tt * ft + yy * fy + xx * fx) + ph  # [N, d, 8]
    return (amp * torch.sin(ang)).sum(-1)  # [N, d]


def _long_range_pairs(rng, grid, M):
    T, Hh, W = grid
    N = T * Hh * W
    pairs = []
    while len(pairs) < M:
        r, s = rng.integers(0, N, size=2)
        tr, yr, xr = r // (Hh * W), (r // W) % Hh, r % W
        ts, ys, xs = s // (Hh * W), (s // W) % Hh, s % W
        if abs(tr - ts) + abs(yr - ys) + abs(xr - xs) >= 16:
            pairs.append((int(r), int(s)))
    return pairs


def make_inputs(cfg: Config, device="cpu"):
    """Returns dict(q, k, v, proj) as bf16 torch tensors on ``device``.

    q, k, v: [B, H, N, d] contiguous; proj: [d, d] (None when cfg.linear is False).
    """
    device = torch.device(device)
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    rng = np.random.default_rng(cfg.seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)

    # scalar draws, fixed order: per (b, h): field params, K offset; then W_proj; then pairs
    fparams = []
    koff = np.empty((B, H, d))
    for b in range(B):
        for h in range(H):
            ft = rng.uniform(0.0, 2.0, size=(d, 8))
            fy = rng.uniform(0.0, 2.0, size=(d, 8))
            fx = rng.uniform(0.0, 2.0, size=(d, 8))
            ph = rng.uniform(0.0, 2.0 * math.pi, size=(d, 8))
            amp = rng.normal(0.0, 0.5, size=(d, 8))  # N(0, 1/4): 8 terms of variance a^2/2
            fparams.append((ft, fy, fx, ph, amp))
            koff[b, h] = rng.normal(0.0, 2.0, size=d)  # N(0, 4)
    w = rng.normal(0.0, 1.0 / math.sqrt(d), size=(d, d))
    pairs = None
    if cfg.kind == "longrange":
        M = int(round(0.05 * N))
        pairs = _long_range_pairs(rng, cfg.grid, M)
        dirs = rng.normal(0.0, 1.0, size=(M, d))
        dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
        dirs *= math.sqrt(d) / 2.0

    q = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    for b in range(B):
        for h in range(H):
            i = b * H + h
            nq = torch.randn((N, d), generator=gen, device=device, dtype=torch.float32)
            nk = torch.randn((N, d), generator=gen, device=device, dtype=torch.float32)
            nv = torch.randn((N, d), generator=gen, device=device, dtype=torch.float32)
            off = torch.as_tensor(koff[b, h], device=device, dtype=torch.float32)
            if cfg.kind == "iid":
                qf, kf = nq, nk + off
            else:
                F = _field_head(fparams[i], cfg.grid, device)
                qf = F + cfg.noise * nq
                kf = F + cfg.noise * nk + off
                if pairs is not None:
                    idx_r = torch.as_tensor([p[0] for p in pairs], device=device)
                    idx_s = torch.as_tensor([p[1] for p in pairs], device=device)
                    u = torch.as_tensor(dirs, device=device, dtype=torch.float32)
                    qf.index_add_(0, idx_r, u)
                    qf.index_add_(0, idx_s, u)
                    kf.index_add_(0, idx_r, u)
                    kf.index_add_(0, idx_s, u)
            q[b, h] = qf.to(torch.bfloat16)
            k[b, h] = kf.to(torch.bfloat16)
            v[b, h] = nv.to(torch.bfloat16)
    proj = torch.as_tensor(w, dtype=torch.float32).to(torch.bfloat16).to(device) if cfg.linear else None
    return {"q": q, "k": k, "v": v, "proj": proj}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (host copy), for passing to C code."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def make_linear_inputs(M: int, K: int, N: int, seed: int, device="cpu", bias: bool = True):
    """Inputs of one linear layer of the transformer: dict(x bf16 [M][K], w bf16 [N][K],
    bias bf16 [N] or None), row-major as a torch Linear takes them.

    x: N(0, 1) entries times a per-token magnitude exp(N(0, 1/4)), and K/64 outlier
    channels (every 64th) scaled by 8, the structure that makes per-block activation scales
    matter; w: N(0, 1/K) (unit output variance per unit input); bias: N(0, 0.02^2).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    x *= torch.exp(0.5 * torch.randn((M, 1), generator=gen, device=device, dtype=torch.float32))
    x[:, ::64] *= 8.0
    x = x.to(torch.bfloat16)
    w = (torch.randn((N, K), generator=gen, device=device, dtype=torch.float32) / math.sqrt(K)).to(torch.bfloat16)
    b = None
    if bias:
        b = (0.02 * torch.randn((N,), generator=gen, device=device, dtype=torch.float32)).to(torch.bfloat16)
    return {"x": x, "w": w, "bias": b}


def make_projection_inputs(B: int, N: int, H: int, d: int, seed: int, device="cpu"):
    """A QKV projection output and RMSNorm weights: dict(qkv bf16 [B, N, 3*H*d], gq, gk bf16
    [H*d]). qkv ~ N(0, 1) times a per-token magnitude exp(N(0, 1/4)) per part, plus a
    per-channel offset N(0, 1/4) on the k part (the channel bias that K smoothing removes);
    gq, gk ~ 1 + N(0, 0.1^2)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    D = H * d
    x = torch.randn((B, N, 3, D), generator=gen, device=device, dtype=torch.float32)
    x *= torch.exp(0.5 * torch.randn((B, N, 3, 1), generator=gen, device=device, dtype=torch.float32))
    x[:, :, 1, :] += 0.5 * torch.randn((D,), generator=gen, device=device, dtype=torch.float32)
    g = 1.0 + 0.1 * torch.randn((2, D), generator=gen, device=device, dtype=torch.float32)
    return {"qkv": x.reshape(B, N, 3 * D).to(torch.bfloat16), "gq": g[0].to(torch.bfloat16),
            "gk": g[1].to(torch.bfloat16)}
