"""CPU oracle for the sparse-linear attention (SLA) backward pass (test infrastructure only).

Only the tests and the benchmark's CPU-baseline leg use this module; the GPU library never
imports it. Plain numpy in fp64, one head at a time, [N, d] arrays, written block by block
in the order the method defines, with no fusion.

SLA is trainable: it is fine-tuned so that the model learns which connections matter
(news.qq.com explainer, "First key: attention" and "From training to deployment"); SageSLA,
its quantized form, only replaces it at inference. Fine-tuning needs the gradients of the
unquantized SLA forward, which is (per head, blocks of `blk` tokens, kept lists `idx`):

    sparse part:  O_s[i] = softmax(Q_i K_J^T / sqrt(d)) V_J over the tokens J of the key
                  blocks kept by query block i;  lse = the row log-sum-exp
    linear part:  phi = softmax over the d channels;  H_j = sum_{t in j} phi(K_t)^T V_t,
                  z_j = sum_{t in j} phi(K_t);  H^c_i, z^c_i = sums over the blocks NOT kept;
                  O_l = phi(Q) H^c_i / (phi(Q) . z^c_i)   (0 when nothing is left out)
    output:       O = O_s + O_l W   (W: [d, d], row vector times W; W = None: no linear part)

The selection (top-k of pooled scores) is piecewise constant in the inputs, so its
derivative is zero wherever it is defined: the backward takes `idx` as fixed.

Given dO = dL/dO, the backward returns dL/dQ, dL/dK, dL/dV and dL/dW by the chain rule
through each of the steps above (softmax rows: dS = P * (dP - rowsum(P * dP)); the
channel softmax phi: dx = phi * (dphi - phi . dphi); the ratio u / s: du = dO_l / s,
ds = -(dO_l . O_l) / s; complements: a block's state gradient is the sum of the complement
gradients of the query blocks that left it out).
"""
from __future__ import annotations

import numpy as np


def _blocks(N, blk):
    Nb = (N + blk - 1) // blk
    return Nb, [slice(b * blk, min(N, (b + 1) * blk)) for b in range(Nb)]


def _kept_tokens(idx_row, sl):
    return np.concatenate([np.arange(sl[j].start, sl[j].stop) for j in sorted(int(t) for t in idx_row)])


def _softmax_rows(x):
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def _complement(idx_row, Nb):
    keep = np.zeros(Nb, bool)
    keep[np.asarray(idx_row, int)] = True
    return np.flatnonzero(~keep)


def sla_forward(q, k, v, w, idx, blk=64):
    """fp64 SLA forward of one head. q, k, v: [N, d]; w: [d, d] or None; idx: [Nb, k_sel].
    Returns dict(out, out_s, out_l, lse) ([N, d] each, lse [N])."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    N, d = q.shape
    Nb, sl = _blocks(N, blk)
    scale = 1.0 / np.sqrt(d)
    out_s = np.zeros((N, d))
    lse = np.zeros(N)
    for i in range(Nb):
        cols = _kept_tokens(idx[i], sl)
        s = q[sl[i]] @ k[cols].T * scale
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        out_s[sl[i]] = (p / l[:, None]) @ v[cols]
        lse[sl[i]] = m + np.log(l)
    out_l = np.zeros((N, d))
    if w is not None:
        phq, phk = _softmax_rows(q), _softmax_rows(k)
        H = np.stack([phk[sl[j]].T @ v[sl[j]] for j in range(Nb)])
        z = np.stack([phk[sl[j]].sum(axis=0) for j in range(Nb)])
        for i in range(Nb):
            comp = _complement(idx[i], Nb)
            if comp.size == 0:
                continue
            Hc, zc = H[comp].sum(axis=0), z[comp].sum(axis=0)
            out_l[sl[i]] = (phq[sl[i]] @ Hc) / (phq[sl[i]] @ zc)[:, None]
    y = out_l @ np.asarray(w, np.float64) if w is not None else np.zeros((N, d))
    return dict(out=out_s + y, out_s=out_s, out_l=out_l, lse=lse)


def sla_backward(q, k, v, w, idx, dout, blk=64):
    """Gradients of L = sum(dout * O) for the fp64 SLA forward above.
    Returns dict(dq, dk, dv, dw) (dw None when w is None), plus the sparse and linear
    parts of dq, dk, dv separately (dq_s, dk_s, dv_s, dq_l, dk_l, dv_l)."""
    q, k, v, dout = (np.asarray(a, np.float64) for a in (q, k, v, dout))
    N, d = q.shape
    Nb, sl = _blocks(N, blk)
    scale = 1.0 / np.sqrt(d)
    fw = sla_forward(q, k, v, w, idx, blk)

    # sparse part: the softmax rows recomputed from the saved row log-sum-exp
    dq_s, dk_s, dv_s = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for i in range(Nb):
        cols = _kept_tokens(idx[i], sl)
        p = np.exp(q[sl[i]] @ k[cols].T * scale - fw["lse"][sl[i]][:, None])
        do = dout[sl[i]]
        dv_s[cols] += p.T @ do
        dp = do @ v[cols].T
        D = (do * fw["out_s"][sl[i]]).sum(axis=1)  # = rowsum(p * dp)
        ds = p * (dp - D[:, None])
        dq_s[sl[i]] += ds @ k[cols] * scale
        dk_s[cols] += ds.T @ q[sl[i]] * scale

    dq_l, dk_l, dv_l = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    dw = None
    if w is not None:
        w = np.asarray(w, np.float64)
        dw = fw["out_l"].T @ dout
        dol = dout @ w.T
        phq, phk = _softmax_rows(q), _softmax_rows(k)
        H = np.stack([phk[sl[j]].T @ v[sl[j]] for j in range(Nb)])
        z = np.stack([phk[sl[j]].sum(axis=0) for j in range(Nb)])
        dH, dz = np.zeros_like(H), np.zeros_like(z)
        dphq = np.zeros((N, d))
        for i in range(Nb):
            comp = _complement(idx[i], Nb)
            if comp.size == 0:
                continue
            Hc, zc = H[comp].sum(axis=0), z[comp].sum(axis=0)
            u = phq[sl[i]] @ Hc
            s = phq[sl[i]] @ zc
            ol = u / s[:, None]
            du = dol[sl[i]] / s[:, None]
            ds = -(dol[sl[i]] * ol).sum(axis=1) / s
            dphq[sl[i]] = du @ Hc.T + ds[:, None] * zc[None, :]
            dHc = phq[sl[i]].T @ du
            dzc = phq[sl[i]].T @ ds
            for j in comp:
                dH[j] += dHc
                dz[j] += dzc
        dphk = np.zeros((N, d))
        for j in range(Nb):
            dphk[sl[j]] = v[sl[j]] @ dH[j].T + dz[j][None, :]
            dv_l[sl[j]] = phk[sl[j]] @ dH[j]
        dq_l = phq * (dphq - (phq * dphq).sum(axis=1, keepdims=True))
        dk_l = phk * (dphk - (phk * dphk).sum(axis=1, keepdims=True))
    return dict(dq=dq_s + dq_l, dk=dk_s + dk_l, dv=dv_s + dv_l, dw=dw, dq_s=dq_s, dk_s=dk_s, dv_s=dv_s,
                dq_l=dq_l, dk_l=dk_l, dv_l=dv_l, lse=fw["lse"], out=fw["out"], out_s=fw["out_s"],
                out_l=fw["out_l"])


def sla_backward_rows(q, k, v, w, idx, dout, qblocks, kblocks, blk=64):
    """The same gradients as sla_backward, for the rows of some blocks only: dq on the query
    blocks `qblocks`, dk and dv on the key blocks `kblocks` (for inputs too long to
    differentiate whole). The sparse part needs, per key block, every query block that keeps
    it; the linear part needs the complement-state gradients of every query block, which
    are cheap (one 128 x 128 product each). Returns dict(dq, dk, dv) of {block: rows}."""
    q, k, v, dout = (np.asarray(a, np.float64) for a in (q, k, v, dout))
    N, d = q.shape
    Nb, sl = _blocks(N, blk)
    scale = 1.0 / np.sqrt(d)

    def sparse_rows(i):
        cols = _kept_tokens(idx[i], sl)
        s = q[sl[i]] @ k[cols].T * scale
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        p /= p.sum(axis=1, keepdims=True)
        o_s = p @ v[cols]
        do = dout[sl[i]]
        dp = do @ v[cols].T
        D = (do * o_s).sum(axis=1)
        return cols, p, p * (dp - D[:, None])

    dq = {i: np.zeros((sl[i].stop - sl[i].start, d)) for i in qblocks}
    dk = {j: np.zeros((sl[j].stop - sl[j].start, d)) for j in kblocks}
    dv = {j: np.zeros((sl[j].stop - sl[j].start, d)) for j in kblocks}
    for i in qblocks:
        cols, p, ds = sparse_rows(i)
        dq[i] += ds @ k[cols] * scale
    keepers = {j: [i for i in range(Nb) if j in set(int(t) for t in idx[i])] for j in kblocks}
    for j in kblocks:
        for i in keepers[j]:
            cols, p, ds = sparse_rows(i)
            at = np.flatnonzero((cols >= sl[j].start) & (cols < sl[j].stop))
            dv[j] += p[:, at].T @ dout[sl[i]]
            dk[j] += ds[:, at].T @ q[sl[i]] * scale

    if w is not None:
        w = np.asarray(w, np.float64)
        phq, phk = _softmax_rows(q), _softmax_rows(k)
        H = np.stack([phk[sl[j]].T @ v[sl[j]] for j in range(Nb)])
        z = np.stack([phk[sl[j]].sum(axis=0) for j in range(Nb)])
        dH, dz = np.zeros_like(H), np.zeros_like(z)
        # C[i][j] = 1 when query block i leaves key block j out: every complement sum at
        # once as one product with the 0/1 matrix (the same sums over the blocks not kept)
        C = np.ones((Nb, Nb))
        for i in range(Nb):
            C[i, np.asarray(idx[i], int)] = 0.0
        Hc_all = (C @ H.reshape(Nb, -1)).reshape(H.shape)
        zc_all = C @ z
        for i in range(Nb):
            if not C[i].any():
                continue
            Hc, zc = Hc_all[i], zc_all[i]
            u = phq[sl[i]] @ Hc
            s = phq[sl[i]] @ zc
            ol = u / s[:, None]
            dol = dout[sl[i]] @ w.T
            du = dol / s[:, None]
            dsv = -(dol * ol).sum(axis=1) / s
            if i in dq:
                dph = du @ Hc.T + dsv[:, None] * zc[None, :]
                p_ = phq[sl[i]]
                dq[i] += p_ * (dph - (p_ * dph).sum(axis=1, keepdims=True))
            dHc = phq[sl[i]].T @ du
            dzc = phq[sl[i]].T @ dsv
            for j in kblocks:
                if C[i, j]:
                    dH[j] += dHc
                    dz[j] += dzc
        for j in kblocks:
            p_ = phk[sl[j]]
            dph = v[sl[j]] @ dH[j].T + dz[j][None, :]
            dk[j] += p_ * (dph - (p_ * dph).sum(axis=1, keepdims=True))
            dv[j] += p_ @ dH[j]
    return dict(dq=dq, dk=dk, dv=dv)
