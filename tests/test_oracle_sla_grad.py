"""Pins for the SLA backward oracle (oracle/sla_grad.py) against facts that do not come from
it: central finite differences of its own forward in fp64 (directional and per element),
torch autograd of dense softmax attention where every block is kept and the linear part is
off, the C oracle's unquantized forward, and invariants the mathematics fixes (rows of the
sparse probabilities sum to one; softmax is shift-invariant over its row). CPU only."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import sla_grad as G


def make(N, d, seed, ksel, blk, linear=True, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, d)) * scale
    k = rng.standard_normal((N, d)) * scale
    v = rng.standard_normal((N, d))
    w = rng.standard_normal((d, d)) / np.sqrt(d) if linear else None
    dout = rng.standard_normal((N, d))
    Nb = (N + blk - 1) // blk
    idx = np.stack([rng.choice(Nb, ksel, replace=False) for _ in range(Nb)]).astype(np.int32)
    return q, k, v, w, dout, idx


def loss(q, k, v, w, idx, dout, blk):
    return float((G.sla_forward(q, k, v, w, idx, blk)["out"] * dout).sum())


CASES = [
    # N, d, seed, ksel, blk: a partial last block in each
    (150, 16, 1, 1, 64),
    (150, 16, 2, 2, 64),
    (70, 8, 3, 2, 16),
    (97, 12, 4, 3, 16),
]


@pytest.mark.parametrize("N,d,seed,ksel,blk", CASES)
def test_directional_finite_differences(N, d, seed, ksel, blk):
    q, k, v, w, dout, idx = make(N, d, seed, ksel, blk)
    g = G.sla_backward(q, k, v, w, idx, dout, blk)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    args = dict(q=q, k=k, v=v, w=w)
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"]), ("w", g["dw"])):
        u = rng.standard_normal(args[name].shape)
        ap, am = dict(args), dict(args)
        ap[name] = args[name] + eps * u
        am[name] = args[name] - eps * u
        fd = (loss(ap["q"], ap["k"], ap["v"], ap["w"], idx, dout, blk) -
              loss(am["q"], am["k"], am["v"], am["w"], idx, dout, blk)) / (2 * eps)
        an = float((grad * u).sum())
        assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (name, fd, an)


def test_elementwise_finite_differences():
    N, d, blk = 150, 16, 64
    q, k, v, w, dout, idx = make(N, d, 7, 1, blk)
    g = G.sla_backward(q, k, v, w, idx, dout, blk)
    eps = 1e-6
    # first token, a middle token, tokens of the partial last block
    for name, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        for t, c in ((0, 0), (70, 5), (128, 15), (149, 3)):
            args = dict(q=q.copy(), k=k.copy(), v=v.copy())
            args[name][t, c] += eps
            lp = loss(args["q"], args["k"], args["v"], w, idx, dout, blk)
            args[name][t, c] -= 2 * eps
            lm = loss(args["q"], args["k"], args["v"], w, idx, dout, blk)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[t, c]) <= 1e-6 * (abs(grad[t, c]) + 1.0), (name, t, c, fd, grad[t, c])


def test_dense_equals_autograd_attention():
    """Every block kept and no linear part: plain softmax attention, differentiated by torch."""
    N, d, blk = 150, 16, 64
    q, k, v, _, dout, _ = make(N, d, 8, 1, blk, linear=False)
    Nb = 3
    idx = np.tile(np.arange(Nb, dtype=np.int32), (Nb, 1))
    g = G.sla_backward(q, k, v, None, idx, dout, blk)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    o = torch.softmax(tq @ tk.T / np.sqrt(d), dim=-1) @ tv
    (o * torch.tensor(dout)).sum().backward()
    for a, b in ((g["dq"], tq.grad), (g["dk"], tk.grad), (g["dv"], tv.grad)):
        assert np.allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["out"], o.detach().numpy(), rtol=1e-10, atol=1e-12)
    assert g["dw"] is None


def test_forward_matches_c_oracle_unquantized():
    """The numpy forward against the C oracle's unquantized SLA forward (an independent
    implementation), on bf16-exact inputs with the C oracle's own selection."""
    rng = np.random.default_rng(9)
    N, d = 200, 128
    def bf(x):
        f = np.asarray(x, np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        return r, (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qb, q = bf(rng.standard_normal((N, d)))
    kb, k = bf(rng.standard_normal((N, d)) + rng.standard_normal(d) * 2)
    vb, v = bf(rng.standard_normal((N, d)))
    wb, w = bf(rng.standard_normal((d, d)) / np.sqrt(d))
    r = O.sagesla_head(qb, kb, vb, wb, 0.34, quant=False)
    f = G.sla_forward(q, k, v, w, r["idx"], 64)
    assert np.allclose(f["out"], r["out"][:N], rtol=1e-9, atol=1e-11)
    assert np.allclose(f["out_s"], r["out_s"][:N], rtol=1e-9, atol=1e-11)
    assert np.allclose(f["out_l"], r["out_l"][:N], rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("N,d,seed,ksel,blk", CASES)
def test_invariants(N, d, seed, ksel, blk):
    q, k, v, w, dout, idx = make(N, d, seed, ksel, blk)
    g = G.sla_backward(q, k, v, w, idx, dout, blk)
    # each query row's probabilities sum to one: the value gradients of the sparse part sum
    # (over tokens) to the column sums of dout
    assert np.allclose(g["dv_s"].sum(axis=0), dout.sum(axis=0), rtol=1e-10, atol=1e-10)
    # softmax over a row is shift-invariant: sum_j dS_ij = 0, so the key gradients sum to zero
    assert np.allclose(g["dk_s"].sum(axis=0), 0.0, atol=1e-10)
    # the channel softmax phi is shift-invariant per token: the linear part's q and k
    # gradients sum to zero over the channels of each token
    assert np.allclose(g["dq_l"].sum(axis=1), 0.0, atol=1e-12)
    assert np.allclose(g["dk_l"].sum(axis=1), 0.0, atol=1e-12)
    # the linear part is linear in W, so dL/dW . W = sum(dout * O_l W)
    assert np.isclose((g["dw"] * w).sum(), (dout * (g["out_l"] @ w)).sum(), rtol=1e-10)


def test_linear_off_when_all_blocks_kept():
    N, d, blk = 150, 16, 64
    q, k, v, w, dout, _ = make(N, d, 10, 1, blk)
    idx = np.tile(np.arange(3, dtype=np.int32), (3, 1))
    g = G.sla_backward(q, k, v, w, idx, dout, blk)
    assert not g["dq_l"].any() and not g["dk_l"].any() and not g["dv_l"].any() and not g["dw"].any()


@pytest.mark.parametrize("linear", [False, True])
def test_rows_match_whole_backward(linear):
    """The row-sampled gradients equal the whole backward's rows (same formulas, taken a
    block at a time)."""
    N, d, blk = 300, 16, 32
    q, k, v, w, dout, idx = make(N, d, 11, 3, blk, linear=linear)
    g = G.sla_backward(q, k, v, w, idx, dout, blk)
    qb, kb = [0, 4, 9], [1, 5, 9]
    r = G.sla_backward_rows(q, k, v, w, idx, dout, qb, kb, blk)
    for i in qb:
        assert np.allclose(r["dq"][i], g["dq"][i * blk:min(N, (i + 1) * blk)], rtol=1e-10, atol=1e-12)
    for j in kb:
        assert np.allclose(r["dk"][j], g["dk"][j * blk:min(N, (j + 1) * blk)], rtol=1e-10, atol=1e-12)
        assert np.allclose(r["dv"][j], g["dv"][j * blk:min(N, (j + 1) * blk)], rtol=1e-10, atol=1e-12)
