"""GPU parity of the SLA training path at the headline size (Wan2.1-14B 720p attention:
B=1, H=40, N=75,600, topk 0.1, linear branch on), in the launch configuration bench.py
times, on sampled rows: the whole forward and backward run on the GPU; the oracle
(oracle/sla_grad.py, sla_backward_rows) computes dQ on three query blocks and dK, dV on three
key blocks (first, middle, the ragged last) of the first and the last head, from the
oracle's own selection. Bars as in test_parity_sla_train.py."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import sla_grad as G
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import cos

pytestmark = pytest.mark.gpu


def test_sla_train_full_size_sampled():
    cfg = synth.CONFIGS["wan14b-720p"]
    print("\n[case] sla-train full: H=%d N=%d topk=%g" % (cfg.H, cfg.N, cfg.topk), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    q, k, v, proj = x["q"], x["k"], x["v"], x["proj"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 77)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    out, ws = S.sla_fwd(q, k, v, proj, topk=cfg.topk)
    idx_gpu = S.sla_workspace_views(ws, cfg.B, cfg.H, cfg.N, topk=cfg.topk, linear=True)["idx"].cpu().numpy()
    dq, dk, dv, _ = S.sla_bwd(q, k, v, dout, ws, proj=proj, topk=cfg.topk)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    N, Nb = cfg.N, O.num_blocks(cfg.N)
    ks = S.ksel(N, cfg.topk)
    qbl, kbl = [0, Nb // 2, Nb - 1], [0, Nb // 2 + 7, Nb - 1]
    w = O.bf16_to_f64(synth.bf16_bits(proj))
    for h in (0, cfg.H - 1):
        qb, kb, vb, db = (synth.bf16_bits(t[0, h]) for t in (q, k, v, dout))
        idx = O.select(O.scores(O.pool(qb), O.pool(kb)), ks)
        assert all(set(idx_gpu[h][r].tolist()) == set(idx[r].tolist()) for r in range(Nb)), "kept sets differ"
        ref = G.sla_backward_rows(O.bf16_to_f64(qb), O.bf16_to_f64(kb), O.bf16_to_f64(vb), w, idx,
                                  O.bf16_to_f64(db), qbl, kbl)
        for what, got, blocks in (("dQ", dq, qbl), ("dK", dk, kbl), ("dV", dv, kbl)):
            want = np.concatenate([ref[what.lower()][b] for b in blocks])
            g = np.concatenate([got[0, h, 64 * b:min(N, 64 * b + 64)].cpu().numpy().astype(np.float64)
                                for b in blocks])
            c, e, m = cos(g, want), float(np.abs(g - want).max()), float(np.abs(want).max())
            print("  head %d %s: cos %.7f maxabs %.3g (max|g| %.3g)" % (h, what, c, e, m), flush=True)
            assert c >= 0.999 and e <= 2e-2 * m, (what, c, e, m)


def test_sla_train_max_length():
    """The longest sequence the library accepts (2^20 tokens, 16384 key blocks: the
    transposed kept rows of the dK/dV kernel are 512 words, its staging limit), one head,
    linear branch off. dQ on three query blocks against the oracle; over all tokens the
    value gradients sum to the column sums of dO (each probability row sums to one), within
    the bf16 rounding of the probabilities."""
    cfg = synth.scaled(synth.CONFIGS["wan14b-720p"], H=1, grid=(16, 256, 256), seed=43, name="max-length")
    print("\n[case] sla-train max length: H=%d N=%d topk=%g" % (cfg.H, cfg.N, cfg.topk), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 77)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    out, ws = S.sla_fwd(q, k, v, None, topk=cfg.topk)
    idx_gpu = S.sla_workspace_views(ws, cfg.B, cfg.H, cfg.N, topk=cfg.topk, linear=False)["idx"][0].cpu().numpy()
    dq, dk, dv = S.sla_bwd(q, k, v, dout, ws, topk=cfg.topk)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    N, Nb = cfg.N, O.num_blocks(cfg.N)
    assert Nb == 16384
    ks = S.ksel(N, cfg.topk)
    qb, kb, vb, db = (synth.bf16_bits(t[0, 0]) for t in (q, k, v, dout))
    qbl = [0, Nb // 2 + 3, Nb - 1]
    # the oracle's selection for the sampled query blocks only (the rows the backward reads)
    idx = np.zeros((Nb, ks), dtype=np.int32)
    idx[qbl] = O.select(O.scores(O.pool(qb)[qbl], O.pool(kb)), ks)
    assert all(set(idx_gpu[r].tolist()) == set(idx[r].tolist()) for r in qbl), "kept sets differ"
    do64 = O.bf16_to_f64(db)
    sdv = dv[0, 0].double().sum(dim=0).cpu().numpy()
    # the probabilities enter the product rounded to bf16 (2^-9 relative), with errors of
    # independent signs from row to row: six standard deviations of their sum
    bound = 6 * 2.0 ** -9 * np.sqrt((do64 ** 2).sum(axis=0)) + 1e-3
    err = np.abs(sdv - do64.sum(axis=0))
    print("  sum dV - sum dO: max %.3g (bound %.3g)" % (err.max(), bound.min()), flush=True)
    assert np.all(err <= bound)
    ref = G.sla_backward_rows(O.bf16_to_f64(qb), O.bf16_to_f64(kb), O.bf16_to_f64(vb), None, idx, do64, qbl, [])
    want = np.concatenate([ref["dq"][b] for b in qbl])
    g = np.concatenate([dq[0, 0, 64 * b:min(N, 64 * b + 64)].cpu().numpy().astype(np.float64) for b in qbl])
    c, e, m = cos(g, want), float(np.abs(g - want).max()), float(np.abs(want).max())
    print("  dQ: cos %.7f maxabs %.3g (max|g| %.3g)" % (c, e, m), flush=True)
    assert c >= 0.999 and e <= 2e-2 * m, ("dQ", c, e, m)
