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
