"""GPU parity of the SLA training path (unquantized forward + backward) with the oracle
(oracle/sla_grad.py for the gradients, the C oracle for the selection).

Bars, per head:
 * kept sets equal to the oracle's (the cases avoid near-ties; selection near-ties are
   covered by the stage tests);
 * out and O_s: cos >= 0.9999 and max-abs <= 1e-2 (the probabilities enter the PV product
   rounded to bf16, 2^-9 relative; out is stored in bf16); with the linear branch, out
   within 2e-2 (its states are bf16, as in the inference forward);
 * lse within 1e-4 absolute (fp32 scores from exact bf16 products, fp32 log-sum-exp);
 * dQ, dK, dV, dW: cos >= 0.999 and max-abs <= 2e-2 * max|g_ref|. P and dS enter their
   products rounded to bf16 (2^-9 relative each), as do phi, du and the state gradients
   of the linear part; sums of hundreds of such terms keep the error near 1e-3 of the
   largest gradient entries.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import sla_grad as G
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import cos

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides); linear=True adds the linear branch through W_proj
    "ragged": (synth.CONFIGS["tiny"], dict(H=2, grid=(1, 5, 60), topk=0.4, seed=51, linear=False)),
    "field": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 8, 40), topk=0.2, seed=52, linear=False)),
    "one-block": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 1, 37), topk=0.5, seed=53, linear=False)),
    "dense": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 3, 50), topk=1.0, seed=54, linear=False)),
    "ksel-1": (synth.CONFIGS["wan1.3b-480p"], dict(H=1, grid=(2, 10, 40), topk=1e-6, seed=55, linear=False)),
    "lin-ragged": (synth.CONFIGS["tiny"], dict(H=2, grid=(1, 5, 60), topk=0.4, seed=56, linear=True)),
    "lin-field": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 8, 40), topk=0.2, seed=57, linear=True)),
    # more than half the blocks kept: the key blocks' state gradients are summed directly
    "lin-most-kept": (synth.CONFIGS["wan1.3b-480p"], dict(H=1, grid=(2, 8, 40), topk=0.7, seed=58, linear=True)),
    # more key blocks than one complement group holds (300 blocks: groups of 256 + 44)
    "lin-two-groups": (synth.CONFIGS["wan1.3b-480p"], dict(H=1, grid=(3, 10, 640), topk=0.1, seed=59, linear=True)),
    # every block kept: no linear part, dW = 0
    "lin-dense": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 3, 50), topk=1.0, seed=60, linear=True)),
    # two sequences in the batch (dW sums over both)
    "lin-batch2": (synth.CONFIGS["wan1.3b-480p"], dict(B=2, H=2, grid=(1, 5, 60), topk=0.3, seed=61, linear=True)),
}


def _bf16(t):
    return synth.bf16_bits(t)


def _f64(bits):
    return O.bf16_to_f64(bits)


def _run(name):
    cfg, ov = CASES[name]
    cfg = synth.scaled(cfg, name=name, **ov)
    print("\n[case] sla-train %s: H=%d N=%d topk=%g" % (name, cfg.H, cfg.N, cfg.topk), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 1000)
    dout = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    proj = x["proj"]
    out, ws = S.sla_fwd(q, k, v, proj, topk=cfg.topk)
    views = {n: t.clone() for n, t in S.sla_workspace_views(ws, cfg.B, cfg.H, cfg.N, topk=cfg.topk,
                                                             linear=proj is not None).items()}
    grads = S.sla_bwd(q, k, v, dout, ws, proj=proj, topk=cfg.topk)
    torch.cuda.synchronize()
    return cfg, q, k, v, proj, dout, out, views, grads


@pytest.mark.parametrize("name", list(CASES))
def test_sla_train_parity(name):
    cfg, q, k, v, proj, dout, out, views, grads = _run(name)
    dq, dk, dv = grads[:3]
    N = cfg.N
    wb = None if proj is None else _bf16(proj)
    dw_ref = 0.0
    for b, h in [(b, h) for b in range(cfg.B) for h in range(cfg.H)]:
        bh = b * cfg.H + h
        qb, kb, vb, db = (_bf16(t[b, h]) for t in (q, k, v, dout))
        ora = O.sagesla_head(qb, kb, vb, wb, cfg.topk, quant=False)
        gi = views["idx"][bh].cpu().numpy()
        assert all(set(gi[r].tolist()) == set(ora["idx"][r].tolist()) for r in range(len(gi))), "kept sets differ"
        ref = G.sla_backward(_f64(qb), _f64(kb), _f64(vb), None if wb is None else _f64(wb), ora["idx"], _f64(db))
        if ref["dw"] is not None:
            dw_ref = dw_ref + ref["dw"]
        o = out[b, h].float().cpu().numpy()
        os_ = views["os"][bh].float().cpu().numpy()
        for got, want, what in ((o, ref["out"], "out"), (os_, ref["out_s"], "O_s")):
            c, e = cos(got, want), float(np.abs(got - want).max())
            print("  seq %d head %d %s: cos %.7f maxabs %.3g" % (b, h, what, c, e))
            # the linear part's states are bf16 (as in the inference forward): 2e-2 there
            assert c >= 0.9999 and e <= (2e-2 if what == "out" and wb is not None else 1e-2), (what, c, e)
        lse = views["lse"][bh].cpu().numpy().astype(np.float64) * np.log(2.0)
        assert np.abs(lse - ref["lse"]).max() <= 1e-4
        for got, want, what in ((dq, ref["dq"], "dQ"), (dk, ref["dk"], "dK"), (dv, ref["dv"], "dV")):
            g = got[b, h].cpu().numpy().astype(np.float64)
            c, e, m = cos(g, want), float(np.abs(g - want).max()), float(np.abs(want).max())
            print("  seq %d head %d %s: cos %.7f maxabs %.3g (max|g| %.3g)" % (b, h, what, c, e, m))
            assert c >= 0.999 and e <= 2e-2 * m, (what, c, e, m)
    assert N == q.shape[2]
    if proj is not None:
        dw = grads[3].cpu().numpy().astype(np.float64)
        if isinstance(dw_ref, float):  # every block kept: no linear part
            assert not dw.any()
        else:
            c, e, m = cos(dw, dw_ref), float(np.abs(dw - dw_ref).max()), float(np.abs(dw_ref).max())
            print("  dW: cos %.7f maxabs %.3g (max|g| %.3g)" % (c, e, m))
            assert c >= 0.999 and e <= 2e-2 * m, ("dW", c, e, m)
