"""GPU parity of the content-adaptive kept-block count (sagesla_adaptive_ksel and
sagesla_fwd_adaptive) against the oracle.

Bars:
- per-row counts equal the oracle's wherever the oracle's margin exceeds 1e-12 (the
  masses are fp64 sums in different orders on the two sides);
- per-head counts equal the oracle's count from its own rows when no row is that close;
- every head's output, kept lists and linear part equal, bit for bit, sagesla_fwd's on
  that head alone at topk = k_head / Nb (the adaptive forward is the fixed-count forward
  at the head's count);
- outputs against the oracle's adaptive head: cosine >= 0.9995 and max-abs <= 2e-2, as
  for the fixed-count forward;
- at the Wan2.1-14B 720p shape: sampled heads' counts against the oracle, and the
  fixed-count identity on two heads.
"""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import cos, mask_mismatch

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides, topk_min, topk_max, tau)
    "ragged-field": (synth.CONFIGS["wan1.3b-480p"], dict(H=3, grid=(3, 10, 21), seed=51), 0.05, 0.5, 0.6),
    "tiles-ragged": (synth.CONFIGS["wan14b-720p"], dict(H=3, grid=(4, 20, 33), seed=52), 0.05, 0.25, 0.9),
    "longrange": (synth.CONFIGS["i2v-a14b-720p"], dict(H=2, grid=(3, 24, 40), seed=53), 0.1, 0.3, 0.5),
    "iid-no-linear": (synth.CONFIGS["tiny"], dict(H=2, seed=54, linear=False), 0.05, 0.8, 0.7),
    # tau = 1 and topk_max = 1: every row needs every block, so every head keeps all of
    # them and its linear part is zero
    "all-kept": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 8, 40), seed=55), 0.1, 1.0, 1.0),
    # a clamp from below: tiny tau
    "clamp-low": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 8, 40), seed=56), 0.2, 0.4, 0.01),
    "single-block": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 1, 37), seed=57), 0.1, 1.0, 0.5),
}


def _cfg(name):
    cfg, ov, tmin, tmax, tau = CASES[name]
    return synth.scaled(cfg, name=name, **ov), tmin, tmax, tau


def _oracle_counts(qb, kb, N, tau, kmin, kmax):
    sc = O.scores(O.pool(qb), O.pool(kb))
    kr, margin = O.adaptive_k(sc, N, tau)
    return kr, margin, O.adaptive_ksel(kr, kmin, kmax), sc


@pytest.mark.parametrize("name", list(CASES))
def test_adaptive_parity(name):
    cfg, tmin, tmax, tau = _cfg(name)
    N, Nb, BH = cfg.N, O.num_blocks(cfg.N), cfg.B * cfg.H
    print("\n[case] %s: H=%d N=%d topk %g..%g tau %g" % (name, cfg.H, N, tmin, tmax, tau), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    linear = x["proj"] is not None
    ws = torch.empty(S.adaptive_workspace_size(cfg.B, cfg.H, N, topk_min=tmin, topk_max=tmax, linear=linear),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # poison
    out, k_rows, k_head = S.fwd_adaptive(x["q"], x["k"], x["v"], x["proj"], topk_min=tmin, topk_max=tmax, tau=tau,
                                         workspace=ws)
    torch.cuda.synchronize()
    views = S.adaptive_workspace_views(ws, cfg.B, cfg.H, N, topk_min=tmin, topk_max=tmax, linear=linear)
    kmin, kmax = O.ksel(tmin, Nb), O.ksel(tmax, Nb)
    kr_g, kh_g = k_rows.cpu().numpy(), k_head.cpu().numpy()
    idx_g = views["idx"].cpu().numpy()
    keys_g = views["keys"].cpu().numpy()
    out_g = out.float().cpu().numpy()
    bits = {n: synth.bf16_bits(x[n]) for n in ("q", "k", "v")}
    wbits = synth.bf16_bits(x["proj"]) if linear else None

    # the stage entry point on the pooled means gives the same counts
    kr2, kh2 = S.adaptive_ksel(views["qbar"], views["kbart"], cfg.B, cfg.H, N, topk_min=tmin, topk_max=tmax, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(kr2, k_rows) and torch.equal(kh2, k_head)

    for bh in range(BH):
        b, h = divmod(bh, cfg.H)
        q, k, v = bits["q"][b, h], bits["k"][b, h], bits["v"][b, h]
        kr_o, margin, kh_o, sc = _oracle_counts(q, k, N, tau, kmin, kmax)
        sure = margin > 1e-12
        assert np.array_equal(kr_g[bh][sure], kr_o[sure]), (bh, np.nonzero(kr_g[bh] != kr_o)[0])
        # the score keys the selection reused decode to the oracle's fp64 scores
        u = keys_g[bh].view(np.uint64)
        top = np.uint64(1 << 63)
        s_g = np.where(u & top, u & ~top, ~u).view(np.float64)
        assert np.allclose(s_g, sc, rtol=1e-12, atol=1e-12)
        if sure.all():
            assert kh_g[bh] == kh_o, (bh, kh_g[bh], kh_o)
        ks = int(kh_g[bh])
        print("  head %d: k_head %d (oracle %d, range %d..%d), mean k_i %.2f" % (bh, ks, kh_o, kmin, kmax,
                                                                              kr_g[bh].mean()), flush=True)
        assert kmin <= ks <= kmax
        assert (idx_g[bh][:, ks:] == -1).all()
        # the fixed-count forward on this head alone, at the head's count
        sl = lambda t: t[b:b + 1, h:h + 1].contiguous()  # noqa: E731
        topk = ks / Nb
        assert O.ksel(topk, Nb) == ks
        wsf = S.alloc_workspace(sl(x["q"]), topk, linear)
        of = S.fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["proj"], topk=topk, workspace=wsf)
        torch.cuda.synchronize()
        vf = S.workspace_views(wsf, 1, 1, N, topk=topk, linear=linear)
        assert np.array_equal(vf["idx"][0].cpu().numpy(), idx_g[bh][:, :ks])
        assert torch.equal(of[0, 0], out[b, h]), bh
        if linear and ks < Nb:
            assert torch.equal(vf["y"][0], views["y"][bh])
        # against the oracle's adaptive head (its own selection at its own count)
        if sure.all():
            r = O.sagesla_head_adaptive(q, k, v, wbits, tmin, tmax, tau, quant=True)
            assert r["ksel"] == ks
            assert (r["idx"][:, ks:] == -1).all()
            # kept sets equal except near-ties of the scores (rows left out below)
            flips = mask_mismatch(idx_g[bh][:, :ks], r["idx"][:, :ks], sc)
            assert len(flips) <= 1, flips
            ok = np.ones(N, bool)
            for i in flips:
                ok[i * 64:(i + 1) * 64] = False
            want = r["out"][:N][ok]
            got = out_g[b, h][ok]
            c, err = cos(got, want), np.max(np.abs(got - want))
            print("  head %d: cos %.6f maxabs %.3g flips %d" % (bh, c, err, len(flips)), flush=True)
            assert c >= 0.9995 and err <= 2e-2
    del ws, out, x


def test_adaptive_rejects_bad_arguments():
    q = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    for tmin, tmax, tau in [(0.0, 0.5, 0.5), (0.6, 0.5, 0.5), (0.1, 1.5, 0.5), (0.1, 0.5, 0.0), (0.1, 0.5, 1.01)]:
        with pytest.raises(S.SageSLAError):
            S.fwd_adaptive(q, q, q, None, topk_min=tmin, topk_max=tmax, tau=tau)


def test_full_size_adaptive_wan14b_720p():
    cfg = synth.CONFIGS["wan14b-720p"]
    tmin, tmax, tau = 0.05, 0.25, 0.9
    N, Nb = cfg.N, O.num_blocks(cfg.N)
    print("\n[case] wan14b-720p adaptive: H=%d N=%d tau %g" % (cfg.H, N, tau), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    out, k_rows, k_head = S.fwd_adaptive(x["q"], x["k"], x["v"], x["proj"], topk_min=tmin, topk_max=tmax, tau=tau)
    torch.cuda.synchronize()
    kr_g, kh_g = k_rows.cpu().numpy(), k_head.cpu().numpy()
    kmin, kmax = O.ksel(tmin, Nb), O.ksel(tmax, Nb)
    print("  k_head: %s" % kh_g.tolist(), flush=True)
    assert ((kh_g >= kmin) & (kh_g <= kmax)).all()
    for h in sorted({0, 17, cfg.H - 1}):
        q, k = synth.bf16_bits(x["q"][0, h]), synth.bf16_bits(x["k"][0, h])
        kr_o, margin, kh_o, _ = _oracle_counts(q, k, N, tau, kmin, kmax)
        sure = margin > 1e-12
        assert np.array_equal(kr_g[h][sure], kr_o[sure]), h
        if sure.all():
            assert kh_g[h] == kh_o
    for h in (0, cfg.H - 1):
        sl = lambda t: t[0:1, h:h + 1].contiguous()  # noqa: E731
        topk = int(kh_g[h]) / Nb
        of = S.fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["proj"], topk=topk)
        torch.cuda.synchronize()
        assert torch.equal(of[0, 0], out[0, h]), h
    del out, x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tau", [0.05, 0.2, 0.5])
def test_adaptive_equal_scores_at_the_boundary(tau):
    # key blocks 0..7 are one block repeated, shifted along a direction shared with every
    # query: they carry the top scores of every row, all exactly equal, so the count
    # crosses tau inside a run of equal scores and those blocks are taken in index order
    rng = np.random.default_rng(61)
    N, d = 64 * 40, 128
    u = rng.normal(0, 1, d)
    u *= 3.0 / np.linalg.norm(u)
    q = rng.normal(0, 1, (N, d)) + u
    k = rng.normal(0, 1, (N, d))
    blk = rng.normal(0, 1, (64, d)) + u
    k[:512] = np.tile(blk, (8, 1))
    v = rng.normal(0, 1, (N, d))
    to = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).reshape(1, 1, N, d).cuda()  # noqa
    tq, tk, tv = to(q), to(k), to(v)
    print("\n[case] equal scores at the boundary: N=%d tau %g" % (N, tau), flush=True)
    out, k_rows, k_head = S.fwd_adaptive(tq, tk, tv, None, topk_min=0.01, topk_max=1.0, tau=tau)
    torch.cuda.synchronize()
    qb, kb, vb = (synth.bf16_bits(t[0, 0]) for t in (tq, tk, tv))
    Nb = O.num_blocks(N)
    kr_o, margin, kh_o, sc = _oracle_counts(qb, kb, N, tau, O.ksel(0.01, Nb), O.ksel(1.0, Nb))
    # the planted ties are exact on both sides
    top = np.argsort(-sc, axis=1, kind="stable")[:, :8]
    assert (np.sort(top, axis=1) == np.arange(8)).all()
    assert (sc[:, :8] == sc[:, :1]).all()
    kr_g = k_rows[0].cpu().numpy()
    sure = margin > 1e-12
    assert sure.mean() > 0.9
    assert np.array_equal(kr_g[sure], kr_o[sure])
    if sure.all():
        assert int(k_head[0]) == kh_o
    # the counts land inside the run of equal scores for the smaller tau
    if tau <= 0.2:
        assert ((kr_o > 1) & (kr_o <= 8)).any()
