"""GPU stage parity at sizes the oracle finishes in seconds: every intermediate the
library leaves in its workspace is compared with the oracle's stage of the same name.

Bars: pooled means, K mean, V max, INT8/FP8 codes and their scales bit-exact (the sums
are exact in fp64 for these inputs, and both sides take every rounding decision in
fp32 with the same expressions); kept sets equal except near-ties (pooled-score gap
< 1e-5); linear states within 1e-5 relative; the sparse part O_s and the projected
linear part y = O_l W within cos >= 0.9995 and max-abs <= 2e-2 per head, and the
output within the same bars.
"""
import ctypes as C
import numpy as np
import pytest
import torch

import oracle as O
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import cos, decode_qk_codes, decode_v_codes, mask_mismatch

pytestmark = pytest.mark.gpu

CASES = {
    # name: (config, overrides)
    "tiny": (synth.CONFIGS["tiny"], {}),
    "ragged-field": (synth.CONFIGS["wan1.3b-480p"], dict(H=3, grid=(3, 10, 21), topk=0.3, seed=21)),
    "tiles-ragged": (synth.CONFIGS["wan14b-720p"], dict(H=2, grid=(4, 20, 33), seed=22)),
    "longrange": (synth.CONFIGS["i2v-a14b-720p"], dict(H=2, grid=(3, 24, 40), seed=23)),
    "one-block": (synth.CONFIGS["tiny"], dict(H=2, grid=(1, 1, 37), seed=24)),
    "ksel-1": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 16, 40), topk=1e-6, seed=25)),
    # more query blocks than one complement group holds (300 blocks: groups of 256 + 44)
    "two-groups": (synth.CONFIGS["wan1.3b-480p"], dict(H=1, grid=(3, 10, 640), seed=26)),
    # edge cases: one token; exactly one full block; a complement of a single block
    # (ksel = Nb - 1); the linear branch off with sparse selection (no projection)
    "single-token": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 1, 1), seed=28)),
    "exact-block": (synth.CONFIGS["tiny"], dict(H=1, grid=(1, 1, 64), seed=29)),
    "one-block-linear": (synth.CONFIGS["wan1.3b-480p"], dict(H=1, grid=(1, 4, 80), topk=0.8, seed=30)),
    "linear-off": (synth.CONFIGS["wan1.3b-480p"], dict(H=2, grid=(2, 8, 40), topk=0.2, seed=31, linear=False)),
}


def _run(name):
    cfg, ov = CASES[name]
    cfg = synth.scaled(cfg, name=name, **ov) if ov else cfg
    print("\n[case] %s: H=%d N=%d topk=%g seed=%d" % (name, cfg.H, cfg.N, cfg.topk, cfg.seed), flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    ws = S.alloc_workspace(x["q"], cfg.topk, x["proj"] is not None)
    ws.fill_(0xFF)  # poison: every region the call reads must have been written by it
    out = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=cfg.topk, workspace=ws)
    torch.cuda.synchronize()
    views = S.workspace_views(ws, cfg.B, cfg.H, cfg.N, topk=cfg.topk, linear=x["proj"] is not None)
    host = {k: (v.float() if v.dtype == torch.bfloat16 else v).cpu().numpy() for k, v in views.items()}
    bits = {n: synth.bf16_bits(x[n]) for n in ("q", "k", "v")}
    wbits = synth.bf16_bits(x["proj"]) if x["proj"] is not None else None
    return cfg, x, ws, out, host, bits, wbits


@pytest.mark.parametrize("name", list(CASES))
def test_stage_parity(name):
    cfg, x, ws, out, g, bits, wbits = _run(name)
    N, Nb = cfg.N, O.num_blocks(cfg.N)
    ksel = O.ksel(cfg.topk, Nb)
    linear = wbits is not None and ksel < Nb
    out_h = out.float().cpu().numpy()
    for bh in range(cfg.B * cfg.H):
        b, h = divmod(bh, cfg.H)
        q, k, v = bits["q"][b, h], bits["k"][b, h], bits["v"][b, h]
        # pooling
        qbar, kbar = O.pool(q), O.pool(k)
        assert np.array_equal(g["qbar"][bh], qbar)
        assert np.array_equal(g["kbart"][bh].T, kbar)
        # K mean and V max
        qz = O.quantize_head(q, k, v)
        assert np.array_equal(g["kmean"][bh], qz["kmean"])
        assert np.array_equal(g["vamax"][bh] / np.float32(448.0), qz["sv"])
        # codes and scales
        assert np.array_equal(g["sq"][bh], qz["sq"])
        assert np.array_equal(decode_qk_codes(g["q8"][bh]), qz["q8"])
        assert np.array_equal(g["sk"][bh], qz["sk"])
        assert np.array_equal(decode_qk_codes(g["k8"][bh]), qz["k8"])
        v8 = decode_v_codes(g["v8"][bh])
        assert np.array_equal(v8[:N], qz["v8"]) and np.all(v8[N:] == 0)
        # selection
        sc = O.scores(qbar, kbar)
        ora_idx = np.stack([O.order_best_first(sc[i], row) for i, row in enumerate(O.select(sc, ksel))])
        flips = mask_mismatch(g["idx"][bh], ora_idx, sc)
        assert len(flips) <= max(1, Nb // 50)
        # processing order: best block first (up to near-ties), then strictly ascending
        for i in range(Nb):
            gi = g["idx"][bh][i]
            assert np.all(np.diff(gi[1:]) > 0)
            if i not in flips and gi[0] != ora_idx[i][0]:
                assert abs(sc[i][gi[0]] - sc[i][ora_idx[i][0]]) < 1e-5
        if linear:
            H, z = O.linear_states(k, v)
            # S_j = [H_j^T ; z_j] in bf16: each element within half a bf16 ulp (+ fp32 slack)
            St = np.concatenate([H.transpose(0, 2, 1), z[:, None, :]], axis=1)
            hs = g["hs"][bh]
            assert np.all(np.abs(hs - St) <= 2.0 ** -8 * np.abs(St) + 1e-6 * np.max(np.abs(St)))
            tot = St.sum(0)
            assert np.max(np.abs(g["htot"][bh] - tot)) <= 1e-5 * np.max(np.abs(tot))
            # union of each group's kept sets, with the per-query-block masks
            gidx = g["idx"][bh]
            # (the blocks NOT kept when more than half are kept)
            G = S.GROUP
            comp = 2 * ksel > Nb
            member = [(set(range(Nb)) - set(gidx[i].tolist())) if comp else set(gidx[i].tolist())
                      for i in range(Nb)]
            for grp in range((Nb + G - 1) // G):
                rows = range(G * grp, min(Nb, G * grp + G))
                want = sorted(set().union(*(member[i] for i in rows)))
                cnt = int(g["ucount"][bh][grp])
                assert cnt == len(want) and list(g["ulist"][bh][grp][:cnt]) == want
                um = g["umask"][bh][grp].view(np.uint32).T  # [G][ceil(Nb/32)]: bit p of row qb
                for qi, i in enumerate(rows):
                    got = [p for p in range(32 * um.shape[1]) if (um[qi][p // 32] >> (p % 32)) & 1]
                    assert got == [p for p, j in enumerate(want) if j in member[i]]
                assert not um[len(rows):].any()
            # complement states: total minus the kept blocks (with the GPU's kept sets)
            for i in range(Nb):
                keep = np.zeros(Nb, bool)
                keep[gidx[i]] = True
                want_c = St[~keep].sum(0)
                err = np.max(np.abs(g["hc"][bh][i] - want_c))
                assert err <= 4e-3 * np.max(np.abs(want_c)), (i, err)
        # outputs against the oracle run on the same inputs (its own mask)
        r = O.sagesla_head(q, k, v, wbits, cfg.topk, quant=True)
        ok_rows = np.ones(N, bool)
        for i in flips:
            ok_rows[i * 64:(i + 1) * 64] = False
        want = r["out"][:N][ok_rows]
        got = out_h[b, h][ok_rows]
        assert cos(got, want) >= 0.9995, (bh, cos(got, want))
        assert np.max(np.abs(got - want)) <= 2e-2
        if linear:
            W = O.bf16_to_f64(wbits)
            y_want = (r["out_l"][:N] @ W)[ok_rows]
            y_got = g["y"][bh][ok_rows].astype(np.float64)
            assert cos(y_got, y_want) >= 0.9995, (bh, cos(y_got, y_want))
            assert np.max(np.abs(y_got - y_want)) <= 2e-2
    # O_s alone: rerun the sparse stage without the linear part on the same workspace
    if linear:
        os_ = torch.empty_like(out)
        st = S.lib().sagesla_sparse_attn(
            *(ws.data_ptr() + S.workspace_layout(cfg.B, cfg.H, N, topk=cfg.topk, linear=True)[n]
              for n in ("q8", "sq", "k8", "sk", "v8", "vamax", "idx")),
            None, cfg.B, cfg.H, N, 128, 64, cfg.topk, os_.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        os_h = os_.float().cpu().numpy()
        for bh in range(cfg.B * cfg.H):
            b, h = divmod(bh, cfg.H)
            r = O.sagesla_head(bits["q"][b, h], bits["k"][b, h], bits["v"][b, h], wbits, cfg.topk)
            c = cos(os_h[b, h], r["out_s"][:N])
            assert c >= 0.9995, c


@pytest.mark.parametrize("name", ["tiny", "tiles-ragged"])
def test_deterministic_and_finite(name):
    cfg, x, ws, out, g, bits, wbits = _run(name)
    out2 = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=cfg.topk)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out, out2)


def test_dense_topk_one_matches_oracle():
    cfg = synth.scaled(synth.CONFIGS["i2v-a14b-720p"], H=2, grid=(2, 12, 20), seed=26, topk=1.0)
    print("\n[case] dense topk=1 N=%d" % cfg.N, flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    out = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=1.0)  # proj given, branch empty
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    bits = {n: synth.bf16_bits(x[n]) for n in ("q", "k", "v")}
    for h in range(cfg.H):
        r = O.sagesla_head(bits["q"][0, h], bits["k"][0, h], bits["v"][0, h], None, 1.0)
        assert cos(o[0, h], r["out"][:cfg.N]) >= 0.9995
        assert np.max(np.abs(o[0, h] - r["out"][:cfg.N])) <= 2e-2


def test_batch_of_two():
    from dataclasses import replace
    cfg = replace(synth.scaled(synth.CONFIGS["wan1.3b-480p"], H=2, grid=(2, 10, 19), seed=27, topk=0.25),
                  B=2)
    print("\n[case] B=2 N=%d" % cfg.N, flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    out = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=cfg.topk)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    bits = {n: synth.bf16_bits(x[n]) for n in ("q", "k", "v")}
    w = synth.bf16_bits(x["proj"])
    for b in range(2):
        for h in range(2):
            r = O.sagesla_head(bits["q"][b, h], bits["k"][b, h], bits["v"][b, h], w, cfg.topk)
            assert cos(o[b, h], r["out"][:cfg.N]) >= 0.9995


@pytest.mark.parametrize("grid", [(1, 1, 37), (4, 20, 33)])
def test_small_scores_partial_block(grid):
    """Q and K scaled by 2^-10: the logit scale a = s_q s_k / sqrt(d) log2(e) falls near
    1e-10, where a masked key's INT_MIN score no longer underflows the exponent on its own.
    The keys past N in the partial last block must still take no part. (A power-of-two
    factor leaves the pooled means, the scores' order and the INT8 codes unchanged.)"""
    cfg = synth.scaled(synth.CONFIGS["wan14b-720p"], H=2, grid=grid, seed=32)
    print("\n[case] small scores N=%d" % cfg.N, flush=True)
    x = synth.make_inputs(cfg, device="cuda")
    for n in ("q", "k"):
        x[n] = x[n] * 2.0 ** -10
    out = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=cfg.topk)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    bits = {n: synth.bf16_bits(x[n]) for n in ("q", "k", "v")}
    w = synth.bf16_bits(x["proj"])
    for h in range(cfg.H):
        r = O.sagesla_head(bits["q"][0, h], bits["k"][0, h], bits["v"][0, h], w, cfg.topk, quant=True)
        assert cos(o[0, h], r["out"][:cfg.N]) >= 0.9995
        assert np.max(np.abs(o[0, h] - r["out"][:cfg.N])) <= 2e-2


def _planted_tie_inputs(nq=16, nk=16, v0=4.0):
    """Scores near 180 whose planted gaps (about 1.2e-5, just over the 1e-5 near-tie
    bound) are narrower than one fp32 step there (1.5e-5): every query token is
    (w_i, v0 + e_i, v0, ..., v0) and every key token (1, v0, ..., v0), except that channel 0
    of the first tokens of key block j adds 18 j bf16 steps of 2^-7, so the pooled
    channel-0 mean grows by 18 j 2^-7 / 64 and s_ij by w_i times that over sqrt(128).
    Query blocks differ in w_i and e_i, which moves where the fp32 roundings fall."""
    N = 64 * max(nq, nk)
    q = np.full((N, 128), v0, np.float32)
    k = np.full((N, 128), v0, np.float32)
    k[:, 0] = 1.0
    for i in range(nq):
        q[64 * i:64 * (i + 1), 0] = 0.0625 + (i % 4) * 2.0 ** -10
        q[64 * i:64 * (i + 1), 1] = v0 + (i // 4) * 2.0 ** -5
    for j in range(nk):
        n, t = 18 * j, 0
        while n > 0:
            a = min(n, 120)
            k[64 * j + t, 0] = 1.0 + a * 2.0 ** -7
            n, t = n - a, t + 1
    v = np.random.default_rng(33).standard_normal((N, 128)).astype(np.float32)
    return q, k, v


def test_select_exact_fp64_near_ties():
    """The selection keys are the fp64 scores themselves: with planted score gaps of about
    1.2e-5 at |s| ~ 180 (fp32 step 1.5e-5 there), the kept sets must equal the oracle's
    exactly, up to the 1e-5 near-tie rule, which these gaps exceed."""
    q, k, v = _planted_tie_inputs()
    N = q.shape[0]
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).reshape(1, 1, N, 128).cuda()
    tq, tk, tv = to(q), to(k), to(v)
    topk = 0.5
    ws = S.alloc_workspace(tq, topk, False)
    S.fwd(tq, tk, tv, None, topk=topk, workspace=ws)
    torch.cuda.synchronize()
    g = S.workspace_views(ws, 1, 1, N, topk=topk, linear=False)["idx"].cpu().numpy()[0]
    qb, kb = O.pool(synth.bf16_bits(tq[0, 0])), O.pool(synth.bf16_bits(tk[0, 0]))
    sc = O.scores(qb, kb)
    Nb, ks = sc.shape[1], O.ksel(topk, sc.shape[1])
    ora = np.stack([O.order_best_first(sc[i], row) for i, row in enumerate(O.select(sc, ks))])
    # the case is hard for fp32 keys: in some row the boundary pair shares an fp32 value
    srt = np.sort(sc, axis=1)[:, ::-1]
    gap = srt[:, ks - 1] - srt[:, ks]
    assert gap.min() > 1e-5 and np.abs(srt[0, 0]) > 128
    assert np.any(np.float32(srt[:, ks - 1]) == np.float32(srt[:, ks]))
    assert mask_mismatch(g, ora, sc) == []
    assert np.array_equal(g, ora)


@pytest.mark.parametrize("Nb", [37, 300, 700, 1500, 2300])
def test_select_stage_every_row_length(Nb):
    """The selection stage alone, on pooled means drawn directly, at row lengths that take
    each of its paths: the keys held in registers (up to 8, 16 or 32 per lane: rows of up
    to 512, 1024 and 2048 blocks) and read from LDS (longer rows). Kept sets and their
    processing order equal the oracle's, up to near-ties."""
    rng = np.random.default_rng(40 + Nb)
    H, d, topk = 2, 128, 0.1
    N = 64 * Nb - 5  # a ragged last block
    qbar = rng.standard_normal((H, Nb, d)) + rng.standard_normal((H, 1, d))
    kbar = rng.standard_normal((H, Nb, d)) * 0.5 + rng.standard_normal((H, 1, d))
    ks = O.ksel(topk, Nb)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tq, tk = dev(qbar), dev(np.transpose(kbar, (0, 2, 1)))  # kbart: [BH][d][Nb]
    idx = torch.full((H, Nb, ks), -7, dtype=torch.int32, device="cuda")
    st = S.lib().sagesla_select(tq.data_ptr(), tk.data_ptr(), 1, H, N, d, 64, topk, idx.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    for h in range(H):
        sc = O.scores(qbar[h], kbar[h])
        ora = np.stack([O.order_best_first(sc[i], row) for i, row in enumerate(O.select(sc, ks))])
        near = set(mask_mismatch(g[h], ora, sc))
        for r in range(Nb):
            if r in near:
                continue
            assert np.array_equal(g[h, r], ora[r]), (h, r)


def test_grouped_stages_and_descriptor_forward_equal_fwd():
    """sagesla_pool_select + sagesla_linear_states (or sagesla_quantize) + the complement
    and sparse stages, and sagesla_fwd_tensors, compute exactly what sagesla_fwd does."""
    from sparse_attention_sagesla_amd import _lib
    cfg = synth.scaled(synth.CONFIGS["wan14b-720p"], H=2, grid=(4, 20, 33), seed=22, name="grouped")
    x = synth.make_inputs(cfg, device="cuda")
    q, k, v, proj = x["q"], x["k"], x["v"], x["proj"]
    B, H, N, topk = cfg.B, cfg.H, cfg.N, cfg.topk
    L = S.lib()
    sp = torch.cuda.current_stream().cuda_stream
    ref_ws = S.alloc_workspace(q, topk, True)
    ref = S.fwd(q, k, v, proj, topk=topk, workspace=ref_ws)
    for use_states in (True, False):
        ws = S.alloc_workspace(q, topk, True)
        ws.fill_(0xFF)
        P = {n: ws.data_ptr() + o for n, o in S.workspace_layout(B, H, N, topk=topk, linear=True).items()}
        out = torch.empty_like(q)
        st = L.sagesla_pool_select(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, 128, 64, topk, P["qbar"],
                                   P["kbart"], P["ksum"], P["vamax_blk"], P["q8"], P["sq"], P["kmean"], P["vamax"],
                                   P["idx"], sp)
        assert st == 0
        if use_states:
            st = L.sagesla_linear_states(k.data_ptr(), v.data_ptr(), P["kmean"], P["vamax"], B, H, N, 128, 64,
                                         P["k8"], P["sk"], P["v8"], P["hs"], P["hpart"], P["htot"], sp)
            assert st == 0
            st = L.sagesla_linear_complement(q.data_ptr(), P["idx"], P["hs"], P["htot"], proj.data_ptr(), B, H, N,
                                             128, 64, topk, P["ulist"], P["umask"], P["ucount"], P["hc"], P["y"], sp)
            assert st == 0
        else:
            st = L.sagesla_quantize(k.data_ptr(), v.data_ptr(), P["kmean"], P["vamax"], B, H, N, 128, 64, P["k8"],
                                    P["sk"], P["v8"], sp)
            assert st == 0
        st = L.sagesla_sparse_attn(P["q8"], P["sq"], P["k8"], P["sk"], P["v8"], P["vamax"], P["idx"],
                                   P["y"] if use_states else None, B, H, N, 128, 64, topk, out.data_ptr(), sp)
        assert st == 0
        torch.cuda.synchronize()
        gv, rv = S.workspace_views(ws, B, H, N, topk=topk), S.workspace_views(ref_ws, B, H, N, topk=topk)
        for name in ("qbar", "kbart", "kmean", "vamax", "q8", "sq", "k8", "sk", "v8", "idx"):
            assert torch.equal(gv[name], rv[name]), name
        if use_states:
            assert torch.equal(out, ref)
        else:
            ref_s = S.fwd(q, k, v, None, topk=topk)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_s)
    # the descriptor forward
    out = torch.empty_like(q)
    ws = S.alloc_workspace(q, topk, True)
    d = _lib.tensor_desc
    st = L.sagesla_fwd_tensors(*(C.byref(d(t)) for t in (q, k, v, proj)), topk, 64, C.byref(d(out)),
                               C.byref(d(ws)), sp)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
