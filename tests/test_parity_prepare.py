"""GPU parity of the producer-side fusion (sagesla_prepare): RMSNorm of q and k from the QKV
projection output, the attention layout, and the pool stage in the same pass.

Bars: q, k, v bit-exact against oracle/prepare.py (both sides take every rounding in the
same precision: fp64 mean square, fp32 scale and products, bf16 round-to-nearest-even);
pooled means, K block sums, V block maxima, Q codes and scales bit-exact against the
attention oracle applied to the oracle's normalized tensors; and the forward run from the
prepared workspace (sagesla_fwd_prepared) gives the bits sagesla_fwd gives on those tensors.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import prepare as OP
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import decode_qk_codes

pytestmark = pytest.mark.gpu

CASES = {"ragged": (1, 3, 200, 0.3, 71), "two-batches": (2, 2, 64, 0.5, 72), "wide": (1, 8, 1000, 0.1, 73),
         # the Wan2.1-14B 720p attention (pool outputs checked on the first and last head)
         "wan14b-720p": (1, 40, 75600, 0.1, 74)}


@pytest.mark.parametrize("name", list(CASES))
def test_prepare_parity(name):
    B, H, N, topk, seed = CASES[name]
    d, eps = 128, 1e-6
    print("\n[case] prepare %s: B=%d H=%d N=%d" % (name, B, H, N), flush=True)
    inp = synth.make_projection_inputs(B, N, H, d, seed, device="cuda")
    proj = torch.randn((d, d), generator=torch.Generator(device="cuda").manual_seed(seed), device="cuda") / d ** 0.5
    proj = proj.to(torch.bfloat16)
    q, k, v, ws = S.prepare(inp["qkv"], inp["gq"], inp["gk"], H, eps=eps, topk=topk)
    out = S.fwd_prepared(q, k, v, ws, proj=proj, topk=topk)
    torch.cuda.synchronize()
    views = S.workspace_views(ws, B, H, N, topk=topk)
    g = {n: t.cpu().numpy() for n, t in views.items() if n in ("qbar", "kbart", "ksum", "vamax_blk", "q8", "sq")}
    ref = S.fwd(q, k, v, proj, topk=topk)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    qkv = synth.bf16_bits(inp["qkv"])
    gq, gk = synth.bf16_bits(inp["gq"]), synth.bf16_bits(inp["gk"])
    qg, kg, vg = (synth.bf16_bits(t) for t in (q, k, v))
    for b in range(B):
        oq, ok, ov = OP.prepare(qkv[b], gq, gk, H, d, eps)
        assert np.array_equal(qg[b], oq) and np.array_equal(kg[b], ok) and np.array_equal(vg[b], ov)
        for h in ((0, H - 1) if H > 8 else range(H)):
            bh = b * H + h
            qbar, kbar = O.pool(oq[h]), O.pool(ok[h])
            assert np.array_equal(g["qbar"][bh], qbar)
            assert np.array_equal(g["kbart"][bh].T, kbar)
            qz = O.quantize_head(oq[h], ok[h], ov[h])
            assert np.array_equal(g["sq"][bh], qz["sq"])
            assert np.array_equal(decode_qk_codes(g["q8"][bh]), qz["q8"])
            vabs = np.abs(O.bf16_to_f64(ov[h]))
            vmax = np.stack([vabs[64 * j:64 * j + 64].max(axis=0) for j in range(O.num_blocks(N))])
            assert np.array_equal(g["vamax_blk"][bh].astype(np.float64), vmax)
            ksum = np.stack([O.bf16_to_f64(ok[h])[64 * j:64 * j + 64].sum(axis=0) for j in range(O.num_blocks(N))])
            assert np.allclose(g["ksum"][bh], ksum, rtol=1e-15, atol=0)
