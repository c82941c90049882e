"""GPU parity of the W8A8 linear layer with the oracle (oracle/w8a8.py).

Bars: the INT8 codes and fp32 scales of weights and activations bit-exact (both sides take
every rounding decision in fp32 with the same expressions; padding rows zero); y within
2^-8 |y_ref| + 2^-14 max|y_ref| of the oracle's fp64 product of the oracle's own codes.
The GPU sums each 128-channel block's integer product exactly (int32), scales it by one
fp32 product sx*sw (2^-24 relative) and adds it into an fp32 accumulator (2^-24 of the
running sum per block), then rounds y to bf16 (2^-9 relative): the first term covers the
output rounding, the second the accumulation over up to a few hundred blocks.
"""
import numpy as np
import pytest
import torch

import oracle.w8a8 as OW
import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import synth
from _helpers import decode_w8a8_tiles

pytestmark = pytest.mark.gpu


def _bits(t):
    return synth.bf16_bits(t)


def _y_bound(ref):
    return 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * np.abs(ref).max()


CASES = {
    # name: (M, K, N, bias, seed)
    "ragged": (300, 384, 256, True, 41),
    "one-row": (1, 128, 256, False, 42),
    "tiles": (513, 640, 768, True, 43),
    "odd-kb": (1000, 1152, 512, False, 44),
    "exact-tile": (256, 1024, 512, True, 45),
}


@pytest.mark.parametrize("name", list(CASES))
def test_w8a8_parity(name):
    M, K, N, with_bias, seed = CASES[name]
    print("\n[case] w8a8 %s: M=%d K=%d N=%d bias=%s" % (name, M, K, N, with_bias), flush=True)
    inp = synth.make_linear_inputs(M, K, N, seed, device="cuda", bias=with_bias)
    x, w, b = inp["x"], inp["w"], inp["bias"]
    sz = S.w8a8_sizes(M, N, K)
    Mp = sz["sx"] // (4 * (K // 128))
    w8, sw = S.w8a8_quant_weight(w)
    x8, sx = S.w8a8_quant_act(x)
    y = S.w8a8_gemm(x8, sx, w8, sw, M, N, K, bias=b)
    y2 = S.w8a8_linear(x, w8, sw, N, bias=b)
    torch.cuda.synchronize()

    xb, wb = _bits(x), _bits(w)
    qx, sxo = OW.quant_act(xb)
    qw, swo = OW.quant_weight(wb)
    # weights: codes and block scales
    gw = decode_w8a8_tiles(w8.cpu().numpy(), N // 32, K)
    assert np.array_equal(gw, qw)
    assert np.array_equal(sw.cpu().numpy(), swo)
    # activations: codes, scales, zero padding rows
    gx = decode_w8a8_tiles(x8.cpu().numpy(), Mp // 32, K)
    assert np.array_equal(gx[:M], qx)
    assert not gx[M:].any()
    gs = sx.cpu().numpy()
    assert gs.shape == (K // 128, Mp)
    assert np.array_equal(gs[:, :M], sxo.T)
    assert not gs[:, M:].any()
    # the product
    ref = OW.gemm(qx, sxo, qw, swo, None if b is None else _bits(b))
    got = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = _y_bound(ref)
    assert np.all(err <= bound), (err.max(), np.unravel_index(np.argmax(err - bound), err.shape))
    # the whole layer in one call gives the same bits
    assert torch.equal(y, y2)


def test_w8a8_full_size_sampled_rows():
    """A projection of the Wan2.1-14B transformer at 720p (75,600 tokens, 5120 -> 5120),
    checked on rows spread over every row tile class, the last row included."""
    M, K, N = 75600, 5120, 5120
    print("\n[case] w8a8 full: M=%d K=%d N=%d" % (M, K, N), flush=True)
    inp = synth.make_linear_inputs(M, K, N, 46, device="cuda", bias=True)
    x, w, b = inp["x"], inp["w"], inp["bias"]
    w8, sw = S.w8a8_quant_weight(w)
    x8, sx = S.w8a8_quant_act(x)
    y = S.w8a8_gemm(x8, sx, w8, sw, M, N, K, bias=b)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 255, 256, 4097, 37811, 75519, 75520, 75599])
    xr = _bits(x[torch.as_tensor(rows, device="cuda")])
    qx, sxo = OW.quant_act(xr)  # quantization is per row: a row subset quantizes alike
    qw, swo = OW.quant_weight(_bits(w))
    ref = OW.gemm(qx, sxo, qw, swo, _bits(b))
    got = y[torch.as_tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= _y_bound(ref))
    assert np.array_equal(sx[:, torch.as_tensor(rows, device="cuda")].cpu().numpy(), sxo.T)
    assert np.array_equal(sw.cpu().numpy(), swo)
    assert torch.isfinite(y).all()
