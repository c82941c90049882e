"""Pins for the oracle's smoothing and quantization stages.

SageAttention maps values to 8-bit integers (TurboDiffusion explainer, news.qq.com,
section "First key: attention"); each small block shares one scale factor and outliers
are smoothed into range first (same page, section "Third key"). The pins are the exact
error bounds of symmetric rounding, exactness of the integer dot product, and the
shift invariance that K-mean smoothing must have.
"""
import numpy as np
import torch

import oracle as O


def _bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_int8_block_quant_bounds():
    rng = np.random.default_rng(0)
    N, d = 64 * 5 + 9, 128
    x = (rng.normal(size=(N, d)) * rng.uniform(0.01, 30, size=(N, 1))).astype(np.float32)
    x[64:128] = 0.0  # an all-zero block
    q8, s = O.quant_blocks(x, 64)
    assert q8.shape == (6 * 64, d) and s.shape == (6,)
    assert np.all(q8[N:] == 0)  # padded rows
    assert s[1] == 0 and np.all(q8[64:128] == 0)
    for i in range(6):
        blk = x[i * 64:min(N, (i + 1) * 64)]
        codes = q8[i * 64:i * 64 + len(blk)].astype(np.float64)
        amax = np.abs(blk).max()
        if amax == 0:
            continue
        assert s[i] == np.float32(amax / np.float32(127.0))
        assert np.abs(codes).max() == 127
        err = np.abs(blk - s[i] * codes)
        assert np.all(err <= s[i] * 0.5 * (1 + 1e-5))


def test_int8_round_half_even():
    # amax = 127 -> inv = 1, so codes are rne(x) exactly
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49]], np.float32)
    x = np.repeat(x, 2, axis=0)
    x = np.pad(x, ((0, 0), (0, 120)))
    q8, s = O.quant_blocks(x, 64)
    assert s[0] == 1.0
    assert list(q8[0, :8]) == [127, 0, 2, 2, 0, -2, -2, 3]


def test_dot_i8_exact():
    rng = np.random.default_rng(1)
    for _ in range(50):
        a = rng.integers(-127, 128, 128).astype(np.int8)
        b = rng.integers(-127, 128, 128).astype(np.int8)
        assert O.dot_i8(a, b) == int(a.astype(np.int64) @ b.astype(np.int64))
    ext = np.full(128, -127, np.int8)
    assert O.dot_i8(ext, ext) == 127 * 127 * 128


def test_v_fp8_bounds():
    rng = np.random.default_rng(2)
    N, d = 333, 128
    v = (rng.normal(size=(N, d)) * rng.uniform(0.001, 50, size=(1, d))).astype(np.float32)
    vb = _bits(v)
    vv = O.bf16_to_f64(vb)
    v8, sv = O.quant_v(vb)
    dec = O.e4m3_decode(v8)
    amax = np.abs(vv).max(0)
    assert np.array_equal(sv, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32))
    # the largest element of each channel lands on +-448
    arg = np.abs(vv).argmax(0)
    assert np.all(np.abs(dec[arg, np.arange(d)]) == 448.0)
    recon = dec * sv[None, :].astype(np.float64)
    err = np.abs(vv - recon)
    normal = np.abs(dec) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(vv[normal]) * (1 + 1e-5) + 1e-30)
    sub = ~normal
    assert np.all(err[sub] <= (sv[None, :] * 2.0 ** -10 * (1 + 1e-5)).repeat(N, 0)[sub])


def test_k_mean_shift_invariance():
    """K + c (c per channel, exact in bf16) moves the mean by exactly c."""
    rng = np.random.default_rng(3)
    N, d = 1000, 128
    k = np.clip(np.round(rng.normal(size=(N, d)) * 16) / 16, -4, 4).astype(np.float32)
    mu = O.k_mean(_bits(k))
    c = np.where(np.arange(d) % 2 == 0, 8.0, -4.0).astype(np.float32)
    mu2 = O.k_mean(_bits(k + c))
    assert np.allclose(mu2 - c, mu, rtol=0, atol=2e-6)
    # and matches the library mean of the same values
    assert np.array_equal(mu, np.mean(k.astype(np.float64), axis=0).astype(np.float32))


def test_quantize_head_smoothing_removes_offset():
    """After smoothing, a large per-channel K offset no longer sets the INT8 scale."""
    rng = np.random.default_rng(4)
    N, d = 640, 128
    k = rng.normal(size=(N, d)).astype(np.float32)
    off = (rng.normal(size=d) * 2).astype(np.float32)
    q = rng.normal(size=(N, d)).astype(np.float32)
    v = rng.normal(size=(N, d)).astype(np.float32)
    a = O.quantize_head(_bits(q), _bits(k), _bits(v))
    b = O.quantize_head(_bits(q), _bits(k + off), _bits(v))
    # scales of the offset K equal those of the plain K up to bf16 rounding of k+off
    assert np.allclose(a["sk"], b["sk"], rtol=0.08)
    assert np.mean(np.abs(a["k8"].astype(int) - b["k8"].astype(int)) <= 1) > 0.99
    # without smoothing the offset would dominate amax and crush the code spread
    assert np.std(b["k8"].astype(float)) > 0.9 * np.std(a["k8"].astype(float))
