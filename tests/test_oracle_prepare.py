"""Pins for the producer-side oracle (oracle/prepare.py): facts of RMSNorm that do not come
from its code. CPU only."""
import numpy as np

from oracle import prepare as P


def bf16(x):
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_constant_rows_normalize_to_unit_magnitude():
    # a row of one repeated value c has rms |c|: every output is sign(c) (eps negligible)
    D = 256
    for c in (3.0, -0.015625, 96.0):
        x = bf16(np.full((1, D), c))
        out = P.rmsnorm(x, bf16(np.ones(D)), 1e-12)
        assert np.all(val(out) == np.sign(c))


def test_power_of_two_scaling_is_invisible():
    # scaling a row by 2^k scales r by 2^-k exactly (fp64 sqrt of a 4^k multiple, eps = 0)
    rng = np.random.default_rng(1)
    D = 512
    x = bf16(rng.standard_normal((4, D)))
    g = bf16(1 + 0.1 * rng.standard_normal(D))
    a = P.rmsnorm(x, g, 0.0)
    for k in (-3, 2, 5):
        xs = bf16(val(x) * 2.0 ** k)
        assert np.array_equal(P.rmsnorm(xs, g, 0.0), a)


def test_unit_mean_square_and_weight():
    rng = np.random.default_rng(2)
    D = 1024
    x = bf16(rng.standard_normal((8, D)) * np.exp(rng.standard_normal((8, 1))))
    ones = bf16(np.ones(D))
    n = val(P.rmsnorm(x, ones, 1e-6))
    # mean square 1 up to the bf16 roundings (2^-9 relative per element)
    ms = (n * n).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 4e-3)
    # the weight multiplies after the first rounding: g = 2 doubles the output exactly
    twos = bf16(np.full(D, 2.0))
    assert np.array_equal(val(P.rmsnorm(x, twos, 1e-6)), 2 * n)


def test_eps_dominates_tiny_rows():
    # ss / D << eps: r -> 1 / sqrt(eps), the output is x / sqrt(eps)
    D = 128
    x = bf16(np.full((1, D), 2.0 ** -20))
    out = P.rmsnorm(x, bf16(np.ones(D)), 1.0)
    assert np.allclose(val(out), 2.0 ** -20, rtol=2 ** -8)


def test_prepare_layout_and_copy():
    rng = np.random.default_rng(3)
    N, H, d = 5, 3, 4
    qkv = bf16(rng.standard_normal((N, 3 * H * d)))
    g = bf16(np.ones(H * d))
    q, k, v = P.prepare(qkv, g, g, H, d, 1e-6)
    assert q.shape == (H, N, d) and v.shape == (H, N, d)
    for h in range(H):
        assert np.array_equal(v[h], qkv[:, 2 * H * d + h * d:2 * H * d + (h + 1) * d])
        assert np.array_equal(q[h], P.rmsnorm(qkv[:, :H * d], g, 1e-6)[:, h * d:(h + 1) * d])
