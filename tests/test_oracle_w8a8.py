"""Pins for the W8A8 oracle (oracle/w8a8.py) against facts that do not come from it:
exact integer arithmetic on power-of-two block scales, per-element quantization bounds,
the closed-form error bound against the unquantized product, exact scaling, and brute
force integer products. CPU only."""
import numpy as np
import pytest

from oracle import w8a8 as W


def bf16_exact(a):
    """float64 values that bf16 holds exactly -> bf16 bit patterns."""
    f = np.asarray(a, np.float32)
    u = f.view(np.uint32)
    assert np.all(f.astype(np.float64) == np.asarray(a, np.float64)) and np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def bf16_round(a):
    """Round float64 to bf16 (RNE) -> (bits, decoded values)."""
    f = np.asarray(a, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def power_blocks(rng, rows, cols, brows, exps):
    """Integers in [-127, 127] times 2^e per (brows x 128) block, each block holding a
    +-127: its scale is then exactly 2^e and its codes are the integers."""
    ints = rng.integers(-127, 128, size=(rows, cols))
    val = np.empty((rows, cols))
    for a in range(0, rows, brows):
        for b in range(0, cols, 128):
            blk = ints[a:a + brows, b:b + 128]
            blk[0, 0] = 127 if rng.random() < 0.5 else -127
            val[a:a + brows, b:b + 128] = blk * 2.0 ** exps[a // brows, b // 128]
    return ints, val


def test_exact_power_of_two_scales():
    rng = np.random.default_rng(11)
    M, K, N = 40, 384, 256
    ex = rng.integers(-6, 7, size=(M, K // 128))
    ew = rng.integers(-6, 7, size=(N // 128, K // 128))
    xi, xv = power_blocks(rng, M, K, 1, ex)
    wi, wv = power_blocks(rng, N, K, 128, ew)
    qx, sx = W.quant_act(bf16_exact(xv))
    qw, sw = W.quant_weight(bf16_exact(wv))
    assert np.array_equal(qx, xi) and np.array_equal(qw, wi)
    assert np.array_equal(sx, (2.0 ** ex).astype(np.float32))
    assert np.array_equal(sw, (2.0 ** ew).astype(np.float32))
    # every product and partial sum is exact in fp64 (integers below 2^53 times 2^e)
    y = W.gemm(qx, sx, qw, sw)
    assert np.array_equal(y, xv @ wv.T)


def test_bias_is_added():
    rng = np.random.default_rng(12)
    M, K, N = 8, 128, 128
    x, _ = bf16_round(rng.standard_normal((M, K)))
    w, _ = bf16_round(rng.standard_normal((N, K)) / np.sqrt(K))
    b, bv = bf16_round(rng.standard_normal(N))
    y0 = W.linear(x, w)
    y1 = W.linear(x, w, b)
    # y1 = y0 + b up to one fp64 rounding of the sum
    assert np.all(np.abs(y1 - y0 - bv) <= 1e-15 * (np.abs(y0) + np.abs(bv)) * 4)


def test_quantization_bounds_and_zero_blocks():
    rng = np.random.default_rng(13)
    M, K, N = 33, 256, 256
    xv = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    xv[5, 128:] = 0.0  # an all-zero activation block
    wv = rng.standard_normal((N, K)) / 16
    wv[128:, :128] = 0.0  # an all-zero weight block
    x, xd = bf16_round(xv)
    w, wd = bf16_round(wv)
    qx, sx = W.quant_act(x)
    qw, sw = W.quant_weight(w)
    assert sx[5, 1] == 0 and not qx[5, 128:].any()
    assert sw[1, 0] == 0 and not qw[128:, :128].any()
    sxe = np.repeat(sx.astype(np.float64), 128, axis=1)
    swe = np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)
    # half a step, plus the fp32 roundings of 127/amax, of x * inv and of amax/127
    # (each 2^-24 relative, on values up to 127 steps): under 3e-5 of a step
    assert np.all(np.abs(xd - sxe * qx) <= sxe * (0.5 + 3e-5))
    assert np.all(np.abs(wd - swe * qw) <= swe * (0.5 + 3e-5))
    # each non-zero block reaches the full code range
    for m in range(M):
        for b in range(K // 128):
            blk = qx[m, 128 * b:128 * b + 128]
            assert np.abs(blk).max() == (127 if sx[m, b] > 0 else 0)


def test_error_bound_against_unquantized():
    rng = np.random.default_rng(14)
    M, K, N = 17, 512, 256
    x, xd = bf16_round(rng.standard_normal((M, K)))
    w, wd = bf16_round(rng.standard_normal((N, K)) / np.sqrt(K))
    qx, sx = W.quant_act(x)
    qw, sw = W.quant_weight(w)
    y = W.gemm(qx, sx, qw, sw)
    ref = xd @ wd.T
    # |x w - s_x q_x s_w q_w| <= |x| e_w + |w| e_x + e_x e_w per element, e = s / 2
    ex = np.repeat(sx.astype(np.float64), 128, axis=1) / 2
    ew = np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1) / 2
    bound = np.abs(xd) @ ew.T + ex @ np.abs(wd).T + ex @ ew.T
    assert np.all(np.abs(y - ref) <= bound * (1 + 1e-9))
    # and the layer is a close approximation overall
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) < 2e-2


@pytest.mark.parametrize("f", [4.0, 0.25])
def test_power_of_two_scaling_is_exact(f):
    rng = np.random.default_rng(15)
    M, K, N = 9, 256, 128
    x, xd = bf16_round(rng.standard_normal((M, K)))
    w, _ = bf16_round(rng.standard_normal((N, K)))
    x2 = bf16_exact(xd * f)
    q1, s1 = W.quant_act(x)
    q2, s2 = W.quant_act(x2)
    assert np.array_equal(q1, q2) and np.array_equal(s2, s1 * np.float32(f))
    assert np.array_equal(W.linear(x2, w), W.linear(x, w) * f)


def test_integer_products_brute_force():
    rng = np.random.default_rng(16)
    M, K, N = 5, 256, 128
    qx = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    ones_x = np.ones((M, K // 128), np.float32)
    ones_w = np.ones((N // 128, K // 128), np.float32)
    y = W.gemm(qx, ones_x, qw, ones_w)
    want = np.array([[sum(int(qx[m, k]) * int(qw[n, k]) for k in range(K)) for n in range(N)] for m in range(M)])
    assert np.array_equal(y, want.astype(np.float64))


def test_row_range():
    rng = np.random.default_rng(17)
    x, _ = bf16_round(rng.standard_normal((6, 128)))
    w, _ = bf16_round(rng.standard_normal((128, 128)))
    full = W.linear(x, w)
    part = W.linear(x, w, rows=(2, 4))
    assert np.array_equal(part[2:4], full[2:4]) and np.isnan(part[:2]).all() and np.isnan(part[4:]).all()
