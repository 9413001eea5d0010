"""Pins for the oracle's calibration (no GPU).

sigma^2 = E[(KV_full - mu)^2] is the cost-minimising variance ('Speculative KV
coding', what q should look like), measured per (kv, head, channel) on a small
calibration set ('early results'); p_hat is the symbol histogram.
"""
import numpy as np
import pytest
import torch

from oracle import skvref as R
from lossless_kv_cache_scalar_amd import synth


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_histogram_is_bincount():
    w = synth.WORKLOADS["tiny_bf16"]
    x, mu = synth.generate(w)
    xn = x.numpy().view(np.uint16)
    cal = R.Calibrator(R.make_shape(1, 2, 256, 64))
    cal.accumulate(xn, mu.numpy().view(np.uint16))
    sigma, hist = cal.finalize()
    np.testing.assert_array_equal(hist, np.bincount(xn.ravel(), minlength=65536))


def test_constant_residual_gives_its_magnitude():
    rng = np.random.default_rng(1)
    a = np.float32(0.125)
    xv = rng.integers(-8, 8, (1, 2, 1, 64, 64)).astype(np.float32)  # exact in bf16
    x = _bf16_bits(xv)
    mu = _bf16_bits(xv - a)
    cal = R.Calibrator(R.make_shape(1, 1, 64, 64))
    cal.accumulate(x, mu)
    sigma, _ = cal.finalize()
    assert np.all(sigma == a)


def test_alternating_residual():
    xv = np.zeros((1, 2, 1, 10, 8), np.float32)
    mu_v = np.where(np.arange(10)[None, None, None, :, None] % 2 == 0, 0.5, -0.5) * np.ones_like(xv)
    cal = R.Calibrator(R.make_shape(1, 1, 10, 8))
    cal.accumulate(_bf16_bits(xv), _bf16_bits(mu_v))
    sigma, _ = cal.finalize()
    assert np.all(sigma == 0.5)


def test_sigma_minimises_gaussian_code_length():
    """Perturbing the calibrated sigma up or down raises the mean of
    -log N(x; mu, sigma^2) over the calibration data."""
    w = synth.WORKLOADS["tiny_bf16"]
    x, mu = synth.generate(w)
    xn, mn = x.numpy().view(np.uint16), mu.numpy().view(np.uint16)
    cal = R.Calibrator(R.make_shape(1, 2, 256, 64))
    cal.accumulate(xn, mn)
    sigma, _ = cal.finalize()
    xv = (xn.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mv = (mn.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r2 = ((xv - mv) ** 2).transpose(0, 1, 2, 4, 3).reshape(-1, 256)  # [channel, token]

    def nll(s):
        return (0.5 * np.log(2 * np.pi * s[:, None] ** 2) + r2 / (2 * s[:, None] ** 2)).mean(1)

    s = sigma.astype(np.float64)
    base = nll(s)
    assert np.all(nll(s * 1.01) > base) and np.all(nll(s * 0.99) > base)


def test_streaming_order_is_call_then_token():
    """Two calls of 100 and 156 tokens equal one call over the concatenation."""
    w = synth.WORKLOADS["tiny_bf16"]
    x, mu = synth.generate(w)
    xn, mn = x.numpy().view(np.uint16), mu.numpy().view(np.uint16)
    one = R.Calibrator(R.make_shape(1, 2, 256, 64))
    one.accumulate(xn, mn)
    two = R.Calibrator(R.make_shape(1, 2, 100, 64))
    two.accumulate(np.ascontiguousarray(xn[:, :, :, :100]), np.ascontiguousarray(mn[:, :, :, :100]))
    two.shape = R.make_shape(1, 2, 156, 64)
    two.accumulate(np.ascontiguousarray(xn[:, :, :, 100:]), np.ascontiguousarray(mn[:, :, :, 100:]))
    s1, h1 = one.finalize()
    s2, h2 = two.finalize()
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(h1, h2)


def test_non_finite_symbols_and_means():
    x = np.full((1, 2, 1, 4, 8), 0x3F80, np.uint16)  # 1.0
    x[0, 0, 0, 0, :] = 0x7FC0  # NaN: counted in hist, skipped in sigma
    x[0, 0, 0, 1, :] = 0xFF80  # -inf
    mu = np.full_like(x, 0x3F00)  # 0.5
    mu[0, 1, 0, 2, :] = 0x7F80  # +inf prediction reads as 0
    cal = R.Calibrator(R.make_shape(1, 1, 4, 8))
    cal.accumulate(x, mu)
    sigma, hist = cal.finalize()
    assert hist[0x7FC0] == 8 and hist[0xFF80] == 8 and hist[0x3F80] == 48
    assert np.all(sigma[:8] == 0.5)  # K: two finite tokens, residual 0.5
    expect_v = np.float32(np.sqrt((3 * 0.25 + 1.0) / 4))
    assert np.all(sigma[8:] == expect_v)
    empty = R.Calibrator(R.make_shape(1, 1, 1, 8))
    xx = np.full((1, 2, 1, 1, 8), 0x7FC0, np.uint16)
    empty.accumulate(xx, xx)
    s, _ = empty.finalize()
    assert np.all(s == 1.0)


def test_e4m3_values_and_fp32_mean():
    vals = np.array([R.value(1, v) for v in range(256)])
    xb = np.arange(256, dtype=np.uint8).reshape(1, 2, 1, 16, 8)
    mu = np.zeros((1, 2, 1, 16, 8), np.float32)
    cal = R.Calibrator(R.make_shape(1, 1, 16, 8, R.SYM_E4M3, R.MU_F32))
    cal.accumulate(xb, mu)
    sigma, hist = cal.finalize()
    assert np.all(hist == 1)
    v = vals.reshape(2, 16, 8)
    for kv in range(2):
        for d in range(8):
            col = v[kv, :, d]
            col = col[np.isfinite(col)]
            assert sigma[kv * 8 + d] == np.float32(np.sqrt(np.mean(col ** 2)))
