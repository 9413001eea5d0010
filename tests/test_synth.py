"""The input generator (no coding arithmetic): shapes, determinism, and the
FP8-residual predictor's defining property."""
import numpy as np
import torch

from lossless_kv_cache_scalar_amd import synth


def test_layers_drawn_alone_match_the_whole_cache():
    w = synth.WORKLOADS["qwen3_0.6b_bf16"].with_tokens(40, layers=3)
    x, mu = synth.generate(w)
    x1, mu1 = synth.generate(w, layers=range(1, 2))
    assert x.shape == (3, 2, 8, 40, 128) and torch.equal(x[1:2], x1) and torch.equal(mu[1:2], mu1)


def test_fp8_block_predictor_is_the_block_fp8_round_trip():
    """mu = e4m3(x / s) * s per 32-channel block, s = amax / 448: every residual
    is within half an e4m3 step of the scaled value, values representable in
    the block's e4m3 grid come back exactly, and the block maximum is exact."""
    w = synth.WORKLOADS["qwen3_32b_bf16_fp8res"].with_tokens(64, layers=1)
    x, mu = synth.generate(w)
    xf = (x.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mf = (mu.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xb = xf.reshape(-1, 32)
    mb = mf.reshape(-1, 32)
    s = np.abs(xb).max(1, keepdims=True) / 448.0
    v = np.abs(xb) / s
    # e4m3 step at v: 2^(floor(log2 v) - 3) for normal values, 2^-9 below 2^-6
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 1e-300))) - 3), 2.0 ** -9)
    err = np.abs(xb - mb) / s
    # mu is rounded to bf16 after the round trip: allow one bf16 rounding of mu
    assert np.all(err <= 0.5 * step + np.abs(mb) / s * 2.0 ** -8 + 1e-12)
    amax_pos = np.abs(xb).argmax(1)
    rows = np.arange(xb.shape[0])
    assert np.allclose(mb[rows, amax_pos], xb[rows, amax_pos], rtol=2.0 ** -8)
    assert 0.0 < np.mean(err == 0) < 1.0
