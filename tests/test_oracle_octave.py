"""Pins for the oracle's magnitude-conditioned sigma (octave mode; no GPU).

The pages name a static per-channel sigma as a cost of the early model, the
residual's size varying with context ("Speculative KV coding", "下一步计划").
Octave mode looks sigma up per (channel, octave of |mu'|); these tests fix the
octave rule with numpy's frexp, the table layout through the lane substreams,
the calibration estimator by brute force, and the reduction to channel mode.
"""
import numpy as np
import pytest

from lossless_kv_cache_scalar_amd import synth
from oracle import skvref as R

from test_oracle_coder import _cache, _lane_bytes_from_chunk


def _exp_field(v):
    """fp32 biased exponent field of v via frexp: floor(log2|v|) + 127, 0 for 0 and subnormals."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(np.abs(v))  # |v| = m 2^e, m in [0.5, 1)
    return np.where(np.abs(v) >= 2.0 ** -126, e + 126, 0)


def _octave(mup, sigma_c):
    sg = np.maximum(np.asarray(sigma_c, dtype=np.float32), np.float32(2.0 ** -100))
    return np.clip(_exp_field(mup) - _exp_field(sg) - 1, 0, R.OCTAVES - 1)


def _mu_prime(mu_f32):
    return np.where(np.isfinite(mu_f32), mu_f32, np.float32(0)).astype(np.float32)


def _shape(w, mode=R.SIGMA_OCTAVE, tokens=None):
    return R.make_shape(w.layers, w.kv_heads, tokens or w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, mode)


def _mu_f32(w, mu):
    if w.mu_fmt == R.MU_BF16:
        return (mu.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return mu.astype(np.float32)


@pytest.mark.parametrize("tokens,head_dim,fmt", [(256, 128, 0), (300, 64, 0), (200, 128, 1)])
def test_octave_chunk_is_the_lane_substreams(tokens, head_dim, fmt):
    """In octave mode substream l is the range code of scalars l, l + 64, ...
    with each scalar's scale taken from its channel's table at the octave of
    its mean (non-finite means read as 0, so octave 0)."""
    w = synth.Workload("t", 1, 1, 2, head_dim, tokens, fmt, 1 if fmt else 0, 0.02, 1, 64)
    x, mu = _cache(w)
    mu = mu.copy()
    if w.mu_fmt == R.MU_BF16:
        mu.reshape(-1)[::97] = 0x7FC0
        mu.reshape(-1)[::89] = 0xFF80
    else:
        mu.reshape(-1)[::97] = np.nan
    rng = np.random.default_rng(tokens + head_dim)
    table = np.exp(rng.uniform(-7, 0, (w.n_channels, R.OCT_STRIDE))).astype(np.float32)
    table[::7, 0] = 0.0  # sigma_c = 0: the grid is set by 2^-100
    m = R.Model(fmt, rng.integers(0, 50, 65536 if fmt == 0 else 256).astype(np.uint64))
    bits, offs = m.encode(_shape(w), x, mu, table.reshape(-1))
    xs = x.reshape(-1, tokens * head_dim)
    mus = _mu_f32(w, mu).reshape(-1, tokens * head_dim)
    ntb = (tokens + 255) // 256
    up = 0 if fmt == 0 else 8
    for c in range(len(offs) - 1):
        row, blk = divmod(c, ntb)
        lo_i, hi_i = blk * 256 * head_dim, min(tokens, (blk + 1) * 256) * head_dim
        lanes = _lane_bytes_from_chunk(bits[int(offs[c]):int(offs[c + 1])])
        trow = table[row * head_dim:(row + 1) * head_dim]
        for l in range(64):
            idx = np.arange(lo_i + l, hi_i, 64)
            ch = idx % head_dim
            j = _octave(_mu_prime(mus[row, idx]), trow[ch, 0])
            sc = R.scale(trow[ch, 1 + j])
            clo, chi = m.cum_pair(mus[row, idx], sc, xs[row, idx].astype(np.uint32))
            want = R.rc_encode_seq(clo.astype(np.uint64) << up, (chi - clo).astype(np.uint64) << up)
            assert bytes(lanes[l]) == bytes(want), (c, l)


def test_flat_octave_table_equals_channel_mode():
    """A table whose eight octave sigmas all equal the channel's codes exactly
    as channel mode with that sigma."""
    w = synth.WORKLOADS["qwen3_0.6b_bf16"].with_tokens(300, layers=1)
    x, mu = _cache(w)
    rng = np.random.default_rng(3)
    sigma = (0.02 * np.exp(rng.standard_normal(w.n_channels))).astype(np.float32)
    table = np.repeat(sigma[:, None], R.OCT_STRIDE, axis=1)
    m = R.Model(0, rng.integers(0, 9, 65536).astype(np.uint64))
    b0, o0 = m.encode(_shape(w, R.SIGMA_CHANNEL), x, mu, sigma)
    b1, o1 = m.encode(_shape(w, R.SIGMA_OCTAVE), x, mu, np.ascontiguousarray(table.reshape(-1)))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(b0, b1)


@pytest.mark.parametrize("name", ["qwen3_32b_bf16_fp8res", "qwen3_0.6b_e4m3"])
def test_octave_calibration_is_the_per_octave_rms(name):
    """Entry 0 is the channel sigma of channel mode; entry 1 + j is the rms
    residual over the channel's calibration scalars in octave j (by frexp),
    or the channel sigma when fewer than 16 fell there."""
    w = synth.WORKLOADS[name].with_tokens(96, layers=1)
    w = synth.Workload(w.name, w.index, 1, w.kv_heads, w.head_dim, 96, w.sym_fmt, w.mu_fmt, w.sigma_k,
                       2, 96, w.mu_kind)
    c0 = R.Calibrator(_shape(w, R.SIGMA_CHANNEL, tokens=96))
    c1 = R.Calibrator(_shape(w, R.SIGMA_OCTAVE, tokens=96))
    xs, ms = [], []
    for j in range(2):
        x, mu = _cache(w, seed=w.calib_seed(j), tokens=96)
        c0.accumulate(x, mu)
        c1.accumulate(x, mu)
        xs.append(x)
        ms.append(mu)
    sig, h0 = c0.finalize()
    tab, h1 = c1.finalize()
    tab = tab.reshape(-1, R.OCT_STRIDE)
    np.testing.assert_array_equal(tab[:, 0], sig)
    np.testing.assert_array_equal(h0, h1)
    D = w.head_dim
    # brute force: values, means and residuals by channel
    def by_channel(a):
        return a.reshape(w.layers * 2 * w.kv_heads, -1, D).transpose(0, 2, 1).reshape(w.n_channels, -1)
    if w.sym_fmt == R.SYM_BF16:
        v = np.concatenate([by_channel((x.view(np.uint16).astype(np.uint32) << 16).view(np.float32)) for x in xs], 1)
    else:
        import torch
        v = np.concatenate([by_channel(torch.from_numpy(x.view(np.uint8).copy()).view(torch.float8_e4m3fn)
                                       .to(torch.float32).numpy()) for x in xs], 1)
    mp = np.concatenate([by_channel(_mu_prime(_mu_f32(w, mu))) for mu in ms], 1)
    fin = np.isfinite(v)
    r2 = np.where(fin, (v.astype(np.float64) - mp.astype(np.float64)) ** 2, 0.0)
    j = _octave(mp, sig[:, None])
    for q in range(R.OCTAVES):
        sel = fin & (j == q)
        n = sel.sum(1)
        rms = np.sqrt(np.where(sel, r2, 0).sum(1) / np.maximum(n, 1))
        want = np.where(n >= 16, rms, sig).astype(np.float32)
        np.testing.assert_allclose(tab[:, 1 + q], want, rtol=2e-7)
        assert np.array_equal(tab[n < 16, 1 + q], sig[n < 16])


@pytest.mark.parametrize("name", ["qwen3_32b_bf16_fp8res", "qwen3_0.6b_e4m3", "tiny_bf16"])
def test_octave_roundtrip(name):
    w = synth.WORKLOADS[name]
    if name != "tiny_bf16":
        w = w.with_tokens(300, layers=1)
    cal = R.Calibrator(_shape(w, tokens=w.calib_tokens))
    x, mu = _cache(w, seed=w.calib_seed(0), tokens=w.calib_tokens)
    cal.accumulate(x, mu)
    tab, hist = cal.finalize()
    x, mu = _cache(w)
    m = R.Model(w.sym_fmt, hist)
    sh = _shape(w)
    bits, offs = m.encode(sh, x, mu, tab)
    out, st = m.decode(sh, bits, offs, mu, tab)
    assert st == R.OK and np.array_equal(out, x)


def _bits_per_scalar(w, mode):
    cal = R.Calibrator(_shape(w, mode, tokens=w.calib_tokens))
    for j in range(4):
        cal.accumulate(*_cache(w, seed=w.calib_seed(j), tokens=w.calib_tokens))
    sig, hist = cal.finalize()
    x, mu = _cache(w)
    bits, _ = R.Model(w.sym_fmt, hist).encode(_shape(w, mode), x, mu, sig)
    return 8.0 * bits.size / x.size


def test_octave_mode_saves_bits_where_the_residual_scales_with_mu():
    """Block-FP8 round-trip residuals grow with |mu|: per-octave sigma codes
    them in well under the per-channel bits; on the mixture workload, whose
    residual does not depend on |mu|, it costs next to nothing."""
    fp8 = synth.WORKLOADS["qwen3_32b_bf16_fp8res"].with_tokens(512, layers=1)
    b0, b1 = _bits_per_scalar(fp8, R.SIGMA_CHANNEL), _bits_per_scalar(fp8, R.SIGMA_OCTAVE)
    assert b1 < b0 - 0.4, (b0, b1)
    mix = synth.WORKLOADS["qwen3_32b_bf16"].with_tokens(512, layers=1)
    c0, c1 = _bits_per_scalar(mix, R.SIGMA_CHANNEL), _bits_per_scalar(mix, R.SIGMA_OCTAVE)
    assert abs(c1 - c0) < 0.03, (c0, c1)
