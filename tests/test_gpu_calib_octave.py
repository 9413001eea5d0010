"""Octave-mode calibration on the GPU against the oracle, bin by bin.

The calibration state is compared with the oracle's sums after several calls:
per channel the fp64 sum of squares and the count, and per (channel, fp32
exponent field of mu') the same pair, bit for bit. The means of one call span
far more exponent fields than the kernel keeps in LDS at once (24 below the
channel's largest, plus field 0), and include zeros, subnormals, non-finite
values (read as 0) and the largest finite field (254); some symbols are
non-finite (skipped). The calls use different exponent ranges, so a bin held in
LDS by one call is updated in global memory by another.

The state's layout is the library's own and not part of its interface: S (fp64
[channels]) | n (u64 [channels]) | hist (u64 [symbols]) | So (fp64 [256][channels])
| no (u64 [256][channels]). The oracle keeps its bins channel-major.
"""
import numpy as np
import pytest
import torch

from lossless_kv_cache_scalar_amd import skv
from oracle import skvref as R

from gpu_util import DEV, ensure_built

pytestmark = pytest.mark.gpu

LAYERS, KV_HEADS, HEAD_DIM, TOKENS = 1, 3, 64, 300   # 384 channels: one full block of 256 and a ragged one
RANGES = [(-40, 10), (-10, 30), (-60, -20)]         # log2 |mu| per call


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _f32_to_bf16_bits(a):
    return (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _call_data(rng, sym, mu_fmt, call):
    nch = LAYERS * 2 * KV_HEADS * HEAD_DIM
    n = nch * TOKENS
    lo, hi = RANGES[call]
    mag = np.exp2(rng.uniform(lo, hi, n)) * rng.choice([-1.0, 1.0], n)
    mag[rng.random(n) < 0.1] = 0.0
    m = mag.astype(np.float32)
    m[rng.random(n) < 0.02] = np.float32(3e-39)          # fp32 subnormal: field 0
    # [rows][tokens][head_dim] with rows = layers * 2 * kv_heads; channel c = (row, d)
    m3 = m.reshape(-1, TOKENS, HEAD_DIM)
    if call == 0:
        m3[0, :, 5] = 0.0                                # a channel whose means are all zero this call
    if call == 1:
        m3[1, ::3, 6] = np.float32(3.0e38)               # field 254, the largest finite one
    with np.errstate(over="ignore"):                   # near 3e38 some symbols overflow to inf: skipped
        x32 = (m * (1.0 + 0.05 * rng.standard_normal(n))).astype(np.float32)
    if mu_fmt == R.MU_BF16:
        mu = _f32_to_bf16_bits(m)
        mu[::97] = 0x7FC0                                # NaN, read as 0
        mu[::89] = 0xFF80                                # -inf, read as 0
        mu[::83] = 0x0003                                # bf16 subnormal
    else:
        mu = m.copy()
        mu[::97] = np.float32("nan")
        mu[::89] = np.float32("-inf")
    if sym == R.SYM_BF16:
        x = _f32_to_bf16_bits(x32)
        x[::101] = 0x7F80                                # +inf: skipped
        x[::103] = 0xFFC1                                # NaN: skipped
    else:
        x = rng.integers(0, 256, n).astype(np.uint8)     # includes the two NaN patterns
    return np.ascontiguousarray(x), np.ascontiguousarray(mu)


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


@pytest.mark.parametrize("sym,mu_fmt", [(R.SYM_BF16, R.MU_BF16), (R.SYM_BF16, R.MU_F32),
                                        (R.SYM_E4M3, R.MU_BF16), (R.SYM_E4M3, R.MU_F32)])
def test_octave_bins_bit_exact(sym, mu_fmt):
    rng = np.random.default_rng(4242 + 10 * sym + mu_fmt)
    sh = skv.shape(LAYERS, KV_HEADS, TOKENS, HEAD_DIM, sym, mu_fmt, skv.SIGMA_OCTAVE)
    rsh = R.make_shape(LAYERS, KV_HEADS, TOKENS, HEAD_DIM, sym, mu_fmt, R.SIGMA_OCTAVE)
    state = torch.empty(skv.calib_state_size(sh), dtype=torch.uint8, device=DEV)
    assert skv.calib_reset(state, sh) == skv.OK
    cal = R.Calibrator(rsh)
    for call in range(len(RANGES)):
        x, mu = _call_data(rng, sym, mu_fmt, call)
        assert skv.calib_accumulate(state, sh, _dev(x), _dev(mu)) == skv.OK
        cal.accumulate(x, mu)
    torch.cuda.synchronize()

    nch = LAYERS * 2 * KV_HEADS * HEAD_DIM
    nsym = 65536 if sym == R.SYM_BF16 else 256
    raw = state.cpu().numpy()
    o = 0

    def take(count, dtype):
        nonlocal o
        a = raw[o:o + 8 * count].view(dtype)
        o += 8 * count
        return a

    S, n, hist = take(nch, np.float64), take(nch, np.uint64), take(nsym, np.uint64)
    So, no = take(256 * nch, np.float64), take(256 * nch, np.uint64)
    assert o == raw.size
    np.testing.assert_array_equal(S.view(np.uint64), cal.S.view(np.uint64))
    np.testing.assert_array_equal(n, cal.n)
    np.testing.assert_array_equal(hist, cal.hist)
    np.testing.assert_array_equal(no.reshape(256, nch).T, cal.no.reshape(nch, 256))
    np.testing.assert_array_equal(So.reshape(256, nch).T.view(np.uint64), cal.So.reshape(nch, 256).view(np.uint64))
    # the data reach far outside one call's window: many fields per channel are occupied
    occupied = (cal.no.reshape(nch, 256) > 0).sum(axis=1)
    assert occupied.min() > 40

    sigma = torch.empty(skv.sigma_floats(sh), dtype=torch.float32, device=DEV)
    hist_out = torch.empty(nsym, dtype=torch.int64, device=DEV)
    assert skv.calib_finalize(state, sh, sigma, hist_out) == skv.OK
    torch.cuda.synchronize()
    rtable, rhist = cal.finalize()
    np.testing.assert_array_equal(sigma.cpu().numpy(), rtable)
    np.testing.assert_array_equal(hist_out.cpu().numpy().view(np.uint64), rhist)
