"""GPU parity of the adaptive p_hat (phat_mode 1, e4m3): stream bytes, offsets,
decoded symbols and status words bit-exact against the oracle on the same
seeded inputs, on the drifting workload and the 32K-token FP8 cache at reduced
size, on ragged shapes (every scale period, chunks of one to eight epochs, an
epoch boundary at the start of a short chunk's last partial batch), in both
sigma modes and with both mean formats, and on corrupt payloads."""
import dataclasses

import numpy as np
import pytest
import torch

from lossless_kv_cache_scalar_amd import skv, synth
from oracle import skvref as R

from gpu_util import DEV, ensure_built, gpu_calibrate, gpu_roundtrip, np_mu, np_sym, oracle_calibrate, shapes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _check(w, x, mu, sigma, hist):
    sh, rsh = shapes(w)
    assert sh.phat_mode == 1 and rsh.phat_mode == 1
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, x.to(DEV), mu.to(DEV), torch.from_numpy(sigma).to(DEV),
                                                torch.from_numpy(hist.view(np.int64)).to(DEV))
    assert st_e == skv.OK and st_d == skv.OK, (skv.status_string(st_e), skv.status_string(st_d))
    m = R.Model(1, hist)
    xn, mn = np_sym(x, 1), np_mu(mu, w.mu_fmt)
    rbits, roffs = m.encode(rsh, xn, mn, sigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    assert torch.equal(out.cpu(), x)
    rout, st = m.decode(rsh, bits, offs, mn, sigma)
    assert st == R.OK and np.array_equal(rout, xn)
    return bits, offs, m, rsh, mn


@pytest.mark.parametrize("name,mode", [("qwen3_0.6b_e4m3_drift_adapt", 0), ("qwen3_0.6b_e4m3_drift_adapt", 1),
                                       ("qwen3_32b_e4m3_32k_adapt", 0), ("qwen3_32b_e4m3_32k_adapt", 1)])
def test_adaptive_workloads_reduced(name, mode):
    w = dataclasses.replace(synth.WORKLOADS[name], sigma_mode=mode).with_tokens(600, layers=2)
    seqs = [synth.calibration_set(w, j) for j in range(2)]
    sigma, hist = gpu_calibrate(w, seqs)
    rsigma, rhist = oracle_calibrate(w, seqs)
    np.testing.assert_array_equal(sigma.cpu().numpy(), rsigma)
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint64), rhist)
    x, mu = synth.generate(w)
    _check(w, x, mu, rsigma, rhist)


@pytest.mark.parametrize("tokens,head_dim,mu_fmt,mode", [
    (1, 64, 0, 0), (65, 64, 1, 0), (33, 128, 0, 0), (300, 128, 1, 1), (256, 512, 0, 0), (40, 512, 1, 1),
    (257, 256, 0, 0), (300, 32, 1, 0), (511, 16, 0, 1), (3, 8, 1, 0), (257, 256, 1, 1), (300, 256, 0, 1),
    (256, 512, 1, 0), (300, 64, 0, 1)])
def test_adaptive_ragged_shapes(tokens, head_dim, mu_fmt, mode):
    """65 x 64 and 33 x 128 put an epoch boundary right at the start of the
    last partial batch; 256 x 512 has 32 epochs per chunk."""
    w = synth.Workload("adapt_ragged", 7, 1, 2, head_dim, tokens, 1, mu_fmt, 0.05, 1, 64, "drift", mode, 1)
    rng = np.random.default_rng(tokens * 3 + head_dim + mu_fmt)
    x, mu = synth.generate(w)
    per = R.OCT_STRIDE if mode else 1
    sigma = np.ascontiguousarray((0.05 * np.exp(rng.standard_normal(w.n_channels * per))).astype(np.float32))
    sigma[::13] = 0.0
    hist = rng.integers(0, 200, 256).astype(np.uint64)
    _check(w, x, mu, sigma, hist)


def test_adaptive_corrupt_payload_status_matches_oracle():
    w = synth.WORKLOADS["qwen3_0.6b_e4m3_drift_adapt"].with_tokens(300, layers=1)
    seqs = [synth.calibration_set(w, 0)]
    rsigma, rhist = oracle_calibrate(w, seqs)
    x, mu = synth.generate(w)
    bits, offs, m, rsh, mn = _check(w, x, mu, rsigma, rhist)
    sh, _ = shapes(w)
    rng = np.random.default_rng(9)
    sigma = torch.from_numpy(rsigma).to(DEV)
    hist = torch.from_numpy(rhist.view(np.int64)).to(DEV)
    for trial in range(4):
        bad = bits.copy()
        c = int(rng.integers(0, len(offs) - 1))
        pos = rng.integers(int(offs[c]) + 128, int(offs[c + 1]), size=24)
        bad[pos] ^= rng.integers(1, 256, size=24).astype(np.uint8)
        buf = skv.Buffers(sh, device=DEV)
        got = torch.empty_like(x, device=DEV)
        buf.decode(mu.to(DEV), sigma, hist, got, bits=torch.from_numpy(bad).to(DEV),
                   offsets=torch.from_numpy(offs.view(np.int64)).to(DEV))
        torch.cuda.synchronize()
        rout, st_ref = m.decode(rsh, bad, offs, mn, rsigma)
        assert int(buf.status.item()) == st_ref, (trial, c)
        if st_ref == R.OK:
            assert np.array_equal(np_sym(got.cpu(), 1), rout)


def test_adaptive_bf16_is_refused():
    sh = skv.shape(1, 1, 256, 64, 0, 0, 0, 1)
    z = torch.zeros(256 * 64 * 2, dtype=torch.int16, device=DEV)
    sigma = torch.zeros(2 * 64, dtype=torch.float32, device=DEV)
    hist = torch.zeros(65536, dtype=torch.int64, device=DEV)
    big = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    buf_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    rc = skv.encode(sh, z, z, sigma, hist, big, 1 << 20, big, big, 1 << 20, buf_status)
    assert rc == skv.ERR_UNSUPPORTED
