"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact: stream bytes, offsets, decoded symbols,
calibrated sigma and histogram."""
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


def _workload(name):
    """A named workload; "<name>_oct" not in the table: that workload coded in octave mode."""
    if name in synth.WORKLOADS:
        return synth.WORKLOADS[name]
    assert name.endswith("_oct")
    return dataclasses.replace(synth.WORKLOADS[name[:-4]], name=name, sigma_mode=1)


def _reduced(name, layers=2, tokens=600, calib_seqs=2):
    w = _workload(name)
    if not name.startswith("tiny_bf16"):
        w = w.with_tokens(tokens, layers=layers)
    return w, min(calib_seqs, w.calib_seqs)


CASES = ["tiny_bf16", "qwen3_0.6b_bf16", "qwen3_0.6b_e4m3", "qwen3_32b_bf16", "qwen3_32b_e4m3_32k", "qwen3_32b_bf16_fp8res",
         "qwen3_32b_bf16_fp8res_oct", "qwen3_0.6b_e4m3_oct", "tiny_bf16_oct"]


@pytest.mark.parametrize("name", CASES)
def test_calibration_bit_exact(name):
    w, ns = _reduced(name)
    seqs = [synth.calibration_set(w, j) for j in range(ns)]
    sigma, hist = gpu_calibrate(w, seqs)
    rsigma, rhist = oracle_calibrate(w, seqs)
    np.testing.assert_array_equal(sigma.cpu().numpy(), rsigma)
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint64), rhist)


@pytest.mark.parametrize("name", CASES)
def test_encode_decode_bit_exact(name):
    w, ns = _reduced(name)
    seqs = [synth.calibration_set(w, j) for j in range(ns)]
    rsigma, rhist = oracle_calibrate(w, seqs)
    x, mu = synth.generate(w)
    sh, rsh = shapes(w)
    sigma = torch.from_numpy(rsigma).to(DEV)
    hist = torch.from_numpy(rhist.view(np.int64)).to(DEV)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, x.to(DEV), mu.to(DEV), sigma, hist)
    assert st_e == skv.OK and st_d == skv.OK
    m = R.Model(w.sym_fmt, rhist)
    xn, mn = np_sym(x, w.sym_fmt), np_mu(mu, w.mu_fmt)
    rbits, roffs = m.encode(rsh, xn, mn, rsigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    assert torch.equal(out.cpu(), x)
    # the oracle decodes the GPU stream too
    rout, st = m.decode(rsh, bits, offs, mn, rsigma)
    assert st == R.OK and np.array_equal(rout, xn)


def test_every_bf16_pattern_and_degenerate_inputs():
    rng = np.random.default_rng(7)
    x = rng.permutation(65536).astype(np.uint16).reshape(1, 2, 1, 512, 64)
    mu = (x.astype(np.int64) + rng.integers(-40, 40, x.shape)).clip(0, 65535).astype(np.uint16)
    mu.reshape(-1)[::101] = 0x7FC0
    mu.reshape(-1)[::103] = 0xFF80
    mu.reshape(-1)[::107] = 0x0001  # subnormal
    sigma = np.exp(rng.uniform(-30, 30, 128)).astype(np.float32)
    sigma[::9] = 0.0
    sigma[1::9] = 1e-38
    hist = rng.integers(0, 50, 65536).astype(np.uint64)
    sh, rsh = skv.shape(1, 1, 512, 64), R.make_shape(1, 1, 512, 64)
    xt = torch.from_numpy(x.view(np.int16)).to(DEV)
    mt = torch.from_numpy(mu.view(np.int16)).to(DEV)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, xt, mt, torch.from_numpy(sigma).to(DEV),
                                                torch.from_numpy(hist.view(np.int64)).to(DEV))
    assert st_e == skv.OK and st_d == skv.OK
    rbits, roffs = R.Model(0, hist).encode(rsh, x, mu, sigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), x)


@pytest.mark.parametrize("mu_fmt", [0, 1])
def test_every_e4m3_pattern(mu_fmt):
    rng = np.random.default_rng(8 + mu_fmt)
    n = 2 * 2 * 300 * 64
    x = rng.permutation(np.tile(np.arange(256, dtype=np.uint8), n // 256 + 1)[:n]).reshape(1, 2, 2, 300, 64)
    vals = np.nan_to_num(np.array([R.value(1, v) for v in range(256)]), nan=0.0)
    muf = (vals[x] + rng.standard_normal(x.shape) * np.exp(rng.uniform(-6, 6, x.shape))).astype(np.float32)
    muf.reshape(-1)[::37] = np.nan
    muf.reshape(-1)[::41] = np.inf     # read as 0
    muf.reshape(-1)[::43] = -1e30      # far beyond +-448: bf16 keeps it, the guesses clamp
    muf.reshape(-1)[::47] = 600.0
    if mu_fmt == 0:
        mu = torch.from_numpy(muf).to(torch.bfloat16).view(torch.int16)
        mun = mu.numpy().view(np.uint16)
    else:
        mu = torch.from_numpy(muf)
        mun = muf
    sigma = np.exp(rng.uniform(-10, 6, 2 * 2 * 64)).astype(np.float32)
    sigma[::5] = 0.0
    hist = rng.integers(0, 1000, 256).astype(np.uint64)
    sh, rsh = skv.shape(1, 2, 300, 64, 1, mu_fmt), R.make_shape(1, 2, 300, 64, 1, mu_fmt)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, torch.from_numpy(x).to(DEV), mu.to(DEV),
                                                torch.from_numpy(sigma).to(DEV),
                                                torch.from_numpy(hist.view(np.int64)).to(DEV))
    assert st_e == skv.OK and st_d == skv.OK
    rbits, roffs = R.Model(1, hist).encode(rsh, x, np.ascontiguousarray(mun), sigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    np.testing.assert_array_equal(out.cpu().numpy(), x)


@pytest.mark.parametrize("tokens,head_dim,sym,mu_fmt", [
    (1, 64, 0, 0), (3, 128, 0, 0), (300, 64, 1, 0), (257, 8, 0, 0), (40, 512, 1, 0), (511, 16, 0, 0), (2, 32, 1, 0),
    (1, 64, 0, 1), (3, 128, 0, 1), (257, 8, 0, 1), (511, 16, 0, 1), (2, 32, 1, 1), (300, 64, 1, 1)])
def test_ragged_shapes(tokens, head_dim, sym, mu_fmt):
    w = synth.Workload("ragged", 1, 2, 3, head_dim, tokens, sym, mu_fmt, 0.02, 1, 64)
    rng = np.random.default_rng(tokens + head_dim + 1000 * mu_fmt)
    x, mu = synth.generate(w)
    sigma = (0.02 * np.exp(rng.standard_normal(w.n_channels))).astype(np.float32)
    hist = rng.integers(0, 9, 65536 if sym == 0 else 256).astype(np.uint64)
    sh, rsh = shapes(w)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, x.to(DEV), mu.to(DEV), torch.from_numpy(sigma).to(DEV),
                                                torch.from_numpy(hist.view(np.int64)).to(DEV))
    assert st_e == skv.OK and st_d == skv.OK
    rbits, roffs = R.Model(sym, hist).encode(rsh, np_sym(x, sym), np_mu(mu, mu_fmt), sigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    assert torch.equal(out.cpu(), x)


@pytest.mark.parametrize("tokens,head_dim,sym,mu_fmt", [
    (3, 128, 0, 0), (300, 64, 1, 0), (257, 8, 0, 0), (40, 512, 1, 0), (600, 256, 0, 0),
    (40, 512, 0, 0), (257, 256, 1, 0), (40, 512, 0, 1), (257, 256, 1, 1), (300, 256, 0, 1), (40, 512, 1, 1)])
def test_ragged_shapes_octave_mode(tokens, head_dim, sym, mu_fmt):
    """Octave mode on every scale period (head_dim 8 .. 512), both symbol and
    mean formats, and ragged chunks, with a random table (zero, tiny and large
    sigmas) and non-finite means."""
    w = synth.Workload("ragged_oct", 1, 2, 3, head_dim, tokens, sym, mu_fmt, 0.02, 1, 64, "mixture", 1)
    rng = np.random.default_rng(tokens + head_dim + 7)
    x, mu = synth.generate(w)
    mu = mu.clone()
    if mu_fmt == 0:
        mu.view(-1)[::97] = 0x7FC0   # NaN means read as 0
        mu.view(-1)[::89] = -128     # 0xFF80 = -inf
    else:
        mu.view(-1)[::97] = float("nan")
        mu.view(-1)[::89] = float("-inf")
    table = np.exp(rng.uniform(-9, 1, (w.n_channels, R.OCT_STRIDE))).astype(np.float32)
    table[::5, 0] = 0.0
    table[::7, 3] = 0.0
    sigma = np.ascontiguousarray(table.reshape(-1))
    hist = rng.integers(0, 9, 65536 if sym == 0 else 256).astype(np.uint64)
    sh, rsh = shapes(w)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, x.to(DEV), mu.to(DEV), torch.from_numpy(sigma).to(DEV),
                                                torch.from_numpy(hist.view(np.int64)).to(DEV))
    assert st_e == skv.OK and st_d == skv.OK
    rbits, roffs = R.Model(sym, hist).encode(rsh, np_sym(x, sym), np_mu(mu, mu_fmt), sigma)
    np.testing.assert_array_equal(offs, roffs)
    np.testing.assert_array_equal(bits, rbits)
    assert torch.equal(out.cpu(), x)


def _tiny_inputs():
    w = synth.WORKLOADS["tiny_bf16"]
    rsigma, rhist = oracle_calibrate(w, [synth.calibration_set(w, 0)])
    x, mu = synth.generate(w)
    sh, rsh = shapes(w)
    return w, sh, x.to(DEV), mu.to(DEV), torch.from_numpy(rsigma).to(DEV), torch.from_numpy(rhist.view(np.int64)).to(DEV)


def test_capacity_error_is_reported():
    w, sh, x, mu, sigma, hist = _tiny_inputs()
    buf = skv.Buffers(sh, device=DEV)
    rc = skv.encode(sh, x, mu, sigma, hist, buf.bits, 1000, buf.offsets, buf.workspace, buf.ws_bytes, buf.status)
    assert rc == skv.OK
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.ERR_CAPACITY
    assert int(buf.offsets[-1].item()) > 1000


def test_corrupt_stream_is_reported():
    w, sh, x, mu, sigma, hist = _tiny_inputs()
    buf = skv.Buffers(sh, device=DEV)
    buf.encode(x, mu, sigma, hist)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.OK
    bad = buf.bits.clone()
    bad[0] ^= 1  # header length no longer adds up
    out = torch.empty_like(x)
    buf.decode(mu, sigma, hist, out, bits=bad)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.ERR_CORRUPT


@pytest.mark.parametrize("name", ["tiny_bf16", "qwen3_0.6b_e4m3"])
def test_corrupt_payload_status_matches_oracle(name):
    """Garbage inside a chunk's coded words (headers intact) drives the
    decoder's search into and past the alphabet's ends; the GPU must finish,
    and report corruption exactly when the oracle does."""
    w, ns = _reduced(name, layers=1, tokens=300)
    seqs = [synth.calibration_set(w, j) for j in range(ns)]
    rsigma, rhist = oracle_calibrate(w, seqs)
    x, mu = synth.generate(w)
    sh, rsh = shapes(w)
    sigma = torch.from_numpy(rsigma).to(DEV)
    hist = torch.from_numpy(rhist.view(np.int64)).to(DEV)
    bits, offs, out, st_e, st_d = gpu_roundtrip(sh, x.to(DEV), mu.to(DEV), sigma, hist)
    assert st_e == skv.OK and st_d == skv.OK
    m = R.Model(w.sym_fmt, rhist)
    mn = np_mu(mu, w.mu_fmt)
    rng = np.random.default_rng(7)
    for trial in range(4):
        bad = bits.copy()
        c = int(rng.integers(0, len(offs) - 1))
        lo, hi = int(offs[c]) + 128, int(offs[c + 1])  # past the chunk's length header
        pos = rng.integers(lo, hi, size=24)
        bad[pos] ^= rng.integers(1, 256, size=24).astype(np.uint8)
        buf = skv.Buffers(sh, device=DEV)
        dev_bits = torch.from_numpy(bad).to(DEV)
        got = torch.empty_like(x, device=DEV)
        buf.decode(mu.to(DEV), sigma, hist, got, bits=dev_bits, offsets=torch.from_numpy(offs.view(np.int64)).to(DEV))
        torch.cuda.synchronize()
        st_gpu = int(buf.status.item())
        rout, st_ref = m.decode(rsh, bad, offs, mn, rsigma)
        assert st_gpu == st_ref, (trial, c, st_gpu, st_ref)
        if st_ref == R.OK:
            assert np.array_equal(np_sym(got.cpu(), w.sym_fmt), rout)


def test_bad_sigma_is_reported():
    w, sh, x, mu, sigma, hist = _tiny_inputs()
    buf = skv.Buffers(sh, device=DEV)
    bad = sigma.clone()
    bad[3] = float("nan")
    bad[5] = -1.0
    buf.encode(x, mu, bad, hist)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.ERR_ARG


def test_encode_is_deterministic():
    w, sh, x, mu, sigma, hist = _tiny_inputs()
    a = skv.Buffers(sh, device=DEV)
    b = skv.Buffers(sh, device=DEV)
    a.encode(x, mu, sigma, hist)
    b.encode(x, mu, sigma, hist)
    torch.cuda.synchronize()
    n = a.stream_bytes()
    assert n == b.stream_bytes() and torch.equal(a.bits[:n], b.bits[:n]) and torch.equal(a.offsets, b.offsets)


def test_kernel_timing_records_each_launch():
    w, sh, x, mu, sigma, hist = _tiny_inputs()
    buf = skv.Buffers(sh, device=DEV)
    out = torch.empty_like(x)
    skv.timing_start(16)
    buf.encode(x, mu, sigma, hist)
    buf.decode(mu, sigma, hist, out)
    rec = skv.timing_stop(16)
    assert [k for k, _ in rec] == ["model", "k_encode", "model", "k_decode"]
    assert all(ms > 0 for _, ms in rec)
    assert torch.equal(out, x)
    buf.encode(x, mu, sigma, hist)  # recording is off again: nothing recorded, nothing breaks
    torch.cuda.synchronize()
