"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times: decode(encode(x)) == x over the whole cache, and sampled chunks of the
GPU stream byte-equal to the oracle's encoding of the same chunks (and decoded
by the oracle back to x).  Calibration is compared with the oracle on the same
sequences."""
import numpy as np
import pytest
import torch

from lossless_kv_cache_scalar_amd import skv, synth
from oracle import skvref as R

from gpu_util import DEV, ensure_built, np_mu, np_sym

pytestmark = pytest.mark.gpu

NAMES = ["tiny_bf16", "qwen3_0.6b_bf16", "qwen3_0.6b_e4m3", "qwen3_32b_bf16", "qwen3_32b_e4m3_32k", "qwen3_32b_bf16_fp8res",
         "qwen3_32b_bf16_fp8res_oct"]
CALIB_SEQS = 2  # the launch configuration does not depend on the calibration set's size


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


@pytest.mark.parametrize("name", NAMES)
def test_full_size_roundtrip_and_sampled_oracle_parity(name):
    w = synth.WORKLOADS[name]
    print(f"[fullsize] {name}: {w.n_scalars} scalars", flush=True)
    ns = min(CALIB_SEQS, w.calib_seqs)
    csh = skv.shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    seqs = [synth.calibration_set(w, j, device=DEV) for j in range(ns)]
    sigma, hist = skv.calibrate_sequences(csh, seqs, device=DEV)
    torch.cuda.synchronize()
    # calibration parity on the same sequences
    cal = R.Calibrator(R.make_shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode))
    for cx, cm in seqs:
        cal.accumulate(np_sym(cx, w.sym_fmt), np_mu(cm, w.mu_fmt), nthreads=16)
    rsigma, rhist = cal.finalize()
    np.testing.assert_array_equal(sigma.cpu().numpy(), rsigma)
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint64), rhist)
    del seqs

    x, mu = synth.generate(w, device=DEV)
    sh = skv.shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    buf = skv.Buffers(sh, device=DEV)
    buf.encode(x, mu, sigma, hist)
    out = torch.empty_like(x)
    buf.decode(mu, sigma, hist, out)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.OK, skv.status_string(int(buf.status.item()))
    assert torch.equal(out, x), "decode(encode(x)) != x"
    offs = buf.offsets.cpu().numpy().view(np.uint64)
    assert offs[0] == 0 and np.all(np.diff(offs.astype(np.int64)) >= 128)
    bits_per_scalar = 8.0 * (offs[-1] + 8 * len(offs)) / w.n_scalars
    print(f"[fullsize] {name}: {offs[-1]} bytes, {bits_per_scalar:.4f} bits/scalar", flush=True)

    # sampled chunks against the oracle, one by one
    model = R.Model(w.sym_fmt, rhist)
    rsh = R.make_shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    per_ch = R.OCT_STRIDE if w.sigma_mode == R.SIGMA_OCTAVE else 1
    nc = len(offs) - 1
    ntb = (w.tokens + 255) // 256
    rng = np.random.default_rng(sum(map(ord, name)))
    picks = sorted(set([0, nc - 1, ntb - 1] + rng.integers(0, nc, 40).tolist()))
    xr = x.view(-1, w.tokens, w.head_dim)
    mr = mu.view(-1, w.tokens, w.head_dim)
    for c in picks:
        row, blk = divmod(c, ntb)
        t0 = blk * 256
        t1 = min(w.tokens, t0 + 256)
        xc = np_sym(xr[row, t0:t1], w.sym_fmt).ravel()
        mc = np_mu(mr[row, t0:t1], w.mu_fmt).ravel()
        sc = np.ascontiguousarray(rsigma[row * w.head_dim * per_ch:(row + 1) * w.head_dim * per_ch])
        want = model.encode_chunk(rsh, c, xc, mc, sc)
        got = buf.bits[int(offs[c]):int(offs[c + 1])].cpu().numpy()
        assert np.array_equal(got, want), f"chunk {c} differs from the oracle"
        dec = np.zeros_like(xc)
        assert model.decode_chunk(rsh, c, got, mc, sc, dec) == R.OK and np.array_equal(dec, xc)
    del x, mu, out, buf
    torch.cuda.empty_cache()
