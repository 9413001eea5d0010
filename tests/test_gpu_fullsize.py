"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times: the whole GPU stream (every byte and every offset) equals the oracle's
encoding of the whole cache, decode(encode(x)) == x over the whole cache,
sampled chunks of the GPU stream decode back to x in the oracle, and
calibration equals the oracle's on the same sequences.  Encode and decode
statuses are each checked after their own call."""
import time

import numpy as np
import pytest
import torch

from lossless_kv_cache_scalar_amd import skv, synth
from oracle import skvref as R

from gpu_util import DEV, ensure_built, np_mu, np_sym

pytestmark = pytest.mark.gpu

NAMES = ["tiny_bf16", "qwen3_0.6b_bf16", "qwen3_0.6b_e4m3", "qwen3_32b_bf16", "qwen3_32b_e4m3_32k", "qwen3_32b_bf16_fp8res",
         "qwen3_32b_bf16_fp8res_oct", "qwen3_0.6b_e4m3_drift", "qwen3_0.6b_e4m3_drift_adapt", "qwen3_32b_e4m3_32k_adapt"]
CALIB_SEQS = 2  # the launch configuration does not depend on the calibration set's size
ORACLE_THREADS = 16  # the host's CPU share on a one-GPU machine


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


@pytest.mark.parametrize("name", NAMES)
def test_full_size_whole_stream_equals_oracle(name):
    w = synth.WORKLOADS[name]
    print(f"[fullsize] {name}: {w.n_scalars} scalars", flush=True)
    ns = min(CALIB_SEQS, w.calib_seqs)
    csh = skv.shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    seqs = [synth.calibration_set(w, j, device=DEV) for j in range(ns)]
    sigma, hist = skv.calibrate_sequences(csh, seqs, device=DEV)
    torch.cuda.synchronize()
    cal = R.Calibrator(R.make_shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode))
    for cx, cm in seqs:
        cal.accumulate(np_sym(cx, w.sym_fmt), np_mu(cm, w.mu_fmt), nthreads=ORACLE_THREADS)
    rsigma, rhist = cal.finalize()
    np.testing.assert_array_equal(sigma.cpu().numpy(), rsigma)
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint64), rhist)
    del seqs

    x, mu = synth.generate(w, device=DEV)
    sh = skv.shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode)
    buf = skv.Buffers(sh, device=DEV)
    buf.encode(x, mu, sigma, hist)
    torch.cuda.synchronize()
    st = int(buf.status.item())
    assert st == skv.OK, "encode: " + skv.status_string(st)
    out = torch.empty_like(x)
    buf.decode(mu, sigma, hist, out)
    torch.cuda.synchronize()
    st = int(buf.status.item())
    assert st == skv.OK, "decode: " + skv.status_string(st)
    assert torch.equal(out, x), "decode(encode(x)) != x"
    del out
    offs = buf.offsets.cpu().numpy().view(np.uint64)
    gbits = buf.bits[: int(offs[-1])].cpu().numpy()
    print(f"[fullsize] {name}: {offs[-1]} bytes, {8.0 * (offs[-1] + 8 * len(offs)) / w.n_scalars:.4f} bits/scalar",
          flush=True)

    # the whole cache through the oracle (chunk-parallel over host threads)
    xn, mn = np_sym(x, w.sym_fmt), np_mu(mu, w.mu_fmt)
    del x, mu, buf
    torch.cuda.empty_cache()
    model = R.Model(w.sym_fmt, rhist)
    rsh = R.make_shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode)
    t0 = time.perf_counter()
    rbits, roffs = model.encode(rsh, xn, mn, rsigma, nthreads=ORACLE_THREADS)
    print(f"[fullsize] {name}: oracle encode of the whole cache {time.perf_counter() - t0:.1f}s", flush=True)
    assert np.array_equal(offs, roffs), "offsets differ from the oracle"
    if not np.array_equal(gbits, rbits):
        first = int(np.argmax(gbits != rbits))
        c = int(np.searchsorted(offs, first, side="right")) - 1
        pytest.fail(f"stream bytes differ from the oracle (first difference in chunk {c})")

    # sampled chunks of the GPU stream decoded by the oracle, one by one
    per_ch = R.OCT_STRIDE if w.sigma_mode == R.SIGMA_OCTAVE else 1
    nc = len(offs) - 1
    ntb = (w.tokens + 255) // 256
    rng = np.random.default_rng(sum(map(ord, name)))
    picks = sorted(set([0, nc - 1, ntb - 1] + rng.integers(0, nc, 16).tolist()))
    xr = xn.reshape(-1, w.tokens, w.head_dim)
    mr = mn.reshape(-1, w.tokens, w.head_dim)
    for c in picks:
        row, blk = divmod(c, ntb)
        t0, t1 = blk * 256, min(w.tokens, blk * 256 + 256)
        xc = np.ascontiguousarray(xr[row, t0:t1]).ravel()
        mc = np.ascontiguousarray(mr[row, t0:t1]).ravel()
        sc = np.ascontiguousarray(rsigma[row * w.head_dim * per_ch:(row + 1) * w.head_dim * per_ch])
        dec = np.zeros_like(xc)
        got = gbits[int(offs[c]):int(offs[c + 1])]
        assert model.decode_chunk(rsh, c, got, mc, sc, dec) == R.OK and np.array_equal(dec, xc), f"chunk {c}"


def test_full_size_encode_is_deterministic():
    """Chunks go to waves in whatever order the waves reach the chunk counter,
    and offsets come from the look-back: two encodes of the 32B bf16 cache in
    the launch configuration bench.py times give the same bytes and offsets."""
    w = synth.WORKLOADS["qwen3_32b_bf16"]
    csh = skv.shape(w.layers, w.kv_heads, w.calib_tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    sigma, hist = skv.calibrate_sequences(csh, [synth.calibration_set(w, 0, device=DEV)], device=DEV)
    x, mu = synth.generate(w, device=DEV)
    sh = skv.shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode)
    a = skv.Buffers(sh, device=DEV)
    b = skv.Buffers(sh, device=DEV)
    a.encode(x, mu, sigma, hist)
    b.encode(x, mu, sigma, hist)
    torch.cuda.synchronize()
    assert int(a.status.item()) == skv.OK and int(b.status.item()) == skv.OK
    n = a.stream_bytes()
    assert n == b.stream_bytes()
    assert torch.equal(a.offsets, b.offsets) and torch.equal(a.bits[:n], b.bits[:n])
