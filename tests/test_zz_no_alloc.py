"""skv_decode_static (no allocation, the workspace in the library's static
device array) against skv_decode through the C ABI: identical decoded caches
and status words on two calls in a row, the second with a smaller input, and
on a corrupt stream."""
import numpy as np
import pytest
import torch

from lossless_kv_cache_scalar_amd import skv, synth

from gpu_util import DEV, ensure_built, oracle_calibrate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _encoded(w):
    rsigma, rhist = oracle_calibrate(w, [synth.calibration_set(w, 0)])
    x, mu = synth.generate(w)
    sh = skv.shape(w.layers, w.kv_heads, w.tokens, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode)
    sigma = torch.from_numpy(rsigma).to(DEV)
    hist = torch.from_numpy(rhist.view(np.int64)).to(DEV)
    buf = skv.Buffers(sh, device=DEV)
    x, mu = x.to(DEV), mu.to(DEV)
    buf.encode(x, mu, sigma, hist)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == skv.OK
    return sh, buf, x, mu, sigma, hist


def _both(sh, buf, mu, sigma, hist, x_like, bits=None):
    bits = buf.bits if bits is None else bits
    ref = torch.full_like(x_like, 0x55 if x_like.dtype == torch.uint8 else 0x5555)
    got = torch.full_like(ref, 0x33)
    buf.decode(mu, sigma, hist, ref, bits=bits)
    st_static = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    rc = skv.decode_static(sh, bits, bits.numel(), buf.offsets, mu, sigma, hist, got, st_static)
    assert rc == skv.OK, skv.status_string(rc)
    torch.cuda.synchronize()
    return ref, got, int(buf.status.item()), int(st_static.item())


@pytest.mark.parametrize("first,second", [("qwen3_32b_bf16", "tiny_bf16"), ("qwen3_0.6b_e4m3", "qwen3_32b_e4m3_32k")])
def test_static_decode_equals_decode_twice(first, second):
    big = synth.WORKLOADS[first].with_tokens(600, layers=2)
    small = synth.WORKLOADS[second]
    small = small if small.name == "tiny_bf16" else small.with_tokens(300, layers=1)
    assert small.n_scalars < big.n_scalars
    for w in (big, small):
        sh, buf, x, mu, sigma, hist = _encoded(w)
        ref, got, st_ref, st_got = _both(sh, buf, mu, sigma, hist, x)
        assert st_ref == skv.OK and st_got == skv.OK
        assert torch.equal(ref, x) and torch.equal(got, ref)


def test_static_decode_octave_and_corrupt():
    w = synth.WORKLOADS["qwen3_32b_bf16_fp8res_oct"].with_tokens(300, layers=1)
    sh, buf, x, mu, sigma, hist = _encoded(w)
    ref, got, st_ref, st_got = _both(sh, buf, mu, sigma, hist, x)
    assert st_ref == st_got == skv.OK and torch.equal(got, x)
    bad = buf.bits.clone()
    bad[0] ^= 1  # the first chunk's header no longer adds up
    ref, got, st_ref, st_got = _both(sh, buf, mu, sigma, hist, x, bits=bad)
    assert st_ref == st_got == skv.ERR_CORRUPT
