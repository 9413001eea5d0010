"""Helpers shared by the GPU tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs."""
import numpy as np
import torch

from lossless_kv_cache_scalar_amd import build as B
from lossless_kv_cache_scalar_amd import skv, synth
from oracle import skvref as R

DEV = torch.device("cuda:0")


def ensure_built():
    if not B.is_built():
        B.build()
    skv.load()


def np_sym(t: torch.Tensor, sym_fmt: int) -> np.ndarray:
    a = t.cpu().contiguous().numpy()
    return np.ascontiguousarray(a.view(np.uint16 if sym_fmt == 0 else np.uint8))


def np_mu(t: torch.Tensor, mu_fmt: int) -> np.ndarray:
    a = t.cpu().contiguous().numpy()
    return np.ascontiguousarray(a.view(np.uint16) if mu_fmt == 0 else a)


def shapes(w: synth.Workload, tokens=None):
    t = w.tokens if tokens is None else tokens
    return (skv.shape(w.layers, w.kv_heads, t, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode),
            R.make_shape(w.layers, w.kv_heads, t, w.head_dim, w.sym_fmt, w.mu_fmt, w.sigma_mode, w.phat_mode))


def gpu_calibrate(w, seqs):
    sh, _ = shapes(w, w.calib_tokens)
    sigma, hist = skv.calibrate_sequences(sh, [(x.to(DEV), m.to(DEV)) for x, m in seqs], device=DEV)
    torch.cuda.synchronize()
    return sigma, hist


def oracle_calibrate(w, seqs):
    _, rsh = shapes(w, w.calib_tokens)
    cal = R.Calibrator(rsh)
    for x, m in seqs:
        cal.accumulate(np_sym(x, w.sym_fmt), np_mu(m, w.mu_fmt))
    return cal.finalize()


def gpu_roundtrip(sh, x, mu, sigma, hist, bits_cap=None):
    """Encode then decode on the GPU; returns (bits, offsets, decoded, enc_status, dec_status)."""
    buf = skv.Buffers(sh, device=DEV)
    cap = buf.bits.numel() if bits_cap is None else bits_cap
    rc = skv.encode(sh, x, mu, sigma, hist, buf.bits, cap, buf.offsets, buf.workspace, buf.ws_bytes, buf.status)
    assert rc == skv.OK, skv.status_string(rc)
    torch.cuda.synchronize()
    enc_status = int(buf.status.item())
    out = torch.full_like(x, 0x55 if x.dtype == torch.uint8 else 0x5555)
    rc = skv.decode(sh, buf.bits, buf.bits.numel(), buf.offsets, mu, sigma, hist, out, buf.workspace, buf.ws_bytes, buf.status)
    assert rc == skv.OK, skv.status_string(rc)
    torch.cuda.synchronize()
    dec_status = int(buf.status.item())
    offs = buf.offsets.cpu().numpy().view(np.uint64).copy()
    bits = buf.bits[: int(min(offs[-1], cap))].cpu().numpy().copy()
    return bits, offs, out, enc_status, dec_status
