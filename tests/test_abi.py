"""The C-ABI library loads and exports what include/skv.h declares (no GPU needed);
its host-side size queries agree with the oracle's."""
import os
import re

import pytest

from lossless_kv_cache_scalar_amd import build as B
from lossless_kv_cache_scalar_amd import skv
from oracle import skvref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not B.is_built():
        B.build()
    return skv.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "skv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(skv_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(skv.EXPORTS)


def test_status_strings(lib):
    for code in range(8):
        assert skv.status_string(code)
    assert skv.status_string(99) == "unknown status"


@pytest.mark.parametrize("dims", [(1, 2, 256, 64), (28, 8, 2048, 128), (2, 3, 300, 8), (1, 1, 1, 512), (64, 8, 32768, 128)])
@pytest.mark.parametrize("fmt", [(0, 0), (1, 1), (1, 0)])
def test_sizes_match_oracle(lib, dims, fmt):
    sh = skv.shape(*dims, *fmt)
    rs = R.make_shape(*dims, *fmt)
    assert skv.num_chunks(sh) == R.num_chunks(rs)
    assert skv.encode_bound(sh) == R.encode_bound(rs)
    assert skv.workspace_size(sh) > 0
    nch = dims[0] * 2 * dims[1] * dims[3]
    assert skv.calib_state_size(sh) == 16 * nch + 8 * (65536 if fmt[0] == 0 else 256)


@pytest.mark.parametrize("bad,code", [((0, 1, 1, 64), skv.ERR_ARG), ((1, 1, 1, 96), skv.ERR_UNSUPPORTED),
                                      ((1, 1, 1, 12), skv.ERR_UNSUPPORTED), ((1, 0, 1, 64), skv.ERR_ARG)])
def test_bad_shapes_rejected(lib, bad, code):
    import ctypes as C
    n = C.c_int64(0)
    assert lib.skv_num_chunks(C.byref(skv.shape(*bad)), C.byref(n)) == code
    assert lib.skv_encode(C.byref(skv.shape(*bad)), *([None] * 5), 0, None, None, 0, None, None) == code


def test_sigma_mode_checks_and_sizes(lib):
    """The sigma and p_hat modes are validated (adaptive p_hat needs e4m3
    symbols, as in the oracle); octave mode adds 256 fp64/u64 bin pairs per
    channel to the calibration state and a scale per channel and octave to the
    workspace; the chunking is unchanged."""
    import ctypes as C
    n = C.c_int64(0)
    bad = skv.shape(1, 1, 256, 64, 0, 0, 2)
    assert lib.skv_num_chunks(C.byref(bad), C.byref(n)) == skv.ERR_ARG
    bad = skv.shape(1, 1, 256, 64)
    bad.phat_mode = 2
    assert lib.skv_num_chunks(C.byref(bad), C.byref(n)) == skv.ERR_ARG
    assert lib.skv_num_chunks(C.byref(skv.shape(1, 1, 256, 64, 0, 0, 0, 1)), C.byref(n)) == skv.ERR_UNSUPPORTED
    assert lib.skv_num_chunks(C.byref(skv.shape(1, 1, 256, 64, 1, 0, 0, 1)), C.byref(n)) == skv.OK
    assert R.num_chunks(R.make_shape(1, 1, 256, 64, 0, 0, 0, 1)) == -1  # the oracle refuses it too
    ch, oc = skv.shape(2, 4, 300, 128), skv.shape(2, 4, 300, 128, 0, 0, skv.SIGMA_OCTAVE)
    nch = 2 * 2 * 4 * 128
    assert skv.num_chunks(oc) == skv.num_chunks(ch) and skv.encode_bound(oc) == skv.encode_bound(ch)
    assert skv.calib_state_size(oc) == skv.calib_state_size(ch) + 16 * 256 * nch
    assert skv.workspace_size(oc) >= skv.workspace_size(ch) + 8 * 7 * nch
    assert skv.sigma_floats(oc) == 9 * nch and skv.sigma_floats(ch) == nch
    assert R.num_chunks(R.make_shape(2, 4, 300, 128, 0, 0, R.SIGMA_OCTAVE)) == skv.num_chunks(oc)


def test_null_pointers_rejected(lib):
    sh = skv.shape(1, 2, 256, 64)
    assert skv.encode(sh, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, stream=0) == skv.ERR_ARG
    assert skv.decode(sh, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, stream=0) == skv.ERR_ARG


def test_timing_argument_checks(lib):
    import ctypes as C
    n = C.c_int32(-1)
    assert lib.skv_timing_start(0) == skv.ERR_ARG
    assert lib.skv_timing_start((1 << 20) + 1) == skv.ERR_ARG
    assert lib.skv_timing_stop(None, None, 0, C.byref(n)) == skv.ERR_ARG  # not recording
    assert lib.skv_timing_stop(None, None, 4, C.byref(n)) == skv.ERR_ARG
    names = [skv.load().skv_timed_kernel_name(i).decode() for i in range(4)]
    assert names == ["model", "k_encode", "k_decode", "unknown"]


def test_decode_static_host_checks(lib):
    """skv_decode_static validates on the host before touching a device: null
    pointers, and a shape whose decode workspace exceeds the static scratch."""
    import ctypes as C
    p = C.c_void_p(4096)  # never dereferenced: the calls below return before any launch
    small = skv.shape(1, 1, 256, 64)
    assert lib.skv_decode_static(C.byref(small), None, 0, p, p, p, p, p, p, None) == skv.ERR_ARG
    huge = skv.shape(2048, 8, 256, 512, 0, 0, skv.SIGMA_OCTAVE)  # 16.8 million channels
    assert lib.skv_decode_static(C.byref(huge), p, 4096, p, p, p, p, p, p, None) == skv.ERR_SCRATCH
    assert skv.status_string(skv.ERR_SCRATCH).startswith("shape needs more")


def test_workspace_does_not_grow_with_the_cache(lib):
    """The encoder's scratch is two slots per wave of its grid (at most one
    16-wave block per compute unit), so past a few thousand chunks the
    workspace grows only by the 8-byte published size of each chunk: under
    1 GB for the 32K-token Qwen3-32B e4m3 cache (4.3e9 scalars)."""
    a = skv.workspace_size(skv.shape(64, 8, 8192, 128, 1, 0))
    b = skv.workspace_size(skv.shape(64, 8, 32768, 128, 1, 0))
    assert b < 1 << 30
    assert b - a <= 8 * (131072 - 32768) + 4096


def test_short_arrays_are_refused_before_any_call(lib):
    """The binding checks each tensor argument against the shape (the library
    reads whole arrays through raw pointers), and so does the oracle's numpy
    wrapper: a sigma array for one kv head, given a shape with two, is refused
    on both sides instead of read past its end."""
    import numpy as np
    import torch
    sh = skv.shape(1, 2, 300, 128)
    n = 2 * 2 * 300 * 128
    x = torch.zeros(n, dtype=torch.int16)
    mu = torch.zeros(n, dtype=torch.int16)
    hist = torch.zeros(65536, dtype=torch.int64)
    short = torch.zeros(2 * 128)
    with pytest.raises(skv.SkvError, match="sigma"):
        skv.encode(sh, x, mu, short, hist, 0, 0, 0, 0, 0, 0)
    with pytest.raises(skv.SkvError, match="sigma"):
        skv.decode(sh, 0, 0, 0, mu, short, hist, x, 0, 0, 0)
    with pytest.raises(skv.SkvError, match="x_out"):
        skv.decode_static(sh, 0, 0, 0, mu, torch.zeros(4 * 128), hist, x[: n // 2], 0)
    with pytest.raises(skv.SkvError, match="mu"):
        skv.encode(sh, x, mu[:-1], torch.zeros(4 * 128), hist, 0, 0, 0, 0, 0, 0)
    with pytest.raises(skv.SkvError, match="contiguous"):
        skv.encode(sh, x.view(2, -1).t(), mu, torch.zeros(4 * 128), hist, 0, 0, 0, 0, 0, 0)
    rsh = R.make_shape(1, 2, 300, 128)
    xn = np.zeros(n, dtype=np.uint16)
    with pytest.raises(ValueError, match="sigma"):
        R.Model(0, np.ones(65536, dtype=np.uint64)).encode(rsh, xn, xn, np.zeros(2 * 128, dtype=np.float32))
