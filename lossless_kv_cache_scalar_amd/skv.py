"""Python binding of libskv (include/skv.h): argument marshalling only.

Every step of the coding path runs in the library's HIP kernels; this module
turns torch tensors into device pointers and the current torch stream into a
hipStream_t.  There is no fallback: if the library is not built, importing the
entry points raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libskv.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_CAPACITY, ERR_CORRUPT, ERR_TABLE, ERR_SCRATCH = range(8)
STATIC_SCRATCH_BYTES = 16 << 20  # SKV_STATIC_SCRATCH_BYTES
SYM_BF16, SYM_E4M3 = 0, 1
MU_BF16, MU_F32 = 0, 1
SIGMA_CHANNEL, SIGMA_OCTAVE = 0, 1
PHAT_STATIC, PHAT_ADAPTIVE = 0, 1
OCTAVES = 8
OCT_STRIDE = 1 + OCTAVES

# every function skv.h declares, in declaration order
EXPORTS = ["skv_status_string", "skv_num_chunks", "skv_encode_bound", "skv_workspace_size",
           "skv_calib_state_size", "skv_calib_reset", "skv_calib_accumulate", "skv_calib_finalize",
           "skv_calibrate", "skv_encode", "skv_decode", "skv_decode_static", "skv_timing_start", "skv_timing_stop",
           "skv_timed_kernel_name"]


class SkvShape(C.Structure):
    _fields_ = [("layers", C.c_int64), ("kv_heads", C.c_int64), ("tokens", C.c_int64),
                ("head_dim", C.c_int64), ("sym_fmt", C.c_int32), ("mu_fmt", C.c_int32),
                ("sigma_mode", C.c_int32), ("phat_mode", C.c_int32)]


class SkvError(RuntimeError):
    pass


_lib = None


def load():
    """Load libskv.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SkvError(f"libskv is not built ({LIB_PATH} missing); run python -m lossless_kv_cache_scalar_amd.build")
    L = C.CDLL(LIB_PATH)
    vp, i64, sz, i32p = C.c_void_p, C.c_int64, C.c_size_t, C.c_void_p
    sp = C.POINTER(SkvShape)
    L.skv_status_string.restype = C.c_char_p
    L.skv_status_string.argtypes = [C.c_int]
    for name in ("skv_num_chunks",):
        getattr(L, name).argtypes = [sp, C.POINTER(C.c_int64)]
    for name in ("skv_encode_bound", "skv_workspace_size", "skv_calib_state_size"):
        getattr(L, name).argtypes = [sp, C.POINTER(C.c_size_t)]
    L.skv_calib_reset.argtypes = [vp, sp, vp]
    L.skv_calib_accumulate.argtypes = [vp, sp, vp, vp, vp]
    L.skv_calib_finalize.argtypes = [vp, sp, vp, vp, vp]
    L.skv_calibrate.argtypes = [sp, i64, vp, vp, vp, vp, vp, vp]
    L.skv_encode.argtypes = [sp, vp, vp, vp, vp, vp, sz, vp, vp, sz, i32p, vp]
    L.skv_decode.argtypes = [sp, vp, sz, vp, vp, vp, vp, vp, vp, sz, i32p, vp]
    L.skv_decode_static.argtypes = [sp, vp, sz, vp, vp, vp, vp, vp, i32p, vp]
    L.skv_timing_start.argtypes = [C.c_int32]
    L.skv_timing_stop.argtypes = [C.POINTER(C.c_int32), C.POINTER(C.c_float), C.c_int32, C.POINTER(C.c_int32)]
    L.skv_timed_kernel_name.argtypes = [C.c_int32]
    for name in EXPORTS[1:]:
        getattr(L, name).restype = C.c_int
    L.skv_timed_kernel_name.restype = C.c_char_p
    _lib = L
    return L


def shape(layers, kv_heads, tokens, head_dim, sym_fmt=SYM_BF16, mu_fmt=MU_BF16, sigma_mode=SIGMA_CHANNEL,
          phat_mode=PHAT_STATIC) -> SkvShape:
    return SkvShape(int(layers), int(kv_heads), int(tokens), int(head_dim), int(sym_fmt), int(mu_fmt),
                    int(sigma_mode), int(phat_mode))


def sigma_floats(sh: SkvShape) -> int:
    """Length of the sigma array for a shape: one per channel, or OCT_STRIDE per channel in octave mode."""
    nch = sh.layers * 2 * sh.kv_heads * sh.head_dim
    return nch * (OCT_STRIDE if sh.sigma_mode == SIGMA_OCTAVE else 1)


def status_string(code: int) -> str:
    return load().skv_status_string(int(code)).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise SkvError(f"{what}: {status_string(rc)} ({rc})")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _fits(t, nbytes: int, what: str):
    """A tensor argument must be contiguous and hold at least nbytes (the
    library reads and writes whole arrays through raw pointers); integer
    addresses pass unchecked, as in C."""
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise SkvError(f"{what}: not contiguous")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise SkvError(f"{what}: {have} bytes, the shape needs {nbytes}")


def _offsets(sh: SkvShape, offsets):
    """offsets holds n_chunks + 1 entries (an invalid shape is left to the
    library, which returns its status code)."""
    n = C.c_int64(0)
    if load().skv_num_chunks(C.byref(sh), C.byref(n)) == OK:
        _fits(offsets, 8 * (n.value + 1), "offsets")


def _state(sh: SkvShape, state):
    n = C.c_size_t(0)
    if load().skv_calib_state_size(C.byref(sh), C.byref(n)) == OK:
        _fits(state, n.value, "state")


def _n_scalars(sh: SkvShape) -> int:
    return sh.layers * 2 * sh.kv_heads * sh.tokens * sh.head_dim


def _model_args(sh: SkvShape, mu, sigma, hist):
    n = _n_scalars(sh)
    _fits(mu, n * (2 if sh.mu_fmt == MU_BF16 else 4), "mu")
    _fits(sigma, 4 * sigma_floats(sh), "sigma")
    _fits(hist, 8 * (65536 if sh.sym_fmt == SYM_BF16 else 256), "hist")


def _symbols(sh: SkvShape, x, what: str):
    _fits(x, _n_scalars(sh) * (2 if sh.sym_fmt == SYM_BF16 else 1), what)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def num_chunks(sh: SkvShape) -> int:
    n = C.c_int64(0)
    _check(load().skv_num_chunks(C.byref(sh), C.byref(n)), "skv_num_chunks")
    return n.value


def _size(fn, sh):
    n = C.c_size_t(0)
    _check(getattr(load(), fn)(C.byref(sh), C.byref(n)), fn)
    return n.value


def encode_bound(sh: SkvShape) -> int:
    return _size("skv_encode_bound", sh)


def workspace_size(sh: SkvShape) -> int:
    return _size("skv_workspace_size", sh)


def calib_state_size(sh: SkvShape) -> int:
    return _size("skv_calib_state_size", sh)


# ---- raw entry points: same names and arguments as skv.h ----
def calib_reset(state, sh: SkvShape, stream=None) -> int:
    _state(sh, state)
    return load().skv_calib_reset(_ptr(state), C.byref(sh), _stream(stream))


def calib_accumulate(state, seq_shape: SkvShape, x, mu, stream=None) -> int:
    _state(seq_shape, state)
    _symbols(seq_shape, x, "x")
    _fits(mu, _n_scalars(seq_shape) * (2 if seq_shape.mu_fmt == MU_BF16 else 4), "mu")
    return load().skv_calib_accumulate(_ptr(state), C.byref(seq_shape), _ptr(x), _ptr(mu), _stream(stream))


def calib_finalize(state, sh: SkvShape, sigma, hist, stream=None) -> int:
    _state(sh, state)
    _fits(sigma, 4 * sigma_floats(sh), "sigma")
    _fits(hist, 8 * (65536 if sh.sym_fmt == SYM_BF16 else 256), "hist")
    return load().skv_calib_finalize(_ptr(state), C.byref(sh), _ptr(sigma), _ptr(hist), _stream(stream))


def calibrate(seq_shape: SkvShape, n_seq: int, x, mu, sigma, hist, state, stream=None) -> int:
    n = _n_scalars(seq_shape) * max(int(n_seq), 0)
    _fits(x, n * (2 if seq_shape.sym_fmt == SYM_BF16 else 1), "x")
    _fits(mu, n * (2 if seq_shape.mu_fmt == MU_BF16 else 4), "mu")
    _fits(sigma, 4 * sigma_floats(seq_shape), "sigma")
    _fits(hist, 8 * (65536 if seq_shape.sym_fmt == SYM_BF16 else 256), "hist")
    _state(seq_shape, state)
    return load().skv_calibrate(C.byref(seq_shape), int(n_seq), _ptr(x), _ptr(mu), _ptr(sigma), _ptr(hist),
                                _ptr(state), _stream(stream))


def encode(sh: SkvShape, x, mu, sigma, hist, bits, bits_cap: int, offsets, workspace, workspace_bytes: int,
           status, stream=None) -> int:
    _symbols(sh, x, "x")
    _model_args(sh, mu, sigma, hist)
    _fits(bits, int(bits_cap), "bits")
    _offsets(sh, offsets)
    _fits(workspace, int(workspace_bytes), "workspace")
    _fits(status, 4, "status")
    return load().skv_encode(C.byref(sh), _ptr(x), _ptr(mu), _ptr(sigma), _ptr(hist), _ptr(bits), int(bits_cap),
                             _ptr(offsets), _ptr(workspace), int(workspace_bytes), _ptr(status), _stream(stream))


def decode(sh: SkvShape, bits, bits_bytes: int, offsets, mu, sigma, hist, x_out, workspace, workspace_bytes: int,
           status, stream=None) -> int:
    _fits(bits, int(bits_bytes), "bits")
    _offsets(sh, offsets)
    _model_args(sh, mu, sigma, hist)
    _symbols(sh, x_out, "x_out")
    _fits(workspace, int(workspace_bytes), "workspace")
    _fits(status, 4, "status")
    return load().skv_decode(C.byref(sh), _ptr(bits), int(bits_bytes), _ptr(offsets), _ptr(mu), _ptr(sigma), _ptr(hist), _ptr(x_out),
                             _ptr(workspace), int(workspace_bytes), _ptr(status), _stream(stream))


def decode_static(sh: SkvShape, bits, bits_bytes: int, offsets, mu, sigma, hist, x_out, status, stream=None) -> int:
    _fits(bits, int(bits_bytes), "bits")
    _offsets(sh, offsets)
    _model_args(sh, mu, sigma, hist)
    _symbols(sh, x_out, "x_out")
    _fits(status, 4, "status")
    return load().skv_decode_static(C.byref(sh), _ptr(bits), int(bits_bytes), _ptr(offsets), _ptr(mu), _ptr(sigma),
                                    _ptr(hist), _ptr(x_out), _ptr(status), _stream(stream))


# ---- buffers sized for a shape (torch allocates, the library fills) ----
class Buffers:
    """Device buffers for one cache shape: workspace, stream, offsets, status."""

    def __init__(self, sh: SkvShape, device="cuda"):
        self.shape = sh
        self.n_chunks = num_chunks(sh)
        self.bound = encode_bound(sh)
        self.ws_bytes = workspace_size(sh)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.bits = torch.empty((self.bound + 15) // 16 * 16, dtype=torch.uint8, device=device)
        self.offsets = torch.empty(self.n_chunks + 1, dtype=torch.int64, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def encode(self, x, mu, sigma, hist, stream=None, status=None) -> None:
        """skv_encode into this object's stream; the status word is self.status unless given."""
        _check(encode(self.shape, x, mu, sigma, hist, self.bits, self.bits.numel(), self.offsets, self.workspace,
                      self.ws_bytes, self.status if status is None else status, stream), "skv_encode")

    def decode(self, mu, sigma, hist, x_out, bits=None, offsets=None, stream=None, status=None) -> None:
        """skv_decode of this object's stream (or the given one); the status word is self.status unless given."""
        bits = self.bits if bits is None else bits
        offsets = self.offsets if offsets is None else offsets
        _check(decode(self.shape, bits, bits.numel(), offsets, mu, sigma, hist, x_out, self.workspace,
                      self.ws_bytes, self.status if status is None else status, stream), "skv_decode")

    def stream_bytes(self) -> int:
        return int(self.offsets[-1].item())


def timing_start(capacity: int) -> None:
    """Start recording per-kernel HIP-event timings of the library's launches."""
    _check(load().skv_timing_start(int(capacity)), "skv_timing_start")


def timing_stop(capacity: int = 1 << 16):
    """Stop recording; [(kernel name, ms), ...] in launch order."""
    L = load()
    ids = (C.c_int32 * capacity)()
    ms = (C.c_float * capacity)()
    n = C.c_int32(0)
    _check(L.skv_timing_stop(ids, ms, int(capacity), C.byref(n)), "skv_timing_stop")
    return [(L.skv_timed_kernel_name(ids[i]).decode(), float(ms[i])) for i in range(min(n.value, capacity))]


def calibrate_sequences(seq_shape: SkvShape, seqs, device="cuda", stream=None):
    """sigma and hist from an iterable of (x, mu) device tensors, each of seq_shape."""
    nsym = 65536 if seq_shape.sym_fmt == SYM_BF16 else 256
    state = torch.empty(calib_state_size(seq_shape), dtype=torch.uint8, device=device)
    sigma = torch.empty(sigma_floats(seq_shape), dtype=torch.float32, device=device)
    hist = torch.empty(nsym, dtype=torch.int64, device=device)
    _check(calib_reset(state, seq_shape, stream), "skv_calib_reset")
    for x, mu in seqs:
        _check(calib_accumulate(state, seq_shape, x, mu, stream), "skv_calib_accumulate")
    _check(calib_finalize(state, seq_shape, sigma, hist, stream), "skv_calib_finalize")
    return sigma, hist
