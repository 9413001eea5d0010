"""ctypes wrapper around the CPU oracle (oracle/skvref.c).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product package
never does.  Everything here is argument marshalling; the arithmetic is in the
C file, which cites the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "skvref.c")
LIB = os.path.join(HERE, "libskvref.so")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_CORRUPT, ERR_TABLE = 0, 1, 2, 4, 5, 6
SYM_BF16, SYM_E4M3 = 0, 1
MU_BF16, MU_F32 = 0, 1
SIGMA_CHANNEL, SIGMA_OCTAVE = 0, 1
PHAT_STATIC, PHAT_ADAPTIVE = 0, 1
OCTAVES = 8
OCT_STRIDE = 1 + OCTAVES  # octave-mode sigma table per channel: [sigma_c, sigma_c,0 .. sigma_c,7]
EXP_BINS = 256


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math, IEEE denormals)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", LIB + ".tmp", SRC, "-lm", "-lpthread"]
        subprocess.check_call(cmd)
        os.replace(LIB + ".tmp", LIB)
    return LIB


class Shape(C.Structure):
    _fields_ = [("layers", C.c_int64), ("kv_heads", C.c_int64), ("tokens", C.c_int64),
                ("head_dim", C.c_int64), ("sym_fmt", C.c_int32), ("mu_fmt", C.c_int32),
                ("sigma_mode", C.c_int32), ("phat_mode", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        vp, i64, u64, f32p = C.c_void_p, C.c_int64, C.c_uint64, C.c_void_p
        L.skvref_model_new.restype = vp
        L.skvref_model_new.argtypes = [C.c_int, vp, C.c_double, C.c_double, i64, i64, C.POINTER(C.c_int)]
        L.skvref_model_free.argtypes = [vp]
        L.skvref_model_info.argtypes = [vp, vp]
        L.skvref_model_knots.argtypes = [vp, vp, vp]
        L.skvref_model_ptable.argtypes = [vp, vp]
        L.skvref_cg_many.argtypes = [vp, vp, vp, i64]
        L.skvref_cum_pair_many.argtypes = [vp, vp, vp, vp, vp, vp, i64]
        L.skvref_cum_table.argtypes = [vp, C.c_float, C.c_float, vp]
        L.skvref_bin_many.argtypes = [C.c_int, vp, vp, vp, i64]
        L.skvref_scale_many.argtypes = [vp, vp, i64]
        L.skvref_rank.restype = C.c_uint32
        L.skvref_rank.argtypes = [C.c_int, C.c_uint32]
        L.skvref_unrank.restype = C.c_uint32
        L.skvref_unrank.argtypes = [C.c_int, C.c_uint32]
        L.skvref_value.restype = C.c_double
        L.skvref_value.argtypes = [C.c_int, C.c_uint32]
        L.skvref_num_chunks.restype = i64
        L.skvref_num_chunks.argtypes = [vp]
        L.skvref_encode_bound.restype = u64
        L.skvref_encode_bound.argtypes = [vp]
        L.skvref_encode_m.argtypes = [vp, vp, vp, vp, vp, vp, u64, vp, C.c_int]
        L.skvref_decode_m.argtypes = [vp, vp, vp, vp, vp, vp, vp, C.c_int]
        L.skvref_encode_chunk.restype = u64
        L.skvref_encode_chunk.argtypes = [vp, vp, i64, vp, vp, vp, vp, u64, C.POINTER(C.c_int)]
        L.skvref_decode_chunk.argtypes = [vp, vp, i64, vp, u64, vp, vp, vp]
        L.skvref_calib_accumulate.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, C.c_int]
        L.skvref_calib_finalize.argtypes = [i64, vp, vp, vp]
        L.skvref_calib_finalize_octave.argtypes = [i64, vp, vp, vp, vp, vp]
        L.skvref_adapt_tables.restype = i64
        L.skvref_adapt_tables.argtypes = [vp, vp, vp, i64, vp, i64]
        L.skvref_adapt_params.argtypes = [vp]
        L.skvref_rc_encode_seq.restype = u64
        L.skvref_rc_encode_seq.argtypes = [vp, vp, i64, vp, u64]
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _sizes(shape: Shape, x, mu, sigma):
    """The C code reads whole arrays through raw pointers: refuse short ones."""
    n = shape.layers * 2 * shape.kv_heads * shape.tokens * shape.head_dim
    nsig = shape.layers * 2 * shape.kv_heads * shape.head_dim * (OCT_STRIDE if shape.sigma_mode == SIGMA_OCTAVE else 1)
    for name, a, need in (("x", x, n), ("mu", mu, n), ("sigma", sigma, nsig)):
        if a is not None and np.asarray(a).size < need:
            raise ValueError(f"{name}: {np.asarray(a).size} elements, the shape needs {need}")


def make_shape(layers, kv_heads, tokens, head_dim, sym_fmt=SYM_BF16, mu_fmt=MU_BF16,
               sigma_mode=SIGMA_CHANNEL, phat_mode=PHAT_STATIC) -> Shape:
    return Shape(layers, kv_heads, tokens, head_dim, sym_fmt, mu_fmt, sigma_mode, phat_mode)


def adapt_params():
    """(epoch scalars, prior weight, observation shift, decay shift) of the adaptive p_hat."""
    out = np.zeros(4, dtype=np.int32)
    lib().skvref_adapt_params(_p(out))
    return tuple(int(v) for v in out)


class Model:
    """The integer frequency model for one symbol format.

    ``w_narrow``/``w_wide``/``MG``/``Mp`` are test hooks; the defaults are the
    pages' mixture (0.95, 0.03; p_hat gets the remaining 0.02).
    """

    def __init__(self, fmt: int, hist=None, w_narrow=0.95, w_wide=0.03, MG=-1, Mp=-1):
        L = lib()
        err = C.c_int(0)
        self._hist = None if hist is None else np.ascontiguousarray(hist, dtype=np.uint64)
        hp = None if self._hist is None else _p(self._hist)
        self.ptr = L.skvref_model_new(fmt, hp, w_narrow, w_wide, MG, Mp, C.byref(err))
        if not self.ptr:
            raise ValueError(f"oracle model construction failed (status {err.value})")
        info = np.zeros(5, dtype=np.uint32)
        L.skvref_model_info(self.ptr, _p(info))
        self.fmt = fmt
        self.N, self.T, self.log2T, self.MG, self.Mp = (int(v) for v in info)

    def __del__(self):
        ptr, self.ptr = getattr(self, "ptr", None), None
        if ptr and _lib is not None:
            try:
                _lib.skvref_model_free(ptr)
            except Exception:  # interpreter shutdown
                pass

    def knots(self):
        K = np.zeros(2049, dtype=np.float32)
        D = np.zeros(2049, dtype=np.float32)
        lib().skvref_model_knots(self.ptr, _p(K), _p(D))
        return K, D

    def ptable(self):
        A = np.zeros(self.N + 1, dtype=np.uint32)
        lib().skvref_model_ptable(self.ptr, _p(A))
        return A

    def cg(self, u):
        u = np.ascontiguousarray(u, dtype=np.float32)
        out = np.zeros(u.shape, dtype=np.uint32)
        lib().skvref_cg_many(self.ptr, _p(u), _p(out), u.size)
        return out

    def cum_pair(self, mu, s, b):
        mu = np.ascontiguousarray(mu, dtype=np.float32)
        s = np.ascontiguousarray(s, dtype=np.float32)
        b = np.ascontiguousarray(b, dtype=np.uint32)
        lo = np.zeros(b.shape, dtype=np.uint32)
        hi = np.zeros(b.shape, dtype=np.uint32)
        lib().skvref_cum_pair_many(self.ptr, _p(mu), _p(s), _p(b), _p(lo), _p(hi), b.size)
        return lo, hi

    def cum_table(self, mu: float, sigma: float):
        out = np.zeros(self.N + 1, dtype=np.uint32)
        lib().skvref_cum_table(self.ptr, float(mu), float(sigma), _p(out))
        return out

    # -- whole cache --
    def encode(self, shape: Shape, x, mu, sigma, nthreads=8, cap=None):
        _sizes(shape, x, mu, sigma)
        L = lib()
        nc = L.skvref_num_chunks(C.byref(shape))
        bound = L.skvref_encode_bound(C.byref(shape)) if cap is None else cap
        bits = np.zeros(max(int(bound), 1), dtype=np.uint8)
        offs = np.zeros(nc + 1, dtype=np.uint64)
        st = L.skvref_encode_m(self.ptr, C.byref(shape), _p(x), _p(mu), _p(sigma), _p(bits),
                               int(bound), _p(offs), nthreads)
        if st != OK:
            raise RuntimeError(f"oracle encode failed (status {st})")
        return bits[: int(offs[-1])].copy(), offs

    def decode(self, shape: Shape, bits, offsets, mu, sigma, nthreads=8):
        _sizes(shape, None, mu, sigma)
        L = lib()
        out = np.zeros(mu.shape, dtype=np.uint16 if shape.sym_fmt == SYM_BF16 else np.uint8)
        bits = np.ascontiguousarray(bits, dtype=np.uint8)
        if bits.size == 0:
            bits = np.zeros(1, dtype=np.uint8)
        st = L.skvref_decode_m(self.ptr, C.byref(shape), _p(bits), _p(offsets), _p(mu), _p(sigma),
                               _p(out), nthreads)
        return out, st

    def encode_chunk(self, shape: Shape, chunk: int, x_c, mu_c, sigma_row):
        """Encode one chunk from its own slices (x_c, mu_c start at the chunk)."""
        L = lib()
        cap = 128 + 64 + 3 + 3 * 256 * shape.head_dim
        out = np.zeros(cap, dtype=np.uint8)
        st = C.c_int(0)
        n = L.skvref_encode_chunk(self.ptr, C.byref(shape), chunk, _p(x_c), _p(mu_c), _p(sigma_row),
                                  _p(out), cap, C.byref(st))
        if st.value != OK:
            raise RuntimeError(f"oracle chunk encode failed (status {st.value})")
        return out[:n].copy()

    def adapt_tables(self, shape: Shape, x_c, nsc: int):
        """The p_hat table of every epoch of a chunk with symbols x_c (adaptive mode)."""
        ne = (nsc + adapt_params()[0] - 1) // adapt_params()[0]
        out = np.zeros((max(ne, 1), self.N + 1), dtype=np.uint32)
        x_c = np.ascontiguousarray(x_c)
        n = lib().skvref_adapt_tables(self.ptr, C.byref(shape), _p(x_c), nsc, _p(out), out.shape[0])
        return out[:n]

    def decode_chunk(self, shape: Shape, chunk: int, data, mu_c, sigma_row, out_c):
        data = np.ascontiguousarray(data, dtype=np.uint8)
        buf = data if data.size else np.zeros(1, dtype=np.uint8)
        return lib().skvref_decode_chunk(self.ptr, C.byref(shape), chunk, _p(buf), data.size, _p(mu_c),
                                         _p(sigma_row), _p(out_c))


def rank(fmt, b):
    return lib().skvref_rank(fmt, b)


def unrank(fmt, k):
    return lib().skvref_unrank(fmt, k)


def value(fmt, b):
    return lib().skvref_value(fmt, b)


def bins(fmt: int, b):
    b = np.ascontiguousarray(b, dtype=np.uint32)
    lo = np.zeros(b.shape, dtype=np.float32)
    hi = np.zeros(b.shape, dtype=np.float32)
    lib().skvref_bin_many(fmt, _p(b), _p(lo), _p(hi), b.size)
    return lo, hi


def scale(sigma):
    sigma = np.ascontiguousarray(sigma, dtype=np.float32)
    out = np.zeros(sigma.shape, dtype=np.float32)
    lib().skvref_scale_many(_p(sigma), _p(out), sigma.size)
    return out


def num_chunks(shape: Shape) -> int:
    return int(lib().skvref_num_chunks(C.byref(shape)))


def encode_bound(shape: Shape) -> int:
    return int(lib().skvref_encode_bound(C.byref(shape)))


def rc_encode_seq(c, f) -> bytes:
    """Range-code a sequence of (cum, freq) pairs whose total is 2^24."""
    c = np.ascontiguousarray(c, dtype=np.uint32)
    f = np.ascontiguousarray(f, dtype=np.uint32)
    cap = 3 * c.size + 8
    out = np.zeros(cap, dtype=np.uint8)
    n = lib().skvref_rc_encode_seq(_p(c), _p(f), c.size, _p(out), cap)
    return bytes(out[:n])


def encode(shape: Shape, x, mu, sigma, hist, nthreads=8):
    return Model(shape.sym_fmt, hist).encode(shape, x, mu, sigma, nthreads)


def decode(shape: Shape, bits, offsets, mu, sigma, hist, nthreads=8):
    return Model(shape.sym_fmt, hist).decode(shape, bits, offsets, mu, sigma, nthreads)


class Calibrator:
    """sigma per (layer, kv, head, channel), or per channel and |mu| octave in
    octave mode (a table of OCT_STRIDE floats per channel), and the symbol
    histogram."""

    def __init__(self, shape: Shape):
        self.shape = shape
        nch = shape.layers * 2 * shape.kv_heads * shape.head_dim
        self.S = np.zeros(nch, dtype=np.float64)
        self.n = np.zeros(nch, dtype=np.uint64)
        nb = nch * EXP_BINS if shape.sigma_mode == SIGMA_OCTAVE else 1
        self.So = np.zeros(nb, dtype=np.float64)
        self.no = np.zeros(nb, dtype=np.uint64)
        self.hist = np.zeros(65536 if shape.sym_fmt == SYM_BF16 else 256, dtype=np.uint64)

    def accumulate(self, x, mu, nthreads=8):
        st = lib().skvref_calib_accumulate(C.byref(self.shape), _p(x), _p(mu), _p(self.S), _p(self.n),
                                           _p(self.So), _p(self.no), _p(self.hist), nthreads)
        if st != OK:
            raise RuntimeError(f"oracle calibration failed (status {st})")

    def finalize(self):
        nch = self.S.size
        if self.shape.sigma_mode == SIGMA_OCTAVE:
            table = np.zeros(nch * OCT_STRIDE, dtype=np.float32)
            lib().skvref_calib_finalize_octave(nch, _p(self.S), _p(self.n), _p(self.So), _p(self.no), _p(table))
            return table, self.hist.copy()
        sigma = np.zeros(nch, dtype=np.float32)
        lib().skvref_calib_finalize(nch, _p(self.S), _p(self.n), _p(sigma))
        return sigma, self.hist.copy()
