"""Pins for the oracle's frequency model (no GPU).

Each test checks the oracle against something other than itself: the exact
mixture CDF from scipy's ndtr, torch's round-to-nearest-even conversions,
closed forms, and brute-force invariants.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import ndtr

from oracle import skvref as R

FMTS = [R.SYM_BF16, R.SYM_E4M3]


def exact_mix(z, w_narrow=0.95, w_wide=0.03):
    z = np.asarray(z, dtype=np.float64)
    return (w_narrow * ndtr(z) + w_wide * ndtr(z / 3.0)) / (w_narrow + w_wide)


# ---------------------------------------------------------------- knots
@pytest.mark.parametrize("fmt", FMTS)
def test_knots_are_correctly_rounded_mixture_cdf(fmt):
    """V_j = RN32(MG * G(j/64)), G the 0.95/0.03 Gaussian pair of the mixture
    ("Speculative KV coding", early results), with G taken from scipy's ndtr."""
    m = R.Model(fmt)
    K, D = m.knots()
    j = np.arange(0, 1024)
    exact = m.MG * exact_mix(j / 64.0)
    V = K[1024:2048].astype(np.float64)
    ulp = np.spacing(np.abs(V).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(V - exact) <= 0.5 * ulp + 1e-9 * m.MG)
    # every knot is far from an fp32 rounding boundary, so any accurate erfc rounds the same way
    frac = (exact - V) / ulp
    margin = 0.5 - np.abs(frac)
    assert margin.min() > 1e-6, f"knot {np.argmin(margin)} is ambiguous: margin {margin.min()}"
    assert K[2048] == m.MG


@pytest.mark.parametrize("fmt", FMTS)
def test_knot_table_structure(fmt):
    m = R.Model(fmt)
    K, D = m.knots()
    Kd = K.astype(np.float64)
    assert K[1024] == m.MG / 2 and K[0] == 0.0 and K[2048] == m.MG
    # K_{-j} = MG - K_j exactly
    np.testing.assert_array_equal(Kd[:1024][::-1], m.MG - Kd[1025:])
    # D is the exact difference and non-negative; the top knot has D = 0
    np.testing.assert_array_equal(D[:-1].astype(np.float64), Kd[1:] - Kd[:-1])
    assert D[-1] == 0.0 and np.all(D >= 0)


def _rn32(q):
    """Exact round-to-nearest-even of a non-negative rational to fp32 (normal range)."""
    from fractions import Fraction
    if q == 0:
        return 0.0
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    n, r = divmod(q, ulp)
    if r > ulp / 2 or (r == ulp / 2 and n % 2 == 1):
        n += 1
    return float(n * ulp)


@pytest.mark.parametrize("fmt", FMTS)
def test_knot_pair_below_zero_floors_alike_near_f_one(fmt):
    """The device evaluates f = c - floor(c) with v_fract_f32, which returns the
    float just below 1 where the fp32 difference rounds to 1.0; that happens
    only for c in [-2^-25, 0), i.e. on the knot pair at floor(c) = -1.  There,
    floor(RN(K + f D)) must not depend on which of the two f is used."""
    from fractions import Fraction
    m = R.Model(fmt)
    K, D = m.knots()
    k, d = Fraction(float(K[1023])), Fraction(float(D[1023]))
    below_one = Fraction(float(np.nextafter(np.float32(1), np.float32(0))))
    y_one = _rn32(k + d)
    y_below = _rn32(k + below_one * d)
    assert math.floor(y_one) == math.floor(y_below)
    assert y_one == float(K[1024])  # the pair's top end is the next knot exactly


@pytest.mark.parametrize("fmt", FMTS)
def test_cg_monotone_and_saturating(fmt):
    m = R.Model(fmt)
    rng = np.random.default_rng(1)
    u = np.concatenate([
        rng.uniform(-1100, 1100, 2_000_000),
        rng.uniform(-2, 2, 500_000),
        np.ldexp(rng.uniform(-1, 1, 200_000), rng.integers(-149, 10, 200_000)),
        np.arange(-1025, 1026, 0.25),
        [0.0, -0.0, np.inf, -np.inf, 1e30, -1e30, 1024.0, -1024.0, 1023.9999, -1023.9999],
    ]).astype(np.float32)
    u = np.sort(u)
    cg = m.cg(u).astype(np.int64)
    assert np.all(np.diff(cg) >= 0)
    assert m.cg(np.array([-np.inf], np.float32))[0] == 0
    assert m.cg(np.array([np.inf], np.float32))[0] == m.MG
    assert m.cg(np.array([0.0], np.float32))[0] == m.MG // 2
    assert m.cg(np.array([-0.0], np.float32))[0] == m.MG // 2


@pytest.mark.parametrize("fmt", FMTS)
def test_cg_monotone_over_every_fp32(fmt):
    """Cg is non-decreasing over every fp32 knot coordinate in [-1024, 1024]
    (about 2.2e9 values, walked in value order: the negative patterns from
    -1024 down to -0 by decreasing bits, then +0 up to +1024), not only on
    samples.  A non-decreasing Cg makes cum(k) non-decreasing in k for every
    (mu, sigma), so the only source of each frequency's lower bound is the
    one-count floor the model adds."""
    from concurrent.futures import ThreadPoolExecutor

    m = R.Model(fmt)
    top = int(np.float32(1024.0).view(np.uint32)) + 1   # patterns 0 .. 0x44800000
    chunk = 1 << 24
    # pieces in value order: (lo, hi, negative) over magnitude bit patterns
    pieces = [(max(0, h - chunk), h, True) for h in range(top, 0, -chunk)]
    pieces += [(lo, min(top, lo + chunk), False) for lo in range(0, top, chunk)]

    def run(piece):
        lo, hi, neg = piece
        if neg:  # decreasing magnitude: increasing value
            bits = np.arange(hi - 1, lo - 1, -1, dtype=np.uint32) | np.uint32(0x80000000)
        else:
            bits = np.arange(lo, hi, dtype=np.uint32)
        cg = m.cg(bits.view(np.float32)).astype(np.int64)
        return int(cg[0]), int(cg[-1]), bool(np.all(np.diff(cg) >= 0))

    with ThreadPoolExecutor(max_workers=4) as ex:
        res = list(ex.map(run, pieces))
    prev = -1
    for (lo, hi, neg), (first, last, inside) in zip(pieces, res):
        assert inside and first >= prev, f"Cg decreases in the {'negative' if neg else 'positive'} patterns {lo:#x}..{hi:#x}"
        prev = last
    assert res[0][0] == 0 and prev == m.MG


@pytest.mark.parametrize("fmt", FMTS)
def test_cg_within_interpolation_bound_of_exact(fmt):
    """Linear interpolation between knots h = 1/64 apart is within h^2/8 max|G''|
    of the exact mixture CDF; knot rounding adds 1/2 count and the floor 1."""
    m = R.Model(fmt)
    rng = np.random.default_rng(2)
    u = rng.uniform(-1024, 1024, 1_000_000).astype(np.float32)
    cg = m.cg(u).astype(np.float64)
    exact = m.MG * exact_mix(u.astype(np.float64) / 64.0)
    gpp_max = (0.95 * math.exp(-0.5) / math.sqrt(2 * math.pi) + 0.03 / 9 * math.exp(-0.5) / math.sqrt(2 * math.pi)) / 0.98
    bound = m.MG * (1 / 64) ** 2 / 8 * gpp_max + 0.5 + 1.0
    err = np.abs(cg - exact)
    assert err.max() <= bound, (err.max(), bound)
    # and clearly finer than that on average (catches a wrong segment index)
    assert err.mean() < 0.5 * bound


# ---------------------------------------------------------------- symbols and bins
def _bf16_values(b):
    return (np.asarray(b, np.uint32) << 16).astype(np.uint32).view(np.float32)


def test_rank_is_value_order_bf16():
    b = np.arange(65536, dtype=np.uint32)
    ranks = np.array([R.rank(0, int(v)) for v in b])
    assert sorted(ranks.tolist()) == list(range(65536))
    assert all(R.unrank(0, int(R.rank(0, int(v)))) == v for v in b[::97])
    order = np.argsort(ranks)
    vals = _bf16_values(b[order]).astype(np.float64)
    finite = ~np.isnan(vals)
    assert np.all(np.isnan(vals[:127])) and np.all(np.isnan(vals[-127:]))
    v = vals[finite]
    assert np.all(np.diff(v) >= 0)  # -0 and +0 compare equal, in that order
    assert np.signbit(vals[32767]) and not np.signbit(vals[32768])


def test_rank_is_value_order_e4m3():
    b = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    ranks = np.array([R.rank(1, int(v)) for v in b])
    assert sorted(ranks.tolist()) == list(range(256))
    order = np.argsort(ranks)
    sv = vals[order]
    assert np.isnan(sv[0]) and np.isnan(sv[-1])
    assert np.all(np.diff(sv[1:-1]) >= 0)
    for v in range(256):
        assert R.value(1, v) == vals[v] or (np.isnan(vals[v]) and np.isnan(R.value(1, v)))


def test_bf16_bins_are_rne_preimages():
    """Points inside each bin round (torch fp32 -> bf16, RNE) to the symbol;
    the fp32 neighbours just outside round to the adjacent symbols."""
    b = np.arange(65536, dtype=np.uint32)
    lo, hi = R.bins(0, b)
    m = b & 0x7FFF
    fin = (m >= 1) & (m <= 0x7F7F)
    bb, lo_, hi_ = b[fin], lo[fin], hi[fin]
    to_bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    inner_lo = np.nextafter(lo_, np.float32(np.inf))
    inner_hi = np.nextafter(hi_, np.float32(-np.inf))
    np.testing.assert_array_equal(to_bf(inner_lo), bb)
    np.testing.assert_array_equal(to_bf(inner_hi), bb)
    below = np.nextafter(lo_, np.float32(-np.inf))
    above = np.nextafter(hi_, np.float32(np.inf))
    rank = np.array([R.rank(0, int(v)) for v in bb])
    rb = np.array([R.rank(0, int(v)) for v in to_bf(below)])
    ra = np.array([R.rank(0, int(v)) for v in to_bf(above)])
    np.testing.assert_array_equal(rb, rank - 1)
    np.testing.assert_array_equal(ra, rank + 1)
    # the edge itself is a tie and goes to the even mantissa
    at_lo = to_bf(lo_)
    even = (bb & 1) == 0
    np.testing.assert_array_equal(at_lo[even], bb[even])
    # specials: zeros, infinities, NaNs
    assert R.bins(0, [0x0000]) == (np.float32(0.0), np.float32(2.0 ** -134))
    lo0, hi0 = R.bins(0, [0x8000])
    assert lo0[0] == -(2.0 ** -134) and hi0[0] == 0.0
    lo_inf, hi_inf = R.bins(0, [0x7F80])
    assert to_bf(np.nextafter(lo_inf, np.float32(np.inf)))[0] == 0x7F80 and hi_inf[0] == np.inf
    assert R.bins(0, [0x7FC0])[0][0] == np.inf and R.bins(0, [0xFFC0])[1][0] == -np.inf


def test_e4m3_bins_are_saturating_rne_preimages():
    b = np.arange(256, dtype=np.uint32)
    lo, hi = R.bins(1, b)

    def to_e4(a):
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).clamp(-448, 448)
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    for v in range(256):
        if (v & 0x7F) == 0x7F:
            assert (lo[v], hi[v]) == ((np.inf, np.inf) if v < 128 else (-np.inf, -np.inf))
            continue
        pts = [np.nextafter(lo[v], np.float32(np.inf)), np.nextafter(hi[v], np.float32(-np.inf))]
        pts = [p for p in pts if np.isfinite(p)]
        if np.isinf(hi[v]):
            pts.append(np.float32(1e30))
        if np.isinf(lo[v]):
            pts.append(np.float32(-1e30))
        got = to_e4(np.array(pts, np.float32))
        want = v if (v & 0x7F) else None
        if want is not None:
            assert np.all(got == v), (v, pts, got)
        else:  # zeros: the sign of a rounded tiny value follows the value
            assert np.all((got & 0x7F) == 0)
    # interval ends meet in rank order
    order = np.argsort([R.rank(1, v) for v in range(256)])
    np.testing.assert_array_equal(hi[order][:-1], lo[order][1:])
    assert lo[0x7E] == 432.0 and hi[0x7E] == np.inf and lo[0x01] == 2.0 ** -10


@pytest.mark.parametrize("fmt", FMTS)
def test_every_fp32_rounds_into_its_symbols_bin(fmt):
    """Every fp32 value that is not a NaN (about 4.28e9) rounds, by torch's
    conversion (nearest even; e4m3 saturating at +-448), to a symbol whose
    oracle bin [lo, hi] contains it: the bins cover the whole real line with
    each value in the bin of the symbol it rounds to, not only at the edges."""
    from concurrent.futures import ThreadPoolExecutor

    n_sym = 65536 if fmt == 0 else 256
    LO, HI = R.bins(fmt, np.arange(n_sym, dtype=np.uint32))
    chunk = 1 << 24

    def sym(y):
        t = torch.from_numpy(y)
        if fmt == 0:
            return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return t.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    def run(start):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        nan = ((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x007FFFFF) != 0)
        y = bits[~nan].view(np.float32)
        s_ = sym(y)
        ok = (LO[s_] <= y) & (y <= HI[s_])
        if ok.all():
            return None
        i = int(np.flatnonzero(~ok)[0])
        return float(y[i]), int(s_[i]), float(LO[s_[i]]), float(HI[s_[i]])

    threads = torch.get_num_threads()
    torch.set_num_threads(1)  # the chunks run in parallel threads instead
    try:
        with ThreadPoolExecutor(max_workers=6) as ex:
            bad = [r for r in ex.map(run, range(0, 1 << 32, chunk)) if r is not None]
    finally:
        torch.set_num_threads(threads)
    assert not bad, f"value outside its symbol's bin (y, symbol, lo, hi): {bad[:3]}"


def test_bf16_bin_ends_meet_in_rank_order():
    b = np.array([R.unrank(0, k) for k in range(65536)], dtype=np.uint32)
    lo, hi = R.bins(0, b)
    np.testing.assert_array_equal(hi[:-1], lo[1:])
    assert lo[0] == -np.inf and hi[-1] == np.inf


# ---------------------------------------------------------------- p_hat table
@pytest.mark.parametrize("fmt", FMTS)
def test_ptable_uniform_closed_form(fmt):
    m = R.Model(fmt)
    A = m.ptable().astype(np.int64)
    k = np.arange(m.N + 1, dtype=np.int64)
    np.testing.assert_array_equal(A, k + (m.Mp * k) // m.N)


@pytest.mark.parametrize("fmt", FMTS)
def test_ptable_tracks_smoothed_histogram(fmt):
    rng = np.random.default_rng(3)
    N = 65536 if fmt == 0 else 256
    hist = rng.zipf(1.5, N).astype(np.uint64) * rng.integers(0, 2, N).astype(np.uint64)
    m = R.Model(fmt, hist)
    A = m.ptable().astype(np.int64)
    order = np.array([R.unrank(fmt, k) for k in range(N)])
    h = hist[order].astype(np.float64) + 1
    dq = np.diff(A) - 1
    expect = m.Mp * h / h.sum()
    assert np.all(np.abs(dq - expect) < 1.0 + 1e-9)
    assert A[0] == 0 and A[-1] == N + m.Mp


@pytest.mark.parametrize("fmt", FMTS)
def test_ptable_domain_edges(fmt):
    """The p_hat table's domain is Mp * H(N) <= 2^62 for the exact smoothed
    total H(N) = sum(hist + 1): at the largest admissible total the table is
    the exact integer quotient (no 64-bit product overflows), one count more
    is outside, and so is any histogram whose exact total passes 2^64 (a count
    of 2^64 - 1 whose +1 would wrap to 0 in 64-bit arithmetic, or two large
    counts)."""
    N = 65536 if fmt == 0 else 256
    Mp = R.Model(fmt).Mp
    limit = (1 << 62) // Mp
    hist = np.zeros(N, dtype=np.uint64)
    pos = [R.unrank(fmt, k) for k in (3, N // 2, N - 2)]
    hist[pos[0]] = limit // 3
    hist[pos[1]] = limit // 5
    hist[pos[2]] = limit - N - int(hist[pos[0]]) - int(hist[pos[1]])
    assert int(hist.astype(object).sum()) + N == limit
    A = R.Model(fmt, hist).ptable()
    H = 0
    want = []
    for k in range(N):
        want.append(k + Mp * H // limit)
        H += int(hist[R.unrank(fmt, k)]) + 1
    want.append(N + Mp)
    assert A.tolist() == want
    over = hist.copy()
    over[pos[2]] += np.uint64(1)
    for bad in (over, np.full(N, 0, dtype=np.uint64)):
        if bad is not over:
            bad[pos[1]] = np.uint64(2**64 - 1)
        with pytest.raises(ValueError, match="status 6"):
            R.Model(fmt, bad)
    two = np.zeros(N, dtype=np.uint64)
    two[pos[0]] = two[pos[1]] = np.uint64(2**63)
    with pytest.raises(ValueError, match="status 6"):
        R.Model(fmt, two)


# ---------------------------------------------------------------- the integer model
def _samples(fmt, n, seed):
    rng = np.random.default_rng(seed)
    # a mean in every fp32 binade, both signs (2^-149 .. 2^127)
    e = np.arange(-149, 128)
    every = np.ldexp(1.0 + rng.uniform(0, 1, e.size), e) * np.where(rng.uniform(size=e.size) < 0.5, -1, 1)
    every = np.minimum(np.abs(every), np.finfo(np.float32).max) * np.sign(every)
    n_rest = max(0, n - every.size - 6)
    mu = np.concatenate([
        every,
        rng.standard_normal(n_rest // 2) * np.exp(rng.uniform(-8, 8, n_rest // 2)),
        np.ldexp(rng.uniform(-1, 1, n_rest // 4), rng.integers(-149, -120, n_rest // 4)),  # subnormal
        rng.uniform(-500, 500, n_rest - n_rest // 2 - n_rest // 4),
        [0.0, -0.0, np.nan, np.inf, -np.inf, 3e38],
    ]).astype(np.float32)
    sigma = np.exp(rng.uniform(-20, 20, mu.size)).astype(np.float32)
    sigma[:: 7] = 0.0
    sigma[1:: 11] = 2.0 ** -100
    sigma[2:: 13] = 1e30
    return mu, sigma


@pytest.mark.parametrize("fmt", FMTS)
def test_model_invariants_bruteforce(fmt):
    """For every sample (mu, sigma): cum(0) = 0, cum(N) = T, every freq >= 1,
    and the encoder's per-symbol pair equals the decoder's per-rank table."""
    from concurrent.futures import ThreadPoolExecutor

    mu, sigma = _samples(fmt, 10_000, 4)
    hist = np.random.default_rng(5).integers(0, 1000, 65536 if fmt == 0 else 256).astype(np.uint64)
    m = R.Model(fmt, hist)
    b = np.array([R.unrank(fmt, k) for k in range(m.N)], dtype=np.uint32)

    def check(i):
        cum = m.cum_table(mu[i], sigma[i]).astype(np.int64)
        s = R.scale(np.array([sigma[i]], np.float32))[0]
        lo, hi = m.cum_pair(np.full(m.N, mu[i], np.float32), np.full(m.N, s, np.float32), b)
        ok = (cum[0] == 0 and cum[-1] == m.T and bool(np.all(np.diff(cum) >= 1))
              and np.array_equal(lo, cum[:-1]) and np.array_equal(hi, cum[1:]))
        return None if ok else (float(mu[i]), float(sigma[i]))

    with ThreadPoolExecutor(max_workers=6) as ex:
        bad = [r for r in ex.map(check, range(mu.size)) if r is not None]
    assert not bad, f"model invariants fail at (mu, sigma): {bad[:5]}"


def test_scale_is_correctly_rounded():
    rng = np.random.default_rng(6)
    sigma = np.exp(rng.uniform(-60, 60, 200_000)).astype(np.float32)
    s = R.scale(sigma)
    from fractions import Fraction
    for sg, sc in list(zip(sigma, s))[:2000]:
        exact = Fraction(64) / Fraction(float(sg))
        lo = Fraction(float(np.nextafter(sc, np.float32(0))))
        hi = Fraction(float(np.nextafter(sc, np.float32(np.inf))))
        c = Fraction(float(sc))
        assert abs(exact - c) <= min(abs(exact - lo), abs(exact - hi))
    assert R.scale(np.array([0.0], np.float32))[0] == np.float32(64.0 * 2.0 ** 100)


@pytest.mark.parametrize("fmt", FMTS)
def test_pure_noise_predictor_costs_full_width(fmt):
    """A predictor that carries no information costs the full symbol width
    ("Speculative KV coding", what predicts the KV cache: close to 16 bits).
    With the Gaussian budget set to 0 and an empty histogram every symbol
    gets exactly 256 counts: 16 bits for bf16, 8 for e4m3."""
    N = 65536 if fmt == 0 else 256
    T = 1 << (24 if fmt == 0 else 16)
    m = R.Model(fmt, None, MG=0, Mp=T - N)
    cum = m.cum_table(0.3, 0.01).astype(np.int64)
    assert np.all(np.diff(cum) == T // N)
