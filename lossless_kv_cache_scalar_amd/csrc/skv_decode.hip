// skv_decode.hip -- decode a range-coded KV cache on gfx950.
//
// Persistent grid, one 1024-thread block per CU with the model's tables in
// LDS (knots 16 KB, the inverse of the Gaussian pair's CDF 8 KB, the bf16 p_hat
// table 137 KB); the static e4m3 kernels, whose tables take 28 KB, run five
// 256-thread blocks per CU instead (5 waves per SIMD rather than 4).  Each wavefront decodes whole chunks, taking their ids from a
// counter (the waves of a SIMD issue at different rates, so fixed shares would
// leave the fast ones idle); lane l decodes substream l, the chunk's scalars
// l, l + 64, ...  The model is rebuilt from
// (mu, sigma, hist), as both ends of the coder do ("Speculative KV coding",
// "什么能预测 KV 缓存").
//
// Symbol search.  The decoder needs the unique symbol s with
// r * cum_lo(s) <= d < r * cum_hi(s).  A guess comes from inverting the
// Gaussian pair's CDF at t ~ d / r (fp32, approximate on purpose), twice: at
// t - A(rank of mu), then at t - A(rank of the first guess).  The guess is
// verified with the exact integer model and exact 48-bit products.  The rare
// lanes whose guess misses are then resolved one at a time by the whole wave,
// 64 probes of the exact cumulative count per round (a call with idle lanes,
// in a short chunk's last batch, searches lane by lane instead).  Any exact
// search returns the same symbol, so the output does not depend on the guesses.
//
// Stream reads.  Word w of a lane is word 64 w + l of the chunk's interleaved
// region while w < m, so the lanes' refills read 256 contiguous bytes; each
// lane keeps its next word in flight.  Refills happen once per batch of 8
// symbols, with a wave-wide fallback for a lane that runs short within one.
//
// Adaptive p_hat (e4m3): the wave's count and pair tables in LDS follow the
// decoded symbols and are rebuilt every epoch, exactly where the encoder
// rebuilt them (skv_adapt.hpp).
#include "skv_adapt.hpp"
#include "skv_modeldev.hpp"

namespace skv {

constexpr int kDecBlock = 1024;
constexpr int kDecWaves = kDecBlock / 64;

struct DecArgs {
  Geo g;
  const uint8_t *bits;
  uint64_t bits_bytes;
  const uint64_t *offsets;
  const void *mu;
  const float2 *knots;
  const uint32_t *ptab;
  const uint16_t *a16;
  const uint32_t *abase;
  const int32_t *aflag;
  const float2 *uinv;
  const float2 *etab;
  const uint32_t *prior;  // adaptive p_hat: the counts a chunk starts from (at the symbols' patterns)
  const float2 *scale;   // per channel, or per channel and octave
  const int32_t *eref;   // octave mode: per channel octave reference
  float inv_step;  // kNInv / MG
  void *x_out;
  int32_t *status;
  uint32_t *ctr;   // next chunk id (zeroed by the call before the launch)
};

// Bits of one lane's substream, most significant first; bytes at or past its
// length read as 0.  ib holds the bits before word w.  Whenever w advances,
// issue() loads the dword(s) that hold the new word w into (plo, phi), so the
// next refill finds them in registers.  A full batch starts with top_up(),
// which leaves every lane at least 32 bits; a symbol takes at most 24, so a
// lane falls short within a batch only after a run of expensive symbols, and
// the per-symbol refill is a rare wave-wide branch.  Words w < m are aligned
// dwords of the interleaved region (no masking); the lane's tail words may
// straddle dwords and run past its length.
struct LaneReader {
  const uint8_t *chunk;  // chunk start, 4-byte aligned
  uint32_t csize;        // chunk bytes (a multiple of 4, >= 192)
  uint32_t m;            // interleaved words per lane
  uint32_t tail, len;    // chunk offset of the lane's tail, lane length
  uint32_t ip0;          // chunk offset of the lane's interleaved word 0 (word w: ip0 + 256 w)
  uint32_t ipw;          // ip0 + 256 w, advanced with w (an add where the product would take a shift-add)
  uint32_t w, plo, phi;
  uint64_t ib;  // next bits, left-aligned
  int nib;      // valid bits in ib

  bool fast;    // wave-uniform: at the last issue no lane was past its interleaved words

  __device__ __forceinline__ void issue() {
    const bool tl = w >= m;
    fast = !__any(tl);
    uint32_t a0 = ipw;  // = ip0 + 256 w; an interleaved word never lies past the lane's end
    if (__builtin_expect(!fast, 0)) {
      if (tl) {
        a0 = (tail + 4u * (w - m)) & ~3u;
        if (4u * w >= len) a0 = 0u;  // nothing left: any dword of the chunk, masked off below
      }
    }
    // both dwords on every issue: a load on one branch only would make the
    // compiler wait for it where the branches join
    uint32_t a1 = a0 + 4u;
    if (a1 >= csize) a1 = a0;
    plo = *reinterpret_cast<const uint32_t *>(chunk + a0);
    phi = *reinterpret_cast<const uint32_t *>(chunk + a1);
  }
  // renormalisation bytes taken so far (after the 6 priming bytes)
  __device__ __forceinline__ uint32_t renorm_bytes() const { return (32u * w - (uint32_t)nib) / 8u - 6u; }
  // word w of the lane, from the loads of the last issue (made for this w)
  __device__ __forceinline__ uint32_t word() const {
    if (__builtin_expect(fast, 1) || w < m) return __builtin_bswap32(plo);
    // bytes tail mod 4 .. of phi:plo (two separate registers: no pair to merge)
    uint32_t v = __builtin_bswap32(__builtin_amdgcn_alignbyte(phi, plo, tail & 3u));
    const int valid = (int)len - 4 * (int)w;
    if (valid <= 0) return 0u;
    if (valid < 4) v &= ~(0xFFFFFFFFu >> (8 * valid));
    return v;
  }
  __device__ __forceinline__ void init(uint32_t lane) {
    w = 0;
    ip0 = kHeaderBytes + 4u * lane;
    ipw = ip0;
    issue();
    ib = (uint64_t)word() << 32;
    w = 1;
    ipw += 256u;
    issue();
    ib |= word();
    nib = 64;
    w = 2;
    ipw += 256u;
    issue();
  }
  // word w joins the buffer (nib <= 32)
  __device__ __forceinline__ void refill() {
    ib |= (uint64_t)word() << (32 - nib);
    nib += 32;
    ++w;
    ipw += 256u;
  }
  // at least n valid bits, n <= 24 (wave-wide: the refill is rare)
  __device__ __forceinline__ void ensure(uint32_t n) {
    if (__builtin_expect(__any(nib < (int)n), 0)) {
      if (nib < (int)n) refill();
      issue();
    }
  }
  // at least 32 valid bits before a full batch: one word wherever it fits
  __device__ __forceinline__ void top_up() {
    if (__any(nib <= 32)) {
      if (nib <= 32) refill();
      issue();
    }
  }
  // n in {0, 8, 16, 24}
  __device__ __forceinline__ uint32_t take(uint32_t n) {
    ensure(n);
    const uint32_t v = __builtin_amdgcn_ubfe((uint32_t)(ib >> 32), (0u - n) & 31u, n);
    ib <<= n;
    nib -= (int)n;
    return v;
  }
  // (x << n) | take(n) for x < 2^(64 - n), as two 64-bit shifts: the high
  // word of x << n, and the high word of (low word of x : next bits) << n
  __device__ __forceinline__ uint64_t shift_in(uint64_t x, uint32_t n) {
    ensure(n);
    const uint64_t lo = (((uint64_t)(uint32_t)x << 32) | (uint32_t)(ib >> 32)) << n;
    const uint64_t r = ((x << n) & 0xFFFFFFFF00000000ull) | (lo >> 32);
    ib <<= n;
    nib -= (int)n;
    return r;
  }
};

// bf16 pattern of x, rounded to nearest even, in the low half of a zero word:
// v_cvt_pk_bf16_f32 with 0.0 as the second operand (written out so that the
// compiler knows the high half is zero and masks nothing)
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t v;
  asm("v_cvt_pk_bf16_f32 %0, %1, 0" : "=v"(v) : "v"(x));
  return v;
}

// e4m3 pattern of a guessed value e, rounded to nearest even: the hardware
// conversion (OCP e4m3).  Beyond +-464 it gives a NaN pattern, which is still
// a symbol: such a guess misses and the exact search finds the answer, so the
// guesses skip the clamp.  The instruction writes the low 16 bits only: the
// word starts at zero, and the second operand 0.0 converts to a zero byte.
__device__ __forceinline__ uint32_t e4m3_rne_bits(float e) {
  uint32_t v = 0;
  asm("v_cvt_pk_fp8_f32 %0, %1, 0" : "+v"(v) : "v"(e));
  return v;
}

// A(k) for a guess; k is the table index (bf16: tix_bf16; e4m3: the pattern)
template <int SYM, int TAB>
__device__ __forceinline__ uint32_t a_guess(const ModelTabs &t, uint32_t k) {
  if (SYM != SKV_SYM_BF16) return TAB == kTabPattern ? __float_as_uint(t.ep[k].z) : t.ab[2u * k];
  return a_one<TAB>(t, k);
}

// The symbol whose bin holds the value where the Gaussian pair's CDF reaches
// t - A(k): the inverse table gives the knot coordinate, mu + u sigma / 64 the
// value, and rounding to the symbol format the guess.  ts is t in steps of the
// inverse table (kNInv / MG counts per step).  A first guess, whose only use is
// the A of its bin, takes a table point instead of interpolating within the
// step: the point below t for e4m3 (kGuessFloor; its bins are wide), the
// nearest one for bf16 (kGuessNearest).
constexpr int kGuessInterp = 0, kGuessFloor = 1, kGuessNearest = 2;
template <int SYM, int TAB, int MODE = kGuessInterp>
__device__ __forceinline__ uint32_t guess_symbol(const ModelTabs &t, const float2 *uinv, float ts, uint32_t k,
                                                 float inv_step, float sinv, float m) {
  float mf = __builtin_fmaf((float)a_guess<SYM, TAB>(t, k), -inv_step, ts);
  mf = __builtin_fminf(__builtin_fmaxf(mf, 0.0f), (float)kNInv - 0.5f);
  // mf >= 0: truncation is the floor; the nearest point is at most kNInv, the
  // table's last entry
  const int ii = MODE == kGuessNearest ? (int)(mf + 0.5f) : (int)mf;
  const float2 ud = uinv[ii];
  const float uu = MODE == kGuessInterp ? __builtin_fmaf(__builtin_amdgcn_fractf(mf), ud.y, ud.x) : ud.x;
  const float e = __builtin_fmaf(uu, sinv, m);
  return SYM == SKV_SYM_BF16 ? bf16_rne_bits(e) : e4m3_rne_bits(e);
}

// The exact rank: the largest k with r * (cum(k) << up) <= d.  Known so far:
// that holds at lo and fails at hi (hi = N: no bound), and the rank k0 was
// probed: it holds (below = false) or fails (below = true) there.  Gallop away
// from k0 towards the answer, then bisect.
template <int SYM, int TAB>
__device__ uint32_t search_rank(const ModelTabs &t, uint32_t k0, bool below, uint32_t lo, uint32_t hi, uint64_t d,
                                uint32_t r, int up, float m, float s) {
  const uint32_t N = SYM == SKV_SYM_BF16 ? 65536u : 256u;
  auto leq = [&](uint32_t k) -> bool { return mul24(r, cum_rank<SYM, TAB>(t, k, m, s) << up) <= d; };
  if (below) {
    hi = min(hi, k0);
    uint32_t step = 1;
    while (hi - lo > 1) {
      const uint32_t p = hi - lo > step ? hi - step : lo;
      if (p == lo) break;
      if (leq(p)) {
        lo = p;
        break;
      }
      hi = p;
      step <<= 1;
    }
  } else {
    lo = max(lo, k0);
    uint32_t step = 1;
    while (hi - lo > 1) {
      const uint32_t p = hi - lo > step ? lo + step : hi;
      if (p == hi || p >= N) break;
      if (leq(p)) {
        lo = p;
        step <<= 1;
      } else {
        hi = p;
        break;
      }
    }
  }
  while (hi - lo > 1) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (leq(mid)) lo = mid; else hi = mid;
  }
  return lo;
}

// verify symbol g: d - r*cum_lo and whether it lies in [0, r*freq).  The
// difference is taken modulo 2^64: when d < r*cum_lo it wraps above 2^63, far
// beyond r*freq < 2^48, so one unsigned compare decides.  below: d < r*cum_lo.
template <int SYM, int TAB>
__device__ __forceinline__ bool verify(const ModelTabs &t, uint32_t g, float m, float s, uint64_t d, uint32_t r,
                                       int up, uint32_t &clo, uint32_t &chi, uint64_t &dd, uint64_t &pf,
                                       bool &below) {
  model_pair<SYM, TAB>(t, g, m, s, clo, chi);
  // r 2^up times the counts: one 32 x 32-bit multiply-add each (r 2^up < 2^32)
  const uint32_t ru = r << up;
  const uint64_t plo = (uint64_t)ru * clo;
  pf = (uint64_t)ru * (chi - clo);
  dd = d - plo;
  below = d < plo;
  return dd < pf;
}

// A lane's next kBatch predictor means (symbols i0, i0 + 64, ...), raw.
template <int MU>
struct MuBatch {
  uint32_t v[kBatch];
  __device__ __forceinline__ uint32_t one(const void *mu, uint32_t i) const {
    return MU == SKV_MU_BF16 ? (uint32_t) static_cast<const uint16_t *>(mu)[i] : static_cast<const uint32_t *>(mu)[i];
  }
  __device__ __forceinline__ void load_full(const void *mu, uint32_t i0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = one(mu, i0 + kLanes * j);
  }
  __device__ __forceinline__ float get(int j) const {
    return mu_finite_wave(MU == SKV_MU_BF16 ? __uint_as_float(v[j] << 16) : __uint_as_float(v[j]));
  }
};

// A lane whose guess missed, on its own (for the rare calls where not every
// lane of the wave is active): one secant step in rank space from the guess's
// exact counts, then galloping and bisection.
template <int SYM, int TAB>
__device__ __forceinline__ void resolve_alone(const ModelTabs &t, bool ok, bool below, uint32_t &gs,
                                              uint32_t &clo, uint32_t &chi, float m, float sj, uint64_t d, uint32_t r,
                                              uint64_t &dd, uint64_t &pf, bool &corrupt) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  constexpr int up = BF ? 0 : 8;
  constexpr uint32_t N = BF ? 65536u : 256u;
  if (!ok) {
    // one secant step in rank space on the guess's exact counts
    const uint32_t kg = BF ? rank_bf16(gs) : rank_e4m3(gs);
    const float tq = (float)(uint32_t)(d >> 16) * (65536.0f * __builtin_amdgcn_rcpf((float)(r << up)));
    const float st = (tq - (float)clo) * __builtin_amdgcn_rcpf((float)(chi - clo));
    int step = (int)__builtin_floorf(__builtin_fminf(__builtin_fmaxf(st, -70000.0f), 70000.0f));
    step = below ? min(step, -1) : max(step, 1);
    const int k2 = min(max((int)kg + step, 0), (int)N - 1);
    uint32_t lo = below ? 0u : kg + 1, hi = below ? kg : N;  // holds at lo, fails at hi
    if (lo < hi && (uint32_t)k2 >= lo && (uint32_t)k2 < hi) {
      gs = BF ? unrank_bf16((uint32_t)k2) : unrank_e4m3((uint32_t)k2);
      bool below2;
      if (!verify<SYM, TAB>(t, gs, m, sj, d, r, up, clo, chi, dd, pf, below2)) {
        const uint32_t ks = search_rank<SYM, TAB>(t, (uint32_t)k2, below2, lo, hi, d, r, up, m, sj);
        gs = BF ? unrank_bf16(ks) : unrank_e4m3(ks);
        if (!verify<SYM, TAB>(t, gs, m, sj, d, r, up, clo, chi, dd, pf, below2)) {
          corrupt = true;  // no symbol holds d
          dd = 0;
        }
      }
    } else {
      corrupt = true;  // d beyond the last symbol
      dd = 0;
    }
  }
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// The lanes whose guess missed, one at a time, with the whole wave (every lane
// must be active): lane L's answer is the largest rank k with r * cum(k) <= d,
// and the wave evaluates cum at 64 ranks per round.  The first round takes the 64 ranks next to the
// guess on the side the verify pointed to (about 94% of misses end there);
// later rounds spread 64 probes over the remaining bracket [lo, hi), so a
// bracket of 65,536 ranks needs three more rounds at most.  cum(lo) <= t <
// cum(hi) holds throughout (cum(0) = 0, cum(N) = T), and the counts at both
// ends are kept, so the answer's pair comes with the last round.
template <int SYM, int TAB>
__device__ __forceinline__ void resolve_misses(const ModelTabs &t, bool miss, bool below, uint32_t &gs, uint32_t &clo,
                                            uint32_t &chi, float m, float s, uint64_t d, uint32_t r, uint64_t &dd,
                                            uint64_t &pf, bool &corrupt) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  constexpr int up = BF ? 0 : 8;
  constexpr uint32_t N = BF ? 65536u : 256u;
  constexpr uint32_t T = BF ? (1u << 24) : (1u << 16);
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t kg = BF ? rank_bf16(gs) : rank_e4m3(gs);
  uint64_t pend = __ballot(miss);
  while (pend) {
    const int L = __builtin_ctzll(pend);
    pend &= pend - 1;
    const float mL = __uint_as_float(lane_u32(__float_as_uint(m), L));
    const float sL = __uint_as_float(lane_u32(__float_as_uint(s), L));
    const uint64_t dL = ((uint64_t)lane_u32((uint32_t)(d >> 32), L) << 32) | lane_u32((uint32_t)d, L);
    const uint32_t rL = lane_u32(r, L);
    const uint32_t kgL = lane_u32(kg, L);
    uint32_t lo, hi, clo_b, chi_b, start;
    if ((__ballot(below) >> L) & 1) {
      lo = 0, clo_b = 0, hi = kgL, chi_b = lane_u32(clo, L);
      start = hi > 64u ? hi - 64u : 0u;
    } else {
      lo = kgL + 1u, clo_b = lane_u32(chi, L), hi = N, chi_b = T;
      start = lo;
    }
    for (int round = 0; hi - lo > 1u && round < 8; ++round) {
      uint32_t kj;
      if (hi - lo <= 64u) kj = lo + lane;
      else if (round == 0) kj = start + lane;
      else kj = lo + (uint32_t)(((uint64_t)(hi - lo) * lane) >> 6);
      const bool valid = kj < hi;
      const uint32_t cj = cum_rank<SYM, TAB>(t, valid ? kj : lo, mL, sL);
      const uint64_t bal = __ballot(valid && mul24(rL, cj << up) <= dL);
      if (bal == 0) {  // even the first probe lies above the answer
        hi = lane_u32(kj, 0);
        chi_b = lane_u32(cj, 0);
        continue;
      }
      const int js = 63 - __builtin_clzll(bal);
      lo = lane_u32(kj, js);
      clo_b = lane_u32(cj, js);
      if (js < 63 && ((__ballot(valid) >> (js + 1)) & 1)) {
        hi = lane_u32(kj, js + 1);
        chi_b = lane_u32(cj, js + 1);
      }
    }
    if (lane == (uint32_t)L) {
      gs = BF ? unrank_bf16(lo) : unrank_e4m3(lo);
      clo = clo_b;
      chi = chi_b;
      const uint64_t plo = mul24(r, clo << up);
      pf = mul24(r, (chi - clo) << up);
      dd = d - plo;
      if (hi - lo != 1u || d < plo || dd >= pf) {  // no symbol holds d
        corrupt = true;
        dd = 0;
        pf = (uint64_t)r << 16;  // keeps the renormalisation within 3 bytes
      }
    }
  }
}

// Decode one symbol of a lane: returns its pattern and advances the coder.
// FULL: every lane of the wave is active (full batches), so a miss is always
// resolved by the whole wave and the lane-alone search is not compiled in; the
// batch loop inlines this eight times, and the smaller code stays in the
// instruction cache.
template <int SYM, int MU, int TAB, bool FULL>
__device__ __forceinline__ uint32_t decode_symbol(const DecArgs &a, const ModelTabs &t, const float2 *uinv,
                                                  LaneReader &br, uint64_t &d, uint32_t &r,
                                                  bool &corrupt, float m, uint32_t mraw, float sj, float sinvj) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  constexpr int up = BF ? 0 : 8;
  __builtin_assume(r < (1u << 24));
  // ---- guess: invert the Gaussian pair's CDF at t - A(k), first with k the
  // rank of mu, then with k the rank of that first guess (the one-count floor
  // makes A(k) grow by one per rank, which matters near zero)
  // t = d / r in units of the inverse table's step
  const float ts = (float)(uint32_t)(d >> 16) * (a.inv_step * 65536.0f * __builtin_amdgcn_rcpf((float)(r << up)));
  // (any start serves: a non-finite bf16 mean starts from its own pattern)
  uint32_t kmu;
  if (BF) kmu = tix_bf16(MU == SKV_MU_F32 ? bf16_rne_bits(m) : mraw);
  else kmu = e4m3_rne_bits(m);
  // the first guess at a table point (A/B runs, k_decode: e4m3 with the point
  // below t -1.4% on the 32K e4m3 cache and -2.7% on the 0.6B one, with the
  // nearest point slower; bf16 with the nearest point -1.5% on the 32B cache,
  // with the point below t unchanged; a second guess at a table point too
  // +6% on e4m3)
  uint32_t gs = guess_symbol<SYM, TAB, BF ? kGuessNearest : kGuessFloor>(t, uinv, ts, kmu, a.inv_step, sinvj, m);
  gs = guess_symbol<SYM, TAB>(t, uinv, ts, BF ? tix_bf16(gs) : gs, a.inv_step, sinvj, m);
  // ---- verify exactly
  uint32_t clo, chi;
  uint64_t dd, pf;
  bool below;
  const bool ok = verify<SYM, TAB>(t, gs, m, sj, d, r, up, clo, chi, dd, pf, below);
  if (__builtin_expect(__any(!ok), 0)) {
    if (FULL || __ballot(1) == ~0ull) resolve_misses<SYM, TAB>(t, !ok, below, gs, clo, chi, m, sj, d, r, dd, pf, corrupt);
    else resolve_alone<SYM, TAB>(t, ok, below, gs, clo, chi, m, sj, d, r, dd, pf, corrupt);
  }
  // ---- update and renormalise
  const uint32_t n8 = __builtin_clz((uint32_t)(pf >> 16)) & 24u;  // pf >= r >= 2^16: clz & ~7
  d = br.shift_in(dd, n8);
  r = __builtin_amdgcn_alignbit((uint32_t)(pf >> 32), (uint32_t)pf, 24u - n8);  // (pf << n8) >> 24 < 2^24
  return gs;
}

// AD: adaptive p_hat (e4m3): the wave's pair table and counts in `aw`, reset
// from the block's static pairs and prior at every chunk, rebuilt every epoch
// from the symbols decoded so far (the encoder rebuilds from the same ones).
template <int SYM, int MU, int PER, int OCT, int TAB, bool AD>
__device__ __forceinline__ void decode_chunks(const DecArgs &a, const ModelTabs &t0, const float2 *uinv, AdaptLds *aw,
                                              const uint32_t *s_pairs, const uint32_t *s_prior) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  const Geo &g = a.g;
  ModelTabs t = t0;
  if (AD) t.ab = aw->pairs;
  const int lane = threadIdx.x & 63;
  const uint32_t D = (uint32_t)g.D;
  constexpr int kStep = kLanes * kBatch;  // scalars of one batch of the wave
  for (;;) {
    // chunk ids in increasing order from a counter: a wave that finishes
    // early takes more, so no wave waits on a fixed share at the end
    uint32_t cid = 0;
    if (lane == 0) cid = atomicAdd(a.ctr, 1u);
    const int64_t chunk = (int64_t)__builtin_amdgcn_readfirstlane(__shfl(cid, 0, 64));
    if (chunk >= g.n_chunks) break;
    const int64_t row = chunk / g.ntb, blk = chunk - row * g.ntb;
    const int64_t tok = min<int64_t>(kChunkTokens, g.tokens - blk * kChunkTokens);
    const int nsc = (int)(tok * g.D);
    const int64_t base = (row * g.tokens + blk * kChunkTokens) * g.D;

    // ---- header: lane lengths, the interleaved word count m, the tails' offsets
    const uint64_t o0 = a.offsets[chunk], o1 = a.offsets[chunk + 1];
    const uint64_t nbytes = o1 >= o0 ? o1 - o0 : 0;
    bool corrupt = o1 < o0 || o1 > a.bits_bytes || nbytes < (uint64_t)kHeaderBytes || (o0 & 3u) != 0 ||
                   nbytes > 0xFFFFFFFFull;
    uint32_t len = corrupt ? 0u : (uint32_t) reinterpret_cast<const uint16_t *>(a.bits + o0)[lane];
    uint32_t mw = len >> 2;
    for (int off = 32; off > 0; off >>= 1) mw = min(mw, (uint32_t)__shfl_xor((int)mw, off, 64));
    uint32_t inc = len - 4u * mw;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(inc, off, 64);
      if (lane >= off) inc += v;
    }
    const uint32_t tails = __shfl(inc, 63, 64);
    const uint64_t total = (uint64_t)kHeaderBytes + 4ull * kLanes * mw + tails;  // = 128 + sum of lengths
    if (!corrupt && ((total + 3) & ~3ull) != nbytes) corrupt = true;
    if (len == 0) corrupt = true;
    if (__any(corrupt)) {  // the whole chunk is flagged and nothing of it is read
      set_status(a.status, SKV_ERR_CORRUPT);
      continue;
    }
    LaneReader br;
    // the chunk's start is the same for the whole wave: in SGPRs, so the
    // lanes' stream reads take a scalar base and a 32-bit lane offset
    br.chunk = a.bits + (((uint64_t)lane_u32((uint32_t)(o0 >> 32), 0) << 32) | lane_u32((uint32_t)o0, 0));
    br.csize = (uint32_t)nbytes;
    br.m = mw;
    br.tail = kHeaderBytes + 4u * kLanes * mw + inc - (len - 4u * mw);
    br.len = len;
    br.init((uint32_t)lane);
    uint64_t d = (uint64_t)br.take(24) << 24;
    d |= br.take(24);
    uint32_t range = (uint32_t)(kW48 >> 24);
    if (AD) adapt_start(*aw, s_pairs, s_prior, lane);

    // ---- symbols: lane l decodes scalars l, l + 64, ... of the chunk; symbol
    // k has channel (l + 64 k) mod D, which repeats with period PER = max(2, D / 64),
    // a divisor of kBatch
    float s[PER], sinv[PER];
    int32_t er[PER];  // octave mode: the channels' octave references
    uint32_t cb[PER]; // octave mode: the channels' column in the row's [octave][d] scale table
    const float2 *srow = a.scale + (OCT ? row * kOctaves * g.D : 0);
    const uint32_t lgD = (uint32_t)__builtin_ctz(D);
    // octave mode, full batches: the row's table from scalar registers, a
    // scale pair at byte offset (octave << (lgD + 3)) + 8 d
    const char *srow_b = reinterpret_cast<const char *>(OCT ? wave_uniform(srow) : srow);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t ch = row * g.D + ((lane + kLanes * j) & (D - 1));
      if (OCT) {
        er[j] = a.eref[ch];
        cb[j] = (uint32_t)((lane + kLanes * j) & (D - 1));
      } else {
        const float2 sc = a.scale[ch];
        s[j] = sc.x;
        sinv[j] = sc.y;
      }
    }
    // wait for the scales here: a wait inside the symbol loop would also wait
    // for the loads in flight on every trip
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (OCT) asm volatile("" ::"v"(er[j]));
      else asm volatile("" ::"v"(s[j]), "v"(sinv[j]));
    }
    const void *mu_ch = MU == SKV_MU_BF16 ? (const void *)(static_cast<const uint16_t *>(a.mu) + base)
                                          : (const void *)(static_cast<const float *>(a.mu) + base);
    void *x_ch = BF ? (void *)(static_cast<uint16_t *>(a.x_out) + base) : (void *)(static_cast<uint8_t *>(a.x_out) + base);
    const int nk = lane < nsc ? (nsc - lane + kLanes - 1) / kLanes : 0;
    const int nfull = nsc / kStep;
    // two mean buffers used by turns (the next batch loads into the other
    // one), so no batch is copied from one set of registers to the other
    MuBatch<MU> mA, mB;
    if (nfull > 0) {
      mA.load_full(mu_ch, lane);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) asm volatile("" ::"v"(mA.v[j]));
    }
    auto batch = [&](int b, MuBatch<MU> &cur, MuBatch<MU> &nxt) __attribute__((always_inline)) {
      const uint32_t i0 = (uint32_t)lane + (uint32_t)b * kStep;
      // this batch's means were loaded one batch ago; wait for them here, once
      // per batch, and not inside the symbols
#pragma unroll
      for (int j = 0; j < kBatch; ++j) asm volatile("" ::"v"(cur.v[j]));
      // octave mode: the batch's scales, read at its start (the means are here)
      // and before the next batch's loads: loads complete in order, so the
      // first symbol's wait for them leaves the next batch in flight
      float2 sb[kBatch];
      float mj[kBatch];  // (octave mode: the means, converted once)
      if (OCT) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          mj[j] = cur.get(j);
          sb[j] = *reinterpret_cast<const float2 *>(srow_b + ((octave_of(mj[j], er[j % PER]) << (lgD + 3)) +
                                                             (cb[j % PER] << 3)));
        }
      }
      if (b + 1 < nfull) nxt.load_full(mu_ch, i0 + kStep);  // in flight meanwhile
      if (AD && b > 0 && b % kAdaptBatches == 0) adapt_rebuild(*aw, g.Mp, lane);  // a new epoch
      uint32_t packed[AD ? kBatch / 4 : 1];  // the batch's e4m3 symbols, four to a word (adaptive mode)
      br.top_up();
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const uint32_t gs =
            decode_symbol<SYM, MU, TAB, true>(a, t, uinv, br, d, range, corrupt, OCT ? mj[j] : cur.get(j), cur.v[j],
                                        OCT ? sb[j].x : s[j % PER], OCT ? sb[j].y : sinv[j % PER]);
        if (AD) packed[j / 4] = (j % 4 == 0 ? 0u : packed[j / 4]) | (gs << (8 * (j % 4)));
        if (BF) static_cast<uint16_t *>(x_ch)[i0 + kLanes * j] = (uint16_t)gs;
        else static_cast<uint8_t *>(x_ch)[i0 + kLanes * j] = (uint8_t)gs;
      }
      // the batch's symbols join the epoch's counts after its table reads
      // (LDS operations complete in order: an atomic among the reads would make
      // every later read wait for it)
      if (AD) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) adapt_count(*aw, (packed[j / 4] >> (8 * (j % 4))) & 0xFFu);
      }
    };
    for (int b = 0; b < nfull; b += 2) {
      batch(b, mA, mB);
      if (b + 1 < nfull) batch(b + 1, mB, mA);
    }
    MuBatch<MU> &cur = mA;
    // the last, partial batch of a short chunk: symbol by symbol (an epoch
    // boundary can only fall at its start)
    if (AD && nfull > 0 && nfull % kAdaptBatches == 0 && nsc > nfull * kStep) adapt_rebuild(*aw, g.Mp, lane);
    for (int k = nfull * kBatch; k < nk; ++k) {
      const uint32_t i = (uint32_t)lane + (uint32_t)k * kLanes;
      const int j = k & (kBatch - 1);
      const uint32_t mraw = cur.one(mu_ch, i);
      const float m = MU == SKV_MU_BF16 ? mu_from_bf16(mraw) : mu_from_f32(__uint_as_float(mraw));
      float sj, sij;
      if (OCT) {
        int32_t e = er[0];
        uint32_t b0 = cb[0];
#pragma unroll
        for (int q = 1; q < PER; ++q) {
          if (j % PER == q) {
            e = er[q];
            b0 = cb[q];
          }
        }
        const float2 sc = srow[(octave_of(m, e) << lgD) + b0];
        sj = sc.x;
        sij = sc.y;
      } else {
        sj = s[0];
        sij = sinv[0];
#pragma unroll
        for (int q = 1; q < PER; ++q) {
          if (j % PER == q) {
            sj = s[q];
            sij = sinv[q];
          }
        }
      }
      const uint32_t gs = decode_symbol<SYM, MU, TAB, false>(a, t, uinv, br, d, range, corrupt, m, mraw, sj, sij);
      if (AD) adapt_count(*aw, gs);
      if (BF) static_cast<uint16_t *>(x_ch)[i] = (uint16_t)gs;
      else static_cast<uint8_t *>(x_ch)[i] = (uint8_t)gs;
    }
    // a substream of n renormalisations holds n + 1 bytes
    if (br.renorm_bytes() + 1 != len) corrupt = true;
    if (corrupt) set_status(a.status, SKV_ERR_CORRUPT);
  }
}

// The decoder's LDS tables in one block, the small ones first: every table
// then starts below 64 KB, so a table read takes its base as the LDS
// instruction's immediate offset and its index by one shift (a separate base
// register costs a three-operand shift-add, twice the issue time of a shift).
template <bool AD>
struct alignas(16) DecAdaptBlock {
  uint32_t prior[256];
  AdaptLds w[kDecWaves];
};
template <>
struct DecAdaptBlock<false> {};

template <bool BF, bool AD>
struct DecLds {
  float4 ep[BF || AD ? 1 : 256];  // static e4m3: bins and p_hat pairs by pattern
  float2 kn[kNKnot];
  float2 ui[kNInv + 1];
  uint32_t ab[BF ? kNWin + 2 : (AD ? 512 : 2)];  // (even length: the next table stays 8-byte aligned)
  float2 et[BF || !AD ? 1 : 256];
  uint32_t a16w[BF ? kNWin * kWinEntries / 2 : 1];
  DecAdaptBlock<AD> ad;
};

// Threads per block: the static e4m3 kernels in channel mode with head_dim
// up to 256 have 28 KB of LDS tables and fit 5 waves per SIMD in registers,
// so they run as 256-thread blocks, 5 to a CU; the others keep one 1024-thread
// block per CU (the bf16 tables fill the LDS, the adaptive kernels keep 16
// waves' tables beside them, and the octave and 512-channel e4m3 kernels would
// spill at 96 registers).
template <int SYM, int PER, int OCT, int AD>
struct DecBlockOf {
  static constexpr bool small = SYM != SKV_SYM_BF16 && !AD && !OCT && PER <= 4;
  static constexpr int value = small ? 256 : kDecBlock;
  static constexpr int per_cu = small ? 5 : 1;
};

template <int SYM, int MU, int PER, int OCT, int AD>
__global__ __attribute__((amdgpu_flat_work_group_size(1, DecBlockOf<SYM, PER, OCT, AD>::value),
                          amdgpu_waves_per_eu(DecBlockOf<SYM, PER, OCT, AD>::small ? 5 : 4)))
void k_decode(DecArgs a) {
  constexpr int kB = DecBlockOf<SYM, PER, OCT, AD>::value;
  constexpr bool BF = SYM == SKV_SYM_BF16;
  static_assert(!(BF && AD), "adaptive p_hat is e4m3 only");
  __shared__ DecLds<BF, AD != 0> lds;
  float2 *s_kn = lds.kn;
  float2 *s_ui = lds.ui;
  uint32_t *s_a16w = lds.a16w;
  uint32_t *s_ab = lds.ab;
  float2 *s_et = lds.et;

  const bool win = BF ? *a.aflag != 0 : true;
  for (int i = threadIdx.x; i < kNKnot; i += kB) s_kn[i] = a.knots[i];
  for (int i = threadIdx.x; i <= kNInv; i += kB) s_ui[i] = a.uinv[i];
  if (BF) {
    if (win) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(a.a16);
      for (int i = threadIdx.x; i < kNWin * kWinEntries / 2; i += kB) s_a16w[i] = src[i];
      for (int i = threadIdx.x; i <= kNWin; i += kB) s_ab[i] = a.abase[i];
    }
  } else if (AD) {
    // (A(k), A(k + 1)) side by side at the pattern of rank k
    for (int i = threadIdx.x; i < 512; i += kB) s_ab[i] = a.ptab[(tix_e4m3((uint32_t)i >> 1) ^ 0x80u) + (i & 1)];
    for (int i = threadIdx.x; i < 256; i += kB) s_et[i] = a.etab[i];
  } else {
    for (int i = threadIdx.x; i < 256; i += kB) {
      const uint32_t j = tix_e4m3((uint32_t)i) ^ 0x80u;
      const float2 e = a.etab[i];
      lds.ep[i] = make_float4(e.x, e.y, __uint_as_float(a.ptab[j]), __uint_as_float(a.ptab[j + 1]));
    }
  }
  AdaptLds *aw = nullptr;
  const uint32_t *s_prior = nullptr;
  if constexpr (AD != 0) {
    for (int i = threadIdx.x; i < 256; i += kB) lds.ad.prior[i] = a.prior[i];
    aw = &lds.ad.w[__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))];
    s_prior = lds.ad.prior;
  }
  __syncthreads();
  const ModelTabs t{s_kn, reinterpret_cast<const uint16_t *>(s_a16w), s_ab, a.ptab, s_et, lds.ep};
  // static e4m3: guesses, verify and probes read the per-pattern table (no
  // table index per lookup; k_decode -2% on the 0.6B e4m3 cache, -0.7% on the
  // 32K one), which replaces the bins and the rank-ordered pairs in LDS
  if constexpr (!BF && AD == 0) {
    decode_chunks<SYM, MU, PER, OCT, kTabPattern, false>(a, t, s_ui, aw, s_ab, s_prior);
  } else {
    if (!BF || win) decode_chunks<SYM, MU, PER, OCT, kTabLdsAll, AD != 0>(a, t, s_ui, aw, s_ab, s_prior);
    else decode_chunks<SYM, MU, PER, OCT, kTabGlobal, AD != 0>(a, t, s_ui, aw, s_ab, s_prior);
  }
}

template <int SYM, int MU, int PER, int OCT, int AD>
static void launch_dec_one(const DecArgs &a, hipStream_t st) {
  using B = DecBlockOf<SYM, PER, OCT, AD>;
  const int64_t need = (a.g.n_chunks + B::value / 64 - 1) / (B::value / 64);
  const int64_t slots = device_cu_count() * B::per_cu;
  const unsigned blocks = (unsigned)(need < slots ? need : slots);
  hipLaunchKernelGGL((k_decode<SYM, MU, PER, OCT, AD>), dim3(blocks), dim3(B::value), 0, st, a);
}

template <int SYM, int MU, int AD>
static void launch_dec_kernel(const DecArgs &a, hipStream_t st) {
  // the scale period of a lane's symbols: max(2, head_dim / 64); the sigma mode
  const int per = a.g.D >= 512 ? 8 : (a.g.D >= 256 ? 4 : 2);
  if (a.g.octave) {
    if (per == 8) launch_dec_one<SYM, MU, 8, 1, AD>(a, st);
    else if (per == 4) launch_dec_one<SYM, MU, 4, 1, AD>(a, st);
    else launch_dec_one<SYM, MU, 2, 1, AD>(a, st);
  } else {
    if (per == 8) launch_dec_one<SYM, MU, 8, 0, AD>(a, st);
    else if (per == 4) launch_dec_one<SYM, MU, 4, 0, AD>(a, st);
    else launch_dec_one<SYM, MU, 2, 0, AD>(a, st);
  }
}

hipError_t launch_decode(const Geo &g, const uint8_t *bits, uint64_t bits_bytes, const uint64_t *offsets,
                         const void *mu, const Workspace &ws, void *x_out, int32_t *status, hipStream_t st) {
  DecArgs a{g, bits, bits_bytes, offsets, mu, ws.knots, ws.ptab, ws.a16, ws.abase, ws.aflag, ws.uinv, ws.etab,
            ws.prior, ws.scale, ws.eref, (float)kNInv / (float)g.MG, x_out, status, ws.ctr};
  timing_mark(kTimeDecode, false, st);
  if (g.sym_fmt == SKV_SYM_BF16) {
    if (g.mu_fmt == SKV_MU_BF16) launch_dec_kernel<SKV_SYM_BF16, SKV_MU_BF16, 0>(a, st);
    else launch_dec_kernel<SKV_SYM_BF16, SKV_MU_F32, 0>(a, st);
  } else if (g.adapt) {
    if (g.mu_fmt == SKV_MU_BF16) launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_BF16, 1>(a, st);
    else launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_F32, 1>(a, st);
  } else {
    if (g.mu_fmt == SKV_MU_BF16) launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_BF16, 0>(a, st);
    else launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_F32, 0>(a, st);
  }
  timing_mark(kTimeDecode, true, st);
  return hipGetLastError();
}

}  // namespace skv
