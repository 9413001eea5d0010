// skv_modeldev.hpp -- the integer frequency model as device code, shared by the
// encoder and the decoder so that both take every integer decision the same way.
//
// cum_lo(b) = A(rank b) + Cg(u(lo(b))), cum_hi(b) = A(rank b + 1) + Cg(u(hi(b))):
// the mixture q ("Speculative KV coding", "早期结果") integrated over the bin of
// b, in counts, with one count per symbol as a floor.
#pragma once

#include "skv_internal.hpp"

namespace skv {

// exact 48-bit product of two values below 2^24: v_mul_u32_u24 + v_mul_hi_u32_u24
__device__ __forceinline__ uint64_t mul24(uint32_t a, uint32_t b) {
  __builtin_assume(a < (1u << 24));
  __builtin_assume(b < (1u << 24));
  return (uint64_t)a * (uint64_t)b;
}

// Where the bf16 p_hat table A lives for a kernel.
enum { kTabGlobal = 0,    // A from global memory only (the 16-bit window image does not fit)
       kTabLdsAll = 1,    // all 1024 windows in LDS
       kTabPattern = 2 }; // static e4m3: bins and (A(k), A(k + 1)) in one table by pattern

struct ModelTabs {
  const float2 *kn;      // LDS: knots (K_j, D_j)
  const uint16_t *a16;   // LDS: window image (bf16), window slots as tix_bf16 orders them
  const uint32_t *ab;    // LDS: window bases (bf16); e4m3: (A(k), A(k + 1)) at 2 b, 2 b + 1 for the pattern b of rank k
  const uint32_t *ptab;  // global: full table A in rank order
  const float2 *et;      // LDS: e4m3 bins
  const float4 *ep;      // LDS, kTabPattern: per e4m3 pattern (lower edge, upper edge, A(k), A(k + 1))
};

// A(k) and A(k + 1) of bf16 rank k, given as its table index ti = k ^ 0x8000
template <int TAB>
__device__ __forceinline__ void a_pair(const ModelTabs &t, uint32_t ti, uint32_t &alo, uint32_t &ahi) {
  if (TAB == kTabGlobal) {
    const uint32_t k = ti ^ 0x8000u;
    alo = t.ptab[k];
    ahi = t.ptab[k + 1];
    return;
  }
  const uint32_t w = ti >> 6;
  const uint32_t e = ti + w;  // = 65 w + (ti mod 64)
  const uint32_t base = t.ab[w];
  alo = base + t.a16[e];
  ahi = base + t.a16[e + 1];
}

// A(k) alone of bf16 rank k < N, given as its table index ti = k ^ 0x8000
template <int TAB>
__device__ __forceinline__ uint32_t a_one(const ModelTabs &t, uint32_t ti) {
  if (TAB == kTabGlobal) return t.ptab[ti ^ 0x8000u];
  const uint32_t w = ti >> 6;
  // entry ti + w, addressed in bytes as one add-and-shift
  return t.ab[w] + *reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(t.a16) + ((ti + w) << 1));
}

// cum_lo and cum_hi of symbol b in model units (bf16: total 2^24, e4m3: 2^16)
template <int SYM, int TAB>
__device__ __forceinline__ void model_pair(const ModelTabs &t, uint32_t b, float m, float s, uint32_t &clo,
                                           uint32_t &chi) {
  if (SYM == SKV_SYM_BF16) {
    // p_hat part first: it depends on b alone, so its table reads are in flight
    // while the Gaussian pair is evaluated
    uint32_t alo, ahi;
    a_pair<TAB>(t, tix_bf16(b), alo, ahi);
    // The bin of a finite non-zero b is [(b-1):8000, b:8000] in fp32 bits for
    // b > 0 and the same pair swapped for b < 0; Cg is monotone, so the lower
    // count is the min of the two.  +-0, +-inf and NaN take the general edges
    // (the counts are complete before that rare branch, which redoes them, so
    // the table reads and their sums stay in one block).
    uint64_t spm;
    const uint32_t eA = bf16_hi_bits(b, spm);  // (b << 16) | 0x8000
    const uint32_t eB = eA - 0x10000u;
    const uint32_t cA = cg_eval(t.kn, u_of(__uint_as_float(eA), m, s));
    const uint32_t cB = cg_eval(t.kn, u_of(__uint_as_float(eB), m, s));
    clo = alo + min(cA, cB);
    chi = ahi + max(cA, cB);
    if (__builtin_expect(spm != 0, 0)) {
      if (bf16_special(b)) {
        a_pair<TAB>(t, tix_bf16(b), alo, ahi);
        float lo, hi;
        bf16_bin(b, lo, hi);
        clo = alo + cg_eval(t.kn, u_of(lo, m, s));
        chi = ahi + cg_eval(t.kn, u_of(hi, m, s));
      }
    }
  } else if (TAB == kTabPattern) {
    const float4 q = t.ep[b];
    clo = __float_as_uint(q.z) + cg_eval(t.kn, u_of(q.x, m, s));
    chi = __float_as_uint(q.w) + cg_eval(t.kn, u_of(q.y, m, s));
  } else {
    const float2 e = t.et[b];
    const uint2 p = reinterpret_cast<const uint2 *>(t.ab)[b];
    clo = p.x + cg_eval(t.kn, u_of(e.x, m, s));
    chi = p.y + cg_eval(t.kn, u_of(e.y, m, s));
  }
}

// cum(k) = cum_lo(unrank k) for 0 <= k < N, cum(N) = T (decoder probes)
template <int SYM, int TAB>
__device__ __forceinline__ uint32_t cum_rank(const ModelTabs &t, uint32_t k, float m, float s) {
  if (SYM == SKV_SYM_BF16) {
    if (k >= 65536u) return 1u << 24;
    // lower edge of a finite non-zero b: half an ulp below (b > 0) or above
    // (b < 0) in fp32 bits; +-0, +-inf and NaN take the general edge
    const uint32_t b = unrank_bf16(k);
    uint32_t e = (b & 0x8000u) ? ((b << 16) | 0x8000u) : ((b << 16) - 0x8000u);
    const bool special = bf16_special(b);
    if (__builtin_expect(__any(special), 0)) {
      if (special) e = __float_as_uint(bf16_lo_edge(b));
    }
    return a_one<TAB>(t, k ^ 0x8000u) + cg_eval(t.kn, u_of(__uint_as_float(e), m, s));
  } else {
    if (k >= 256u) return 1u << 16;
    if (TAB == kTabPattern) {
      const float4 q = t.ep[unrank_e4m3(k)];
      return __float_as_uint(q.z) + cg_eval(t.kn, u_of(q.x, m, s));
    }
    const uint32_t pb = unrank_e4m3(k);
    return t.ab[2u * pb] + cg_eval(t.kn, u_of(t.et[pb].x, m, s));
  }
}

}  // namespace skv
