// skv_adapt.hpp -- the adaptive p_hat of e4m3 caches, as device code shared by
// the encoder and the decoder.
//
// The online entropy-estimation page keeps decayed symbol counts, C_t(s) =
// alpha C_{t-1}(s) + delta(s, s_t) ("虚拟滑动窗口的设计原理"), one window per
// layer-head ("针对 KV 缓存的局部性优化"), rebuilds the CDF only now and then
// ("计算优化技巧": lazy rebuilds) and starts from a calibrated prior
// ("局限性与应对": cold start).  Here the window is one chunk, coded by one
// wave: the wave keeps its counts and its p_hat pair table in LDS, every lane
// adds its symbols to the counts as it codes them (integer LDS atomics, so the
// order does not matter), and after every epoch of 4096 scalars the whole wave
// rebuilds the table from the counts and decays them:
//   H(0) = 0, H(k+1) = H(k) + C(k) + 1, A(k) = k + floor(Mp H(k) / H(256)),
//   C(k) <- floor(3 C(k) / 4).
// Epoch 0 codes with the static table.  The counts start at floor(3 C_0 / 4),
// C_0 the prior (the static table's p_hat counts scaled to
// SKV_ADAPT_PRIOR_WEIGHT): the decay of an epoch's counts comes before the
// epoch adds its symbols, C_{e+1} = floor(3 C_e / 4) + n_e, and the rebuild
// at the end of epoch e therefore decays the counts after building the table.
#pragma once

#include "skv_internal.hpp"

namespace skv {

static_assert(kAdaptEpoch % (kLanes * kBatch) == 0, "an epoch is a whole number of wave batches");

// One wave's adaptive state: the pairs (A(k), A(k + 1)) at 2 b and 2 b + 1 and
// the counts at b, for the pattern b of rank k (a coded symbol reads its pair
// and adds to its count with no index arithmetic; only the rebuild maps ranks
// to patterns; pairs in rank order instead made k_encode 4% and k_decode 3-4%
// slower on the e4m3 caches).
// 16-byte aligned: a pair is read as one 64-bit LDS access, which is slow at
// an address that is not a multiple of 8.
struct alignas(16) AdaptLds {
  uint32_t pairs[512];
  uint32_t cnt[256];
};

// Every lane's LDS accesses before this point are complete and seen by every
// lane's accesses after it (one wave: its LDS operations execute in order once
// issued; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// A chunk starts from the static pairs and the decayed prior counts (both in
// the block's LDS, 512 and 256 words; the prior at the symbols' patterns).
__device__ __forceinline__ void adapt_start(AdaptLds &w, const uint32_t *__restrict__ static_pairs,
                                            const uint32_t *__restrict__ prior, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) w.pairs[lane + 64 * j] = static_pairs[lane + 64 * j];
#pragma unroll
  for (int j = 0; j < 4; ++j) w.cnt[lane + 64 * j] = prior[lane + 64 * j];
  wave_lds_sync();
}

// floor(a / b) for a < 2^31, b >= 1, a / b < 2^12: a float estimate within one
// of the quotient, then one integer correction each way.
__device__ __forceinline__ uint32_t small_quotient(uint32_t a, uint32_t b, float rb) {
  uint32_t q = (uint32_t)((float)a * rb);
  if ((q + 1u) * b <= a) ++q;
  if (q * b > a) --q;
  return q;
}

// End of an epoch: the table from the counts, then the counts decayed.  Lane l
// holds ranks 4 l .. 4 l + 3; the smoothed counts are summed in rank order by
// a wave scan.  Mp * H(256) stays below 2^31: the counts total at most the
// prior weight plus four epochs of observations.
__device__ __forceinline__ void adapt_rebuild(AdaptLds &w, uint32_t Mp, int lane) {
  wave_lds_sync();  // every lane's count of the epoch is in
  uint32_t c[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = w.cnt[unrank_e4m3((uint32_t)(4 * lane + j))];
    s += c[j] + 1u;
  }
  uint32_t inc = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(inc, off, 64);
    if (lane >= off) inc += v;
  }
  const uint32_t total = __shfl(inc, 63, 64);
  const float rt = 1.0f / (float)total;
  uint32_t H = inc - s;
  uint32_t A[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    A[j] = (uint32_t)(4 * lane + j) + small_quotient(Mp * H, total, rt);  // A(256) = 256 + Mp: H = total there
    if (j < 4) H += c[j] + 1u;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t pb = unrank_e4m3((uint32_t)(4 * lane + j));
    w.pairs[2 * pb] = A[j];
    w.pairs[2 * pb + 1] = A[j + 1];
    w.cnt[pb] = (c[j] * ((1u << kAdaptDecayShift) - 1u)) >> kAdaptDecayShift;
  }
  wave_lds_sync();
}

// a coded symbol (e4m3 pattern b) joins the counts of the epoch
__device__ __forceinline__ void adapt_count(AdaptLds &w, uint32_t b) { atomicAdd(&w.cnt[b & 0xFFu], 1u); }

}  // namespace skv
