// skv_internal.hpp -- shared definitions of the HIP implementation (gfx950).
//
// The model and stream format implemented here (constants, bins, the knot
// table of the Gaussian pair, the p_hat table, the range coder, chunks and
// lanes) are those of speculative KV coding: q = 0.95 N(mu, sigma^2) +
// 0.03 N(mu, (3 sigma)^2) + 0.02 p_hat integrated over each symbol's bin
// ("Speculative KV coding", sections "q 应是什么样的", "早期结果",
// "原生 FP8 KV 缓存"), made integer with a one-count floor per symbol and
// coded by a 48-bit byte range coder in 64 lane substreams per chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skv.h"

namespace skv {

constexpr int kChunkTokens = 256;
constexpr int kLanes = 64;        // one wavefront: one lane per substream
constexpr int kBatch = 8;         // symbols a lane loads ahead at a time
constexpr int kKnotsPerUnit = 64; // knot spacing 1/64 in z
constexpr int kUMax = 1024;       // knots cover |z| <= 16
constexpr int kNKnot = 2 * kUMax + 1;
constexpr int kHeaderBytes = 2 * kLanes;
constexpr int kWavesPerBlock = 4;
// bf16 p_hat table as held in LDS: windows of 64 ranks, each stored as 65 u16
// offsets from the window's u32 base (the 65th is the next window's first rank),
// so A(k) and A(k+1) come from one window: 133 KB + 4 KB for all 65536 ranks.
constexpr int kWinRanks = 64;
constexpr int kWinEntries = kWinRanks + 1;
constexpr int kNWin = 65536 / kWinRanks;
// inverse of the Gaussian-pair CDF (counts -> knot coordinate), decoder guesses
constexpr int kNInv = 1024;
constexpr int kOctaves = SKV_OCTAVES;
constexpr int kExpBins = 256;  // fp32 exponent fields (calibration bins in octave mode)
// adaptive p_hat (e4m3): epoch length in scalars of a chunk, the prior's
// weight, alpha = 1 - 2^-kAdaptDecayShift per epoch
constexpr int kAdaptEpoch = SKV_ADAPT_EPOCH;
constexpr uint32_t kAdaptPriorWeight = SKV_ADAPT_PRIOR_WEIGHT;
constexpr int kAdaptDecayShift = 2;
constexpr int kAdaptBatches = kAdaptEpoch / (64 * 8);  // wave batches of 8 symbols per lane in an epoch
constexpr uint64_t kW48 = 0xFFFFFFFFFFFFull;
constexpr uint64_t kTop40 = 1ull << 40;

// Everything a kernel needs to know about the shape and the model constants.
struct Geo {
  int64_t layers, heads, tokens, D;
  int64_t ntb;       // 256-token blocks per row
  int64_t rows;      // layers * 2 * heads
  int64_t n_chunks;
  int sym_fmt, mu_fmt;
  int octave;        // sigma per (channel, octave of |mu'|) instead of per channel
  int adapt;         // adaptive p_hat (e4m3): per-chunk decayed counts, tables rebuilt every epoch
  uint32_t N;        // alphabet: 65536 or 256
  uint32_t log2T;    // 24 or 16
  uint32_t MG, Mp;   // Gaussian-pair and p_hat budgets, MG + Mp = 2^log2T - N
  uint32_t lane_cap; // encoder scratch bytes per lane (multiple of 4)
  int64_t enc_blocks; // encoder grid: min(chunks / 16 rounded up, compute units); two scratch slots per wave
};

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Optional per-kernel timing (skv_timing_start .. skv_timing_stop): while it
// is on, timing_mark records a HIP event on `st` before (end = false) and after
// (end = true) each main launch.
enum TimedKernel { kTimeModel = 0, kTimeEncode, kTimeDecode, kTimeCount };
void timing_mark(int kernel, bool end, hipStream_t st);

// ---- workspace layout (encode and decode share it) ----
struct Workspace {
  float2 *knots;      // kNKnot (K_j, K_{j+1} - K_j)
  uint32_t *ptab;     // N + 1: A(k) = k + Qhat(k)
  uint16_t *a16;      // kNWin * kWinEntries: A(64w + j) - A(64w) (bf16)
  uint32_t *abase;    // kNWin + 1: A(64w)
  int32_t *aflag;     // 1 when every window's offsets fit 16 bits
  uint64_t *psum;     // per 1024 ranks: sum of hist + 1 (table build)
  float2 *uinv;       // kNInv + 1: (u, du) at y = m * MG / kNInv
  float2 *etab;       // 256 e4m3 bins (lo, hi), indexed by pattern
  uint32_t *prior;    // adaptive p_hat: the decayed counts C_0, at the symbols' patterns
  float2 *scale;      // per channel (octave mode: per channel and octave): (s, ~1/s), s = RN32(64 / max(sigma, 2^-100))
  int32_t *eref;      // octave mode, per channel: E(max(sigma_c, 2^-100)) + 1; octave = clamp(E(mu') - eref, 0, 7)
  uint64_t *flags;    // n_chunks published sizes / prefixes (encode)
  uint32_t *ctr;      // next chunk id (encode)
  uint8_t *scratch;   // 2 slots per encoder wave (enc_blocks * 16 waves), 64 * lane_cap bytes each (encode)
};

// ---- symbol order ----
__device__ __forceinline__ uint32_t rank_bf16(uint32_t b) { return b ^ ((b & 0x8000u) ? 0xFFFFu : 0x8000u); }
__device__ __forceinline__ uint32_t unrank_bf16(uint32_t k) { return k ^ ((k & 0x8000u) ? 0x8000u : 0xFFFFu); }
// Index of bf16 pattern b in the device image of the p_hat window table:
// rank_bf16(b) ^ 0x8000, that is b for b < 0x8000 and b ^ 0x7FFF above (two
// instructions: a sign-bit extract and one bitwise op).  The image stores the
// window of ranks [64 w, 64 w + 64) in slot w ^ (kNWin / 2), so consecutive
// ranks of a window stay consecutive.
__device__ __forceinline__ uint32_t tix_bf16(uint32_t b) {
  // neg = all ones for b >= 0x8000 (bit 15 sign-extended), then b ^ (neg & 0x7FFF)
  // as one three-input bitwise op (truth table 0x6c over (neg, b, 0x7FFF));
  // written out because the compiler turns the plain C into compare + select + xor
  uint32_t t;
  asm("v_bfe_i32 %0, %1, 15, 1\n\tv_bitop3_b32 %0, %0, %1, %2 bitop3:0x6c" : "=&v"(t) : "v"(b), "s"(0x7FFFu));
  return t;
}
__device__ __forceinline__ uint32_t rank_e4m3(uint32_t b) { return b ^ ((b & 0x80u) ? 0xFFu : 0x80u); }
// e4m3 table index of pattern b < 256: rank ^ 0x80 = b ^ (b >= 0x80 ? 0x7F : 0),
// the same two instructions as tix_bf16 on 8 bits
__device__ __forceinline__ uint32_t tix_e4m3(uint32_t b) {
  uint32_t t;
  asm("v_bfe_i32 %0, %1, 7, 1\n\tv_bitop3_b32 %0, %0, %1, %2 bitop3:0x6c" : "=&v"(t) : "v"(b), "s"(0x7Fu));
  return t;
}
__device__ __forceinline__ uint32_t unrank_e4m3(uint32_t k) { return k ^ ((k & 0x80u) ? 0x80u : 0xFFu); }

// bf16 bin of pattern b: the fp32 values that round (nearest-even) to b.
// Magnitude m in [1, 0x7F7F]: [m - half ulp, m + half ulp] in fp32 bit
// arithmetic; +-0 meet at 0; +-inf reach +-inf; NaN bins are empty at +-inf.
__device__ __forceinline__ void bf16_bin(uint32_t b, float &lo, float &hi) {
  uint32_t m = b & 0x7FFFu;
  uint32_t sh = m << 16;
  uint32_t a = m == 0 ? 0u : sh - 0x8000u;
  uint32_t c = sh + 0x8000u;
  if (m >= 0x7F80u) {
    c = 0x7F800000u;
    if (m > 0x7F80u) a = 0x7F800000u;
  }
  uint32_t sgn = (b & 0x8000u) << 16;
  lo = __uint_as_float(sgn ? (c | sgn) : a);
  hi = __uint_as_float(sgn ? (a | sgn) : c);
}

// (b << 16) | 0x8000 for a bf16 pattern b < 2^16: the fp32 bits of the bin
// edge half an ulp beyond b's magnitude (the upper edge for b > 0, the lower
// one for b < 0; the other edge is these bits less 0x10000).  spm gets the
// wave's mask of lanes whose b may be special (+-0, +-inf, NaN: bins that need
// bf16_bin), from one class test of the pattern read as fp32 (signaling and
// quiet NaN, -inf, -0, +0, +inf), so the common case costs a shift, an or and
// the test, and the branch on the mask is scalar.  A lane the test flags by
// mistake would only take the general edges, which hold for every pattern.
__device__ __forceinline__ uint32_t bf16_hi_bits(uint32_t b, uint64_t &spm) {
  const uint32_t bf = b << 16;
  // written out: the compiler's own form of this test goes through fp64
  asm("v_cmp_class_f32_e64 %0, %1, %2" : "=s"(spm) : "v"(bf), "s"(0x267u));
  uint32_t e;
  asm("v_or_b32 %0, 0x8000, %1" : "=v"(e) : "v"(bf));  // an or, not the shift-or the compiler would fuse
  return e;
}
// the lane's own test: magnitude 0 or at least 0x7F80
__device__ __forceinline__ bool bf16_special(uint32_t b) { return ((b << 17) - (1u << 17)) >= (0x7F7Fu << 17); }

__device__ __forceinline__ float bf16_lo_edge(uint32_t b) {
  float lo, hi;
  bf16_bin(b, lo, hi);
  return lo;
}

// a pointer that is the same for the whole wave, moved to scalar registers so
// that loads through it take a scalar base and a 32-bit lane offset
template <typename T>
__device__ __forceinline__ const T *wave_uniform(const T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const T *>(((uint64_t)hi << 32) | lo);
}

// octave of a scalar with finite mean m in a channel with reference eref
__device__ __forceinline__ uint32_t octave_of(float m, int32_t eref) {
  const int32_t e = (int32_t)((__float_as_uint(m) >> 23) & 0xFFu);
  return (uint32_t)min(max(e - eref, 0), kOctaves - 1);
}

// predictor mean in fp32; a non-finite mean reads as 0
__device__ __forceinline__ float mu_from_bf16(uint32_t bits16) {
  float f = __uint_as_float(bits16 << 16);
  return __builtin_isfinite(f) ? f : 0.0f;
}
__device__ __forceinline__ float mu_from_f32(float f) { return __builtin_isfinite(f) ? f : 0.0f; }
// the same rule where a whole wave reads means: one class test per lane, and the
// select only on the rare step where some lane's mean is not finite
__device__ __forceinline__ float mu_finite_wave(float f) {
  const bool bad = !__builtin_isfinite(f);
  if (__builtin_expect(__any(bad), 0)) f = bad ? 0.0f : f;
  return f;
}

// knot coordinate u = RN(RN(e - mu) * s); the build turns contraction off
__device__ __forceinline__ float u_of(float e, float mu, float s) {
  float t = e - mu;
  return t * s;
}

// Gaussian-pair CDF in counts: straight line between knots 1/64 apart in z,
// at f = c - floor(c) in fp32.  v_fract_f32 returns exactly that difference
// except where it rounds to 1.0 (c in [-2^-25, 0)), where it returns the float
// just below 1; that case only reaches the knot pair at floor(c) = -1, whose
// interpolated count floors to the same integer at either f (a property of the
// knot tables of both symbol formats).
__device__ __forceinline__ uint32_t cg_eval(const float2 *__restrict__ kn, float u) {
  float c = __builtin_fminf(__builtin_fmaxf(u, -(float)kUMax), (float)kUMax);
  int i;  // floor(c) as an integer in one instruction (|c| <= 1024)
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(i) : "v"(c));
  float f = __builtin_amdgcn_fractf(c);
  float2 kd = kn[i + kUMax];
  float y = __builtin_fmaf(f, kd.y, kd.x);
  return (uint32_t)y;
}

__device__ __forceinline__ uint32_t bswap32(uint32_t v) { return __builtin_bswap32(v); }

// first error wins
__device__ __forceinline__ void set_status(int32_t *status, int32_t code) { atomicCAS(status, 0, code); }

// ---- launchers (defined in the .hip files) ----
hipError_t launch_model(const Geo &g, const float *sigma, const uint64_t *hist, const Workspace &ws,
                        int32_t *status, hipStream_t st);
hipError_t launch_encode(const Geo &g, const void *x, const void *mu, const Workspace &ws, uint8_t *bits,
                         uint64_t bits_cap, uint64_t *offsets, int32_t *status, hipStream_t st);
hipError_t launch_decode(const Geo &g, const uint8_t *bits, uint64_t bits_bytes, const uint64_t *offsets, const void *mu,
                         const Workspace &ws, void *x_out, int32_t *status, hipStream_t st);
hipError_t launch_clear_status(int32_t *status, uint32_t *ctr, hipStream_t st);
hipError_t launch_calib_reset(const Geo &g, void *state, hipStream_t st);
hipError_t launch_calib_accumulate(const Geo &g, void *state, const void *x, const void *mu, hipStream_t st);
hipError_t launch_calib_finalize(const Geo &g, const void *state, float *sigma, uint64_t *hist, hipStream_t st);

}  // namespace skv
