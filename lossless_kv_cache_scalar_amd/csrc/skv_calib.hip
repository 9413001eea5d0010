// skv_calib.hip -- calibration of sigma and p_hat on gfx950.
//
// sigma^2 = E[(KV_full - mu)^2] is the cost-minimising variance ("Speculative
// KV coding", "q 应是什么样的"), measured per (layer, kv, head, channel) on a
// small calibration set and frozen ("同一模型的优化版本", "早期结果"); p_hat is
// the calibration symbol histogram ("早期结果").  Results are deterministic:
// one thread owns a channel and sums its fp64 squares in token order, and the
// histogram uses integer atomics only.
//
// Octave mode (sigma per channel and octave of |mu'|) also keeps, per channel,
// the same sums split by the fp32 exponent field of mu'.
//
// State layout: S (fp64 [channels]) | n (u64 [channels]) | hist (u64 [N]),
// then in octave mode So (fp64 [256][channels]) | no (u64 [256][channels]),
// exponent-major so that a wave's 64 channels read one bin side by side.
#include "skv_internal.hpp"

namespace skv {

struct CalState {
  double *S;
  uint64_t *n;
  uint64_t *hist;
  double *So;    // octave mode only
  uint64_t *no;
};

static CalState cal_state(const Geo &g, void *state) {
  int64_t nch = g.rows * g.D;
  CalState c;
  c.S = static_cast<double *>(state);
  c.n = reinterpret_cast<uint64_t *>(c.S + nch);
  c.hist = c.n + nch;
  c.So = reinterpret_cast<double *>(c.hist + g.N);
  c.no = reinterpret_cast<uint64_t *>(c.So + nch * kExpBins);
  return c;
}

__global__ void k_fill_u64(uint64_t *p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_calib_reset(const Geo &g, void *state, hipStream_t st) {
  // S, n, hist (and So, no) are all 8-byte words
  int64_t words = 2 * g.rows * g.D * (g.octave ? 1 + kExpBins : 1) + g.N;
  hipLaunchKernelGGL(k_fill_u64, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     static_cast<uint64_t *>(state), words);
  return hipGetLastError();
}

__device__ __forceinline__ double e4m3_value(uint32_t b) {
  uint32_t c = b & 0x7Fu;
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -v : v;
}

// One thread per channel: over the call's tokens in order, S += RN(r * r);
// in octave mode the same square also goes to the bin of mu's exponent field.
// The loads of kCalUnroll tokens are issued before any of them is added, so a
// wave keeps that many loads of x and of mu in flight; the additions stay in
// token order.
constexpr int kCalUnroll = 8;
constexpr int kCalThreads = 256;

// Octave mode: the bins one call touches are cached in LDS. A first pass over
// the call's means finds the channel's largest exponent field emax; the window
// holds the kOctWin fields below and up to emax (from field 1) plus field 0
// (zero and subnormal means). Each window bin is read from the state before
// the first token and written back after the last, so every bin still adds its
// squares in token order, and the bin's count is kept as a u32 added to the
// state's u64 at the end. A mean below 2^-(kOctWin - 1) of the channel's
// largest updates its bin in global memory directly. (Updating every bin in
// global memory made each token wait for the previous one's store: 3.2 ms per
// call of 512 tokens on the 32B geometry.)
constexpr int kOctWin = 24;
constexpr int kOctSlots = kOctWin + 1;  // slot kOctWin holds field 0

struct CalOctLds {
  double s[kOctSlots][kCalThreads];  // [slot][thread]: a wave's 64 lanes read side by side
  uint32_t n[kOctSlots][kCalThreads];  // a launch covers at most 2^31 tokens
};
constexpr int64_t kOctSegTokens = int64_t(1) << 31;
template <int OCT>
struct CalLdsOf {
  using T = CalOctLds;
};
template <>
struct CalLdsOf<0> {
  using T = uint32_t;  // channel mode uses no LDS
};

template <int SYM, int MU, int OCT>
struct CalAcc {
  double acc;
  uint64_t cnt;
  // octave mode
  CalOctLds *lds;
  uint32_t base;  // exponent field of window slot 0
  double *So;
  uint64_t *no;
  int64_t c, nch;
  __device__ __forceinline__ void add(uint32_t xb, uint32_t mb) {
    double v;
    bool fin;
    if (SYM == SKV_SYM_BF16) {
      const float f = __uint_as_float(xb << 16);
      fin = __builtin_isfinite(f);
      v = (double)f;
    } else {
      fin = (xb & 0x7Fu) != 0x7Fu;
      v = fin ? e4m3_value(xb) : 0.0;
    }
    if (!fin) return;
    const float m = MU == SKV_MU_BF16 ? mu_from_bf16(mb) : mu_from_f32(__uint_as_float(mb));
    const double r = v - (double)m;
    const double rr = r * r;
    acc = acc + rr;
    ++cnt;
    if (OCT) {
      const uint32_t e = (__float_as_uint(m) >> 23) & 0xFFu;
      uint32_t slot = e - base;  // e < base wraps above the window
      if (slot >= (uint32_t)kOctWin) slot = kOctSlots;
      if (e == 0) slot = kOctWin;
      if (slot < (uint32_t)kOctSlots) {
        double &sv = lds->s[slot][threadIdx.x];
        sv = sv + rr;
        __hip_atomic_fetch_add(&lds->n[slot][threadIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
        const int64_t k = (int64_t)e * nch + c;
        So[k] = So[k] + rr;
        no[k] = no[k] + 1;
      }
    }
  }
};

template <int SYM, int MU, int OCT>
__global__ __launch_bounds__(kCalThreads) void k_calib_sums(const void *__restrict__ x, const void *__restrict__ mu,
                                                            double *__restrict__ S, uint64_t *__restrict__ n,
                                                            double *__restrict__ So, uint64_t *__restrict__ no,
                                                            int64_t rows, int64_t tokens, int64_t D, int64_t t0,
                                                            int64_t t1) {
  // tokens [t0, t1) of the call; only octave mode uses LDS, each thread its
  // own column of it, so no barrier
  __shared__ typename CalLdsOf<OCT>::T lds_oct;
  const int64_t nch = rows * D;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  const int64_t row = c / D, d = c % D;
  auto xload = [&](int64_t i) -> uint32_t {
    return SYM == SKV_SYM_BF16 ? (uint32_t) static_cast<const uint16_t *>(x)[i]
                               : (uint32_t) static_cast<const uint8_t *>(x)[i];
  };
  auto mload = [&](int64_t i) -> uint32_t {
    return MU == SKV_MU_BF16 ? (uint32_t) static_cast<const uint16_t *>(mu)[i] : static_cast<const uint32_t *>(mu)[i];
  };
  auto mexp = [&](uint32_t mb) -> uint32_t {
    const float m = MU == SKV_MU_BF16 ? mu_from_bf16(mb) : mu_from_f32(__uint_as_float(mb));
    return (__float_as_uint(m) >> 23) & 0xFFu;
  };
  const int64_t i0 = row * tokens * D + d;
  CalAcc<SYM, MU, OCT> a{S[c], n[c], nullptr, 0u, So, no, c, nch};
  if (OCT) {
    uint32_t emax = 0;
    int64_t t = t0;
    for (; t + kCalUnroll <= t1; t += kCalUnroll) {
      uint32_t mb[kCalUnroll];
#pragma unroll
      for (int u = 0; u < kCalUnroll; ++u) mb[u] = mload(i0 + (t + u) * D);
#pragma unroll
      for (int u = 0; u < kCalUnroll; ++u) emax = max(emax, mexp(mb[u]));
    }
    for (; t < t1; ++t) emax = max(emax, mexp(mload(i0 + t * D)));
    // a finite mean has a field of at most 254, so the window ends by 254
    a.base = emax >= (uint32_t)kOctWin ? emax - (kOctWin - 1) : 1u;
    a.lds = reinterpret_cast<CalOctLds *>(&lds_oct);
#pragma unroll
    for (int s = 0; s < kOctSlots; ++s) {
      const uint32_t e = s == kOctWin ? 0u : a.base + s;
      a.lds->s[s][threadIdx.x] = So[(int64_t)e * nch + c];
      a.lds->n[s][threadIdx.x] = 0;
    }
  }
  int64_t t = t0;
  for (; t + kCalUnroll <= t1; t += kCalUnroll) {
    uint32_t xb[kCalUnroll], mb[kCalUnroll];
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) {
      xb[u] = xload(i0 + (t + u) * D);
      mb[u] = mload(i0 + (t + u) * D);
    }
#pragma unroll
    for (int u = 0; u < kCalUnroll; ++u) a.add(xb[u], mb[u]);
  }
  for (; t < t1; ++t) a.add(xload(i0 + t * D), mload(i0 + t * D));
  S[c] = a.acc;
  n[c] = a.cnt;
  if (OCT) {
#pragma unroll
    for (int s = 0; s < kOctSlots; ++s) {
      const int64_t k = (int64_t)(s == kOctWin ? 0u : a.base + s) * nch + c;
      So[k] = a.lds->s[s][threadIdx.x];
      no[k] = no[k] + a.lds->n[s][threadIdx.x];
    }
  }
}

// Histogram: LDS counters for a window of 32768 bins, packed two 16-bit
// counts per word; a block takes a tile of at most 65535 symbols so no count
// can overflow, then adds its non-zero counts to the u64 histogram.
constexpr int kHistWindow = 32768;
constexpr int64_t kHistTile = 65535;

template <int SYM>
__global__ __launch_bounds__(1024) void k_calib_hist(const void *__restrict__ x, int64_t n, uint64_t *__restrict__ hist,
                                                     uint32_t win0) {
  __shared__ uint32_t cnt[kHistWindow / 2];
  const uint32_t nbins = SYM == SKV_SYM_BF16 ? kHistWindow : 256;
  for (uint32_t i = threadIdx.x; i < nbins / 2; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * kHistTile;
  const int64_t t1 = min<int64_t>(n, t0 + kHistTile);
  for (int64_t i = t0 + threadIdx.x; i < t1; i += blockDim.x) {
    uint32_t b = SYM == SKV_SYM_BF16 ? (uint32_t) static_cast<const uint16_t *>(x)[i]
                                     : (uint32_t) static_cast<const uint8_t *>(x)[i];
    uint32_t rel = b - win0;
    if (rel < nbins) atomicAdd(&cnt[rel >> 1], 1u << (16 * (rel & 1u)));
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nbins; i += blockDim.x) {
    uint32_t v = (cnt[i >> 1] >> (16 * (i & 1u))) & 0xFFFFu;
    if (v) atomicAdd(reinterpret_cast<unsigned long long *>(&hist[win0 + i]), (unsigned long long)v);
  }
}

hipError_t launch_calib_accumulate(const Geo &g, void *state, const void *x, const void *mu, hipStream_t st) {
  CalState cs = cal_state(g, state);
  int64_t nch = g.rows * g.D;
  dim3 grid((unsigned)((nch + kCalThreads - 1) / kCalThreads)), blk(kCalThreads);
  const int sel = (g.sym_fmt == SKV_SYM_BF16 ? 0 : 4) + (g.mu_fmt == SKV_MU_BF16 ? 0 : 2) + g.octave;
#define SKV_SUMS(S_, M_, O_)                                                                                      \
  hipLaunchKernelGGL((k_calib_sums<S_, M_, O_>), grid, blk, 0, st, x, mu, cs.S, cs.n, cs.So, cs.no, g.rows, g.tokens, \
                     g.D, t0, t1)
  // octave mode counts a window bin in 32 bits: at most 2^31 tokens per launch
  const int64_t seg = g.octave ? kOctSegTokens : g.tokens;
  for (int64_t t0 = 0; t0 < g.tokens; t0 += seg) {
    const int64_t t1 = g.tokens - t0 < seg ? g.tokens : t0 + seg;  // (HIP's host min() narrows to int)
    switch (sel) {
      case 0: SKV_SUMS(SKV_SYM_BF16, SKV_MU_BF16, 0); break;
      case 1: SKV_SUMS(SKV_SYM_BF16, SKV_MU_BF16, 1); break;
      case 2: SKV_SUMS(SKV_SYM_BF16, SKV_MU_F32, 0); break;
      case 3: SKV_SUMS(SKV_SYM_BF16, SKV_MU_F32, 1); break;
      case 4: SKV_SUMS(SKV_SYM_E4M3, SKV_MU_BF16, 0); break;
      case 5: SKV_SUMS(SKV_SYM_E4M3, SKV_MU_BF16, 1); break;
      case 6: SKV_SUMS(SKV_SYM_E4M3, SKV_MU_F32, 0); break;
      default: SKV_SUMS(SKV_SYM_E4M3, SKV_MU_F32, 1); break;
    }
  }
#undef SKV_SUMS
  int64_t total = g.rows * g.tokens * g.D;
  dim3 hgrid((unsigned)((total + kHistTile - 1) / kHistTile)), hblk(1024);
  if (g.sym_fmt == SKV_SYM_BF16) {
    for (uint32_t w = 0; w < 65536u; w += kHistWindow)
      hipLaunchKernelGGL(k_calib_hist<SKV_SYM_BF16>, hgrid, hblk, 0, st, x, total, cs.hist, w);
  } else {
    hipLaunchKernelGGL(k_calib_hist<SKV_SYM_E4M3>, hgrid, hblk, 0, st, x, total, cs.hist, 0u);
  }
  return hipGetLastError();
}

// sigma = RN32(sqrt(q)), q = RN64(S / n): start from the fp64 square root and
// settle the fp32 rounding by comparing q with the squares of the midpoints
// between neighbouring fp32 values, which fp64 holds exactly (ties to even).
__device__ float rn32_sqrt(double q) {
  float s = (float)__builtin_sqrt(q);
  for (int it = 0; it < 4; ++it) {
    if (!__builtin_isfinite(s)) break;
    uint32_t sb = __float_as_uint(s);
    float up = __uint_as_float(sb + 1);
    double mu = 0.5 * ((double)s + (double)up);
    double mu2 = mu * mu;
    if (mu2 < q || (mu2 == q && (sb & 1u))) {
      s = up;
      continue;
    }
    if (sb == 0) break;
    float dn = __uint_as_float(sb - 1);
    double md = 0.5 * ((double)s + (double)dn);
    double md2 = md * md;
    if (md2 > q || (md2 == q && (sb & 1u))) {
      s = dn;
      continue;
    }
    break;
  }
  return s;
}

__global__ void k_calib_finalize(const double *__restrict__ S, const uint64_t *__restrict__ n,
                                 const uint64_t *__restrict__ hist_in, float *__restrict__ sigma,
                                 uint64_t *__restrict__ hist_out, int64_t nch, int64_t N) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nch) sigma[i] = n[i] == 0 ? 1.0f : rn32_sqrt(S[i] / (double)n[i]);
  if (i < N) hist_out[i] = hist_in[i];
}

// Octave mode: per channel its sigma_c (as above), then per octave j the
// estimator over the exponent bins that fall in j (see skv.h), added in
// increasing exponent order, or sigma_c below 16 scalars.
__global__ void k_calib_finalize_oct(const double *__restrict__ S, const uint64_t *__restrict__ n,
                                     const double *__restrict__ So, const uint64_t *__restrict__ no,
                                     float *__restrict__ table, int64_t nch) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  const float sc = n[c] == 0 ? 1.0f : rn32_sqrt(S[c] / (double)n[c]);
  float *t = table + c * SKV_OCT_STRIDE;
  t[0] = sc;
  const int base = (int)((__float_as_uint(sc > 0x1p-100f ? sc : 0x1p-100f) >> 23) & 0xFFu) + 1;
  const double *so = So + c;  // bin e at so[e * nch]
  const uint64_t *nn = no + c;
  for (int j = 0; j < kOctaves; ++j) {
    // exponent fields of octave j: [0, base] for j = 0, base + j for 0 < j < 7, [base + 7, 255] for j = 7
    const int e0 = j == 0 ? 0 : base + j;
    const int e1 = j == kOctaves - 1 ? kExpBins - 1 : (j == 0 ? base : base + j);
    double sj = 0.0;
    uint64_t nj = 0;
    for (int e = e0; e <= e1 && e < kExpBins; ++e) {
      sj = sj + so[(int64_t)e * nch];
      nj += nn[(int64_t)e * nch];
    }
    t[1 + j] = nj < 16 ? sc : rn32_sqrt(sj / (double)nj);
  }
}

hipError_t launch_calib_finalize(const Geo &g, const void *state, float *sigma, uint64_t *hist, hipStream_t st) {
  CalState cs = cal_state(g, const_cast<void *>(state));
  int64_t nch = g.rows * g.D;
  int64_t m = nch > (int64_t)g.N ? nch : (int64_t)g.N;
  // channel sigmas (overwritten by the octave tables below in octave mode) and the histogram
  hipLaunchKernelGGL(k_calib_finalize, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, cs.S, cs.n, cs.hist,
                     g.octave ? nullptr : sigma, hist, g.octave ? 0 : nch, (int64_t)g.N);
  if (g.octave)
    hipLaunchKernelGGL(k_calib_finalize_oct, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, cs.S, cs.n, cs.So,
                       cs.no, sigma, nch);
  return hipGetLastError();
}

}  // namespace skv
