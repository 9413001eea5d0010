// skv_model.hip -- per-call model build: knot table, p_hat table, e4m3 bins,
// per-channel scales.  Small kernels; they run before every encode / decode.
#include "skv_internal.hpp"

namespace skv {

// ---------------------------------------------------------------- knots
// Gaussian pair of the mixture, normalised to its weight 0.98 ("Speculative KV
// coding", "早期结果": 0.95 N(mu, sigma^2) + 0.03 N(mu, (3 sigma)^2)):
//   G(z) = (0.95 Phi(z) + 0.03 Phi(z / 3)) / 0.98,  Phi(x) = erfc(-x / sqrt 2) / 2.
// In counts at z = j / 64: V_j = RN32(MG G(j/64)) for 0 <= j < 1024, V_1024 = MG;
// K_j = V_j (j >= 0), MG - V_{-j} (j < 0); the table holds (K_j, K_{j+1} - K_j).
// fp64 erfc is accurate to a few ulp, far inside the distance of every knot's
// exact value from an fp32 rounding boundary, so the rounding is the exact one.
__global__ __launch_bounds__(1024) void k_knots(float2 *__restrict__ out, uint32_t MG) {
  __shared__ float V[kUMax + 1];
  __shared__ float K[kNKnot];
  const double inv_sqrt2 = 0.70710678118654752440;
  for (int j = threadIdx.x; j <= kUMax; j += blockDim.x) {
    if (j == kUMax) {
      V[j] = (float)MG;
    } else {
      double z = (double)j / (double)kKnotsPerUnit;
      double p1 = 0.5 * erfc(-z * inv_sqrt2);
      double p3 = 0.5 * erfc(-(z / 3.0) * inv_sqrt2);
      double g = (0.95 * p1 + 0.03 * p3) / 0.98;
      V[j] = (float)((double)MG * g);
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < kNKnot; j += blockDim.x) {
    int jj = j - kUMax;
    K[j] = jj >= 0 ? V[jj] : (float)MG - V[-jj];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < kNKnot; j += blockDim.x) {
    float d = j + 1 < kNKnot ? K[j + 1] - K[j] : 0.0f;
    out[j] = make_float2(K[j], d);
  }
}

// ---------------------------------------------------------------- p_hat table
// p_hat: the calibration symbol histogram, +1 smoothed, in rank order
// ("早期结果": the empirical bf16 symbol distribution).  H(0) = 0,
// H(k+1) = H(k) + hist[unrank(k)] + 1, Qhat(k) = floor(Mp H(k) / H(N));
// A(k) = k + Qhat(k) carries the one-count floor of every symbol.  The
// quotient is exact: an fp64 estimate, then integer correction steps.
// Domain: Mp * H(N) <= 2^62 with H(N) the exact sum, else SKV_ERR_TABLE and a
// uniform table (every frequency still >= 1).
__device__ __forceinline__ uint64_t floor_div(uint64_t num, uint64_t den) {
  uint64_t q = (uint64_t)((double)num / (double)den);  // within 2 of the quotient
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if (q > 0 && q * den > num) --q;
#pragma unroll
  for (int it = 0; it < 3; ++it)
    if ((q + 1) * den <= num) ++q;
  return q;
}

// Two kernels, one thread per rank, 1024 ranks per block.  k_psums: the
// counts hist[unrank k] + 1 of each block, summed.  k_ptable: H(k) from the
// block sums and a block scan, then A(k); for bf16 also the LDS image of the
// table: window w's base A(64 w) and 65 u16 offsets A(64 w + j) - A(64 w),
// j = 0..64 (window w in slot w ^ 512), clearing aflag when some window's
// offsets do not fit 16 bits.
constexpr int kPtBlock = 1024;

// Sums of counts saturate at 2^64 - 1: a total that reaches it is beyond the
// table's domain anyway, and saturating addition of unsigned values is
// min(exact sum, 2^64 - 1) whatever the order, so no wrapped total can pass
// for a small one.
__device__ __forceinline__ uint64_t sat_add(uint64_t a, uint64_t b) {
  const uint64_t s = a + b;
  return s < a ? ~0ull : s;
}

__device__ __forceinline__ uint64_t rank_count(const uint64_t *__restrict__ hist, uint32_t k, int bf16) {
  return sat_add(hist[bf16 ? unrank_bf16(k) : unrank_e4m3(k)], 1);
}

__device__ __forceinline__ uint64_t block_sum(uint64_t v, uint64_t *red) {
  for (int off = 32; off > 0; off >>= 1) v = sat_add(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t s = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s = sat_add(s, red[i]);
  return s;
}

__global__ __launch_bounds__(kPtBlock) void k_psums(const uint64_t *__restrict__ hist, uint64_t *__restrict__ psum,
                                                    int32_t *__restrict__ aflag, uint32_t N, int bf16) {
  __shared__ uint64_t red[kPtBlock / 64];
  const uint32_t k = blockIdx.x * kPtBlock + threadIdx.x;
  const uint64_t s = block_sum(k < N ? rank_count(hist, k, bf16) : 0, red);
  if (threadIdx.x == 0) psum[blockIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) *aflag = bf16 ? 1 : 0;
}

__global__ __launch_bounds__(kPtBlock) void k_ptable(const uint64_t *__restrict__ hist,
                                                     const uint64_t *__restrict__ psum, uint32_t *__restrict__ A,
                                                     uint16_t *__restrict__ a16, uint32_t *__restrict__ abase,
                                                     int32_t *__restrict__ aflag, uint32_t N, uint32_t Mp, int bf16,
                                                     int32_t *status) {
  __shared__ uint64_t scan[kPtBlock];
  const int t = threadIdx.x;
  const uint32_t nblk = gridDim.x;
  // the total and this block's base from the block sums
  uint64_t base = 0, total = 0;
  for (uint32_t i = 0; i < nblk; ++i) {
    const uint64_t v = psum[i];
    if (i < blockIdx.x) base = sat_add(base, v);
    total = sat_add(total, v);
  }
  const uint32_t k = blockIdx.x * kPtBlock + t;
  const bool active = k < N;
  const uint64_t c = active ? rank_count(hist, k, bf16) : 0;
  scan[t] = c;
  __syncthreads();
  for (int off = 1; off < kPtBlock; off <<= 1) {
    const uint64_t v = t >= off ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  const uint64_t H = base + scan[t] - c;  // H(k), exclusive
  if (total < N || (Mp != 0 && total > (1ull << 62) / Mp)) {  // uniform table: every frequency stays >= 1
    if (blockIdx.x == 0 && t == 0) {
      set_status(status, SKV_ERR_TABLE);
      *aflag = 0;
    }
    if (active) A[k] = k + (uint32_t)(((uint64_t)Mp * k) / N);
    if (k == N - 1) A[N] = N + Mp;
    return;
  }
  if (!active) return;
  const uint32_t ak = k + (uint32_t)floor_div((uint64_t)Mp * H, total);
  A[k] = ak;
  if (k == N - 1) A[N] = N + Mp;
  if (!bf16) return;
  // window image: thread j = 0 of a window holds its base; j = 63 also writes
  // entry 64, A(64 w + 64) - A(64 w).  Window w goes to slot w ^ (kNWin / 2),
  // the order in which tix_bf16 indexes it.
  const uint32_t w = k / kWinRanks, j = k % kWinRanks;
  const uint32_t ws = w ^ (uint32_t)(kNWin / 2);
  const uint32_t a0 = __shfl(ak, 0, 64);  // the window is this wave
  if (j == 0) abase[ws] = ak;
  uint32_t off = ak - a0;
  bool wide = off > 0xFFFFu;
  a16[ws * kWinEntries + j] = (uint16_t)off;
  if (j == kWinRanks - 1) {
    const uint32_t an = k + 1 + (uint32_t)floor_div((uint64_t)Mp * (H + c), total);
    const uint32_t on = an - a0;
    wide = wide || on > 0xFFFFu;
    a16[ws * kWinEntries + kWinRanks] = (uint16_t)on;
    if (w == N / kWinRanks - 1) abase[kNWin] = an;
  }
  if (__any(wide) && j == 0) atomicAnd(aflag, 0);
}

// Adaptive p_hat (e4m3): the prior, the static table's p_hat counts of each
// rank scaled to the prior weight, C_0(k) = floor(SKV_ADAPT_PRIOR_WEIGHT
// (A(k+1) - A(k) - 1) / Mp).  Stored already decayed, floor(alpha C_0(k)):
// the counts a chunk's first epoch adds its symbols to, so that the table of
// epoch 1 is built from C_1 = floor(alpha C_0) + n_0.  Stored at the
// pattern of rank k, as the kernels' count tables are.
__global__ void k_prior(const uint32_t *__restrict__ A, uint32_t *__restrict__ prior, uint32_t Mp) {
  const uint32_t k = threadIdx.x;
  if (k >= 256) return;
  const uint64_t q = (uint64_t)(A[k + 1] - A[k] - 1u) * kAdaptPriorWeight;
  const uint32_t c0 = Mp ? (uint32_t)(q / Mp) : 0u;
  prior[unrank_e4m3(k)] = (c0 * ((1u << kAdaptDecayShift) - 1u)) >> kAdaptDecayShift;  // at the symbol's pattern
}

// ---------------------------------------------------------------- inverse CDF
// For the decoder's first guess only (every decoded symbol is verified
// exactly): u at y = m * MG / kNInv on the knot table's piecewise-linear CDF,
// and the step to the next point.
__global__ __launch_bounds__(1024) void k_uinv(const float2 *__restrict__ knots, float2 *__restrict__ uinv, uint32_t MG) {
  __shared__ float U[kNInv + 1];
  for (int m = threadIdx.x; m <= kNInv; m += blockDim.x) {
    const double y = (double)m * (double)MG / (double)kNInv;
    int lo = 0, hi = kNKnot - 1;  // largest i with K_i <= y, i < kNKnot - 1
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if ((double)knots[mid].x <= y) lo = mid; else hi = mid;
    }
    const float2 kd = knots[lo];
    double u = (double)(lo - kUMax);
    if (kd.y > 0.0f) u += ((y - (double)kd.x) / (double)kd.y);
    U[m] = (float)fmin(fmax(u, -(double)kUMax), (double)kUMax);
  }
  __syncthreads();
  for (int m = threadIdx.x; m <= kNInv; m += blockDim.x)
    uinv[m] = make_float2(U[m], m < kNInv ? U[m + 1] - U[m] : 0.0f);
}

// ---------------------------------------------------------------- e4m3 bins
// OCP e4m3 (bias 7, no infinities, NaN = S.1111.111, max 448).  The bin of a
// code is its round-to-nearest-even preimage with saturation ("原生 FP8 KV
// 缓存": the FP8 symbols are coded under a bin-integrated Gaussian): edges are
// midpoints between neighbouring values, 0 splits +-0, +-448 reach +-inf,
// NaN bins are empty at +-inf.
__device__ double e4m3_mag(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8u + m), (int)e - 10);
}

__global__ void k_etab(float2 *__restrict__ etab) {
  uint32_t b = threadIdx.x;
  if (b >= 256) return;
  uint32_t m = b & 0x7Fu;
  float a, c;
  if (m == 0x7Fu) {
    a = c = __builtin_inff();
  } else {
    a = m == 0 ? 0.0f : (float)(0.5 * (e4m3_mag(m - 1) + e4m3_mag(m)));
    c = m == 0x7Eu ? __builtin_inff() : (float)(0.5 * (e4m3_mag(m) + e4m3_mag(m + 1)));
  }
  etab[b] = (b & 0x80u) ? make_float2(-c, -a) : make_float2(a, c);
}

// ---------------------------------------------------------------- scales
// s_c = RN32(64 / max(sigma_c, 2^-100)): the fp64 quotient of two fp32 values
// rounds to the same fp32 as the exact quotient (53 >= 2 * 24 + 2).
// sigma must be finite and >= 0.  The second member, an approximate 1 / s,
// only steers the decoder's first guesses.
__global__ void k_scale(const float *__restrict__ sigma, float2 *__restrict__ scale, int64_t n, int32_t *status) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float sg = sigma[i];
  if (!(sg >= 0.0f) || !__builtin_isfinite(sg)) {
    set_status(status, SKV_ERR_ARG);
    sg = 1.0f;
  }
  float sp = sg > 0x1p-100f ? sg : 0x1p-100f;
  const float sc = (float)(64.0 / (double)sp);
  scale[i] = make_float2(sc, __builtin_amdgcn_rcpf(sc));
}

// Octave mode: per channel c = row * D + d (one thread), eref = E(max(sigma_c,
// 2^-100)) + 1 and the (s, ~1/s) of its eight octave sigmas, from the
// SKV_OCT_STRIDE table, stored at [row][octave][d] so that the lanes of a wave
// (consecutive channels of one row) read side by side.
__global__ void k_scale_oct(const float *__restrict__ table, float2 *__restrict__ scale, int32_t *__restrict__ eref,
                            int64_t nch, int64_t D, int32_t *status) {
  int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nch) return;
  const int64_t row = c / D, d = c - row * D;
  const float *t = table + c * SKV_OCT_STRIDE;
  bool bad = false;
  float sg0 = t[0];
  if (!(sg0 >= 0.0f) || !__builtin_isfinite(sg0)) {
    bad = true;
    sg0 = 1.0f;
  }
  const float sp0 = sg0 > 0x1p-100f ? sg0 : 0x1p-100f;
  eref[c] = (int32_t)((__float_as_uint(sp0) >> 23) & 0xFFu) + 1;
  for (int j = 0; j < kOctaves; ++j) {
    float sg = t[1 + j];
    if (!(sg >= 0.0f) || !__builtin_isfinite(sg)) {
      bad = true;
      sg = 1.0f;
    }
    const float sp = sg > 0x1p-100f ? sg : 0x1p-100f;
    const float sc = (float)(64.0 / (double)sp);
    scale[(row * kOctaves + j) * D + d] = make_float2(sc, __builtin_amdgcn_rcpf(sc));
  }
  if (bad) set_status(status, SKV_ERR_ARG);
}

// the call's status, and the workspace's chunk counter (the kernels take
// chunk ids from it)
__global__ void k_clear_status(int32_t *status, uint32_t *ctr) {
  if (threadIdx.x == 0) {
    *status = SKV_OK;
    *ctr = 0;
  }
}

hipError_t launch_clear_status(int32_t *status, uint32_t *ctr, hipStream_t st) {
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(64), 0, st, status, ctr);
  return hipGetLastError();
}

hipError_t launch_model(const Geo &g, const float *sigma, const uint64_t *hist, const Workspace &ws,
                        int32_t *status, hipStream_t st) {
  timing_mark(kTimeModel, false, st);
  hipLaunchKernelGGL(k_knots, dim3(1), dim3(1024), 0, st, ws.knots, g.MG);
  const unsigned pblocks = (g.N + kPtBlock - 1) / kPtBlock;
  const int bf = g.sym_fmt == SKV_SYM_BF16 ? 1 : 0;
  hipLaunchKernelGGL(k_psums, dim3(pblocks), dim3(kPtBlock), 0, st, hist, ws.psum, ws.aflag, g.N, bf);
  hipLaunchKernelGGL(k_ptable, dim3(pblocks), dim3(kPtBlock), 0, st, hist, ws.psum, ws.ptab, ws.a16, ws.abase,
                     ws.aflag, g.N, g.Mp, bf, status);
  if (g.adapt) hipLaunchKernelGGL(k_prior, dim3(1), dim3(256), 0, st, ws.ptab, ws.prior, g.Mp);
  hipLaunchKernelGGL(k_uinv, dim3(1), dim3(1024), 0, st, ws.knots, ws.uinv, g.MG);
  if (g.sym_fmt == SKV_SYM_E4M3) hipLaunchKernelGGL(k_etab, dim3(1), dim3(256), 0, st, ws.etab);
  int64_t nch = g.rows * g.D;
  if (g.octave)
    hipLaunchKernelGGL(k_scale_oct, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, sigma, ws.scale, ws.eref,
                       nch, g.D, status);
  else
    hipLaunchKernelGGL(k_scale, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, sigma, ws.scale, nch, status);
  timing_mark(kTimeModel, true, st);
  return hipGetLastError();
}

}  // namespace skv
