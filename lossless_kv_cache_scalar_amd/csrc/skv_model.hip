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
// Domain: Mp * H(N) < 2^62, else SKV_ERR_TABLE.
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

// One block of 1024 threads; thread t owns window t: ranks 64t .. 64t + 63
// (bf16: all 1024 windows; e4m3: the first 4).  Writes the full table A and,
// for bf16, the LDS image: base A(64t) and 65 u16 offsets A(64t + j) - A(64t),
// j = 0..64, flagging a window whose offsets do not fit 16 bits.
__global__ __launch_bounds__(1024) void k_ptable(const uint64_t *__restrict__ hist, uint32_t *__restrict__ A,
                                                 uint16_t *__restrict__ a16, uint32_t *__restrict__ abase,
                                                 int32_t *__restrict__ aflag, uint32_t N, uint32_t Mp, int bf16,
                                                 int32_t *status) {
  __shared__ uint64_t part[1024];
  __shared__ int bad, narrow;
  const int t = threadIdx.x;
  const uint32_t nwin = N / kWinRanks;
  const bool active = (uint32_t)t < nwin;
  const uint32_t k0 = (uint32_t)t * kWinRanks;
  uint64_t s = 0;
  if (active)
    for (int j = 0; j < kWinRanks; ++j) {
      uint32_t k = k0 + j;
      s += hist[bf16 ? unrank_bf16(k) : unrank_e4m3(k)] + 1;
    }
  part[t] = s;
  if (t == 0) {
    bad = 0;
    narrow = 0;
  }
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    uint64_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const uint64_t total = part[1023];
  uint64_t H = part[t] - s;  // exclusive prefix
  if (t == 0 && (total < N || (Mp != 0 && total > (1ull << 62) / Mp))) bad = 1;
  __syncthreads();
  if (bad) {  // uniform table so that every frequency stays >= 1
    if (t == 0) set_status(status, SKV_ERR_TABLE);
    for (uint32_t k = t; k <= N; k += blockDim.x) A[k] = k + (uint32_t)(((uint64_t)Mp * k) / N);
    if (t == 0) *aflag = 0;
    return;
  }
  if (active) {
    uint32_t a0 = 0;
    for (int j = 0; j <= kWinRanks; ++j) {
      const uint32_t k = k0 + j;
      uint32_t ak = k + (uint32_t)floor_div((uint64_t)Mp * H, total);
      if (j < kWinRanks) A[k] = ak;
      if (j == 0) a0 = ak;
      if (bf16) {
        uint32_t off = ak - a0;
        if (off > 0xFFFFu) atomicOr(&narrow, 1);
        a16[t * kWinEntries + j] = (uint16_t)off;
      }
      if (j < kWinRanks) H += hist[bf16 ? unrank_bf16(k) : unrank_e4m3(k)] + 1;
    }
    if (bf16) abase[t] = a0;
  }
  __syncthreads();
  if (t == 0) {
    A[N] = N + Mp;
    if (bf16) abase[nwin] = N + Mp;
    *aflag = bf16 && !narrow ? 1 : 0;
  }
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

__global__ void k_clear_status(int32_t *status) {
  if (threadIdx.x == 0) *status = SKV_OK;
}

hipError_t launch_clear_status(int32_t *status, hipStream_t st) {
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(64), 0, st, status);
  return hipGetLastError();
}

hipError_t launch_model(const Geo &g, const float *sigma, const uint64_t *hist, const Workspace &ws,
                        int32_t *status, hipStream_t st) {
  timing_mark(kTimeModel, false, st);
  hipLaunchKernelGGL(k_knots, dim3(1), dim3(1024), 0, st, ws.knots, g.MG);
  hipLaunchKernelGGL(k_ptable, dim3(1), dim3(1024), 0, st, hist, ws.ptab, ws.a16, ws.abase, ws.aflag, g.N, g.Mp,
                     g.sym_fmt == SKV_SYM_BF16 ? 1 : 0, status);
  hipLaunchKernelGGL(k_uinv, dim3(1), dim3(1024), 0, st, ws.knots, ws.uinv, g.MG);
  if (g.sym_fmt == SKV_SYM_E4M3) hipLaunchKernelGGL(k_etab, dim3(1), dim3(256), 0, st, ws.etab);
  int64_t nch = g.rows * g.D;
  hipLaunchKernelGGL(k_scale, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, st, sigma, ws.scale, nch, status);
  timing_mark(kTimeModel, true, st);
  return hipGetLastError();
}

}  // namespace skv
