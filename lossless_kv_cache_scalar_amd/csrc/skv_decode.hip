// skv_decode.hip -- decode a range-coded KV cache on gfx950.
//
// One wavefront per chunk, lane l decodes substream l: the same 8-scalar
// groups the encoder gave it, so the decoded symbols of a wave step are one
// contiguous 1 KB (bf16) store.  The model is rebuilt from (mu, sigma, hist),
// as both ends of the coder do ("Speculative KV coding", "什么能预测 KV 缓存").
#include "skv_internal.hpp"

namespace skv {

struct DecArgs {
  Geo g;
  const uint8_t *bits;
  uint64_t bits_bytes;
  const uint64_t *offsets;
  const void *mu;
  const float2 *knots;
  const uint32_t *ptab;
  const float2 *etab;
  const float *scale;
  void *x_out;
  int32_t *status;
};

// cum(k) = A(k) + Cg(u(lower edge of unrank(k))), cum(N) = T
template <int SYM>
__device__ __forceinline__ uint32_t cum_rank(const DecArgs &a, const float2 *kn, const float2 *etab_s,
                                             const uint32_t *ptab_s, uint32_t k, float mu, float s) {
  if (SYM == SKV_SYM_BF16) {
    if (k >= 65536u) return 1u << 24;
    return a.ptab[k] + cg_eval(kn, u_of(bf16_lo_edge(unrank_bf16(k)), mu, s));
  } else {
    if (k >= 256u) return 1u << 16;
    return ptab_s[k] + cg_eval(kn, u_of(etab_s[unrank_e4m3(k)].x, mu, s));
  }
}

template <int SYM, int MU>
__global__ __launch_bounds__(256) void k_decode(DecArgs a) {
  __shared__ float2 s_kn[kNKnot];
  __shared__ float2 s_etab[SYM == SKV_SYM_E4M3 ? 256 : 1];
  __shared__ uint32_t s_ptab[SYM == SKV_SYM_E4M3 ? 257 : 1];
  for (int i = threadIdx.x; i < kNKnot; i += blockDim.x) s_kn[i] = a.knots[i];
  if (SYM == SKV_SYM_E4M3) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) s_etab[i] = a.etab[i];
    for (int i = threadIdx.x; i < 257; i += blockDim.x) s_ptab[i] = a.ptab[i];
  }
  __syncthreads();

  const Geo &g = a.g;
  const int lane = threadIdx.x & 63;
  const int64_t chunk = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (chunk >= g.n_chunks) return;
  const int64_t row = chunk / g.ntb, blk = chunk % g.ntb;
  const int64_t tok = min<int64_t>(kChunkTokens, g.tokens - blk * kChunkTokens);
  const int64_t ngroups = tok * g.D / kGroup;
  const int64_t base = (row * g.tokens + blk * kChunkTokens) * g.D;
  const uint32_t N = SYM == SKV_SYM_BF16 ? 65536u : 256u;
  const uint32_t T = SYM == SKV_SYM_BF16 ? (1u << 24) : (1u << 16);
  const int up = SYM == SKV_SYM_BF16 ? 0 : 8;

  // ---- header: lane lengths, their prefix, and consistency with the offsets
  const uint64_t o0 = a.offsets[chunk], o1 = a.offsets[chunk + 1];
  const uint64_t nbytes = o1 >= o0 ? o1 - o0 : 0;
  bool corrupt = o1 < o0 || o1 > a.bits_bytes || nbytes < (uint64_t)kHeaderBytes;
  uint32_t len = 0;
  if (!corrupt) len = (uint32_t)a.bits[o0 + 2 * lane] | ((uint32_t)a.bits[o0 + 2 * lane + 1] << 8);
  uint32_t pre = len;  // inclusive prefix over lanes
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t v = __shfl_up(pre, off, 64);
    if (lane >= off) pre += v;
  }
  const uint32_t total = __shfl(pre, 63, 64);
  uint64_t start = (uint64_t)kHeaderBytes + (pre - len);
  if (!corrupt && (uint64_t)kHeaderBytes + total != nbytes) corrupt = true;
  if (len == 0) corrupt = true;
  // keep every substream inside the chunk whatever the header says
  if (corrupt) len = 0;  // a chunk outside the buffer reads nothing
  if (start > nbytes) start = nbytes;
  if (start + len > nbytes) len = (uint32_t)(nbytes - start);
  const uint8_t *src = a.bits + o0 + start;

  const int d0 = (int)((kGroup * lane) % g.D);
  float s[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) s[j] = a.scale[row * g.D + d0 + j];

  uint32_t pos = 0;
  auto next_byte = [&]() -> uint64_t {
    uint64_t v = pos < len ? src[pos] : 0;
    ++pos;
    return v;
  };
  uint64_t d = 0, range = kW48;
  for (int i = 0; i < 6; ++i) d = (d << 8) | next_byte();
  uint32_t shifts = 0;

  for (int64_t grp = lane; grp < ngroups; grp += kLanes) {
    const int64_t i0 = base + grp * kGroup;
    float mu[kGroup];
    if (MU == SKV_MU_BF16) {
      uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.mu) + i0);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mu[2 * j] = mu_from_bf16(w[j] & 0xFFFFu);
        mu[2 * j + 1] = mu_from_bf16(w[j] >> 16);
      }
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(a.mu) + i0);
      float4 v0 = p[0], v1 = p[1];
      float m8[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) mu[j] = mu_from_f32(m8[j]);
    }
    uint32_t out[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint64_t r = range >> 24;
      const uint64_t q = r << up;
      // t = floor(d / q): the fp64 quotient of exact integers is within one of it
      uint64_t t = q ? (uint64_t)((double)d / (double)q) : 0;
      if (q) {
        uint64_t tq = t * q;
        if (tq > d) t -= 1;
        else if (tq + q <= d) t += 1;
      }
      if (t >= T) {
        corrupt = true;
        t = T - 1;
      }
      // the unique rank k with cum(k) <= t < cum(k + 1), by bisection
      uint32_t lo = 0, hi = N;
      while (hi - lo > 1) {
        uint32_t mid = (lo + hi) >> 1;
        if (cum_rank<SYM>(a, s_kn, s_etab, s_ptab, mid, mu[j], s[j]) <= t) lo = mid; else hi = mid;
      }
      const uint32_t c = cum_rank<SYM>(a, s_kn, s_etab, s_ptab, lo, mu[j], s[j]);
      const uint32_t f = cum_rank<SYM>(a, s_kn, s_etab, s_ptab, lo + 1, mu[j], s[j]) - c;
      d -= r * ((uint64_t)c << up);
      range = r * ((uint64_t)f << up);
      for (int it = 0; it < 6 && range < kTop40; ++it) {
        d = ((d << 8) | next_byte()) & kW48;
        range <<= 8;
        ++shifts;
      }
      out[j] = SYM == SKV_SYM_BF16 ? unrank_bf16(lo) : unrank_e4m3(lo);
    }
    if (SYM == SKV_SYM_BF16) {
      uint4 v;
      v.x = out[0] | (out[1] << 16);
      v.y = out[2] | (out[3] << 16);
      v.z = out[4] | (out[5] << 16);
      v.w = out[6] | (out[7] << 16);
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.x_out) + i0) = v;
    } else {
      uint2 v;
      v.x = out[0] | (out[1] << 8) | (out[2] << 16) | (out[3] << 24);
      v.y = out[4] | (out[5] << 8) | (out[6] << 16) | (out[7] << 24);
      *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(a.x_out) + i0) = v;
    }
  }
  // a substream of n renormalisations holds n + 1 bytes
  if (shifts + 1 != len) corrupt = true;
  if (corrupt) set_status(a.status, SKV_ERR_CORRUPT);
}

template <int SYM, int MU>
static void launch_dec_kernel(const DecArgs &a, hipStream_t st) {
  unsigned blocks = (unsigned)((a.g.n_chunks + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((k_decode<SYM, MU>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, st, a);
}

hipError_t launch_decode(const Geo &g, const uint8_t *bits, uint64_t bits_bytes, const uint64_t *offsets,
                         const void *mu, const Workspace &ws, void *x_out, int32_t *status, hipStream_t st) {
  DecArgs a{g, bits, bits_bytes, offsets, mu, ws.knots, ws.ptab, ws.etab, ws.scale, x_out, status};
  if (g.sym_fmt == SKV_SYM_BF16) {
    if (g.mu_fmt == SKV_MU_BF16) launch_dec_kernel<SKV_SYM_BF16, SKV_MU_BF16>(a, st);
    else launch_dec_kernel<SKV_SYM_BF16, SKV_MU_F32>(a, st);
  } else {
    if (g.mu_fmt == SKV_MU_BF16) launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_BF16>(a, st);
    else launch_dec_kernel<SKV_SYM_E4M3, SKV_MU_F32>(a, st);
  }
  return hipGetLastError();
}

}  // namespace skv
