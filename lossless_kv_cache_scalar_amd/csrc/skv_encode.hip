// skv_encode.hip -- range-code a KV cache on gfx950.
//
// One wavefront per chunk (one (layer, kv, head) row x 256 tokens); lane l
// codes the chunk's 8-scalar groups g = l, l + 64, ... as its own substream.
// A group of 8 bf16 symbols and their 8 predictor means are one 16-byte load
// each, so a wave reads 1 KB of x and of mu per step, contiguous.
//
// Output: each lane writes its bytes to its own scratch slot; a scan over
// chunk sizes gives the offsets, and a compaction kernel writes every chunk
// (u16 length header, then the 64 substreams) at its offset.
#include "skv_internal.hpp"

namespace skv {

// ---- per-lane range coder (48-bit window, byte renormalisation) ----
// The coder spends -log2(f / 2^24) bits per symbol: q(x) integrated over the
// bin is the cost ("KV 缓存并非真正随机": every bit is cross-entropy).
struct Coder {
  uint64_t low, range;
  uint32_t acc;      // pending bytes, big-endian in the low nacc bytes
  uint32_t nacc;
  uint32_t nbytes;   // bytes emitted so far
  uint32_t *out;     // the lane's scratch slot (words, stream byte order)
  uint32_t nw;       // words emitted
  uint32_t capw;     // words the slot holds; a valid model never needs more

  __device__ void init(uint32_t *o, uint32_t cap_words) {
    capw = cap_words;
    low = 0;
    range = kW48;
    acc = 0;
    nacc = 0;
    nbytes = 0;
    out = o;
    nw = 0;
  }

  __device__ void emit(uint32_t byte) {
    acc = (acc << 8) | byte;
    ++nacc;
    ++nbytes;
    if (nacc == 4) {
      if (nw < capw) out[nw] = bswap32(acc);
      ++nw;
      acc = 0;
      nacc = 0;
    }
  }

  // add one to the big-endian number formed by every byte emitted so far
  __device__ void carry() {
    if (nacc) {
      uint32_t mask = (1u << (8 * nacc)) - 1u;
      acc = (acc + 1u) & mask;
      if (acc != 0) return;
    }
    for (int w = (int)min(nw, capw) - 1; w >= 0; --w) {
      uint32_t v = bswap32(out[w]) + 1u;
      out[w] = bswap32(v);
      if (v != 0) return;
    }
  }

  // c, f on the coder's 2^24 total
  __device__ void encode(uint32_t c, uint32_t f) {
    uint64_t r = range >> 24;
    low += r * c;
    if (low >> 48) {
      carry();
      low &= kW48;
    }
    range = r * f;
    for (int it = 0; it < 6 && range < kTop40; ++it) {
      emit((uint32_t)(low >> 40) & 0xFFu);
      low = (low << 8) & kW48;
      range <<= 8;
    }
  }

  __device__ void finish() {
    low = (low + (kTop40 - 1)) & ~(kTop40 - 1);
    if (low >> 48) {
      carry();
      low &= kW48;
    }
    emit((uint32_t)(low >> 40) & 0xFFu);
    if (nacc && nw < capw) out[nw] = bswap32(acc << (8 * (4 - nacc)));
  }
};

struct EncArgs {
  Geo g;
  const void *x, *mu;
  const float2 *knots;
  const uint32_t *ptab;
  const float2 *etab;
  const float *scale;
  uint32_t *lens;
  uint64_t *sizes;
  uint8_t *scratch;
  int32_t *status;
};

// (cum, freq) of symbol b on the model's own total, then scaled to 2^24
template <int SYM>
__device__ __forceinline__ void model_pair(const EncArgs &a, const float2 *kn, const float2 *etab_s,
                                           const uint32_t *ptab_s, uint32_t b, float mu, float s,
                                           uint32_t &c, uint32_t &f) {
  float lo, hi;
  uint32_t k, alo, ahi;
  if (SYM == SKV_SYM_BF16) {
    bf16_bin(b, lo, hi);
    k = rank_bf16(b);
    alo = a.ptab[k];
    ahi = a.ptab[k + 1];
  } else {
    float2 e = etab_s[b];
    lo = e.x;
    hi = e.y;
    k = rank_e4m3(b);
    alo = ptab_s[k];
    ahi = ptab_s[k + 1];
  }
  uint32_t clo = alo + cg_eval(kn, u_of(lo, mu, s));
  uint32_t chi = ahi + cg_eval(kn, u_of(hi, mu, s));
  c = clo;
  f = chi - clo;
  if (SYM == SKV_SYM_E4M3) {
    c <<= 8;
    f <<= 8;
  }
}

template <int SYM, int MU>
__global__ __launch_bounds__(256) void k_encode(EncArgs a) {
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

  // the lane's 8 channels are fixed because 512 is a multiple of head_dim
  const int d0 = (int)((kGroup * lane) % g.D);
  float s[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) s[j] = a.scale[row * g.D + d0 + j];

  Coder cod;
  cod.init(reinterpret_cast<uint32_t *>(a.scratch + ((uint64_t)chunk * kLanes + lane) * g.lane_cap), g.lane_cap / 4);

  for (int64_t grp = lane; grp < ngroups; grp += kLanes) {
    const int64_t i0 = base + grp * kGroup;
    uint32_t sym[kGroup];
    float mu[kGroup];
    if (SYM == SKV_SYM_BF16) {
      uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + i0);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sym[2 * j] = w[j] & 0xFFFFu;
        sym[2 * j + 1] = w[j] >> 16;
      }
    } else {
      uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(a.x) + i0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sym[j] = (v.x >> (8 * j)) & 0xFFu;
        sym[4 + j] = (v.y >> (8 * j)) & 0xFFu;
      }
    }
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
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      uint32_t c, f;
      model_pair<SYM>(a, s_kn, s_etab, s_ptab, sym[j], mu[j], s[j], c, f);
      cod.encode(c, f);
    }
  }
  cod.finish();
  // every frequency >= 1 bounds a lane at 3 bytes per symbol + 1; more means a broken table
  if (cod.nbytes > g.lane_cap) {
    set_status(a.status, SKV_ERR_TABLE);
    cod.nbytes = g.lane_cap;
  }
  a.lens[chunk * kLanes + lane] = cod.nbytes;
  // chunk size = header + every lane's bytes
  uint64_t tot = cod.nbytes;
  for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
  if (lane == 0) a.sizes[chunk] = kHeaderBytes + tot;
}

// ---- exclusive scan of chunk sizes into offsets (one block) ----
__global__ __launch_bounds__(1024) void k_offsets(const uint64_t *__restrict__ sizes, uint64_t *__restrict__ offsets,
                                                  int64_t n, uint64_t cap, int32_t *status) {
  __shared__ uint64_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t i0 = t * per, i1 = min<int64_t>(n, i0 + per);
  uint64_t s = 0;
  for (int64_t i = i0; i < i1; ++i) s += sizes[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    uint64_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  uint64_t run = part[t] - s;
  for (int64_t i = i0; i < i1; ++i) {
    offsets[i] = run;
    run += sizes[i];
  }
  if (t == 1023) {
    offsets[n] = part[1023];
    if (part[1023] > cap) set_status(status, SKV_ERR_CAPACITY);
  }
}

// ---- compaction: header and substreams of one chunk per block ----
__global__ __launch_bounds__(256) void k_compact(const uint32_t *__restrict__ lens, const uint8_t *__restrict__ scratch,
                                                 const uint64_t *__restrict__ offsets, uint8_t *__restrict__ bits,
                                                 uint64_t cap, uint32_t lane_cap) {
  __shared__ uint32_t pre[kLanes + 1];
  const int64_t chunk = blockIdx.x;
  const uint64_t o0 = offsets[chunk], o1 = offsets[chunk + 1];
  if (o1 > cap) return;  // capacity error already recorded; write nothing past the buffer
  const int t = threadIdx.x;
  if (t < kLanes) pre[t + 1] = lens[chunk * kLanes + t];
  if (t == 0) pre[0] = 0;
  __syncthreads();
  if (t == 0)
    for (int l = 1; l <= kLanes; ++l) pre[l] += pre[l - 1];
  __syncthreads();
  uint8_t *dst = bits + o0;
  if (t < kLanes) {
    uint32_t len = pre[t + 1] - pre[t];
    dst[2 * t] = (uint8_t)(len & 0xFFu);
    dst[2 * t + 1] = (uint8_t)(len >> 8);
  }
  const uint32_t total = pre[kLanes];
  const uint8_t *src = scratch + (uint64_t)chunk * kLanes * lane_cap;
  for (uint32_t j = t; j < total; j += blockDim.x) {
    int lo = 0, hi = kLanes;  // lane l holds bytes [pre[l], pre[l+1])
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (pre[mid] <= j) lo = mid; else hi = mid;
    }
    dst[kHeaderBytes + j] = src[(uint64_t)lo * lane_cap + (j - pre[lo])];
  }
}

template <int SYM, int MU>
static void launch_enc_kernel(const EncArgs &a, hipStream_t st) {
  unsigned blocks = (unsigned)((a.g.n_chunks + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL((k_encode<SYM, MU>), dim3(blocks), dim3(64 * kWavesPerBlock), 0, st, a);
}

hipError_t launch_encode(const Geo &g, const void *x, const void *mu, const Workspace &ws, uint8_t *bits,
                         uint64_t bits_cap, uint64_t *offsets, int32_t *status, hipStream_t st) {
  EncArgs a{g, x, mu, ws.knots, ws.ptab, ws.etab, ws.scale, ws.lens, ws.sizes, ws.scratch, status};
  if (g.sym_fmt == SKV_SYM_BF16) {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_BF16, SKV_MU_BF16>(a, st);
    else launch_enc_kernel<SKV_SYM_BF16, SKV_MU_F32>(a, st);
  } else {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_BF16>(a, st);
    else launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_F32>(a, st);
  }
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, st, ws.sizes, offsets, g.n_chunks, bits_cap, status);
  hipLaunchKernelGGL(k_compact, dim3((unsigned)g.n_chunks), dim3(256), 0, st, ws.lens, ws.scratch, offsets, bits,
                     bits_cap, g.lane_cap);
  return hipGetLastError();
}

}  // namespace skv
