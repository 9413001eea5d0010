// skv_encode.hip -- range-code a KV cache on gfx950.
//
// Persistent grid, one 1024-thread block per CU: every table the model needs
// lives in LDS (knots 16 KB; the bf16 p_hat table in its 64-rank-window u16
// layout, 137 KB).  Each wavefront codes whole chunks (one (layer, kv, head)
// row x 256 tokens); lane l codes the chunk's 8-scalar groups l, l + 64, ...
// as its own substream.  A group of 8 bf16 symbols and its 8 predictor means
// are one 16-byte load each, so a wave reads 1 KB of x and of mu per step.
//
// Each lane writes its substream, as whole 32-bit words, to its own scratch
// slot; a scan over chunk sizes gives the offsets and a compaction kernel
// writes every chunk (u16 length header, then the 64 substreams) at its
// offset with coalesced word stores.
#include "skv_internal.hpp"

namespace skv {

constexpr int kEncBlock = 1024;
constexpr int kEncWaves = kEncBlock / 64;

struct EncArgs {
  Geo g;
  const void *x, *mu;
  const float2 *knots;
  const uint32_t *ptab;
  const uint16_t *a16;
  const uint32_t *abase;
  const int32_t *aflag;
  const float2 *etab;
  const float *scale;
  uint32_t *lens;
  uint64_t *sizes;
  uint8_t *scratch;
  int32_t *status;
};

// exact 48-bit product of two values below 2^24: v_mul_u32_u24 + v_mul_hi_u32_u24
__device__ __forceinline__ uint64_t mul24(uint32_t a, uint32_t b) {
  __builtin_assume(a < (1u << 24));
  __builtin_assume(b < (1u << 24));
  return (uint64_t)a * (uint64_t)b;
}

// A carry that ran through all 16 pending bits of the coder register: add one
// to the bits already emitted (the valid low nbits of acc, then stored words).
__device__ __noinline__ uint64_t carry_out(uint64_t acc, int nbits, uint32_t *out, uint32_t nw, uint32_t capw) {
  if (nbits > 0) {
    const uint64_t mask = (1ull << nbits) - 1ull;
    const uint64_t v = ((acc & mask) + 1ull) & mask;
    acc = (acc & ~mask) | v;
    if (v != 0) return acc;
  }
  for (int w = (int)min(nw, capw) - 1; w >= 0; --w) {
    const uint32_t v = __builtin_bswap32(out[w]) + 1u;
    out[w] = __builtin_bswap32(v);
    if (v != 0) break;
  }
  return acc;
}

// One range-coder lane.  X holds the 48-bit window "low" in its low bits and
// the two most recently emitted bytes above it, so most carries resolve by
// plain 64-bit addition; emitted bits collect in acc (nbits valid, the first
// 16 bits shifted out of X are the empty pending bytes of the initial state)
// and leave as whole words.
struct LaneCoder {
  uint64_t X, range, acc;
  int nbits;
  uint32_t nw, capw;
  uint32_t *out;

  __device__ __forceinline__ void init(uint32_t *o, uint32_t cap_words) {
    X = 0;
    range = kW48;
    acc = 0;
    nbits = -16;
    nw = 0;
    capw = cap_words;
    out = o;
  }

  // a valid model never fills the slot; a broken one rewrites its last word
  __device__ __forceinline__ void flush_word() {
    if (nbits >= 32) {
      const uint32_t word = (uint32_t)(acc >> (nbits - 32));
      out[min(nw, capw - 1)] = __builtin_bswap32(word);
      ++nw;
      nbits -= 32;
    }
  }

  // c, f on the coder's 2^24 total (f >= 1)
  __device__ __forceinline__ void encode(uint32_t c, uint32_t f) {
    const uint32_t r = (uint32_t)(range >> 24);
    const uint64_t p = mul24(r, c);
    unsigned int c0, c1;
    const uint32_t xl = __builtin_addc((uint32_t)X, (uint32_t)p, 0u, &c0);
    const uint32_t xh = __builtin_addc((uint32_t)(X >> 32), (uint32_t)(p >> 32), c0, &c1);
    X = ((uint64_t)xh << 32) | xl;
    const bool carry = c1 != 0;
    const uint64_t rg = mul24(r, f);
    const uint32_t n8 = __builtin_clz((uint32_t)(rg >> 16)) & ~7u;  // bytes to shift, x8
    if (__builtin_expect(__any(carry), 0)) {
      if (carry) acc = carry_out(acc, nbits, out, nw, capw);
    }
    const uint32_t outb = __builtin_amdgcn_ubfe((uint32_t)(X >> 32), (0u - n8) & 31u, n8);
    X <<= n8;
    range = rg << n8;
    acc = (acc << n8) | outb;
    nbits += (int)n8;
    flush_word();
  }

  // round low up to a multiple of 2^40, emit the pending bytes and its top byte
  __device__ __forceinline__ uint32_t finish() {
    const uint64_t Xn = (X + (kTop40 - 1)) & ~(kTop40 - 1);
    const bool carry = Xn < X;
    X = Xn;
    if (carry) acc = carry_out(acc, nbits, out, nw, capw);
    acc = (acc << 24) | (X >> 40);
    nbits += 24;
    flush_word();
    if (nbits > 0 && nw < capw) out[nw] = __builtin_bswap32((uint32_t)(acc << (32 - nbits)));
    return 4u * nw + (uint32_t)nbits / 8u;
  }
};

// One group of 8 scalars as loaded: symbols and predictor means.
template <int SYM, int MU>
struct Group {
  uint4 xv;
  uint4 mv0, mv1;  // mv1 only for fp32 means
  __device__ __forceinline__ void load(const EncArgs &a, int64_t i0) {
    if (SYM == SKV_SYM_BF16) {
      xv = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) + i0);
    } else {
      const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(a.x) + i0);
      xv = make_uint4(v.x, v.y, 0u, 0u);
    }
    if (MU == SKV_MU_BF16) {
      mv0 = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.mu) + i0);
    } else {
      const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.mu) + i0);
      mv0 = p[0];
      mv1 = p[1];
    }
  }
  __device__ __forceinline__ uint32_t sym(int j) const {
    const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
    if (SYM == SKV_SYM_BF16) return (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
  }
  __device__ __forceinline__ float mu(int j) const {
    if (MU == SKV_MU_BF16) {
      const uint32_t w[4] = {mv0.x, mv0.y, mv0.z, mv0.w};
      return mu_from_bf16((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    }
    const uint32_t w[8] = {mv0.x, mv0.y, mv0.z, mv0.w, mv1.x, mv1.y, mv1.z, mv1.w};
    return mu_from_f32(__uint_as_float(w[j]));
  }
};

struct EncTables {
  const float2 *kn;
  const uint16_t *a16;
  const uint32_t *ab;
  const float2 *et;
};

// (c, f) of symbol b on the coder's 2^24 total
template <int SYM, bool FAST>
__device__ __forceinline__ void model_pair(const EncArgs &a, const EncTables &t, uint32_t b, float m, float sj,
                                           uint32_t &c, uint32_t &f) {
  if (SYM == SKV_SYM_BF16) {
    // The bin of a finite non-zero b is [(b-1):8000, b:8000] in fp32 bits for
    // b > 0 and the same pair swapped for b < 0; Cg is monotone, so the lower
    // count is the min of the two.  +-0, +-inf and NaN take the general edges.
    const uint32_t eA = (b << 16) | 0x8000u;
    const uint32_t eB = eA - 0x10000u;
    const uint32_t cA = cg_eval(t.kn, u_of(__uint_as_float(eA), m, sj));
    const uint32_t cB = cg_eval(t.kn, u_of(__uint_as_float(eB), m, sj));
    uint32_t glo = min(cA, cB), ghi = max(cA, cB);
    const bool special = ((b << 17) - (1u << 17)) >= (0x7F7Fu << 17);
    if (__builtin_expect(__any(special), 0)) {
      if (special) {
        float lo, hi;
        bf16_bin(b, lo, hi);
        glo = cg_eval(t.kn, u_of(lo, m, sj));
        ghi = cg_eval(t.kn, u_of(hi, m, sj));
      }
    }
    const uint32_t k = rank_bf16(b);
    uint32_t alo, ahi;
    if (FAST) {
      const uint32_t w = k >> 6;
      const uint32_t e = k + w;  // = 65 w + (k mod 64)
      const uint32_t base_w = t.ab[w];
      alo = base_w + t.a16[e];
      ahi = base_w + t.a16[e + 1];
    } else {
      alo = a.ptab[k];
      ahi = a.ptab[k + 1];
    }
    c = alo + glo;
    f = ahi + ghi - c;
  } else {
    const float2 e = t.et[b];
    const uint32_t k = rank_e4m3(b);
    const uint32_t lo = t.ab[k] + cg_eval(t.kn, u_of(e.x, m, sj));
    const uint32_t hi = t.ab[k + 1] + cg_eval(t.kn, u_of(e.y, m, sj));
    c = lo << 8;
    f = (hi - lo) << 8;
  }
}

template <int SYM, int MU, bool FAST>
__device__ __forceinline__ void encode_chunks(const EncArgs &a, const EncTables &t) {
  const Geo &g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int64_t chunk = (int64_t)blockIdx.x * kEncWaves + wave; chunk < g.n_chunks;
       chunk += (int64_t)gridDim.x * kEncWaves) {
    const int64_t row = chunk / g.ntb, blk = chunk - row * g.ntb;
    const int64_t tok = min<int64_t>(kChunkTokens, g.tokens - blk * kChunkTokens);
    const int ngroups = (int)(tok * g.D / kGroup);
    const int64_t base = (row * g.tokens + blk * kChunkTokens) * g.D;

    // the lane's 8 channels are fixed because 512 is a multiple of head_dim
    const int d0 = (kGroup * lane) % (int)g.D;
    float s[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) s[j] = a.scale[row * g.D + d0 + j];

    LaneCoder cod;
    cod.init(reinterpret_cast<uint32_t *>(a.scratch + ((uint64_t)chunk * kLanes + lane) * g.lane_cap),
             g.lane_cap / 4);

    Group<SYM, MU> cur;
    if (lane < ngroups) cur.load(a, base + (int64_t)lane * kGroup);
    for (int grp = lane; grp < ngroups; grp += kLanes) {
      Group<SYM, MU> nxt;
      if (grp + kLanes < ngroups) nxt.load(a, base + (int64_t)(grp + kLanes) * kGroup);  // in flight meanwhile
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        uint32_t c, f;
        model_pair<SYM, FAST>(a, t, cur.sym(j), cur.mu(j), s[j], c, f);
        cod.encode(c, f);
      }
      cur = nxt;
    }
    uint32_t nbytes = cod.finish();
    // every frequency >= 1 bounds a lane at 3 bytes per symbol + 1; more means a broken table
    if (nbytes > g.lane_cap) {
      set_status(a.status, SKV_ERR_TABLE);
      nbytes = g.lane_cap;
    }
    a.lens[chunk * kLanes + lane] = nbytes;
    uint32_t tot = nbytes;
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (lane == 0) a.sizes[chunk] = kHeaderBytes + (uint64_t)tot;
  }
}

template <int SYM, int MU>
__global__ __launch_bounds__(kEncBlock) void k_encode(EncArgs a) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  __shared__ float2 s_kn[kNKnot];
  __shared__ uint32_t s_a16w[BF ? kNWin * kWinEntries / 2 : 1];
  __shared__ uint32_t s_ab[BF ? kNWin + 1 : 257];
  __shared__ float2 s_et[BF ? 1 : 256];

  const bool fast = BF ? *a.aflag != 0 : true;  // windowed p_hat table usable
  for (int i = threadIdx.x; i < kNKnot; i += kEncBlock) s_kn[i] = a.knots[i];
  if (BF) {
    if (fast) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(a.a16);
      for (int i = threadIdx.x; i < kNWin * kWinEntries / 2; i += kEncBlock) s_a16w[i] = src[i];
      for (int i = threadIdx.x; i <= kNWin; i += kEncBlock) s_ab[i] = a.abase[i];
    }
  } else {
    for (int i = threadIdx.x; i < 257; i += kEncBlock) s_ab[i] = a.ptab[i];
    for (int i = threadIdx.x; i < 256; i += kEncBlock) s_et[i] = a.etab[i];
  }
  __syncthreads();
  const EncTables t{s_kn, reinterpret_cast<const uint16_t *>(s_a16w), s_ab, s_et};
  if (fast) encode_chunks<SYM, MU, true>(a, t);
  else encode_chunks<SYM, MU, false>(a, t);
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

// ---- compaction: one block per chunk ----
// The chunk occupies bytes [o0, o1) of the stream: the u16 length header, then
// substream l at [p_l, p_l + len_l), p_l = o0 + 128 + (lengths before l).  A
// wave copies one substream at a time: the aligned words inside it are funnel
// shifts of two scratch words (coalesced stores), and the at most 3 + 3 bytes
// it shares with a neighbour's words are written byte by byte.
__global__ __launch_bounds__(256) void k_compact(const uint32_t *__restrict__ lens_g, const uint8_t *__restrict__ scratch,
                                                 const uint64_t *__restrict__ offsets, uint8_t *__restrict__ bits,
                                                 uint64_t cap, uint32_t lane_cap) {
  __shared__ uint32_t pre[kLanes + 1];
  const int64_t chunk = blockIdx.x;
  const uint64_t o0 = offsets[chunk], o1 = offsets[chunk + 1];
  if (o1 > cap) return;  // capacity error already recorded; write nothing past the buffer
  const int t = threadIdx.x;
  if (t < kLanes) {
    const uint32_t len = lens_g[chunk * kLanes + t];
    bits[o0 + 2 * t] = (uint8_t)(len & 0xFFu);
    bits[o0 + 2 * t + 1] = (uint8_t)(len >> 8);
    uint32_t inc = len;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(inc, off, 64);
      if (t >= off) inc += v;
    }
    pre[t + 1] = inc;
    if (t == 0) pre[0] = 0;
  }
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  for (int l = wave; l < kLanes; l += 4) {
    const uint64_t a = o0 + kHeaderBytes + pre[l];
    const uint64_t b = o0 + kHeaderBytes + pre[l + 1];
    const uint8_t *src = scratch + ((uint64_t)chunk * kLanes + l) * lane_cap;
    const uint64_t wa = (a + 3) & ~3ull, wb = b & ~3ull;  // aligned words fully inside [a, b)
    if (wa < wb) {
      const uint32_t sh = 8 * (uint32_t)((wa - a) & 3);
      const uint32_t *sw0 = reinterpret_cast<const uint32_t *>(src) + ((wa - a) >> 2);
      for (uint64_t q = wa + 4 * (uint64_t)lane; q < wb; q += 256) {
        const uint32_t *sw = sw0 + ((q - wa) >> 2);
        const uint32_t w0 = __builtin_bswap32(sw[0]);
        const uint32_t v = sh ? (w0 << sh) | (__builtin_bswap32(sw[1]) >> (32 - sh)) : w0;
        *reinterpret_cast<uint32_t *>(bits + q) = __builtin_bswap32(v);
      }
      if (lane < 3 && a + lane < wa) bits[a + lane] = src[lane];                       // head
      if (lane < 3 && wb + lane < b) bits[wb + lane] = src[wb + lane - a];             // tail
    } else if (lane < 8 && a + lane < b) {
      bits[a + lane] = src[lane];  // short substream: no whole word inside
    }
  }
}

static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

template <int SYM, int MU>
static void launch_enc_kernel(const EncArgs &a, hipStream_t st) {
  const int64_t need = (a.g.n_chunks + kEncWaves - 1) / kEncWaves;
  const int64_t cus = cu_count();
  const unsigned blocks = (unsigned)(need < cus ? need : cus);
  hipLaunchKernelGGL((k_encode<SYM, MU>), dim3(blocks), dim3(kEncBlock), 0, st, a);
}

hipError_t launch_encode(const Geo &g, const void *x, const void *mu, const Workspace &ws, uint8_t *bits,
                         uint64_t bits_cap, uint64_t *offsets, int32_t *status, hipStream_t st) {
  EncArgs a{g, x, mu, ws.knots, ws.ptab, ws.a16, ws.abase, ws.aflag, ws.etab, ws.scale, ws.lens, ws.sizes,
            ws.scratch, status};
  timing_mark(kTimeEncode, false, st);
  if (g.sym_fmt == SKV_SYM_BF16) {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_BF16, SKV_MU_BF16>(a, st);
    else launch_enc_kernel<SKV_SYM_BF16, SKV_MU_F32>(a, st);
  } else {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_BF16>(a, st);
    else launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_F32>(a, st);
  }
  timing_mark(kTimeEncode, true, st);
  timing_mark(kTimeOffsets, false, st);
  hipLaunchKernelGGL(k_offsets, dim3(1), dim3(1024), 0, st, ws.sizes, offsets, g.n_chunks, bits_cap, status);
  timing_mark(kTimeOffsets, true, st);
  timing_mark(kTimeCompact, false, st);
  hipLaunchKernelGGL(k_compact, dim3((unsigned)g.n_chunks), dim3(256), 0, st, ws.lens, ws.scratch, offsets, bits,
                     bits_cap, g.lane_cap);
  timing_mark(kTimeCompact, true, st);
  return hipGetLastError();
}

}  // namespace skv
