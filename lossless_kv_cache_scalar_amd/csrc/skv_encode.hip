// skv_encode.hip -- range-code a KV cache on gfx950.
//
// Persistent grid, one 1024-thread block per CU: every table the model needs
// lives in LDS (knots 16 KB; the bf16 p_hat table in its 64-rank-window u16
// layout, 137 KB).  Each wavefront codes whole chunks (one (layer, kv, head)
// row x 256 tokens); lane l codes the chunk's scalars l, l + 64, l + 128, ...
// as its own substream, so one wave step reads 64 consecutive scalars of x and
// of mu.  Lanes load their next 8 symbols while coding the current 8.
//
// Each lane writes its substream as whole 32-bit words into a scratch slot,
// word w of lane l at word 64 w + l: a wave's stores land side by side, and
// the first m words of every lane already sit in the stream's interleaved
// layout.  A lane stores its completed word at the start of each batch of 8
// symbols, and within a batch only when its 64-bit accumulator would overflow.  A wave owns two slots and codes its chunks in them by turns: it
// holds at most the chunk it is coding and one whose offset it is still
// waiting for, so the scratch scales with the grid, not with the cache.
//
// With the adaptive p_hat (e4m3), each wave also keeps its chunk's symbol
// counts and p_hat pair table in LDS and rebuilds the table every epoch
// (skv_adapt.hpp); the decoder rebuilds at the same points from the same
// symbols.  Chunk ids come from an atomic counter in increasing
// order; a finished chunk publishes its size, finds its offset by looking back
// over its predecessors' published sizes and prefixes (a single-pass scan:
// every chunk it waits for was taken earlier by a running wave, so the lowest
// unfinished chunk never waits), and its wave then writes the chunk (length
// header, interleaved words, the lanes' remaining bytes, padding) at that
// offset.
#include "skv_adapt.hpp"

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
  const uint32_t *prior;  // adaptive p_hat: the counts a chunk starts from (at the symbols' patterns)
  const float2 *scale;  // per channel, or per channel and octave
  const int32_t *eref;   // octave mode: per channel octave reference
  uint64_t *flags;  // per chunk: kFlagAgg | size, then kFlagIncl | offset + size
  uint32_t *ctr;    // next chunk id
  uint8_t *scratch;
  uint8_t *bits;
  uint64_t bits_cap;
  uint64_t *offsets;
  int32_t *status;
};

// chunk status words of the single-pass scan (0: not yet published)
constexpr uint64_t kFlagAgg = 1ull << 62;   // the chunk's own size
constexpr uint64_t kFlagIncl = 2ull << 62;  // its offset + size
constexpr uint64_t kFlagVal = kFlagAgg - 1;
constexpr uint32_t kSpinLimit = 1u << 20;   // polls of one predecessor before giving up

__device__ __forceinline__ uint64_t flag_load(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Offset of chunk c (> 0) from the published words of its predecessors: lane
// l reads chunks p - l - 64 u, u < kLookBack; the nearest inclusive prefix ends
// the walk, aggregates before it add up.  Returns false when the nearest
// unpublished predecessor is still unpublished after max_spins polls.
constexpr int kLookBack = 8;
__device__ bool look_back(const uint64_t *flags, int64_t c, int lane, uint64_t &excl, uint32_t max_spins) {
  excl = 0;
  int64_t p = c - 1;  // the nearest chunk not yet accounted for
  uint32_t spins = 0;
  for (;;) {
    uint64_t f[kLookBack];
#pragma unroll
    for (int u = 0; u < kLookBack; ++u) {
      const int64_t q = p - lane - (int64_t)kLanes * u;
      f[u] = q >= 0 ? flag_load(flags + q) : kFlagIncl;  // before chunk 0: offset 0
    }
    bool wait = false;
#pragma unroll
    for (int u = 0; u < kLookBack; ++u) {
      if (wait) break;
      const uint64_t st = f[u] >> 62;
      const uint64_t stop = __ballot(st != 1);
      if (stop == 0) {  // 64 aggregates
        excl += wave_sum64(f[u] & kFlagVal);
        p -= kLanes;
        continue;
      }
      const int first = __builtin_ctzll(stop);  // the nearest chunk not holding a plain aggregate
      const uint64_t stf = __shfl(st, first, 64);
      excl += wave_sum64(lane < first || (stf == 2 && lane == first) ? (f[u] & kFlagVal) : 0);
      if (stf == 2) return true;
      p -= first;  // chunk p has not published yet
      wait = true;
    }
    if (wait) {
      if (spins++ >= max_spins) return false;
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// Chunk c's bytes at bits[o0, o0 + size): the header, the interleaved words
// (copied as they sit in the slot), each lane's remaining bytes, zeros.
__device__ __forceinline__ void write_chunk(uint8_t *__restrict__ bits, uint64_t o0, uint64_t size,
                                            const uint8_t *slot, uint32_t len, int lane) {
  reinterpret_cast<uint16_t *>(bits + o0)[lane] = (uint16_t)len;
  uint32_t m = len >> 2;
  for (int off = 32; off > 0; off >>= 1) m = min(m, (uint32_t)__shfl_xor((int)m, off, 64));
  const uint32_t tail = len - 4 * m;
  uint32_t inc = tail;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(inc, off, 64);
    if (lane >= off) inc += v;
  }
  const uint32_t tails = __shfl(inc, 63, 64);
  const uint32_t *sw = reinterpret_cast<const uint32_t *>(slot);
  uint32_t *dw = reinterpret_cast<uint32_t *>(bits + o0 + kHeaderBytes);
  // 16 loads in flight per lane, then their stores
  constexpr int kCopy = 16;
  const uint32_t nwords = kLanes * m;
  for (uint32_t q0 = 0; q0 < nwords; q0 += kLanes * kCopy) {
    uint32_t v[kCopy];
#pragma unroll
    for (int u = 0; u < kCopy; ++u) {
      const uint32_t q = q0 + kLanes * u + (uint32_t)lane;
      v[u] = q < nwords ? sw[q] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kCopy; ++u) {
      const uint32_t q = q0 + kLanes * u + (uint32_t)lane;
      if (q < nwords) dw[q] = v[u];
    }
  }
  // the lane's remaining bytes: its words m, m + 1, ... four at a time
  const uint64_t d0 = o0 + kHeaderBytes + 4ull * kLanes * m + (inc - tail);
  for (uint32_t j0 = 0; j0 < tail; j0 += 16) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = j0 + 4u * u < tail ? sw[(m + (j0 >> 2) + u) * kLanes + (uint32_t)lane] : 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (j0 + u < tail) bits[d0 + j0 + u] = (uint8_t)(v[u >> 2] >> (8 * (u & 3)));
  }
  const uint64_t end = o0 + kHeaderBytes + 4ull * kLanes * m + tails;
  if (lane < 3 && end + lane < o0 + size) bits[end + lane] = 0;
}

// exact 48-bit product of two values below 2^24: v_mul_u32_u24 + v_mul_hi_u32_u24
__device__ __forceinline__ uint64_t mul24(uint32_t a, uint32_t b) {
  __builtin_assume(a < (1u << 24));
  __builtin_assume(b < (1u << 24));
  return (uint64_t)a * (uint64_t)b;
}

// A carry that ran through all 16 pending bits of the coder register: add one
// to the bits already emitted (the valid low nbits of acc, then stored words;
// a lane's word w is out[64 w]).
__device__ __noinline__ uint64_t carry_out(uint64_t acc, int nbits, uint32_t *out, uint32_t nw, uint32_t capw) {
  if (nbits > 0) {
    const uint64_t mask = nbits >= 64 ? ~0ull : (1ull << nbits) - 1ull;
    const uint64_t v = ((acc & mask) + 1ull) & mask;
    acc = (acc & ~mask) | v;
    if (v != 0) return acc;
  }
  for (int w = (int)min(nw, capw) - 1; w >= 0; --w) {
    const uint32_t v = __builtin_bswap32(out[(uint32_t)w * kLanes]) + 1u;
    out[(uint32_t)w * kLanes] = __builtin_bswap32(v);
    if (v != 0) break;
  }
  return acc;
}

// One range-coder lane.  X holds the 48-bit window "low" in its low bits and
// the two most recently emitted bytes above it, so most carries resolve by
// plain 64-bit addition; emitted bits collect in acc (64 - room of them valid;
// the first 16 bits shifted out of X are the empty pending bytes of the
// initial state) and leave as whole words, word w at out[64 w].
struct LaneCoder {
  uint64_t X, acc;
  uint32_t r;  // the 48-bit range over 2^24: only these bits enter the products
  int room;      // 64 - the valid bits in acc
  uint32_t nw, capw;
  uint32_t *out;   // the lane's word 0 in the chunk's slot
  uint8_t *slot;   // the chunk's slot (the same for the whole wave)
  uint32_t off;    // byte offset of the lane's word nw in the slot
  uint32_t q0;     // a completed word not stored yet: word nw - 1 when held
  bool held;

  __device__ __forceinline__ void init(uint8_t *chunk_slot, uint32_t lane, uint32_t cap_words) {
    X = 0;
    r = (uint32_t)(kW48 >> 24);
    acc = 0;
    room = 80;  // -16 valid bits
    nw = 0;
    capw = cap_words;
    slot = chunk_slot;
    out = reinterpret_cast<uint32_t *>(chunk_slot) + lane;
    off = 4u * lane;
    q0 = 0;
    held = false;
  }

  // Stores the lane's oldest complete word, the one that starts at bit
  // 32 - room of acc (room <= 32).  At most 3 bytes per symbol plus the
  // flush: the slot (lane_cap) always has room.
  __device__ __forceinline__ void store_word() {
    const uint32_t word = (uint32_t)(acc >> (32 - room));
    *reinterpret_cast<uint32_t *>(slot + off) = __builtin_bswap32(word);
    ++nw;
    room += 32;
    off += 4u * kLanes;
  }
  // A word completed within a batch waits in q0 and is stored at the next
  // batch's start (a second one stores the first at once).  Loads and stores
  // share one counter, so the wait for a batch's symbols and means, issued a
  // batch earlier, also waited for every store made since; a store late in a
  // batch made the next batch wait for it (k_encode -4.8% on the 32B bf16
  // cache, -1.2% on the 32K e4m3 cache in A/B runs; holding two words cost
  // more selects and saved less).
  __device__ __forceinline__ void queue_word() {
    const uint32_t word = (uint32_t)(acc >> (32 - room));
    if (held) *reinterpret_cast<uint32_t *>(slot + off - 4u * kLanes) = __builtin_bswap32(q0);
    q0 = word;
    held = true;
    ++nw;
    room += 32;
    off += 4u * kLanes;
  }
  __device__ __forceinline__ void drain() {
    if (held) *reinterpret_cast<uint32_t *>(slot + off - 4u * kLanes) = __builtin_bswap32(q0);
    held = false;
  }
  // Before a full batch: the queued words, and a word from every lane that has
  // one, so that a lane holds at most 32 bits, and its symbols add at most 24
  // bits each.
  __device__ __forceinline__ void flush_batch() {
    if (__any(held)) drain();
    if (__any(room <= 32)) {
      if (room <= 32) store_word();
    }
  }

  // c, f on the coder's 2^24 total (f >= 1)
  __device__ __forceinline__ void encode(uint32_t c, uint32_t f) {
    __builtin_assume(r < (1u << 24));
    // the carry out of bit 63 compares the sum with the old X, which the empty
    // asm hides from the optimiser (it would rewrite the test as Xn < r * c and
    // form that product a second time)
    uint64_t Xo = X;
    asm("" : "+v"(Xo));
    const uint64_t Xn = Xo + mul24(r, c);
    const bool carry = Xn < Xo;
    X = Xn;
    // r * f as the two 24-bit multiplies, written out: r also feeds the 32-bit
    // multiply-add above, and the compiler would mask it to 24 bits here
    uint32_t rlo, rhi;
    asm("v_mul_u32_u24 %0, %2, %3\n\tv_mul_hi_u32_u24 %1, %2, %3" : "=&v"(rlo), "=v"(rhi) : "v"(r), "v"(f));
    const uint64_t rg = ((uint64_t)rhi << 32) | rlo;
    // bytes to shift, x8: rg >= 2^16 (f >= 1) makes this clz & ~7; the mask
    // bounds it by 24 whatever rg is, so a lane never emits more than 3 bytes
    // per symbol and never outgrows its slot
    const uint32_t n8 = __builtin_clz((uint32_t)(rg >> 16)) & 24u;
    // room for n8 more bits in acc (n8 > room implies room < 24: a word is complete)
    if (__builtin_expect(__any((int)n8 > room), 0)) {
      if ((int)n8 > room) queue_word();
    }
    if (__builtin_expect(__any(carry), 0)) {
      if (carry) {
        drain();  // the carry may reach the stored words
        acc = carry_out(acc, 64 - room, out, nw, capw);
      }
    }
    // the top n8 bits of X (width 0 reads as 0 whatever the offset)
    const uint32_t outb = __builtin_amdgcn_ubfe((uint32_t)(X >> 32), 32u - n8, n8);
    X <<= n8;
    r = __builtin_amdgcn_alignbit(rhi, rlo, 24u - n8);
    acc = (acc << n8) | outb;
    room -= (int)n8;
  }

  // round low up to a multiple of 2^40, emit the pending bytes and its top byte
  __device__ __forceinline__ uint32_t finish() {
    const uint64_t Xn = (X + (kTop40 - 1)) & ~(kTop40 - 1);
    const bool carry = Xn < X;
    X = Xn;
    drain();
    if (carry) acc = carry_out(acc, 64 - room, out, nw, capw);
    while (room <= 32) store_word();
    acc = (acc << 24) | (X >> 40);
    room -= 24;
    if (room <= 32) store_word();
    const int nbits = 64 - room;
    if (nbits > 0 && nw < capw) out[nw * kLanes] = __builtin_bswap32((uint32_t)(acc << (32 - nbits)));
    return 4u * nw + (uint32_t)nbits / 8u;
  }
};

// A lane's next kBatch symbols and predictor means (symbols i0, i0 + 64, ...).
template <int SYM, int MU>
struct Batch {
  uint32_t xs[kBatch];
  uint32_t ms[kBatch];  // bf16 pattern or fp32 bits
  __device__ __forceinline__ void one(const EncArgs &a, int64_t i, int j) {
    xs[j] = SYM == SKV_SYM_BF16 ? (uint32_t) static_cast<const uint16_t *>(a.x)[i]
                                : (uint32_t) static_cast<const uint8_t *>(a.x)[i];
    ms[j] = MU == SKV_MU_BF16 ? (uint32_t) static_cast<const uint16_t *>(a.mu)[i]
                              : static_cast<const uint32_t *>(a.mu)[i];
  }
  // x and mu are read once: non-temporal loads keep them from displacing the
  // scratch words in L2, which the lanes complete a sector at a time (k_encode
  // -3% and 17% fewer bytes written on the 32B bf16 cache; non-temporal stores
  // for the chunk copy wrote more, as they bypass write combining)
  __device__ __forceinline__ void load_full(const EncArgs &a, int64_t i0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t i = i0 + (int64_t)kLanes * j;
      xs[j] = SYM == SKV_SYM_BF16 ? (uint32_t)__builtin_nontemporal_load(static_cast<const uint16_t *>(a.x) + i)
                                  : (uint32_t)__builtin_nontemporal_load(static_cast<const uint8_t *>(a.x) + i);
      ms[j] = MU == SKV_MU_BF16 ? (uint32_t)__builtin_nontemporal_load(static_cast<const uint16_t *>(a.mu) + i)
                                : __builtin_nontemporal_load(static_cast<const uint32_t *>(a.mu) + i);
    }
  }
  __device__ __forceinline__ float mu(int j) const {
    return mu_finite_wave(MU == SKV_MU_BF16 ? __uint_as_float(ms[j] << 16) : __uint_as_float(ms[j]));
  }
};

struct EncTables {
  const float2 *kn;
  const uint16_t *a16;
  const uint32_t *ab;
  const float2 *et;
  const float4 *ep;
};

// p_hat counts A(rank b), A(rank b + 1) of a bf16 symbol
template <bool FAST>
__device__ __forceinline__ void a_pair_bf16(const EncArgs &a, const EncTables &t, uint32_t b, uint32_t &alo,
                                            uint32_t &ahi) {
  if (FAST) {
    const uint32_t ti = tix_bf16(b);  // the window image's index of rank_bf16(b)
    const uint32_t w = ti >> 6;
    const uint32_t e = ti + w;  // = 65 w + (ti mod 64)
    const uint32_t base_w = t.ab[w];
    alo = base_w + t.a16[e];
    ahi = base_w + t.a16[e + 1];
  } else {
    const uint32_t k = rank_bf16(b);
    alo = a.ptab[k];
    ahi = a.ptab[k + 1];
  }
}

// (c, f) of symbol b on the coder's 2^24 total, for every b but the special
// bf16 ones (+-0, +-inf, NaN), which need model_special: spm is the wave's
// mask of lanes that may hold one (bf16_hi_bits).  The bin of a finite non-zero bf16 b is [(b-1):8000, b:8000]
// in fp32 bits for b > 0 and the same pair swapped for b < 0; Cg is monotone,
// so the lower count is the min of the two.
template <int SYM, bool FAST, bool EP>
__device__ __forceinline__ void model_common(const EncArgs &a, const EncTables &t, uint32_t b, float m, float sj,
                                             uint32_t &c, uint32_t &f, uint64_t &spm) {
  if (SYM == SKV_SYM_BF16) {
    // p_hat part first: it depends on b alone, so its table reads are in flight
    // while the Gaussian pair is evaluated
    uint32_t alo, ahi;
    a_pair_bf16<FAST>(a, t, b, alo, ahi);
    const uint32_t eA = bf16_hi_bits(b, spm);  // (b << 16) | 0x8000
    const uint32_t eB = eA - 0x10000u;
    const uint32_t cA = cg_eval(t.kn, u_of(__uint_as_float(eA), m, sj));
    const uint32_t cB = cg_eval(t.kn, u_of(__uint_as_float(eB), m, sj));
    c = alo + min(cA, cB);
    f = ahi + max(cA, cB) - c;
  } else {
    float2 e;
    uint2 p;  // (A(k), A(k + 1))
    // static p_hat: the bin and the pair in one 16-byte entry per pattern, with
    // no table index to form (k_encode -7% on the 32K e4m3 cache, -4% on the
    // 0.6B one; the adaptive kernels rebuild their pairs in rank order)
    if (EP) {
      const float4 q = t.ep[b];
      e = make_float2(q.x, q.y);
      p = make_uint2(__float_as_uint(q.z), __float_as_uint(q.w));
    } else {
      e = t.et[b];
      p = reinterpret_cast<const uint2 *>(t.ab)[b];
    }
    const uint32_t lo = p.x + cg_eval(t.kn, u_of(e.x, m, sj));
    const uint32_t hi = p.y + cg_eval(t.kn, u_of(e.y, m, sj));
    c = lo << 8;
    f = (hi - lo) << 8;
    spm = 0;
  }
}

// (c, f) of a special bf16 symbol from its general bin edges
template <bool FAST>
__device__ __forceinline__ void model_special(const EncArgs &a, const EncTables &t, uint32_t b, float m, float sj,
                                              uint32_t &c, uint32_t &f) {
  uint32_t alo, ahi;
  a_pair_bf16<FAST>(a, t, b, alo, ahi);
  float lo, hi;
  bf16_bin(b, lo, hi);
  c = alo + cg_eval(t.kn, u_of(lo, m, sj));
  f = ahi + cg_eval(t.kn, u_of(hi, m, sj)) - c;
}

template <int SYM, bool FAST, bool EP>
__device__ __forceinline__ void model_pair(const EncArgs &a, const EncTables &t, uint32_t b, float m, float sj,
                                           uint32_t &c, uint32_t &f) {
  uint64_t spm;
  model_common<SYM, FAST, EP>(a, t, b, m, sj, c, f, spm);
  if (SYM == SKV_SYM_BF16 && __builtin_expect(spm != 0, 0)) {
    if (bf16_special(b)) model_special<FAST>(a, t, b, m, sj, c, f);
  }
}

// AD: adaptive p_hat (e4m3): the wave's pair table and counts in `aw`, reset
// from the block's static pairs and prior at every chunk, rebuilt every epoch.
template <int SYM, int MU, int PER, int OCT, bool FAST, bool AD>
__device__ __forceinline__ void encode_chunks(const EncArgs &a, const EncTables &t0, AdaptLds *aw,
                                              const uint32_t *s_pairs, const uint32_t *s_prior) {
  const Geo &g = a.g;
  EncTables t = t0;
  if (AD) t.ab = aw->pairs;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int D = (int)g.D;
  constexpr int kStep = kLanes * kBatch;  // scalars of one batch of the wave
  (void)wave;
  // A chunk whose look-back would have to wait is finished after the wave has
  // coded its next chunk: by then its predecessors have published.
  int64_t pend = -1;
  uint32_t pend_len = 0;
  uint64_t pend_size = 0;
  // this wave's two scratch slots, used by turns
  // (the wave index read as uniform, so the slot addresses stay in scalar registers)
  const uint64_t wave_gid =
      (uint64_t)blockIdx.x * kEncWaves + (uint64_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint8_t *const slots = a.scratch + wave_gid * 2 * kLanes * (uint64_t)g.lane_cap;
  uint32_t taken = 0;  // chunks this wave has started
  const uint8_t *pend_slot = nullptr;
  auto finalize = [&](int64_t c, uint64_t o0, uint64_t size, uint32_t len, const uint8_t *slot) {
    if (lane == 0) {
      flag_store(a.flags + c, kFlagIncl | (o0 + size));
      a.offsets[c] = o0;
      if (c == g.n_chunks - 1) {
        a.offsets[c + 1] = o0 + size;
        if (o0 + size > a.bits_cap) set_status(a.status, SKV_ERR_CAPACITY);
      }
    }
    // the slot was written by this wave: its stores are complete and visible to
    // its own loads after a workgroup-scope fence (no cache writeback needed)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    if (o0 + size <= a.bits_cap)
      write_chunk(a.bits, o0, size, slot, len, lane);
  };
  for (;;) {
    uint32_t cid = 0;
    if (lane == 0) cid = atomicAdd(a.ctr, 1u);
    const int64_t chunk = (int64_t)__builtin_amdgcn_readfirstlane(__shfl(cid, 0, 64));  // uniform: kept in SGPRs
    if (chunk >= g.n_chunks) {
      if (pend >= 0) {
        uint64_t o0;
        if (!look_back(a.flags, pend, lane, o0, kSpinLimit)) set_status(a.status, SKV_ERR_HIP);
        finalize(pend, o0, pend_size, pend_len, pend_slot);
      }
      break;
    }
    const int64_t row = chunk / g.ntb, blk = chunk - row * g.ntb;
    const int64_t tok = min<int64_t>(kChunkTokens, g.tokens - blk * kChunkTokens);
    const int nsc = (int)(tok * D);
    const int64_t base = (row * g.tokens + blk * kChunkTokens) * g.D;

    // symbol k of the lane has channel (lane + 64 k) mod D; with D a power of
    // two up to 512 that repeats with period PER = max(2, D / 64), which divides kBatch
    float s[PER];
    int32_t er[PER];  // octave mode: the channels' octave references
    uint32_t cb[PER]; // octave mode: the channels' column in the row's [octave][d] scale table
    const float2 *srow = a.scale + (OCT ? row * kOctaves * g.D : 0);
    const uint32_t lgD = (uint32_t)__builtin_ctz(D);
    // octave mode, full batches: the row's table from scalar registers, a
    // scale at byte offset (octave << (lgD + 3)) + 8 d
    const char *srow_b = reinterpret_cast<const char *>(OCT ? wave_uniform(srow) : srow);
    auto scale_at = [&](float m, int j) {
      return *reinterpret_cast<const float *>(srow_b + ((octave_of(m, er[j % PER]) << (lgD + 3)) + (cb[j % PER] << 3)));
    };
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t ch = row * g.D + ((lane + kLanes * j) & (D - 1));
      if (OCT) {
        er[j] = a.eref[ch];
        cb[j] = (uint32_t)((lane + kLanes * j) & (D - 1));
      } else {
        s[j] = a.scale[ch].x;
      }
    }
    // octave mode with at most two channels per lane (head_dim up to 128): the
    // lane's whole scale table, 8 octaves per channel, sits in registers and
    // a symbol picks its scale by three selects on the octave's bits. With
    // the table in memory the next batch's scales are read half a batch
    // ahead, and that read waits for the next batch's means, which have then
    // had only half a batch to arrive (k_encode 18% slower on the FP8-residual
    // cache). Wider heads would need 32 or 64 registers for the table and keep
    // the reads.
    constexpr bool kRegOct = OCT && PER <= 2;
    static_assert(kOctaves == 8, "the scale select takes three octave bits");
    float so[kRegOct ? PER * kOctaves : 1];
    if (kRegOct) {
#pragma unroll
      for (int j = 0; j < PER; ++j)
#pragma unroll
        for (int q = 0; q < kOctaves; ++q) so[j * kOctaves + q] = srow[(q << lgD) + cb[j]].x;
#pragma unroll
      for (int q = 0; q < PER * kOctaves; ++q) asm volatile("" ::"v"(so[q]));
    }
    auto scale_reg = [&](float m, int j) {
      const uint32_t o = octave_of(m, er[j % PER]);
      const float *tb = so + (kRegOct ? (j % PER) * kOctaves : 0);
      const bool o1 = (o & 1u) != 0, o2 = (o & 2u) != 0, o4 = (o & 4u) != 0;
      const float a0 = o1 ? tb[1] : tb[0], a1 = o1 ? tb[3] : tb[2], a2 = o1 ? tb[5] : tb[4], a3 = o1 ? tb[7] : tb[6];
      const float b0 = o2 ? a1 : a0, b1 = o2 ? a3 : a2;
      return o4 ? b1 : b0;
    };
    // wait for the scales here: a wait inside the symbol loop would also wait
    // for the batch loads in flight on every trip
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (OCT) asm volatile("" ::"v"(er[j]));
      else asm volatile("" ::"v"(s[j]));
    }

    LaneCoder cod;
    uint8_t *slot = slots + (uint64_t)(taken & 1u) * kLanes * g.lane_cap;
    ++taken;
    cod.init(slot, (uint32_t)lane, g.lane_cap / 4);
    if (AD) adapt_start(*aw, s_pairs, s_prior, lane);

    const int nk = lane < nsc ? (nsc - lane + kLanes - 1) / kLanes : 0;  // this lane's symbols
    const int nfull = nsc / kStep;                                         // batches every lane fills
    // two batch buffers used by turns (the next batch loads into the other
    // one), so no batch is copied from one set of registers to the other
    Batch<SYM, MU> bA, bB;
    // octave mode with the table in memory: a batch's scales depend on its
    // means; they are read half a batch ahead, once the next batch's means
    // have arrived
    float sA[kBatch], sB[kBatch];
    if (nfull > 0) {
      bA.load_full(a, base + lane);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) asm volatile("" ::"v"(bA.xs[j]), "v"(bA.ms[j]));
      if (OCT && !kRegOct) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) sA[j] = scale_at(bA.mu(j), j);
      }
    }
    auto batch = [&](int b, Batch<SYM, MU> &cur, Batch<SYM, MU> &nxt, float (&sb)[kBatch], float (&sbn)[kBatch])
                     __attribute__((always_inline)) {
      // this batch's symbols and means were loaded one batch ago; wait for
      // them here, once per batch, and not inside the symbols
#pragma unroll
      for (int j = 0; j < kBatch; ++j) asm volatile("" ::"v"(cur.xs[j]), "v"(cur.ms[j]));
      if (b + 1 < nfull) nxt.load_full(a, base + lane + (int64_t)(b + 1) * kStep);  // in flight meanwhile
      if (AD && b > 0 && b % kAdaptBatches == 0) adapt_rebuild(*aw, g.Mp, lane);  // a new epoch
      // software-pipelined by one symbol: symbol j + 1's model pair (its table
      // reads) is issued before symbol j's coder step, whose branches would
      // otherwise keep the reads from starting until the step is done
      // (k_encode -1.5..-3% on the e4m3 caches and -1% on bf16 in A/B runs)
      cod.flush_batch();
      uint32_t c = 0, f = 0;
      model_pair<SYM, FAST, !AD>(a, t, cur.xs[0], cur.mu(0), kRegOct ? scale_reg(cur.mu(0), 0) : OCT ? sb[0] : s[0], c, f);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (OCT && !kRegOct && j == kBatch / 2 && b + 1 < nfull) {
#pragma unroll
          for (int q = 0; q < kBatch; ++q) sbn[q] = scale_at(nxt.mu(q), q);
        }
        uint32_t cn = 0, fn = 0;
        if (j + 1 < kBatch)
          model_pair<SYM, FAST, !AD>(a, t, cur.xs[j + 1], cur.mu(j + 1),
                                kRegOct ? scale_reg(cur.mu(j + 1), j + 1) : OCT ? sb[j + 1] : s[(j + 1) % PER], cn, fn);
        cod.encode(c, f);
        c = cn;
        f = fn;
      }
      // the batch's symbols join the epoch's counts after its table reads: LDS
      // operations complete in order, so an atomic among the reads would make
      // every later read wait for it
      if (AD) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) adapt_count(*aw, cur.xs[j]);
      }
    };
    for (int b = 0; b < nfull; b += 2) {
      batch(b, bA, bB, sA, sB);
      if (b + 1 < nfull) batch(b + 1, bB, bA, sB, sA);
    }
    Batch<SYM, MU> &cur = bA;
    // the last, partial batch of a short chunk: symbol by symbol (an epoch
    // boundary can only fall at its start)
    if (AD && nfull > 0 && nfull % kAdaptBatches == 0 && nsc > nfull * kStep) adapt_rebuild(*aw, g.Mp, lane);
    for (int k = nfull * kBatch; k < nk; ++k) {
      const int64_t i = base + lane + (int64_t)k * kLanes;
      const int j = k & (kBatch - 1);
      cur.one(a, i, 0);
      if (AD) adapt_count(*aw, cur.xs[0]);
      float sj;
      if (OCT) {
        int32_t e = er[0];
        uint32_t b0 = cb[0];
#pragma unroll
        for (int q = 1; q < PER; ++q)
          if (j % PER == q) {
            e = er[q];
            b0 = cb[q];
          }
        sj = srow[(octave_of(cur.mu(0), e) << lgD) + b0].x;
      } else {
        sj = s[0];
#pragma unroll
        for (int q = 1; q < PER; ++q)
          if (j % PER == q) sj = s[q];
      }
      uint32_t c, f;
      model_pair<SYM, FAST, !AD>(a, t, cur.xs[0], cur.mu(0), sj, c, f);
      cod.encode(c, f);
    }
    uint32_t nbytes = cod.finish();
    // every frequency >= 1 bounds a lane at 3 bytes per symbol + 1; more means a broken table
    if (nbytes > g.lane_cap) {
      set_status(a.status, SKV_ERR_TABLE);
      nbytes = g.lane_cap;
    }
    uint32_t tot = nbytes;
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    const uint64_t size = ((uint64_t)kHeaderBytes + tot + 3) & ~3ull;

    // ---- offsets: publish the size; finish the pending chunk, then this one
    // unless it would have to wait
    if (chunk == 0) {
      finalize(0, 0, size, nbytes, slot);
      continue;
    }
    if (lane == 0) flag_store(a.flags + chunk, kFlagAgg | size);
    if (pend >= 0) {
      uint64_t o0;
      if (!look_back(a.flags, pend, lane, o0, kSpinLimit)) set_status(a.status, SKV_ERR_HIP);
      finalize(pend, o0, pend_size, pend_len, pend_slot);
      pend = -1;
    }
    uint64_t o0;
    if (look_back(a.flags, chunk, lane, o0, 0)) {
      finalize(chunk, o0, size, nbytes, slot);
    } else {
      pend = chunk;
      pend_len = nbytes;
      pend_size = size;
      pend_slot = slot;
    }
  }
}

// The encoder's LDS tables in one block, the small ones first: every table
// then starts below 64 KB, so a table read takes its base as the LDS
// instruction's immediate offset and its index by one shift (a separate base
// register costs a three-operand shift-add, twice the issue time of a shift).
template <bool AD>
struct alignas(16) AdaptBlock {
  uint32_t prior[256];
  AdaptLds w[kEncWaves];
};
template <>
struct AdaptBlock<false> {};

template <bool BF, bool AD>
struct EncLds {
  float4 ep[BF || AD ? 1 : 256];  // static e4m3: per pattern (bin edges, A(k), A(k + 1))
  float2 kn[kNKnot];
  uint32_t ab[BF ? kNWin + 2 : 512];  // (even length: the next table stays 8-byte aligned)
  float2 et[BF ? 1 : 256];
  uint32_t a16w[BF ? kNWin * kWinEntries / 2 : 1];
  AdaptBlock<AD> ad;
};

template <int SYM, int MU, int PER, int OCT, int AD>
__global__ __launch_bounds__(kEncBlock) void k_encode(EncArgs a) {
  constexpr bool BF = SYM == SKV_SYM_BF16;
  static_assert(!(BF && AD), "adaptive p_hat is e4m3 only");
  __shared__ EncLds<BF, AD != 0> lds;
  float2 *s_kn = lds.kn;
  uint32_t *s_a16w = lds.a16w;
  uint32_t *s_ab = lds.ab;
  float2 *s_et = lds.et;

  const bool fast = BF ? *a.aflag != 0 : true;  // windowed p_hat table usable
  for (int i = threadIdx.x; i < kNKnot; i += kEncBlock) s_kn[i] = a.knots[i];
  if (BF) {
    if (fast) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(a.a16);
      for (int i = threadIdx.x; i < kNWin * kWinEntries / 2; i += kEncBlock) s_a16w[i] = src[i];
      for (int i = threadIdx.x; i <= kNWin; i += kEncBlock) s_ab[i] = a.abase[i];
    }
  } else {
    // (A(k), A(k + 1)) side by side at the pattern of rank k
    for (int i = threadIdx.x; i < 512; i += kEncBlock) s_ab[i] = a.ptab[(tix_e4m3((uint32_t)i >> 1) ^ 0x80u) + (i & 1)];
    for (int i = threadIdx.x; i < 256; i += kEncBlock) s_et[i] = a.etab[i];
    if constexpr (AD == 0) {
      for (int i = threadIdx.x; i < 256; i += kEncBlock) {
        const uint32_t j = tix_e4m3((uint32_t)i) ^ 0x80u;
        const float2 e = a.etab[i];
        lds.ep[i] = make_float4(e.x, e.y, __uint_as_float(a.ptab[j]), __uint_as_float(a.ptab[j + 1]));
      }
    }
  }
  AdaptLds *aw = nullptr;
  const uint32_t *s_prior = nullptr;
  if constexpr (AD != 0) {
    for (int i = threadIdx.x; i < 256; i += kEncBlock) lds.ad.prior[i] = a.prior[i];
    aw = &lds.ad.w[__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))];
    s_prior = lds.ad.prior;
  }
  __syncthreads();
  const EncTables t{s_kn, reinterpret_cast<const uint16_t *>(s_a16w), s_ab, s_et, lds.ep};
  if (fast) encode_chunks<SYM, MU, PER, OCT, true, AD != 0>(a, t, aw, s_ab, s_prior);
  else encode_chunks<SYM, MU, PER, OCT, false, AD != 0>(a, t, aw, s_ab, s_prior);
}

__global__ void k_enc_reset(uint64_t *__restrict__ flags, int64_t n, uint32_t *__restrict__ ctr) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < n; i += (int64_t)gridDim.x * blockDim.x) flags[i] = 0;
  if (i0 == 0) *ctr = 0;
}

template <int SYM, int MU, int AD>
static void launch_enc_kernel(const EncArgs &a, hipStream_t st) {
  static_assert(kEncWaves == 16, "the workspace holds two scratch slots for each of 16 waves per block");
  // the grid the workspace's scratch slots were sized for
  const unsigned blocks = (unsigned)a.g.enc_blocks;
  // the scale period of a lane's symbols: max(2, head_dim / 64); the sigma mode
#define SKV_ENC(P_, O_) hipLaunchKernelGGL((k_encode<SYM, MU, P_, O_, AD>), dim3(blocks), dim3(kEncBlock), 0, st, a)
  const int per = a.g.D >= 512 ? 8 : (a.g.D >= 256 ? 4 : 2);
  if (a.g.octave) {
    if (per == 8) SKV_ENC(8, 1); else if (per == 4) SKV_ENC(4, 1); else SKV_ENC(2, 1);
  } else {
    if (per == 8) SKV_ENC(8, 0); else if (per == 4) SKV_ENC(4, 0); else SKV_ENC(2, 0);
  }
#undef SKV_ENC
}

hipError_t launch_encode(const Geo &g, const void *x, const void *mu, const Workspace &ws, uint8_t *bits,
                         uint64_t bits_cap, uint64_t *offsets, int32_t *status, hipStream_t st) {
  EncArgs a{g, x, mu, ws.knots, ws.ptab, ws.a16, ws.abase, ws.aflag, ws.etab, ws.prior, ws.scale, ws.eref, ws.flags,
            ws.ctr, ws.scratch, bits, bits_cap, offsets, status};
  hipLaunchKernelGGL(k_enc_reset, dim3(256), dim3(256), 0, st, ws.flags, g.n_chunks, ws.ctr);
  timing_mark(kTimeEncode, false, st);
  if (g.sym_fmt == SKV_SYM_BF16) {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_BF16, SKV_MU_BF16, 0>(a, st);
    else launch_enc_kernel<SKV_SYM_BF16, SKV_MU_F32, 0>(a, st);
  } else if (g.adapt) {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_BF16, 1>(a, st);
    else launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_F32, 1>(a, st);
  } else {
    if (g.mu_fmt == SKV_MU_BF16) launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_BF16, 0>(a, st);
    else launch_enc_kernel<SKV_SYM_E4M3, SKV_MU_F32, 0>(a, st);
  }
  timing_mark(kTimeEncode, true, st);
  return hipGetLastError();
}

}  // namespace skv
