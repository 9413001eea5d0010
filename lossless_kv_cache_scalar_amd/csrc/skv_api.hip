// skv_api.hip -- the C ABI of libskv: argument checks, workspace layout and
// kernel launches on the caller's stream.  Declarations and contracts: skv.h.
#include <math.h>

#include <mutex>

#include "skv_internal.hpp"

using namespace skv;

extern "C" const char *skv_status_string(int status) {
  switch (status) {
    case SKV_OK: return "ok";
    case SKV_ERR_ARG: return "invalid argument";
    case SKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be a multiple of 8 dividing 512)";
    case SKV_ERR_HIP: return "HIP runtime error";
    case SKV_ERR_CAPACITY: return "compressed stream exceeds the output capacity";
    case SKV_ERR_CORRUPT: return "corrupt stream";
    case SKV_ERR_TABLE: return "histogram too large for the p_hat table";
    case SKV_ERR_SCRATCH: return "shape needs more than the library's static scratch (skv_decode_static)";
    default: return "unknown status";
  }
}

namespace skv {
int device_cu_count() {
  static std::mutex mu;
  static int n[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (n[dev] <= 0) {
    int c = 0;
    n[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0 ? c : 256;
  }
  return n[dev];
}
}  // namespace skv

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// shape checks and derived geometry; returns SKV_OK or an error
int make_geo(const skv_shape *sh, Geo &g) {
  if (!sh) return SKV_ERR_ARG;
  if (sh->layers < 1 || sh->kv_heads < 1 || sh->tokens < 1 || sh->head_dim < 1) return SKV_ERR_ARG;
  if (sh->sym_fmt != SKV_SYM_BF16 && sh->sym_fmt != SKV_SYM_E4M3) return SKV_ERR_ARG;
  if (sh->mu_fmt != SKV_MU_BF16 && sh->mu_fmt != SKV_MU_F32) return SKV_ERR_ARG;
  if (sh->sigma_mode != SKV_SIGMA_CHANNEL && sh->sigma_mode != SKV_SIGMA_OCTAVE) return SKV_ERR_ARG;
  if (sh->phat_mode != SKV_PHAT_STATIC && sh->phat_mode != SKV_PHAT_ADAPTIVE) return SKV_ERR_ARG;
  // head_dim a power of two from 8 to 512: a lane's channels then repeat with
  // a period dividing kBatch
  if (sh->head_dim % 8 != 0 || 512 % sh->head_dim != 0) return SKV_ERR_UNSUPPORTED;
  // adaptive p_hat keeps a count per symbol in each chunk's window: e4m3 only
  if (sh->phat_mode == SKV_PHAT_ADAPTIVE && sh->sym_fmt != SKV_SYM_E4M3) return SKV_ERR_UNSUPPORTED;
  if (sh->layers > (1 << 20) || sh->kv_heads > (1 << 16) || sh->tokens > (int64_t(1) << 32)) return SKV_ERR_ARG;
  g.layers = sh->layers;
  g.heads = sh->kv_heads;
  g.tokens = sh->tokens;
  g.D = sh->head_dim;
  g.ntb = (sh->tokens + kChunkTokens - 1) / kChunkTokens;
  g.rows = sh->layers * 2 * sh->kv_heads;
  g.n_chunks = g.rows * g.ntb;
  g.sym_fmt = sh->sym_fmt;
  g.mu_fmt = sh->mu_fmt;
  g.octave = sh->sigma_mode == SKV_SIGMA_OCTAVE ? 1 : 0;
  g.adapt = sh->phat_mode == SKV_PHAT_ADAPTIVE ? 1 : 0;
  g.N = sh->sym_fmt == SKV_SYM_BF16 ? 65536u : 256u;
  g.log2T = sh->sym_fmt == SKV_SYM_BF16 ? 24u : 16u;
  // one count per symbol; the rest split 0.98 : 0.02 between the Gaussian
  // pair and p_hat, the mixture's weights ("Speculative KV coding", "早期结果")
  uint32_t budget = (1u << g.log2T) - g.N;
  g.MG = (uint32_t)llround(0.98 * (double)budget);
  g.Mp = budget - g.MG;
  // most bytes a lane can emit: 3 per symbol (4 * head_dim symbols) + 1
  g.lane_cap = (uint32_t)((3 * 4 * g.D + 1 + 3) / 4 * 4);
  // the encoder's persistent grid: one 16-wave block per compute unit at most
  const int64_t need = (g.n_chunks + 15) / 16;
  const int64_t cus = device_cu_count();
  g.enc_blocks = need < cus ? need : cus;
  return SKV_OK;
}

struct Layout {
  size_t knots, ptab, a16, abase, aflag, psum, uinv, etab, prior, scale, eref, flags, ctr, scratch, total;
};

// The workspace of a call: the model tables, the per-channel scales and the
// chunk counter; an encode also needs the chunks' published sizes and its
// scratch slots (enc = false leaves those two empty).
Layout layout(const Geo &g, bool enc = true) {
  Layout L;
  size_t o = 0;
  L.knots = o; o = align_up(o + sizeof(float2) * kNKnot);
  L.ptab = o;  o = align_up(o + sizeof(uint32_t) * (g.N + 1));
  L.a16 = o;   o = align_up(o + sizeof(uint16_t) * kNWin * kWinEntries);
  L.abase = o; o = align_up(o + sizeof(uint32_t) * (kNWin + 1));
  L.aflag = o; o = align_up(o + sizeof(int32_t));
  L.psum = o;  o = align_up(o + sizeof(uint64_t) * 64);
  L.uinv = o;  o = align_up(o + sizeof(float2) * (kNInv + 1));
  L.etab = o;  o = align_up(o + sizeof(float2) * 256);
  L.prior = o; o = align_up(o + sizeof(uint32_t) * 256);
  L.scale = o; o = align_up(o + sizeof(float2) * (size_t)(g.rows * g.D) * (g.octave ? kOctaves : 1));
  L.eref = o;  o = align_up(o + sizeof(int32_t) * (size_t)(g.octave ? g.rows * g.D : 1));
  L.flags = o; o = align_up(o + (enc ? sizeof(uint64_t) * (size_t)g.n_chunks : 0));
  L.ctr = o;   o = align_up(o + sizeof(uint32_t));
  // two slots per encoder wave: a wave holds at most its current chunk and one
  // whose offset it is still waiting for
  L.scratch = o; o = align_up(o + (enc ? (size_t)g.enc_blocks * 16 * 2 * kLanes * g.lane_cap : 0));
  L.total = o;
  return L;
}

Workspace carve(const Geo &g, void *base, bool enc = true) {
  Layout L = layout(g, enc);
  uint8_t *b = static_cast<uint8_t *>(base);
  Workspace w;
  w.knots = reinterpret_cast<float2 *>(b + L.knots);
  w.ptab = reinterpret_cast<uint32_t *>(b + L.ptab);
  w.a16 = reinterpret_cast<uint16_t *>(b + L.a16);
  w.abase = reinterpret_cast<uint32_t *>(b + L.abase);
  w.aflag = reinterpret_cast<int32_t *>(b + L.aflag);
  w.psum = reinterpret_cast<uint64_t *>(b + L.psum);
  w.uinv = reinterpret_cast<float2 *>(b + L.uinv);
  w.etab = reinterpret_cast<float2 *>(b + L.etab);
  w.prior = reinterpret_cast<uint32_t *>(b + L.prior);
  w.scale = reinterpret_cast<float2 *>(b + L.scale);
  w.eref = reinterpret_cast<int32_t *>(b + L.eref);
  w.flags = reinterpret_cast<uint64_t *>(b + L.flags);
  w.ctr = reinterpret_cast<uint32_t *>(b + L.ctr);
  w.scratch = b + L.scratch;
  return w;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? SKV_OK : SKV_ERR_HIP; }

}  // namespace

extern "C" int skv_num_chunks(const skv_shape *shape, int64_t *n_chunks) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!n_chunks) return SKV_ERR_ARG;
  *n_chunks = g.n_chunks;
  return SKV_OK;
}

extern "C" int skv_encode_bound(const skv_shape *shape, size_t *bytes) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!bytes) return SKV_ERR_ARG;
  size_t nsc = (size_t)(g.rows * g.tokens * g.D);
  *bytes = (size_t)g.n_chunks * (kHeaderBytes + kLanes + 3) + 3 * nsc;
  return SKV_OK;
}

extern "C" int skv_workspace_size(const skv_shape *shape, size_t *bytes) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!bytes) return SKV_ERR_ARG;
  *bytes = layout(g).total;
  return SKV_OK;
}

extern "C" int skv_calib_state_size(const skv_shape *shape, size_t *bytes) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!bytes) return SKV_ERR_ARG;
  *bytes = sizeof(uint64_t) * (size_t)(2 * g.rows * g.D * (g.octave ? 1 + kExpBins : 1) + g.N);
  return SKV_OK;
}

extern "C" int skv_calib_reset(void *state, const skv_shape *shape, void *stream) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!state) return SKV_ERR_ARG;
  return hip_status(launch_calib_reset(g, state, static_cast<hipStream_t>(stream)));
}

extern "C" int skv_calib_accumulate(void *state, const skv_shape *seq_shape, const void *x, const void *mu,
                                    void *stream) {
  Geo g;
  int e = make_geo(seq_shape, g);
  if (e != SKV_OK) return e;
  if (!state || !x || !mu) return SKV_ERR_ARG;
  return hip_status(launch_calib_accumulate(g, state, x, mu, static_cast<hipStream_t>(stream)));
}

extern "C" int skv_calib_finalize(const void *state, const skv_shape *shape, float *sigma, uint64_t *hist,
                                  void *stream) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!state || !sigma || !hist) return SKV_ERR_ARG;
  return hip_status(launch_calib_finalize(g, state, sigma, hist, static_cast<hipStream_t>(stream)));
}

extern "C" int skv_calibrate(const skv_shape *seq_shape, int64_t n_seq, const void *x, const void *mu,
                             float *sigma, uint64_t *hist, void *state, void *stream) {
  Geo g;
  int e = make_geo(seq_shape, g);
  if (e != SKV_OK) return e;
  if (n_seq < 0 || !x || !mu || !sigma || !hist || !state) return SKV_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((e = hip_status(launch_calib_reset(g, state, st))) != SKV_OK) return e;
  const size_t nsc = (size_t)(g.rows * g.tokens * g.D);
  const size_t xb = nsc * (g.sym_fmt == SKV_SYM_BF16 ? 2 : 1);
  const size_t mb = nsc * (g.mu_fmt == SKV_MU_BF16 ? 2 : 4);
  for (int64_t j = 0; j < n_seq; ++j) {
    e = hip_status(launch_calib_accumulate(g, state, static_cast<const uint8_t *>(x) + j * xb,
                                           static_cast<const uint8_t *>(mu) + j * mb, st));
    if (e != SKV_OK) return e;
  }
  return hip_status(launch_calib_finalize(g, state, sigma, hist, st));
}

extern "C" int skv_encode(const skv_shape *shape, const void *x, const void *mu, const float *sigma,
                          const uint64_t *hist, uint8_t *bits, size_t bits_cap, uint64_t *offsets, void *workspace,
                          size_t workspace_bytes, int32_t *status, void *stream) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!x || !mu || !sigma || !hist || !bits || !offsets || !workspace || !status) return SKV_ERR_ARG;
  // the chunk writes store u16 / u32 words at bits + offset, offsets being multiples of 4
  if (!aligned16(x) || !aligned16(mu) || !aligned16(workspace) || !aligned16(bits)) return SKV_ERR_ARG;
  if (workspace_bytes < layout(g).total) return SKV_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws = carve(g, workspace);
  if ((e = hip_status(launch_clear_status(status, ws.ctr, st))) != SKV_OK) return e;
  if ((e = hip_status(launch_model(g, sigma, hist, ws, status, st))) != SKV_OK) return e;
  return hip_status(launch_encode(g, x, mu, ws, bits, bits_cap, offsets, status, st));
}

extern "C" int skv_decode(const skv_shape *shape, const uint8_t *bits, size_t bits_bytes, const uint64_t *offsets,
                          const void *mu, const float *sigma, const uint64_t *hist, void *x_out, void *workspace,
                          size_t workspace_bytes, int32_t *status, void *stream) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!bits || !offsets || !mu || !sigma || !hist || !x_out || !workspace || !status) return SKV_ERR_ARG;
  if (!aligned16(mu) || !aligned16(x_out) || !aligned16(workspace)) return SKV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(bits) & 3u) || (bits_bytes & 3u)) return SKV_ERR_ARG;
  if (workspace_bytes < layout(g).total) return SKV_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws = carve(g, workspace);
  if ((e = hip_status(launch_clear_status(status, ws.ctr, st))) != SKV_OK) return e;
  if ((e = hip_status(launch_model(g, sigma, hist, ws, status, st))) != SKV_OK) return e;
  return hip_status(launch_decode(g, bits, bits_bytes, offsets, mu, ws, x_out, status, st));
}

// ---------------------------------------------------------------- decode without allocation
// skv_decode_static: the decode workspace (model tables, scales, chunk
// counter) lives in this file-scope device array instead of a caller buffer.
// Each GPU holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in: its device address comes from
// hipGetSymbolAddress, resolved once per device (with that device current) on
// the first call there, and only that address is passed to kernels.
namespace {
constexpr size_t kStaticScratchBytes = SKV_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void *g_static_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
int static_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SKV_ERR_HIP;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return SKV_OK;
}
}  // namespace

extern "C" int skv_decode_static(const skv_shape *shape, const uint8_t *bits, size_t bits_bytes,
                                 const uint64_t *offsets, const void *mu, const float *sigma, const uint64_t *hist,
                                 void *x_out, int32_t *status, void *stream) {
  Geo g;
  int e = make_geo(shape, g);
  if (e != SKV_OK) return e;
  if (!bits || !offsets || !mu || !sigma || !hist || !x_out || !status) return SKV_ERR_ARG;
  if (!aligned16(mu) || !aligned16(x_out)) return SKV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(bits) & 3u) || (bits_bytes & 3u)) return SKV_ERR_ARG;
  if (layout(g, false).total > kStaticScratchBytes) return SKV_ERR_SCRATCH;
  void *base = nullptr;
  if ((e = static_scratch(&base)) != SKV_OK) return e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Workspace ws = carve(g, base, false);
  // the counter and the status word are cleared by a kernel, not a memset
  if ((e = hip_status(launch_clear_status(status, ws.ctr, st))) != SKV_OK) return e;
  if ((e = hip_status(launch_model(g, sigma, hist, ws, status, st))) != SKV_OK) return e;
  return hip_status(launch_decode(g, bits, bits_bytes, offsets, mu, ws, x_out, status, st));
}
