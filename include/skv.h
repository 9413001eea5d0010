/*
 * skv.h -- C ABI of libskv, the MI355X (gfx950) speculative-KV-coding library.
 *
 * Speculative KV coding compresses a model's KV cache losslessly: a cheap
 * predictor gives every cache scalar x a mean mu, a calibrated per-(kv, head,
 * channel) sigma gives its spread, and an arithmetic coder spends about
 * -log2 q(x) bits per scalar under the model
 *     q = 0.95 N(mu, sigma^2) + 0.03 N(mu, (3 sigma)^2) + 0.02 p_hat,
 * p_hat being the empirical symbol distribution, integrated over each
 * symbol's bf16 or FP8-e4m3 bin.  Pages: "Speculative KV coding: lossless KV
 * cache compression up to ~4x", sections "q 应是什么样的" (what q should look
 * like), "什么能预测 KV 缓存" (what predicts the KV cache: the coder maps
 * (KV_full, mu, sigma) to bits and (bits, mu, sigma) back), "早期结果" (early
 * results: the mixture, sigma per (kv, head, channel)), "原生 FP8 KV 缓存"
 * (native FP8 cache: bin-integrated model over e4m3 symbols).
 *
 * Stream layout.  A chunk is one (layer, kv, head) row's block of 256 tokens
 * (the last block of a row may be shorter); chunk ids run over rows, then
 * blocks.  Scalar i of a chunk (memory order, i = token * head_dim + channel)
 * goes to lane i mod 64, and each of the 64 lanes range-codes its scalars in
 * order as one substream (48-bit window, byte renormalisation, frequencies on a
 * 2^24 total).  Chunk bytes: 64 little-endian u16 substream lengths; then, with
 * m the fewest whole 4-byte words any substream has, words 0 .. m-1 of the 64
 * substreams interleaved word by word (word w of lane l at 4 (64 w + l)); then
 * the rest of each substream, lane by lane; then zeros up to a multiple of 4
 * bytes.  u64 offsets[c] .. offsets[c+1] delimit chunk c.  The encoder output
 * is a deterministic function of the inputs, byte for byte.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device (HBM) pointers on the current HIP
 *     device; (host) pointers are host memory.  The caller owns every buffer.
 *     The library allocates no device memory: scratch comes from `workspace`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls validate their arguments on the host, then enqueue kernels on the
 *     stream and return without synchronising.
 *   - The return value reports synchronous errors (bad arguments, launch
 *     failures).  Errors that depend on the data are written by the kernels to
 *     `*status` (device int32, cleared by the call itself); read it after the
 *     stream has run.  When *status != SKV_OK the outputs are unspecified but
 *     every kernel stays inside the buffers described here.
 *   - Calls are stateless; concurrent calls must use distinct workspaces.
 *
 * Cache layout (x, mu, x_out): [layers][2 (K=0, V=1)][kv_heads][tokens][head_dim],
 * contiguous, 16-byte aligned.  head_dim must be a multiple of 8 that divides
 * 512 (8 .. 512; Qwen3 uses 128).  Symbols are raw bit patterns.
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum skv_status {
  SKV_OK = 0,
  SKV_ERR_ARG = 1,          /* bad argument (null pointer, bad shape, sigma or p_hat mode, non-finite or negative sigma) */
  SKV_ERR_UNSUPPORTED = 2,  /* head_dim not a multiple of 8 dividing 512; adaptive p_hat with bf16 symbols */
  SKV_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
  SKV_ERR_CAPACITY = 4,     /* the compressed stream does not fit bits_cap */
  SKV_ERR_CORRUPT = 5,      /* the stream does not decode consistently */
  SKV_ERR_TABLE = 6,        /* histogram too large for the p_hat table: its smoothed total
                               H(N) = sum over patterns of (hist + 1), an exact integer, has
                               Mp * H(N) > 2^62 (this includes a total beyond 2^64) */
  SKV_ERR_SCRATCH = 7       /* skv_decode_static: the shape's decode workspace is larger than
                               SKV_STATIC_SCRATCH_BYTES */
};

enum skv_sym_fmt { SKV_SYM_BF16 = 0, SKV_SYM_E4M3 = 1 };
enum skv_mu_fmt { SKV_MU_BF16 = 0, SKV_MU_F32 = 1 };

/*
 * How sigma is resolved per scalar.
 *   SKV_SIGMA_CHANNEL: one sigma per (layer, kv, head, channel); the sigma
 *     array is fp32 [layers][2][kv_heads][head_dim] ("早期结果").
 *   SKV_SIGMA_OCTAVE: sigma also depends on the magnitude of the scalar's mean,
 *     which both ends know (the pages name a static per-channel sigma as a
 *     cost, "下一步计划").  The sigma array is fp32
 *     [layers][2][kv_heads][head_dim][SKV_OCT_STRIDE]: per channel its own
 *     sigma_c, then sigma_c,j for octaves j = 0..7.  A scalar with mean mu'
 *     (mu, or 0 when mu is not finite) takes octave
 *       j = clamp(E(mu') - E(max(sigma_c, 2^-100)) - 1, 0, 7),
 *     E the fp32 biased exponent field (0 for zero and subnormals), and codes
 *     with sigma_c,j.  Calibration sets sigma_c as in channel mode and
 *     sigma_c,j by the same estimator over the channel's scalars in octave j
 *     (their squares summed per exponent field in fp64, the fields of an
 *     octave added in increasing order), or sigma_c when fewer than 16 fell
 *     in the octave.
 */
enum skv_sigma_mode { SKV_SIGMA_CHANNEL = 0, SKV_SIGMA_OCTAVE = 1 };
#define SKV_OCTAVES 8
#define SKV_OCT_STRIDE (1 + SKV_OCTAVES)

/*
 * Which p_hat the coder uses.
 *   SKV_PHAT_STATIC: the calibrated histogram, one table for the whole cache.
 *   SKV_PHAT_ADAPTIVE (e4m3 symbols only, else SKV_ERR_UNSUPPORTED): decayed
 *     symbol counts that follow the data, as the online entropy-estimation
 *     page proposes (decayed counts C_t = alpha C_{t-1} + delta, "虚拟滑动窗口
 *     的设计原理"; one window per layer-head, "针对 KV 缓存的局部性优化"; a
 *     calibrated prior against cold start, "局限性与应对").  The window is one
 *     chunk.  Epoch e of a chunk is its scalars [e E, (e+1) E), E =
 *     SKV_ADAPT_EPOCH, all lanes together.  Epoch 0 codes with the static
 *     table; epoch e+1 with the p_hat table built (as the static one is) from
 *     counts C_{e+1}(k) = floor(alpha C_e(k)) + n_e(k), alpha = 3/4, n_e(k)
 *     the epoch's scalars of rank k, C_0(k) = floor(SKV_ADAPT_PRIOR_WEIGHT *
 *     (the static table's p_hat counts of rank k) / Mp).  Only p_hat adapts;
 *     the mixture weights stay 0.95 / 0.03 / 0.02.
 */
enum skv_phat_mode { SKV_PHAT_STATIC = 0, SKV_PHAT_ADAPTIVE = 1 };
#define SKV_ADAPT_EPOCH 4096
#define SKV_ADAPT_PRIOR_WEIGHT 8192

typedef struct skv_shape {
  int64_t layers;      /* >= 1 */
  int64_t kv_heads;    /* >= 1 */
  int64_t tokens;      /* >= 1; the last 256-token chunk of a row may be shorter */
  int64_t head_dim;    /* multiple of 8 dividing 512 */
  int32_t sym_fmt;     /* enum skv_sym_fmt: symbols are bf16 (uint16 patterns) or e4m3 (uint8 patterns) */
  int32_t mu_fmt;      /* enum skv_mu_fmt: predictor means are bf16 (uint16 patterns) or fp32 */
  int32_t sigma_mode;  /* enum skv_sigma_mode */
  int32_t phat_mode;   /* enum skv_phat_mode (0: the calibrated histogram) */
} skv_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char *skv_status_string(int status);

/* ---------------------------------------------------------------- sizes (host only) */

/* Number of chunks: layers * 2 * kv_heads * ceil(tokens / 256).  Chunk ids run
 * over (layer, kv, head) rows, then 256-token blocks.  Returns SKV_ERR_ARG /
 * SKV_ERR_UNSUPPORTED for a bad shape. */
int skv_num_chunks(const skv_shape *shape, int64_t *n_chunks);

/* Largest possible encoded size in bytes: n_chunks * (128 + 64 + 3) + 3 * n_scalars
 * (a frequency of 1 in 2^24 costs at most 3 bytes; one flush byte per lane; at
 * most 3 bytes of padding per chunk). */
int skv_encode_bound(const skv_shape *shape, size_t *bytes);

/* Device workspace needed by skv_encode and skv_decode for this shape. */
int skv_workspace_size(const skv_shape *shape, size_t *bytes);

/* Device workspace (calibration state) needed by the calibration calls: per
 * channel an fp64 sum of squares and a u64 count, plus the u64 histogram; in
 * octave mode also per channel 256 such pairs, one per exponent field of mu'. */
int skv_calib_state_size(const skv_shape *shape, size_t *bytes);

/* ---------------------------------------------------------------- calibration */
/*
 * sigma^2 = E[(KV_full - mu)^2] minimises the expected code length ("q 应是
 * 什么样的"); it is measured per (layer, kv, head, channel) on a small
 * calibration set and frozen ("同一模型的优化版本", "早期结果"), and p_hat is
 * the calibration set's symbol histogram ("早期结果").
 *
 * Per channel c, over the calibration scalars with a finite symbol value v:
 *   S_c += RN64(r * r), r = RN64(v - mu'), n_c += 1, in call order then token
 *   order (mu' = mu in fp32, or 0 when mu is not finite);
 *   sigma_c = RN32(sqrt(RN64(S_c / n_c))), or 1.0 when n_c = 0.
 * hist[b] counts every symbol pattern b (NaN patterns included).
 * The result is deterministic: sums are fp64 in a fixed order and the
 * histogram uses integer atomics only.
 */

/* Clear a calibration state of skv_calib_state_size(shape) bytes (device). */
int skv_calib_reset(void *state, const skv_shape *shape, void *stream);

/* Add one batch of calibration sequences: x and mu (device) laid out like a
 * cache of shape seq_shape.  seq_shape must match the state's shape in
 * layers, kv_heads, head_dim and formats; tokens may differ per call. */
int skv_calib_accumulate(void *state, const skv_shape *seq_shape, const void *x, const void *mu,
                         void *stream);

/* sigma (device, fp32 [layers][2][kv_heads][head_dim], times SKV_OCT_STRIDE in
 * octave mode) and hist (device, u64 [65536] for bf16, [256] for e4m3, indexed
 * by bit pattern, raw counts) from the state.  The state is left unchanged. */
int skv_calib_finalize(const void *state, const skv_shape *shape, float *sigma, uint64_t *hist,
                       void *stream);

/* Convenience: reset, accumulate n_seq sequences stored back to back (each of
 * shape seq_shape), finalize.  state: skv_calib_state_size(seq_shape) bytes. */
int skv_calibrate(const skv_shape *seq_shape, int64_t n_seq, const void *x, const void *mu,
                  float *sigma, uint64_t *hist, void *state, void *stream);

/* ---------------------------------------------------------------- encode / decode */

/*
 * Encode a cache.
 *   x       (device) symbols, cache layout, bf16 or e4m3 patterns
 *   mu      (device) predictor means, cache layout, bf16 patterns or fp32
 *   sigma   (device) fp32 [layers][2][kv_heads][head_dim] (channel mode) or
 *           [..][head_dim][SKV_OCT_STRIDE] (octave mode), every entry finite
 *           and >= 0 (sigma below 2^-100 is treated as 2^-100)
 *   hist    (device) u64 symbol histogram as produced by skv_calib_finalize
 *   bits    (device) output stream, bits_cap bytes (>= skv_encode_bound
 *           guarantees success); 16-byte aligned, else SKV_ERR_ARG
 *   offsets (device) u64 [n_chunks + 1]: chunk c is bits[offsets[c], offsets[c+1]);
 *           offsets[n_chunks] is the stream's total size
 *   workspace (device) skv_workspace_size(shape) bytes
 *   status  (device) int32: SKV_OK, SKV_ERR_CAPACITY (stream larger than
 *           bits_cap; offsets are still valid), SKV_ERR_ARG (bad sigma),
 *           SKV_ERR_TABLE (histogram too large)
 */
int skv_encode(const skv_shape *shape, const void *x, const void *mu, const float *sigma,
               const uint64_t *hist, uint8_t *bits, size_t bits_cap, uint64_t *offsets,
               void *workspace, size_t workspace_bytes, int32_t *status, void *stream);

/*
 * Decode a cache encoded by skv_encode with the same shape, mu, sigma and hist
 * (the model is not stored in the stream: both ends rebuild it, "什么能预测 KV
 * 缓存").
 *   bits     (device) the stream, 4-byte aligned, bits_bytes readable bytes
 *            (a multiple of 4; skv_encode's buffer qualifies); no read leaves
 *            [bits, bits + bits_bytes) whatever offsets and headers say
 *   offsets  (device) u64 [n_chunks + 1] (a chunk outside bits_bytes, or with
 *            offsets[c+1] < offsets[c], decodes as corrupt)
 *   x_out    (device) decoded symbols, cache layout
 *   status   (device) int32: SKV_OK or SKV_ERR_CORRUPT (header lengths that do
 *            not add up, a quotient outside the frequency total, or a substream
 *            whose length disagrees with what its symbols consumed), or the
 *            model errors of skv_encode
 */
int skv_decode(const skv_shape *shape, const uint8_t *bits, size_t bits_bytes,
               const uint64_t *offsets, const void *mu, const float *sigma, const uint64_t *hist,
               void *x_out, void *workspace, size_t workspace_bytes, int32_t *status, void *stream);

/*
 * Decode without any allocation, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, outputs, status
 * words and stream behaviour as skv_decode, less the workspace: the decode
 * workspace (model tables, per-channel scales, chunk counter) lives in a
 * static device array of SKV_STATIC_SCRATCH_BYTES inside the library, one
 * copy per GPU, held until the process ends.  The first call on a device
 * resolves that array's address (hipGetSymbolAddress) with the device
 * current; no call allocates or frees memory, and the counter and status are
 * cleared by a kernel (no memset).
 * Limit: the shape's decode workspace must fit the array (16 MiB: about two
 * million channels in channel mode, 230 thousand in octave mode, against
 * 131,072 for the Qwen3-32B cache); a larger shape returns SKV_ERR_SCRATCH and
 * enqueues nothing.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two host threads) race
 * and must be serialised by the caller.
 */
#define SKV_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int skv_decode_static(const skv_shape *shape, const uint8_t *bits, size_t bits_bytes,
                      const uint64_t *offsets, const void *mu, const float *sigma, const uint64_t *hist,
                      void *x_out, int32_t *status, void *stream);

/* ---------------------------------------------------------------- kernel timing */

/*
 * Measurement aid, not part of the method.  Between skv_timing_start and
 * skv_timing_stop every main launch of skv_encode / skv_decode (the model
 * build as one record, k_encode, k_decode) is bracketed
 * by two HIP events recorded on the call's own stream, so one kernel's time is
 * known without a profiler and without synchronising between calls.
 * Recording is process-wide and meant for one host thread issuing the calls.
 *
 * skv_timing_start: creates 2 * capacity events on the current device
 *   (1 <= capacity <= 2^20).  SKV_ERR_ARG if recording is already on or the
 *   capacity is out of range, SKV_ERR_HIP if the events cannot be created.
 *   Launches past the capacity go unrecorded.
 * skv_timing_stop: waits for the recorded events, writes the first
 *   min(count, capacity) records (host arrays: kernel id, milliseconds) in
 *   launch order, stores the number recorded in *count (host), releases the
 *   events and stops recording.  SKV_ERR_ARG if recording is off or a pointer
 *   is null; SKV_ERR_HIP if an event could not be read (its time is 0).
 * skv_timed_kernel_name: the name of a kernel id ("model", "k_encode",
 *   "k_decode"; "unknown" otherwise), static storage.
 */
int skv_timing_start(int32_t capacity);
int skv_timing_stop(int32_t *kernel, float *ms, int32_t capacity, int32_t *count);
const char *skv_timed_kernel_name(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* SKV_H */
