/*
 * skvref.c -- CPU oracle for speculative KV coding.  TEST INFRASTRUCTURE ONLY.
 *
 * This is the plain, serial, slow statement of what the coding path computes.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  The product library never links, loads or calls it, and the two
 * share no source, header, table or table generator: every constant below is
 * derived here from its definition.
 *
 * The pages (cited by title and section heading):
 *   [SKV]  "Speculative KV coding: lossless KV cache compression up to ~4x"
 *          (Chinese rendering).  Sections by run-in heading:
 *            "KV 缓存并非真正随机"   (the KV cache is not really random)
 *            "q 应是什么样的"        (what q should look like)
 *            "什么能预测 KV 缓存"    (what predicts the KV cache)
 *            "同一模型的优化版本"    (an optimised version of the same model)
 *            "早期结果"              (early results)
 *            "原生 FP8 KV 缓存"      (native FP8 KV cache)
 *            "下一步计划"            (next steps)
 *   [CO]   "Co-optimising speculative decoding and KV cache compression"
 *          (blog), section "工程实现的关键约束" (key engineering constraints).
 *
 * The pages define the model (a mixture of two Gaussians and an empirical
 * symbol histogram, integrated over each symbol's bin) and say an arithmetic
 * coder turns (KV, mu, sigma) into bits and back.  They do not say how the
 * model is made integer or how the stream is laid out; those readings are
 * restated at each function below.
 *
 * Precision.  Integer frequencies are decided by the fp32 model, and encoder
 * and decoder must take that decision identically (both ends must agree to the
 * bit, [CO] key constraints; [SKV] next steps).  So the model is evaluated in
 * fp32 with a fixed operation order: explicit fmaf() where a fused step is
 * meant, no contraction anywhere else (build with -ffp-contract=off), IEEE
 * denormals.  Knot values are computed in fp64 and rounded once to fp32.
 * Calibration sums are fp64.
 *
 * Parity pins live in tests/test_oracle_*.py; every function here has one.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- status codes and enums (same numeric meaning as the public ABI) ---- */
enum { REF_OK = 0, REF_ERR_ARG = 1, REF_ERR_UNSUPPORTED = 2,
       REF_ERR_CAPACITY = 4, REF_ERR_CORRUPT = 5, REF_ERR_TABLE = 6 };
enum { REF_SYM_BF16 = 0, REF_SYM_E4M3 = 1 };
enum { REF_MU_BF16 = 0, REF_MU_F32 = 1 };

enum { REF_SIGMA_CHANNEL = 0, REF_SIGMA_OCTAVE = 1 };

enum { REF_PHAT_STATIC = 0, REF_PHAT_ADAPTIVE = 1 };

typedef struct {
  int64_t layers, kv_heads, tokens, head_dim;
  int32_t sym_fmt, mu_fmt;
  int32_t sigma_mode, phat_mode;
} ref_shape;

/* ---- model geometry ---- */
#define CHUNK_TOKENS 256
#define LANES 64
#define KNOTS_PER_UNIT 64       /* knot spacing 1/64 in z */
#define U_MAX 1024              /* table covers |z| <= 16 */
#define N_KNOT (2 * U_MAX + 1)
#define HEADER_BYTES (2 * LANES)

typedef struct {
  int fmt;
  uint32_t N;       /* alphabet size: 65536 (bf16) or 256 (e4m3) */
  uint32_t T;       /* frequency total: 2^24 or 2^16 */
  uint32_t log2T;
  uint32_t MG;      /* counts given to the two Gaussian components */
  uint32_t Mp;      /* counts given to the empirical histogram */
  float K[N_KNOT];  /* K[j+U_MAX]: Gaussian-mixture CDF in counts at u = j */
  float D[N_KNOT];  /* K[j+1] - K[j]; 0 at the top knot */
  uint32_t *A;      /* N+1 entries: k + Qhat(k) */
} ref_model;

static float f32_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------ */
/* Symbols and value order.                                                 */
/* The symbols are the cache's own bit patterns (bf16, or FP8 e4m3 for the  */
/* native-FP8 cache, [SKV] "原生 FP8 KV 缓存").  Ranks put the patterns in   */
/* the order of the values they stand for: -NaN < -inf < ... < -0 < +0 <    */
/* ... < +inf < +NaN, so that a cumulative frequency over ranks is a CDF    */
/* over values.                                                             */
/* ------------------------------------------------------------------------ */
uint32_t skvref_rank(int fmt, uint32_t b) {
  if (fmt == REF_SYM_BF16) return b >= 0x8000u ? 0xFFFFu - b : b + 0x8000u;
  return b >= 0x80u ? 0xFFu - b : b + 0x80u;
}

uint32_t skvref_unrank(int fmt, uint32_t k) {
  if (fmt == REF_SYM_BF16) return k >= 0x8000u ? k - 0x8000u : 0xFFFFu - k;
  return k >= 0x80u ? k - 0x80u : 0xFFu - k;
}

/* exact value of an e4m3 code without its sign bit, c in [0, 0x7E] */
static double e4m3_magnitude(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp((double)(8u + m), (int)e - 10);
}

/* Value of symbol b as a double (NaN for NaN patterns). */
double skvref_value(int fmt, uint32_t b) {
  if (fmt == REF_SYM_BF16) return (double)f32_bits(b << 16);
  uint32_t c = b & 0x7Fu;
  if (c == 0x7Fu) return NAN;
  double v = e4m3_magnitude(c);
  return (b & 0x80u) ? -v : v;
}

/*
 * Bin of symbol b: the set of real values that round to it, [lo, hi].
 * The model integrates q over "each bf16 or FP8 bin" ([SKV] "原生 FP8 KV
 * 缓存": the FP8 symbols are coded under a bin-integrated Gaussian).  Reading:
 * the bin is the round-to-nearest-even preimage; for e4m3 the conversion
 * saturates (values beyond 448 round to +-448), so +-448's bins reach +-inf.
 * NaN patterns have empty bins at +-inf; -0 and +0 split the interval at 0.
 * Every finite edge is exact in fp32.
 */
void skvref_bin(int fmt, uint32_t b, float *lo, float *hi) {
  float a, c;  /* magnitude interval [a, c] */
  int neg;
  if (fmt == REF_SYM_BF16) {
    uint32_t m = b & 0x7FFFu;
    neg = (b >> 15) & 1;
    if (m == 0) {
      a = 0.0f;
      c = f32_bits(0x00008000u);                 /* half an ulp of the least subnormal */
    } else if (m < 0x7F80u) {
      a = f32_bits((m << 16) - 0x8000u);         /* value minus half an ulp */
      c = f32_bits((m << 16) + 0x8000u);         /* value plus half an ulp */
    } else if (m == 0x7F80u) {
      a = f32_bits(0x7F7F8000u);                 /* max finite + half an ulp rounds to inf */
      c = INFINITY;
    } else {
      a = INFINITY;
      c = INFINITY;
    }
  } else {
    uint32_t m = b & 0x7Fu;
    neg = (b >> 7) & 1;
    if (m == 0x7Fu) {
      a = INFINITY;
      c = INFINITY;
    } else {
      double va = m == 0 ? 0.0 : 0.5 * (e4m3_magnitude(m - 1) + e4m3_magnitude(m));
      double vc = m == 0x7Eu ? (double)INFINITY : 0.5 * (e4m3_magnitude(m) + e4m3_magnitude(m + 1));
      a = (float)va;
      c = (float)vc;
    }
  }
  if (!neg) { *lo = a; *hi = c; } else { *lo = -c; *hi = -a; }
}

/* ------------------------------------------------------------------------ */
/* Standardisation.  q's Gaussian parts are centred on the predictor mean   */
/* mu with the calibrated per-(kv, head, channel) sigma ([SKV] "q 应是什么样 */
/* 的", "早期结果").  The knot coordinate u = 64 z is formed as              */
/* u = RN(RN(e - mu') * s), s = RN(64 / max(sigma, 2^-100)); mu' is the     */
/* predictor mean in fp32, or 0 when it is not finite.                      */
/* ------------------------------------------------------------------------ */
float skvref_scale(float sigma) {
  float sp = sigma > 0x1p-100f ? sigma : 0x1p-100f;
  return (float)(64.0 / (double)sp);  /* fp64 quotient then fp32: one correct rounding (53 >= 2*24+2) */
}

static float mu_prime(float mu) { return isfinite(mu) ? mu : 0.0f; }

/* symbol i of a bf16 (u16) or e4m3 (u8) array */
static uint32_t sym_at_(int fmt, const void *x, int64_t i) {
  return fmt == REF_SYM_BF16 ? ((const uint16_t *)x)[i] : ((const uint8_t *)x)[i];
}

/*
 * sigma conditioned on the predictor's magnitude (SKV_SIGMA_OCTAVE).  The
 * pages name a static per-channel sigma as a cost, the residual's size
 * varying with position and prompt ([SKV] "下一步计划"); here sigma also
 * depends on |mu'|, a quantity both ends know.  Reading: the octave of a scalar
 * is j = clamp(E(mu') - E(sigma'_c) - 1, 0, 7), E the fp32 biased exponent
 * field (0 for zero and subnormals), sigma'_c = max(sigma_c, 2^-100) the
 * channel's own sigma; sigma is then looked up per (channel, octave).  Table
 * layout per channel: OCT_STRIDE floats, [0] = sigma_c, [1 + j] = sigma_c,j.
 */
#define OCTAVES 8
#define OCT_STRIDE (1 + OCTAVES)
#define OCT_MIN_COUNT 16

static uint32_t exp_field(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return (u >> 23) & 0xFFu;
}

static int octave_of(float mp, float sigma_c) {
  float sg = sigma_c > 0x1p-100f ? sigma_c : 0x1p-100f;
  int j = (int)exp_field(mp) - (int)exp_field(sg) - 1;
  return j < 0 ? 0 : (j > OCTAVES - 1 ? OCTAVES - 1 : j);
}

static float u_of(float e, float mu, float s) {
  float t = e - mu;
  return t * s;
}

/* ------------------------------------------------------------------------ */
/* The two Gaussian components.  q = 0.95 N(mu, s^2) + 0.03 N(mu, (3s)^2)   */
/* + 0.02 p_hat ([SKV] "早期结果"; the wide component is "3 sigma").  The   */
/* Gaussian pair's CDF, normalised to its own weight,                       */
/*   G(z) = (0.95 Phi(z) + 0.03 Phi(z/3)) / 0.98,                           */
/* is tabulated in counts at z = j/64, |j| <= 1024:                         */
/*   V_j = RN32(MG * G(j/64))  (0 <= j < 1024),  V_1024 = MG,               */
/*   K_j = V_j (j >= 0),  K_j = MG - V_{-j} (j < 0),  D_j = K_{j+1} - K_j.  */
/* Between knots G is the straight line through them, evaluated as           */
/*   c = clamp(u, -1024, 1024), i = floor(c), f = RN(c - i),                */
/*   y = fma(f, D_i, K_i),  Cg = floor(y).                                  */
/* All K_j lie on a grid fine enough that D_j is exact, so y meets K_{i+1}  */
/* at the segment's end: Cg is non-decreasing in u, Cg(-inf) = 0 and        */
/* Cg(+inf) = MG.                                                           */
/* ------------------------------------------------------------------------ */
static double phi_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static double mix_cdf(double z, double w_narrow, double w_wide) {
  return (w_narrow * phi_cdf(z) + w_wide * phi_cdf(z / 3.0)) / (w_narrow + w_wide);
}

static int build_knots(ref_model *m, double w_narrow, double w_wide) {
  float V[U_MAX + 1];
  for (int j = 0; j < U_MAX; j++) {
    double z = (double)j / KNOTS_PER_UNIT;
    V[j] = (float)((double)m->MG * mix_cdf(z, w_narrow, w_wide));
  }
  V[U_MAX] = (float)m->MG;
  for (int j = -U_MAX; j <= U_MAX; j++)
    m->K[j + U_MAX] = j >= 0 ? V[j] : (float)m->MG - V[-j];
  for (int j = 0; j < N_KNOT - 1; j++) {
    m->D[j] = m->K[j + 1] - m->K[j];
    /* the difference must be exact, else segment ends would not meet */
    if ((double)m->D[j] != (double)m->K[j + 1] - (double)m->K[j]) return REF_ERR_TABLE;
    if (m->D[j] < 0.0f) return REF_ERR_TABLE;
  }
  m->D[N_KNOT - 1] = 0.0f;
  return REF_OK;
}

uint32_t skvref_cg(const ref_model *m, float u) {
  float c = u;
  if (c < -(float)U_MAX) c = -(float)U_MAX;
  if (c > (float)U_MAX) c = (float)U_MAX;
  float fl = floorf(c);
  int i = (int)fl;
  float f = c - fl;
  float y = fmaf(f, m->D[i + U_MAX], m->K[i + U_MAX]);
  return (uint32_t)y;
}

/* ------------------------------------------------------------------------ */
/* The empirical component p_hat: "the empirical bf16 symbol distribution   */
/* measured on training data" ([SKV] "早期结果"), +1 smoothed.  Its integer */
/* CDF in rank order: H(0) = 0, H(k+1) = H(k) + hist[unrank(k)] + 1,        */
/* Qhat(k) = floor(Mp * H(k) / H(N)) (exact integers; domain Mp*H(N) <= 2^62). */
/* The table stored is A(k) = k + Qhat(k): the "+k" term is the floor of    */
/* one count per symbol that keeps every frequency >= 1.                    */
/* ------------------------------------------------------------------------ */
static int build_ptable(ref_model *m, const uint64_t *hist) {
  uint64_t Htot = 0;
  for (uint32_t k = 0; k < m->N; k++) {
    uint64_t h = hist ? hist[skvref_unrank(m->fmt, k)] : 0;
    /* H(N) is the exact integer sum: one that does not fit 64 bits is outside
       the domain (Htot + h + 1 <= 2^64 - 1 iff h < 2^64 - 1 - Htot) */
    if (h >= UINT64_MAX - Htot) return REF_ERR_TABLE;
    Htot += h + 1;
  }
  if (m->Mp != 0 && Htot > (1ull << 62) / m->Mp) return REF_ERR_TABLE;
  uint64_t H = 0;
  for (uint32_t k = 0; k < m->N; k++) {
    m->A[k] = k + (uint32_t)((uint64_t)m->Mp * H / Htot);
    H += (hist ? hist[skvref_unrank(m->fmt, k)] : 0) + 1;
  }
  m->A[m->N] = m->N + m->Mp;
  return REF_OK;
}

/* ---- model construction ---- */
/*
 * Integer budget (reading): every symbol gets one count (the "+k" floor),
 * the remaining T - N counts are split between the Gaussian pair and p_hat
 * in the mixture's proportion 0.98 : 0.02, MG = round(0.98 (T - N)).
 * T = 2^24 for bf16 and 2^16 for e4m3.  Tests may override the weights and
 * the budget split (MG + Mp must still equal T - N).
 */
ref_model *skvref_model_new(int fmt, const uint64_t *hist, double w_narrow, double w_wide,
                            int64_t MG, int64_t Mp, int *err) {
  *err = REF_ERR_ARG;
  if (fmt != REF_SYM_BF16 && fmt != REF_SYM_E4M3) return NULL;
  ref_model *m = (ref_model *)calloc(1, sizeof(ref_model));
  if (!m) return NULL;
  m->fmt = fmt;
  m->N = fmt == REF_SYM_BF16 ? 65536u : 256u;
  m->log2T = fmt == REF_SYM_BF16 ? 24u : 16u;
  m->T = 1u << m->log2T;
  uint32_t budget = m->T - m->N;
  if (MG < 0) MG = (int64_t)llround(0.98 * (double)budget);
  if (Mp < 0) Mp = (int64_t)budget - MG;
  if (MG + Mp != (int64_t)budget || (MG & 1)) { free(m); return NULL; }
  m->MG = (uint32_t)MG;
  m->Mp = (uint32_t)Mp;
  m->A = (uint32_t *)malloc(sizeof(uint32_t) * (m->N + 1));
  if (!m->A) { free(m); return NULL; }
  int e = build_knots(m, w_narrow, w_wide);
  if (e == REF_OK) e = build_ptable(m, hist);
  if (e != REF_OK) { free(m->A); free(m); *err = e; return NULL; }
  *err = REF_OK;
  return m;
}

ref_model *skvref_model_default(int fmt, const uint64_t *hist, int *err) {
  return skvref_model_new(fmt, hist, 0.95, 0.03, -1, -1, err);
}

void skvref_model_free(ref_model *m) {
  if (m) { free(m->A); free(m); }
}

void skvref_model_info(const ref_model *m, uint32_t *out5) {
  out5[0] = m->N; out5[1] = m->T; out5[2] = m->log2T; out5[3] = m->MG; out5[4] = m->Mp;
}

void skvref_model_knots(const ref_model *m, float *K, float *D) {
  memcpy(K, m->K, sizeof(m->K));
  memcpy(D, m->D, sizeof(m->D));
}

void skvref_model_ptable(const ref_model *m, uint32_t *A) {
  memcpy(A, m->A, sizeof(uint32_t) * (m->N + 1));
}

/*
 * Cumulative frequency at the lower and upper edge of symbol b:
 *   cum_lo = A(rank) + Cg(u(lo)),  cum_hi = A(rank+1) + Cg(u(hi)),
 * so freq = cum_hi - cum_lo >= 1 and the frequencies of all N symbols sum
 * to A(N) + MG = T.  This is q integrated over the bin, in integers.
 */
/* the same with the p_hat table A given (the adaptive tables below) */
static void cum_pair_with(const ref_model *m, const uint32_t *A, float mu, float s, uint32_t b,
                          uint32_t *clo, uint32_t *chi) {
  float lo, hi;
  float mp = mu_prime(mu);
  uint32_t k = skvref_rank(m->fmt, b);
  skvref_bin(m->fmt, b, &lo, &hi);
  *clo = A[k] + skvref_cg(m, u_of(lo, mp, s));
  *chi = A[k + 1] + skvref_cg(m, u_of(hi, mp, s));
}

void skvref_cum_pair(const ref_model *m, float mu, float s, uint32_t b, uint32_t *clo, uint32_t *chi) {
  cum_pair_with(m, m->A, mu, s, b, clo, chi);
}

/* cum(k) for k = 0..N: the lower edge of unrank(k); cum(N) = T. */
static uint32_t cum_rank_with(const ref_model *m, const uint32_t *A, float mp, float s, uint32_t k) {
  if (k >= m->N) return m->T;
  float lo, hi;
  skvref_bin(m->fmt, skvref_unrank(m->fmt, k), &lo, &hi);
  return A[k] + skvref_cg(m, u_of(lo, mp, s));
}

static uint32_t cum_rank(const ref_model *m, float mp, float s, uint32_t k) {
  return cum_rank_with(m, m->A, mp, s, k);
}

/* ------------------------------------------------------------------------ */
/* Adaptive p_hat (phat_mode REF_PHAT_ADAPTIVE; e4m3 symbols only).          */
/* The online entropy-estimation page ([ENT] "虚拟滑动窗口的设计原理") keeps */
/* exponentially decayed symbol counts, C_t(s) = alpha C_{t-1}(s) +         */
/* delta(s, s_t), and estimates P_t = C_t / sum C_t; it keeps one window per */
/* layer-head ("针对 KV 缓存的局部性优化"), rebuilds the CDF lazily every    */
/* N_update tokens rather than per symbol ("计算优化技巧"), and starts the   */
/* counters from a calibrated prior against cold start ("局限性与应对").     */
/* Reading, in integers, so that both ends build identical tables:          */
/*   - the window is one chunk: chunks decode independently, so every chunk */
/*     starts again from the prior;                                         */
/*   - epoch e of a chunk is its scalars i in [e E, (e+1) E), E =           */
/*     ADAPT_EPOCH, in memory order i = token * D + channel (32 tokens at   */
/*     head_dim 128), all 64 lanes together;                                */
/*   - epoch 0 codes with the static table A; epoch e >= 1 with A_e, the    */
/*     table of the p_hat construction above applied to counts C_e in rank  */
/*     order: H(0) = 0, H(k+1) = H(k) + C_e(k) + 1, A_e(k) = k +            */
/*     floor(Mp H(k) / H(N)), A_e(N) = N + Mp;                              */
/*   - C_0(k) = floor(ADAPT_PRIOR_WEIGHT (A(k+1) - A(k) - 1) / Mp), the     */
/*     static table's p_hat counts scaled to a total of about               */
/*     ADAPT_PRIOR_WEIGHT: the calibrated histogram as the prior, worth two */
/*     epochs of observations;                                              */
/*   - C_{e+1}(k) = floor(alpha C_e(k)) + (n_e(k) << ADAPT_OBS_SHIFT),      */
/*     alpha = 1 - 2^-ADAPT_DECAY_SHIFT, n_e(k) the number of epoch-e       */
/*     scalars of rank k: the decay is applied once per epoch, the epoch's  */
/*     observations weigh alike, and a count no longer observed decays to 0 */
/*     (the +1 of the table keeps its symbol's share above zero).           */
/* The mixture weights stay 0.95 / 0.03 / 0.02: only p_hat adapts.          */
/* ------------------------------------------------------------------------ */
#ifndef ADAPT_EPOCH
#define ADAPT_EPOCH 4096
#endif
#ifndef ADAPT_PRIOR_WEIGHT
#define ADAPT_PRIOR_WEIGHT 8192
#endif
#ifndef ADAPT_OBS_SHIFT
#define ADAPT_OBS_SHIFT 0
#endif
#ifndef ADAPT_DECAY_SHIFT
#define ADAPT_DECAY_SHIFT 2
#endif

static void adapt_prior(const ref_model *m, uint32_t *C) {
  for (uint32_t k = 0; k < m->N; k++)
    C[k] = m->Mp ? (uint32_t)((uint64_t)ADAPT_PRIOR_WEIGHT * (m->A[k + 1] - m->A[k] - 1u) / m->Mp) : 0u;
}

static void adapt_rebuild(const ref_model *m, const uint32_t *C, uint32_t *A) {
  uint64_t Htot = 0;
  for (uint32_t k = 0; k < m->N; k++) Htot += (uint64_t)C[k] + 1;
  uint64_t H = 0;
  for (uint32_t k = 0; k < m->N; k++) {
    A[k] = k + (uint32_t)((uint64_t)m->Mp * H / Htot);
    H += (uint64_t)C[k] + 1;
  }
  A[m->N] = m->N + m->Mp;
}

/* C <- floor(alpha C) + (n << ADAPT_OBS_SHIFT) */
static void adapt_step(const ref_model *m, uint32_t *C, const uint32_t *n) {
  const uint64_t a = (1u << ADAPT_DECAY_SHIFT) - 1u;
  for (uint32_t k = 0; k < m->N; k++)
    C[k] = (uint32_t)(((uint64_t)C[k] * a) >> ADAPT_DECAY_SHIFT) + (n[k] << ADAPT_OBS_SHIFT);
}

int64_t skvref_adapt_epoch(void) { return ADAPT_EPOCH; }

void skvref_adapt_params(int32_t *out4) {
  out4[0] = ADAPT_EPOCH; out4[1] = ADAPT_PRIOR_WEIGHT; out4[2] = ADAPT_OBS_SHIFT; out4[3] = ADAPT_DECAY_SHIFT;
}

/* Every epoch table of a chunk of nsc scalars with symbols x_c (encoder
   side: all symbols are known).  Returns n_ep tables of N + 1 entries. */
static uint32_t *adapt_tables(const ref_model *m, const ref_shape *sh, const void *x_c, int64_t nsc, int64_t *n_ep) {
  int64_t ne = (nsc + ADAPT_EPOCH - 1) / ADAPT_EPOCH;
  if (ne < 1) ne = 1;
  uint32_t *T = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(m->N + 1) * (size_t)ne);
  memcpy(T, m->A, sizeof(uint32_t) * (m->N + 1));
  uint32_t C[256], n[256];
  adapt_prior(m, C);
  for (int64_t e = 0; e + 1 < ne; e++) {
    memset(n, 0, sizeof(n));
    for (int64_t i = e * ADAPT_EPOCH; i < (e + 1) * ADAPT_EPOCH && i < nsc; i++)
      n[skvref_rank(m->fmt, sym_at_(sh->sym_fmt, x_c, i))]++;
    adapt_step(m, C, n);
    adapt_rebuild(m, C, T + (size_t)(e + 1) * (m->N + 1));
  }
  *n_ep = ne;
  return T;
}

/* The p_hat tables a chunk's epochs use, for the test suite: n_ep * (N + 1)
   entries written to out (at most cap tables); returns the epoch count. */
int64_t skvref_adapt_tables(const ref_model *m, const ref_shape *sh, const void *x_c, int64_t nsc,
                            uint32_t *out, int64_t cap) {
  int64_t ne;
  uint32_t *T = adapt_tables(m, sh, x_c, nsc, &ne);
  int64_t k = ne < cap ? ne : cap;
  memcpy(out, T, sizeof(uint32_t) * (size_t)(m->N + 1) * (size_t)k);
  free(T);
  return ne;
}

void skvref_cum_table(const ref_model *m, float mu, float sigma, uint32_t *cum) {
  float s = skvref_scale(sigma), mp = mu_prime(mu);
  for (uint32_t k = 0; k <= m->N; k++) cum[k] = cum_rank(m, mp, s, k);
}

/* ------------------------------------------------------------------------ */
/* Range coder ("an arithmetic coder turns (KV_full, mu, sigma) into bits   */
/* and (bits, mu, sigma) back", [SKV] "什么能预测 KV 缓存").  Reading: a    */
/* byte-renormalising range coder on a 48-bit window.                       */
/*   state: low (48 bits, carries propagate into bytes already emitted),    */
/*          range, initially 2^48 - 1.                                      */
/*   encode (c, f) with total 2^L: scale c, f by 2^(24-L) (so the coder     */
/*          always divides by 2^24); r = floor(range / 2^24);               */
/*          low += r*c; range = r*f;                                        */
/*          while range < 2^40: emit the top byte of low, shift low and     */
/*          range left by 8.                                                */
/*   finish: round low up to a multiple of 2^40 (carrying) and emit its top */
/*          byte: exactly one byte, so a substream of n renormalisations    */
/*          has n + 1 bytes.                                                */
/* ------------------------------------------------------------------------ */
#define W48 0xFFFFFFFFFFFFull
#define TOP40 (1ull << 40)

typedef struct {
  uint64_t low, range;
  uint8_t *out;
  size_t n, cap;
  int overflow;
} rc_enc;

static void rc_carry(rc_enc *e) {
  /* add one to the big-endian number formed by the bytes emitted so far */
  size_t i = e->n;
  while (i > 0) {
    i--;
    e->out[i] = (uint8_t)(e->out[i] + 1u);
    if (e->out[i] != 0) return;
  }
}

static void rc_emit(rc_enc *e, uint8_t byte) {
  if (e->n < e->cap) e->out[e->n] = byte; else e->overflow = 1;
  e->n++;
}

static void rc_enc_init(rc_enc *e, uint8_t *out, size_t cap) {
  e->low = 0; e->range = W48; e->out = out; e->n = 0; e->cap = cap; e->overflow = 0;
}

static void rc_encode(rc_enc *e, uint64_t c, uint64_t f) {
  uint64_t r = e->range >> 24;
  e->low += r * c;
  if (e->low >> 48) { rc_carry(e); e->low &= W48; }
  e->range = r * f;
  while (e->range < TOP40) {
    rc_emit(e, (uint8_t)(e->low >> 40));
    e->low = (e->low << 8) & W48;
    e->range <<= 8;
  }
}

static void rc_finish(rc_enc *e) {
  e->low = (e->low + (TOP40 - 1)) & ~(TOP40 - 1);
  if (e->low >> 48) { rc_carry(e); e->low &= W48; }
  rc_emit(e, (uint8_t)(e->low >> 40));
}

/* Decoder: d = code - low, kept below range.  Bytes past the substream end read as 0. */
typedef struct {
  uint64_t d, range;
  const uint8_t *in;
  size_t len, pos;
} rc_dec;

static uint8_t rc_byte(rc_dec *q) {
  uint8_t v = q->pos < q->len ? q->in[q->pos] : 0;
  q->pos++;
  return v;
}

static void rc_dec_init(rc_dec *q, const uint8_t *in, size_t len) {
  q->in = in; q->len = len; q->pos = 0; q->d = 0; q->range = W48;
  for (int i = 0; i < 6; i++) q->d = (q->d << 8) | rc_byte(q);
}

/* ------------------------------------------------------------------------ */
/* Chunks and lanes (reading of the stream layout).                         */
/*   x and mu are [layers][2 (K, V)][kv_heads][tokens][head_dim].           */
/*   A chunk is one (layer, kv, head) row's block of 256 tokens (the last   */
/*   block may be shorter); chunk id = row * ceil(tokens/256) + block.      */
/*   Inside a chunk the scalars are in memory order, i = t * D + d.         */
/*   Scalar i goes to lane i mod 64, and a lane codes its scalars in        */
/*   increasing i.  Each lane is one range-coded substream of len[l] >= 1   */
/*   bytes.                                                                 */
/*   Chunk bytes:                                                           */
/*     u16 len[64], little-endian;                                          */
/*     the interleaved words: with m = min over lanes of floor(len[l] / 4), */
/*       for w = 0 .. m-1, for l = 0 .. 63: bytes 4w .. 4w+3 of lane l;    */
/*     the tails: for l = 0 .. 63, bytes 4m .. len[l]-1 of lane l;          */
/*     zero bytes up to a multiple of 4.                                    */
/*   offsets[0] = 0, chunk c occupies [offsets[c], offsets[c+1]).           */
/* ------------------------------------------------------------------------ */
static int shape_ok(const ref_shape *sh) {
  if (!sh) return REF_ERR_ARG;
  if (sh->layers < 1 || sh->kv_heads < 1 || sh->tokens < 1 || sh->head_dim < 1) return REF_ERR_ARG;
  if (sh->sym_fmt != REF_SYM_BF16 && sh->sym_fmt != REF_SYM_E4M3) return REF_ERR_ARG;
  if (sh->mu_fmt != REF_MU_BF16 && sh->mu_fmt != REF_MU_F32) return REF_ERR_ARG;
  if (sh->sigma_mode != REF_SIGMA_CHANNEL && sh->sigma_mode != REF_SIGMA_OCTAVE) return REF_ERR_ARG;
  if (sh->phat_mode != REF_PHAT_STATIC && sh->phat_mode != REF_PHAT_ADAPTIVE) return REF_ERR_ARG;
  /* adaptive p_hat keeps a count per symbol in each chunk's window: e4m3 only */
  if (sh->phat_mode == REF_PHAT_ADAPTIVE && sh->sym_fmt != REF_SYM_E4M3) return REF_ERR_UNSUPPORTED;
  /* head_dim a power of two from 8 to 512 (a multiple of 8 dividing 512) */
  if (sh->head_dim % 8 != 0 || 512 % sh->head_dim != 0) return REF_ERR_UNSUPPORTED;
  return REF_OK;
}

int64_t skvref_num_chunks(const ref_shape *sh) {
  if (shape_ok(sh) != REF_OK) return -1;
  int64_t ntb = (sh->tokens + CHUNK_TOKENS - 1) / CHUNK_TOKENS;
  return sh->layers * 2 * sh->kv_heads * ntb;
}

/* worst case: 3 bytes per symbol (a frequency of 1 in 2^24), 1 flush byte per
   lane, 3 bytes of padding per chunk */
uint64_t skvref_encode_bound(const ref_shape *sh) {
  int64_t nc = skvref_num_chunks(sh);
  if (nc < 0) return 0;
  uint64_t nsc = (uint64_t)sh->layers * 2 * sh->kv_heads * sh->tokens * sh->head_dim;
  return (uint64_t)nc * (HEADER_BYTES + LANES + 3) + 3 * nsc;
}

static uint32_t sym_at(int fmt, const void *x, int64_t i) {
  if (fmt == REF_SYM_BF16) return ((const uint16_t *)x)[i];
  return ((const uint8_t *)x)[i];
}

static float mu_at(int fmt, const void *mu, int64_t i) {
  if (fmt == REF_MU_BF16) return f32_bits((uint32_t)((const uint16_t *)mu)[i] << 16);
  return ((const float *)mu)[i];
}

typedef struct {
  int64_t row, block, tok, nsc;
  int64_t base;  /* index of the chunk's first scalar in x / mu */
} chunk_geo;

static chunk_geo geometry(const ref_shape *sh, int64_t chunk) {
  chunk_geo g;
  int64_t ntb = (sh->tokens + CHUNK_TOKENS - 1) / CHUNK_TOKENS;
  g.row = chunk / ntb;
  g.block = chunk % ntb;
  g.tok = sh->tokens - g.block * CHUNK_TOKENS;
  if (g.tok > CHUNK_TOKENS) g.tok = CHUNK_TOKENS;
  g.nsc = g.tok * sh->head_dim;
  g.base = g.row * sh->tokens * sh->head_dim + g.block * CHUNK_TOKENS * sh->head_dim;
  return g;
}

/* m: the number of whole 4-byte words every lane has */
static uint64_t common_words(const uint64_t *lens) {
  uint64_t m = lens[0] / 4;
  for (int l = 1; l < LANES; l++)
    if (lens[l] / 4 < m) m = lens[l] / 4;
  return m;
}

/* chunk byte position of byte j of lane l's substream */
static uint64_t lane_byte_pos(const uint64_t *lens, uint64_t m, int l, uint64_t j) {
  if (j < 4 * m) return HEADER_BYTES + 4 * ((j / 4) * LANES + (uint64_t)l) + (j % 4);
  uint64_t p = HEADER_BYTES + 4 * m * LANES;
  for (int k = 0; k < l; k++) p += lens[k] - 4 * m;
  return p + (j - 4 * m);
}

/* sigma floats per channel in the caller's sigma array */
static int64_t sigma_stride(const ref_shape *sh) {
  return sh->sigma_mode == REF_SIGMA_OCTAVE ? OCT_STRIDE : 1;
}

/* Per-channel scales of a row: s[d * OCTAVES + j] (channel mode: the same s
   for every j) and the channel sigmas that fix the octave grid. */
typedef struct {
  float s[512 * OCTAVES];
  float sig[512];
  int octave;
} row_scales;

static void row_scales_init(row_scales *rs, const ref_shape *sh, const float *sigma_row) {
  int64_t D = sh->head_dim;
  rs->octave = sh->sigma_mode == REF_SIGMA_OCTAVE;
  for (int64_t d = 0; d < D; d++) {
    for (int j = 0; j < OCTAVES; j++)
      rs->s[d * OCTAVES + j] = skvref_scale(rs->octave ? sigma_row[d * OCT_STRIDE + 1 + j] : sigma_row[d]);
    rs->sig[d] = rs->octave ? sigma_row[d * OCT_STRIDE] : sigma_row[d];
  }
}

/* the scale of a scalar of channel d whose mean is mu (raw) */
static float scale_at(const row_scales *rs, int64_t d, float mu) {
  int j = rs->octave ? octave_of(mu_prime(mu), rs->sig[d]) : 0;
  return rs->s[d * OCTAVES + j];
}

/*
 * Encode one chunk.  x_c / mu_c point at the chunk's first scalar,
 * sigma_row at the row's sigmas (head_dim of them, or head_dim tables of
 * OCT_STRIDE in octave mode).  Writes at most cap bytes to out;
 * returns the chunk's byte size (which may exceed cap: then *status is
 * REF_ERR_CAPACITY and out holds a prefix).
 */
uint64_t skvref_encode_chunk(const ref_model *m, const ref_shape *sh, int64_t chunk,
                             const void *x_c, const void *mu_c, const float *sigma_row,
                             uint8_t *out, uint64_t cap, int *status) {
  chunk_geo g = geometry(sh, chunk);
  int64_t D = sh->head_dim;
  uint32_t up = 24u - m->log2T;  /* scale to the coder's 2^24 total */
  row_scales *rs = (row_scales *)malloc(sizeof(row_scales));
  row_scales_init(rs, sh, sigma_row);
  size_t lane_cap = (size_t)(3 * 4 * D + 8);
  uint8_t *lane_buf = (uint8_t *)malloc(lane_cap * LANES);
  uint64_t lens[LANES];
  int adaptive = sh->phat_mode == REF_PHAT_ADAPTIVE;
  int64_t n_ep = 1;
  uint32_t *tabs = adaptive ? adapt_tables(m, sh, x_c, g.nsc, &n_ep) : NULL;
  for (int lane = 0; lane < LANES; lane++) {
    rc_enc e;
    rc_enc_init(&e, lane_buf + lane_cap * lane, lane_cap);
    for (int64_t i = lane; i < g.nsc; i += LANES) {
      uint32_t b = sym_at(sh->sym_fmt, x_c, i);
      float mu = mu_at(sh->mu_fmt, mu_c, i);
      const uint32_t *A = adaptive ? tabs + (size_t)(i / ADAPT_EPOCH) * (m->N + 1) : m->A;
      uint32_t clo, chi;
      cum_pair_with(m, A, mu, scale_at(rs, i % D, mu), b, &clo, &chi);
      rc_encode(&e, (uint64_t)clo << up, (uint64_t)(chi - clo) << up);
    }
    rc_finish(&e);
    lens[lane] = e.n;
  }
  free(tabs);
  free(rs);
  uint64_t total = HEADER_BYTES;
  for (int l = 0; l < LANES; l++) total += lens[l];
  uint64_t size = (total + 3) & ~3ull;
  uint64_t mw = common_words(lens);
  *status = REF_OK;
  for (uint64_t p = 0; p < size && p < cap; p++) out[p] = 0;
  for (int l = 0; l < LANES; l++) {
    if (2u * (uint64_t)l + 1 < cap) {
      out[2 * l] = (uint8_t)(lens[l] & 0xFF);
      out[2 * l + 1] = (uint8_t)(lens[l] >> 8);
    }
    for (uint64_t j = 0; j < lens[l]; j++) {
      uint64_t p = lane_byte_pos(lens, mw, l, j);
      if (p < cap) out[p] = lane_buf[lane_cap * l + j];
    }
  }
  free(lane_buf);
  if (size > cap) *status = REF_ERR_CAPACITY;
  return size;
}

/*
 * Decode one chunk of nbytes bytes into x_out_c.  Returns REF_OK or
 * REF_ERR_CORRUPT (the output is then unspecified but every access stays in
 * bounds).  Detected corruption: a header whose lengths do not add up to the
 * chunk, a zero-length substream, a quotient t >= T, and a substream whose
 * decoder does not consume exactly its length (plus the 5 zero bytes that
 * follow the 6-byte priming window).
 */
int skvref_decode_chunk(const ref_model *m, const ref_shape *sh, int64_t chunk,
                        const uint8_t *bytes, uint64_t nbytes, const void *mu_c,
                        const float *sigma_row, void *x_out_c) {
  chunk_geo g = geometry(sh, chunk);
  int64_t D = sh->head_dim;
  uint32_t up = 24u - m->log2T;
  int st = REF_OK;
  if (nbytes < HEADER_BYTES) return REF_ERR_CORRUPT;
  row_scales *rs = (row_scales *)malloc(sizeof(row_scales));
  row_scales_init(rs, sh, sigma_row);
  uint64_t lens[LANES], total = HEADER_BYTES;
  for (int l = 0; l < LANES; l++) {
    lens[l] = (uint64_t)bytes[2 * l] | ((uint64_t)bytes[2 * l + 1] << 8);
    total += lens[l];
    if (lens[l] == 0) st = REF_ERR_CORRUPT;
  }
  if (((total + 3) & ~3ull) != nbytes) {
    st = REF_ERR_CORRUPT;
    for (int l = 0; l < LANES; l++) lens[l] = 0;  /* read nothing */
  }
  uint64_t mw = common_words(lens);
  /* every lane's substream, gathered from the chunk layout, and its decoder */
  uint8_t *lane = (uint8_t *)malloc((size_t)nbytes + 1);
  rc_dec q[LANES];
  uint64_t shifts[LANES];
  for (int l = 0, p = 0; l < LANES; p += (int)lens[l], l++) {
    for (uint64_t j = 0; j < lens[l]; j++) lane[p + j] = bytes[lane_byte_pos(lens, mw, l, j)];
    rc_dec_init(&q[l], lane + p, (size_t)lens[l]);
    shifts[l] = 0;
  }
  /* Epoch by epoch, every lane: an adaptive epoch table needs all lanes'
     symbols of the epochs before it.  With a static p_hat every epoch uses
     A, and the order is immaterial. */
  int adaptive = sh->phat_mode == REF_PHAT_ADAPTIVE;
  uint32_t *At = (uint32_t *)malloc(sizeof(uint32_t) * (m->N + 1));
  memcpy(At, m->A, sizeof(uint32_t) * (m->N + 1));
  uint32_t C[256], n[256];
  if (adaptive) adapt_prior(m, C);
  for (int64_t e0 = 0; e0 < g.nsc; e0 += ADAPT_EPOCH) {
    int64_t e1 = e0 + ADAPT_EPOCH < g.nsc ? e0 + ADAPT_EPOCH : g.nsc;
    memset(n, 0, sizeof(n));
    for (int l = 0; l < LANES; l++) {
      for (int64_t i = e0 + ((l - e0 % LANES) + LANES) % LANES; i < e1; i += LANES) {
        float mu = mu_at(sh->mu_fmt, mu_c, i);
        float mp = mu_prime(mu);
        float sc = scale_at(rs, i % D, mu);
        uint64_t r = q[l].range >> 24;
        uint64_t t = q[l].d / (r << up);
        if (t >= m->T) { st = REF_ERR_CORRUPT; t = m->T - 1; }
        /* the unique k with cum(k) <= t < cum(k+1), by bisection over ranks */
        uint32_t lo = 0, hi = m->N;
        while (hi - lo > 1) {
          uint32_t mid = (lo + hi) / 2;
          if (cum_rank_with(m, At, mp, sc, mid) <= t) lo = mid; else hi = mid;
        }
        uint32_t c = cum_rank_with(m, At, mp, sc, lo);
        uint32_t f = cum_rank_with(m, At, mp, sc, lo + 1) - c;
        q[l].d -= r * ((uint64_t)c << up);
        q[l].range = r * ((uint64_t)f << up);
        while (q[l].range < TOP40) {
          q[l].d = ((q[l].d << 8) | rc_byte(&q[l])) & W48;
          q[l].range <<= 8;
          shifts[l]++;
        }
        uint32_t b = skvref_unrank(m->fmt, lo);
        if (sh->sym_fmt == REF_SYM_BF16) ((uint16_t *)x_out_c)[i] = (uint16_t)b;
        else ((uint8_t *)x_out_c)[i] = (uint8_t)b;
        if (adaptive) n[lo]++;  /* adaptive mode is e4m3 only: lo < 256 */
      }
    }
    if (adaptive && e1 < g.nsc) {
      adapt_step(m, C, n);
      adapt_rebuild(m, C, At);
    }
  }
  for (int l = 0; l < LANES; l++)
    if (lens[l] == 0 || shifts[l] + 1 != lens[l]) st = REF_ERR_CORRUPT;
  free(At);
  free(lane);
  free(rs);
  return st;
}

/* ---- whole-cache encode / decode (chunk-parallel over host threads) ---- */
typedef struct {
  const ref_model *m;
  const ref_shape *sh;
  const void *x, *mu;
  const float *sigma;
  int64_t c0, c1;
  uint8_t *buf;       /* this worker's private output */
  uint64_t buf_cap;
  uint64_t *sizes;    /* per chunk */
  int status;
  /* decode */
  const uint8_t *bits;
  const uint64_t *offsets;
  void *x_out;
} work;

static size_t sym_bytes(const ref_shape *sh) { return sh->sym_fmt == REF_SYM_BF16 ? 2 : 1; }
static size_t mu_bytes(const ref_shape *sh) { return sh->mu_fmt == REF_MU_BF16 ? 2 : 4; }

static void *enc_worker(void *p) {
  work *w = (work *)p;
  uint64_t used = 0;
  w->status = REF_OK;
  for (int64_t c = w->c0; c < w->c1; c++) {
    chunk_geo g = geometry(w->sh, c);
    int st;
    uint64_t n = skvref_encode_chunk(w->m, w->sh, c,
                                     (const uint8_t *)w->x + g.base * sym_bytes(w->sh),
                                     (const uint8_t *)w->mu + g.base * mu_bytes(w->sh),
                                     w->sigma + g.row * w->sh->head_dim * sigma_stride(w->sh),
                                     w->buf + used, w->buf_cap - used, &st);
    if (st != REF_OK) { w->status = st; return NULL; }
    w->sizes[c] = n;
    used += n;
  }
  return NULL;
}

static void *dec_worker(void *p) {
  work *w = (work *)p;
  w->status = REF_OK;
  for (int64_t c = w->c0; c < w->c1; c++) {
    chunk_geo g = geometry(w->sh, c);
    uint64_t a = w->offsets[c], b = w->offsets[c + 1];
    int st = skvref_decode_chunk(w->m, w->sh, c, w->bits + a, b - a,
                                 (const uint8_t *)w->mu + g.base * mu_bytes(w->sh),
                                 w->sigma + g.row * w->sh->head_dim * sigma_stride(w->sh),
                                 (uint8_t *)w->x_out + g.base * sym_bytes(w->sh));
    if (st != REF_OK && w->status == REF_OK) w->status = st;
  }
  return NULL;
}

int skvref_encode_m(const ref_model *m, const ref_shape *sh, const void *x, const void *mu,
                    const float *sigma, uint8_t *bits, uint64_t cap, uint64_t *offsets, int nthreads) {
  int e = shape_ok(sh);
  if (e != REF_OK) return e;
  if (m->fmt != sh->sym_fmt) return REF_ERR_ARG;
  int64_t nc = skvref_num_chunks(sh);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nc) nthreads = (int)nc;
  work *ws = (work *)calloc((size_t)nthreads, sizeof(work));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  uint64_t *sizes = (uint64_t *)calloc((size_t)nc, sizeof(uint64_t));
  uint64_t per_chunk_max = HEADER_BYTES + LANES + 3 + 3ull * CHUNK_TOKENS * (uint64_t)sh->head_dim;
  int st = REF_OK;
  for (int t = 0; t < nthreads; t++) {
    work *w = &ws[t];
    w->m = m; w->sh = sh; w->x = x; w->mu = mu; w->sigma = sigma; w->sizes = sizes;
    w->c0 = nc * t / nthreads;
    w->c1 = nc * (t + 1) / nthreads;
    w->buf_cap = per_chunk_max * (uint64_t)(w->c1 - w->c0);
    w->buf = (uint8_t *)malloc((size_t)w->buf_cap);
    if (!w->buf) st = REF_ERR_ARG;
  }
  if (st == REF_OK) {
    for (int t = 0; t < nthreads; t++) pthread_create(&th[t], NULL, enc_worker, &ws[t]);
    for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; t++) if (ws[t].status != REF_OK) st = ws[t].status;
  }
  if (st == REF_OK) {
    offsets[0] = 0;
    for (int64_t c = 0; c < nc; c++) offsets[c + 1] = offsets[c] + sizes[c];
    if (offsets[nc] > cap) st = REF_ERR_CAPACITY;
    else
      for (int t = 0; t < nthreads; t++)
        memcpy(bits + offsets[ws[t].c0], ws[t].buf, (size_t)(offsets[ws[t].c1] - offsets[ws[t].c0]));
  }
  for (int t = 0; t < nthreads; t++) free(ws[t].buf);
  free(ws); free(th); free(sizes);
  return st;
}

int skvref_decode_m(const ref_model *m, const ref_shape *sh, const uint8_t *bits,
                    const uint64_t *offsets, const void *mu, const float *sigma, void *x_out,
                    int nthreads) {
  int e = shape_ok(sh);
  if (e != REF_OK) return e;
  if (m->fmt != sh->sym_fmt) return REF_ERR_ARG;
  int64_t nc = skvref_num_chunks(sh);
  for (int64_t c = 0; c < nc; c++)
    if (offsets[c + 1] < offsets[c]) return REF_ERR_CORRUPT;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nc) nthreads = (int)nc;
  work *ws = (work *)calloc((size_t)nthreads, sizeof(work));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; t++) {
    work *w = &ws[t];
    w->m = m; w->sh = sh; w->mu = mu; w->sigma = sigma; w->bits = bits; w->offsets = offsets;
    w->x_out = x_out;
    w->c0 = nc * t / nthreads;
    w->c1 = nc * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, dec_worker, w);
  }
  int st = REF_OK;
  for (int t = 0; t < nthreads; t++) {
    pthread_join(th[t], NULL);
    if (ws[t].status != REF_OK && st == REF_OK) st = ws[t].status;
  }
  free(ws); free(th);
  return st;
}

int skvref_encode(const ref_shape *sh, const void *x, const void *mu, const float *sigma,
                  const uint64_t *hist, uint8_t *bits, uint64_t cap, uint64_t *offsets, int nthreads) {
  int e = shape_ok(sh);
  if (e != REF_OK) return e;
  ref_model *m = skvref_model_default(sh->sym_fmt, hist, &e);
  if (!m) return e;
  e = skvref_encode_m(m, sh, x, mu, sigma, bits, cap, offsets, nthreads);
  skvref_model_free(m);
  return e;
}

int skvref_decode(const ref_shape *sh, const uint8_t *bits, const uint64_t *offsets,
                  const void *mu, const float *sigma, const uint64_t *hist, void *x_out, int nthreads) {
  int e = shape_ok(sh);
  if (e != REF_OK) return e;
  ref_model *m = skvref_model_default(sh->sym_fmt, hist, &e);
  if (!m) return e;
  e = skvref_decode_m(m, sh, bits, offsets, mu, sigma, x_out, nthreads);
  skvref_model_free(m);
  return e;
}

/* ------------------------------------------------------------------------ */
/* Calibration.  sigma^2 = E[(KV_full - mu)^2] is the optimum of the coding */
/* cost ([SKV] "q 应是什么样的"), measured per (kv, head, channel) on a     */
/* small calibration set and frozen ([SKV] "同一模型的优化版本", "早期结果"). */
/* Reading: per (layer, kv, head, channel) c, over finite symbol values v:  */
/*   S_c += RN64(r * r), r = RN64(v - mu'), in call order, then token order */
/*   n_c += 1;  sigma_c = RN32(sqrt(RN64(S_c / n_c))), 1.0 when n_c = 0.    */
/* p_hat's histogram counts every symbol pattern (NaNs included).           */
/* Octave mode also sums per (channel, E(mu')), E the fp32 exponent field,  */
/* into So / no (256 bins per channel), in the same order.                   */
/* ------------------------------------------------------------------------ */
#define EXP_BINS 256

typedef struct {
  const ref_shape *sh;
  const void *x, *mu;
  double *S;
  uint64_t *n;
  double *So;     /* octave mode: [channels][EXP_BINS], else NULL */
  uint64_t *no;
  int64_t r0, r1;
} cal_work;

static void *cal_worker(void *p) {
  cal_work *w = (cal_work *)p;
  const ref_shape *sh = w->sh;
  int64_t D = sh->head_dim, T = sh->tokens;
  for (int64_t row = w->r0; row < w->r1; row++) {
    for (int64_t d = 0; d < D; d++) {
      int64_t c = row * D + d;
      double S = w->S[c];
      uint64_t n = w->n[c];
      for (int64_t t = 0; t < T; t++) {
        int64_t i = (row * T + t) * D + d;
        double v = skvref_value(sh->sym_fmt, sym_at(sh->sym_fmt, w->x, i));
        if (!isfinite(v)) continue;
        float mp = mu_prime(mu_at(sh->mu_fmt, w->mu, i));
        double r = v - (double)mp;
        double rr = r * r;
        S = S + rr;
        n++;
        if (w->So) {
          int64_t k = c * EXP_BINS + exp_field(mp);
          w->So[k] = w->So[k] + rr;
          w->no[k]++;
        }
      }
      w->S[c] = S;
      w->n[c] = n;
    }
  }
  return NULL;
}

int skvref_calib_accumulate(const ref_shape *sh, const void *x, const void *mu, double *S,
                            uint64_t *n, double *So, uint64_t *no, uint64_t *hist, int nthreads) {
  int e = shape_ok(sh);
  if (e != REF_OK) return e;
  int64_t rows = sh->layers * 2 * sh->kv_heads;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > rows) nthreads = (int)rows;
  cal_work *ws = (cal_work *)calloc((size_t)nthreads, sizeof(cal_work));
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; t++) {
    ws[t].sh = sh; ws[t].x = x; ws[t].mu = mu; ws[t].S = S; ws[t].n = n;
    ws[t].So = sh->sigma_mode == REF_SIGMA_OCTAVE ? So : NULL;
    ws[t].no = no;
    ws[t].r0 = rows * t / nthreads;
    ws[t].r1 = rows * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, cal_worker, &ws[t]);
  }
  int64_t total = rows * sh->tokens * sh->head_dim;
  for (int64_t i = 0; i < total; i++) hist[sym_at(sh->sym_fmt, x, i)]++;
  for (int t = 0; t < nthreads; t++) pthread_join(th[t], NULL);
  free(ws); free(th);
  return REF_OK;
}

void skvref_calib_finalize(int64_t nch, const double *S, const uint64_t *n, float *sigma) {
  for (int64_t c = 0; c < nch; c++) {
    if (n[c] == 0) { sigma[c] = 1.0f; continue; }
    double q = S[c] / (double)n[c];
    sigma[c] = (float)sqrt(q);
  }
}

/* Octave mode: [0] = sigma_c as above; [1 + j] = the same estimator over the
   channel's scalars in octave j (their exponent bins summed in increasing
   exponent order), or sigma_c when fewer than OCT_MIN_COUNT fell there. */
void skvref_calib_finalize_octave(int64_t nch, const double *S, const uint64_t *n, const double *So,
                                  const uint64_t *no, float *table) {
  for (int64_t c = 0; c < nch; c++) {
    float sc = n[c] == 0 ? 1.0f : (float)sqrt(S[c] / (double)n[c]);
    float *t = table + c * OCT_STRIDE;
    t[0] = sc;
    double Sj[OCTAVES] = {0};
    uint64_t nj[OCTAVES] = {0};
    for (int e = 0; e < EXP_BINS; e++) {
      int j = e - (int)exp_field(sc > 0x1p-100f ? sc : 0x1p-100f) - 1;
      j = j < 0 ? 0 : (j > OCTAVES - 1 ? OCTAVES - 1 : j);
      Sj[j] = Sj[j] + So[c * EXP_BINS + e];
      nj[j] += no[c * EXP_BINS + e];
    }
    for (int j = 0; j < OCTAVES; j++)
      t[1 + j] = nj[j] < OCT_MIN_COUNT ? sc : (float)sqrt(Sj[j] / (double)nj[j]);
  }
}

/* ---- batch helpers for the test suite (plain loops over the functions above) ---- */
void skvref_cg_many(const ref_model *m, const float *u, uint32_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = skvref_cg(m, u[i]);
}

void skvref_cum_pair_many(const ref_model *m, const float *mu, const float *s, const uint32_t *b,
                          uint32_t *clo, uint32_t *chi, int64_t n) {
  for (int64_t i = 0; i < n; i++) skvref_cum_pair(m, mu[i], s[i], b[i], &clo[i], &chi[i]);
}

void skvref_bin_many(int fmt, const uint32_t *b, float *lo, float *hi, int64_t n) {
  for (int64_t i = 0; i < n; i++) skvref_bin(fmt, b[i], &lo[i], &hi[i]);
}

void skvref_scale_many(const float *sigma, float *s, int64_t n) {
  for (int64_t i = 0; i < n; i++) s[i] = skvref_scale(sigma[i]);
}

/* Code one substream of (c, f) pairs (totals already 2^24) with the range coder. */
uint64_t skvref_rc_encode_seq(const uint32_t *c, const uint32_t *f, int64_t n, uint8_t *out, uint64_t cap) {
  rc_enc e;
  rc_enc_init(&e, out, (size_t)cap);
  for (int64_t i = 0; i < n; i++) rc_encode(&e, c[i], f[i]);
  rc_finish(&e);
  return e.n;
}
