/*
 * oracle_driver.c -- drives the CPU oracle (oracle/skvref.c) through round
 * trips and corrupted streams.  tests/test_oracle_sanitized.py builds the two
 * files together with AddressSanitizer and UndefinedBehaviorSanitizer, so any
 * out-of-bounds access, use after free, leak or undefined arithmetic in the
 * oracle's encoder, decoder or model build ends the run with an error.
 *
 * Cases: bf16 and e4m3 symbols, bf16 and fp32 means (NaN and infinite means
 * included), channel and octave sigma (zero, tiny and huge sigmas), static and
 * adaptive p_hat, head_dim 8 .. 512, ragged token counts; then every chunk's
 * bytes corrupted (random byte flips in payload and header, lengths set to
 * their maximum, a chunk cut short) and decoded chunk by chunk, and offsets
 * that run backwards.  The decoder must stay in bounds and report corruption
 * or decode something; the round trips must be exact.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t layers, kv_heads, tokens, head_dim;
  int32_t sym_fmt, mu_fmt, sigma_mode, phat_mode;
} ref_shape;
typedef struct ref_model ref_model;

ref_model *skvref_model_default(int fmt, const uint64_t *hist, int *err);
void skvref_model_free(ref_model *m);
int64_t skvref_num_chunks(const ref_shape *sh);
uint64_t skvref_encode_bound(const ref_shape *sh);
int skvref_encode_m(const ref_model *m, const ref_shape *sh, const void *x, const void *mu, const float *sigma,
                    uint8_t *bits, uint64_t cap, uint64_t *offsets, int nthreads);
int skvref_decode_m(const ref_model *m, const ref_shape *sh, const uint8_t *bits, const uint64_t *offsets,
                    const void *mu, const float *sigma, void *x_out, int nthreads);
int skvref_decode_chunk(const ref_model *m, const ref_shape *sh, int64_t chunk, const uint8_t *bytes,
                        uint64_t nbytes, const void *mu_c, const float *sigma_row, void *x_out_c);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {  /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double unif(void) { return (double)(rnd() >> 11) * 0x1p-53; }

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); fails++; } } while (0)

static void run_case(int sym, int mu_fmt, int sigma_mode, int phat, int64_t tokens, int64_t D) {
  ref_shape sh = {1, 2, tokens, D, sym, mu_fmt, sigma_mode, phat};
  int64_t n = 2 * 2 * tokens * D, nch = 2 * 2 * D, nc = skvref_num_chunks(&sh);
  size_t sb = sym == 0 ? 2 : 1, mb = mu_fmt == 0 ? 2 : 4, per = sigma_mode ? 9 : 1;
  uint32_t N = sym == 0 ? 65536u : 256u;
  uint8_t *x = malloc(n * sb), *mu = malloc(n * mb), *out = malloc(n * sb);
  float *sigma = malloc(sizeof(float) * nch * per);
  uint64_t *hist = malloc(sizeof(uint64_t) * N);
  for (uint32_t k = 0; k < N; k++) hist[k] = rnd() % 1000;
  for (int64_t c = 0; c < nch * (int64_t)per; c++) {
    double u = unif();
    sigma[c] = u < 0.1 ? 0.0f : (u < 0.15 ? 1e-38f : (u < 0.2 ? 1e30f : (float)(0.05 * (0.2 + unif()))));
  }
  for (int64_t i = 0; i < n; i++) {
    float v = (float)((unif() - 0.5) * 8.0);
    uint32_t fb;
    memcpy(&fb, &v, 4);
    if (sym == 0) {
      uint16_t b = (uint16_t)(fb >> 16);
      if (rnd() % 97 == 0) b = (uint16_t)rnd();  /* any pattern, NaN and inf included */
      memcpy(x + 2 * i, &b, 2);
    } else {
      x[i] = (uint8_t)(rnd() % 97 == 0 ? rnd() : (rnd() % 64) + (rnd() % 2) * 128);
    }
    float m = v + (float)((unif() - 0.5) * 0.1);
    if (rnd() % 101 == 0) { uint32_t nanb = 0x7FC00000u; memcpy(&m, &nanb, 4); }
    if (rnd() % 103 == 0) { uint32_t infb = 0xFF800000u; memcpy(&m, &infb, 4); }
    uint32_t mbits;
    memcpy(&mbits, &m, 4);
    if (mu_fmt == 0) { uint16_t h = (uint16_t)(mbits >> 16); memcpy(mu + 2 * i, &h, 2); }
    else memcpy(mu + 4 * i, &m, 4);
  }
  int err;
  ref_model *model = skvref_model_default(sym, hist, &err);
  CHECK(model, "model failed %d", err);
  uint64_t cap = skvref_encode_bound(&sh);
  uint8_t *bits = malloc(cap);
  uint64_t *offs = malloc(sizeof(uint64_t) * (nc + 1));
  int st = skvref_encode_m(model, &sh, x, mu, sigma, bits, cap, offs, 2);
  CHECK(st == 0, "encode %d", st);
  st = skvref_decode_m(model, &sh, bits, offs, mu, sigma, out, 2);
  CHECK(st == 0 && memcmp(out, x, n * sb) == 0, "round trip sym %d mu %d sigma %d phat %d tok %lld D %lld: %d", sym,
        mu_fmt, sigma_mode, phat, (long long)tokens, (long long)D, st);
  /* corrupted chunks, each decoded on its own */
  int64_t ntb = (tokens + 255) / 256;
  for (int64_t c = 0; c < nc; c++) {
    int64_t row = c / ntb, blk = c % ntb;
    int64_t base = (row * tokens + blk * 256) * D;
    uint64_t a = offs[c], len = offs[c + 1] - offs[c];
    for (int trial = 0; trial < 6; trial++) {
      uint64_t clen = len;
      uint8_t *cb = malloc(len + 1);
      memcpy(cb, bits + a, len);
      if (trial < 3) {
        for (int f = 0; f < 16; f++) cb[rnd() % len] ^= (uint8_t)(1 + rnd() % 255);
      } else if (trial == 3) {
        for (int l = 0; l < 64; l++) { cb[2 * l] = 0xFF; cb[2 * l + 1] = 0xFF; }
      } else if (trial == 4) {
        clen = len > 130 ? 130 + rnd() % (len - 130) : len;  /* cut short */
      } else {
        for (uint64_t p = 128; p < len; p++) cb[p] = (uint8_t)rnd();  /* payload replaced, header kept */
      }
      skvref_decode_chunk(model, &sh, c, cb, clen, mu + base * mb, sigma + row * D * per, out + base * sb);
      free(cb);
    }
  }
  if (nc > 1) {  /* offsets that run backwards */
    uint64_t keep = offs[1];
    offs[1] = offs[2] + 1;
    st = skvref_decode_m(model, &sh, bits, offs, mu, sigma, out, 2);
    CHECK(st == 5, "backward offsets not flagged: %d", st);
    offs[1] = keep;
  }
  skvref_model_free(model);
  free(x); free(mu); free(out); free(sigma); free(hist); free(bits); free(offs);
}

int main(void) {
  static const int64_t dims[][2] = {{1, 64}, {3, 128}, {300, 64}, {257, 8}, {40, 512}, {33, 128}, {65, 64}};
  int ncase = 0;
  for (int sym = 0; sym < 2; sym++)
    for (int mu_fmt = 0; mu_fmt < 2; mu_fmt++)
      for (int sm = 0; sm < 2; sm++)
        for (int ph = 0; ph <= sym; ph++)
          for (size_t d = 0; d < sizeof(dims) / sizeof(dims[0]); d++) {
            run_case(sym, mu_fmt, sm, ph, dims[d][0], dims[d][1]);
            ncase++;
          }
  printf("oracle driver: %d cases, %d failures\n", ncase, fails);
  return fails ? 1 : 0;
}
