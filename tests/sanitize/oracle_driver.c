/* Drives every entry point of the CPU oracle (oracle/jas_oracle.c) on small
 * inputs held in exactly sized heap buffers -- padded rows, masks with
 * broadcast and per-query strides, the sink, the causal flag, key lengths
 * (0, inside, past the row, negative), several threads, grouped-query
 * attention -- so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees every access the oracle makes.  Exits 0
 * when every call returns 0 and the outputs pass basic checks (finite
 * probabilities summing with the sink to 1, equal results across thread
 * counts). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int jas_oracle_fwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t N, int64_t ld,
                   const void *scores, const float *mask, int64_t msb, int64_t msh, int64_t msq,
                   int causal, const int32_t *key_len, const float *sink, void *probs,
                   float *p_sink, float *lse, int threads);
int jas_oracle_bwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t N, int64_t ld,
                   const void *probs, const void *dprobs, int causal, const int32_t *key_len,
                   const float *p_sink, void *dscores, float *v, int threads);
int jas_oracle_dsink(int64_t B, int64_t H, int64_t Sq, const float *v, float *d_sink);
int jas_oracle_attn_fwd(int dtype, int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t N,
                        int64_t D, const void *q, const void *k, const void *v, float scale,
                        const float *mask, int64_t msb, int64_t msh, int64_t msq, int causal,
                        const int32_t *key_len, const float *sink, void *out, float *lse,
                        float *p_sink, void *probs, float *scores, int threads);

static uint64_t rng = 88172645463325252ull;
static float urand(void) {  /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (float)((rng >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
}
static uint16_t to_bf16(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)(u >> 16); }
static float from_bits(const void *p, int dtype, int64_t i) {
  if (dtype == 0) return ((const float *)p)[i];
  uint16_t h = ((const uint16_t *)p)[i];
  if (dtype == 1) { uint32_t u = (uint32_t)h << 16; float f; memcpy(&f, &u, 4); return f; }
  /* binary16 */
  int e = (h >> 10) & 31, m = h & 1023; float f;
  if (e == 0) f = ldexpf((float)m, -24); else if (e == 31) f = m ? NAN : INFINITY;
  else f = ldexpf((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -f : f;
}
static void *fill(int dtype, int64_t n, float scale) {
  size_t es = dtype == 0 ? 4 : 2;
  void *p = malloc((size_t)n * es);
  for (int64_t i = 0; i < n; ++i) {
    float x = urand() * scale;
    if (dtype == 0) ((float *)p)[i] = x;
    else ((uint16_t *)p)[i] = to_bf16(x);
  }
  /* binary16: clear the top exponent bit, so every word is a finite value
     below 1 in magnitude */
  if (dtype == 2) for (int64_t i = 0; i < n; ++i) ((uint16_t *)p)[i] &= 0xbbff;
  return p;
}

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); ++fails; } } while (0)

static void softmax_case(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t N, int64_t pad,
                         int with_mask, int per_query_mask, int with_sink, int causal,
                         const int32_t *key_len) {
  const int64_t ld = N + pad, rows = B * H * Sq, span = (rows - 1) * ld + N;
  void *s = fill(dtype, span, 4.0f), *g = fill(dtype, span, 1.0f);
  const size_t es = dtype == 0 ? 4 : 2;
  void *P = calloc((size_t)span, es), *P1 = calloc((size_t)span, es), *dS = calloc((size_t)span, es);
  int64_t msb = 0, msh = 0, msq = 0, mlen = 0;
  float *mask = NULL;
  if (with_mask) {
    if (per_query_mask) { msq = N + 1; msh = Sq * msq; msb = H * msh; mlen = (B - 1) * msb + (H - 1) * msh + (Sq - 1) * msq + N; }
    else { msb = N; mlen = (B - 1) * msb + N; }
    mask = malloc((size_t)mlen * 4);
    for (int64_t i = 0; i < mlen; ++i) mask[i] = (i % 11 == 3) ? -INFINITY : urand();
  }
  float *sink = NULL, *ps = NULL, *ps1 = NULL, *lse = malloc((size_t)rows * 4), *v = NULL;
  if (with_sink) {
    sink = malloc((size_t)H * 4); for (int64_t h = 0; h < H; ++h) sink[h] = urand();
    ps = malloc((size_t)rows * 4); ps1 = malloc((size_t)rows * 4); v = malloc((size_t)rows * 4);
  }
  int r = jas_oracle_fwd(dtype, B, H, Sq, N, ld, s, mask, msb, msh, msq, causal, key_len, sink, P, ps, lse, 1);
  CHECK(r == 0, "fwd returned %d", r);
  r = jas_oracle_fwd(dtype, B, H, Sq, N, ld, s, mask, msb, msh, msq, causal, key_len, sink, P1, ps1, NULL, 3);
  CHECK(r == 0, "fwd (3 threads) returned %d", r);
  for (int64_t row = 0; row < rows; ++row) {
    double sum = ps ? ps[row] : 0.0;
    for (int64_t j = 0; j < N; ++j) {
      float p = from_bits(P, dtype, row * ld + j);
      CHECK(isfinite(p) && p >= 0.0f, "P not a probability at row %lld key %lld", (long long)row, (long long)j);
      sum += p;
    }
    CHECK(sum == 0.0 || fabs(sum - 1.0) < 0.02 * (1 + N / 256), "row %lld sums to %g", (long long)row, sum);
  }
  CHECK(memcmp(P, P1, (size_t)span * es) == 0, "thread count changed P");
  r = jas_oracle_bwd(dtype, B, H, Sq, N, ld, P, g, causal, key_len, ps, dS, v, 2);
  CHECK(r == 0, "bwd returned %d", r);
  if (with_sink) {
    float *ds = malloc((size_t)H * 4);
    r = jas_oracle_dsink(B, H, Sq, v, ds);
    CHECK(r == 0, "dsink returned %d", r);
    free(ds);
  }
  free(s); free(g); free(P); free(P1); free(dS); free(mask); free(sink); free(ps); free(ps1); free(lse); free(v);
}

static void attn_case(int dtype, int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t N, int64_t D,
                      int with_mask, int with_sink, int causal, const int32_t *key_len) {
  void *q = fill(dtype, B * H * Sq * D, 1.0f), *k = fill(dtype, B * Hkv * N * D, 1.0f),
       *v = fill(dtype, B * Hkv * N * D, 1.0f);
  const int64_t rows = B * H * Sq;
  void *out = malloc((size_t)(rows * D) * 2), *probs = malloc((size_t)(rows * N) * 2);
  float *scores = malloc((size_t)(rows * N) * 4), *lse = malloc((size_t)rows * 4);
  float *mask = NULL, *sink = NULL, *ps = NULL;
  int64_t msq = 0;
  if (with_mask) {
    msq = N + 3;
    const int64_t mlen = (Sq - 1) * msq + N;
    mask = malloc((size_t)mlen * 4);
    for (int64_t i = 0; i < mlen; ++i) mask[i] = (i % 13 == 5) ? -INFINITY : urand();
  }
  if (with_sink) {
    sink = malloc((size_t)H * 4); for (int64_t h = 0; h < H; ++h) sink[h] = urand();
    ps = malloc((size_t)rows * 4);
  }
  int r = jas_oracle_attn_fwd(dtype, B, H, Hkv, Sq, N, D, q, k, v, 0.125f, mask, 0, 0, msq, causal,
                              key_len, sink, out, lse, ps, probs, scores, 2);
  CHECK(r == 0, "attn_fwd returned %d", r);
  for (int64_t i = 0; i < rows * D; ++i)
    CHECK(isfinite(from_bits(out, dtype, i)), "attention output not finite at %lld", (long long)i);
  free(q); free(k); free(v); free(out); free(probs); free(scores); free(lse); free(mask); free(sink); free(ps);
}

int main(void) {
  const int32_t kl3[3] = {300, 0, 517}, kl2[2] = {-4, 129};
  for (int dt = 0; dt < 3; ++dt) {
    softmax_case(dt, 2, 3, 5, 257, 0, 0, 0, 0, 0, NULL);
    softmax_case(dt, 2, 3, 5, 257, 7, 1, 0, 1, 0, NULL);
    softmax_case(dt, 3, 2, 9, 300, 4, 1, 1, 1, 1, kl3);
    softmax_case(dt, 2, 1, 40, 33, 1, 0, 0, 1, 1, kl2);
    softmax_case(dt, 1, 2, 3, 1, 0, 1, 0, 1, 0, NULL);
  }
  for (int dt = 1; dt < 3; ++dt) {
    attn_case(dt, 2, 4, 2, 9, 300, 64, 1, 1, 1, kl2);
    attn_case(dt, 1, 2, 1, 5, 1, 16, 0, 1, 0, NULL);
    attn_case(dt, 3, 3, 3, 4, 257, 32, 1, 0, 0, kl3);
  }
  if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
  printf("oracle driver: ok\n");
  return 0;
}
