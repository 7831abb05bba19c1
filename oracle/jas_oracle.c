/*
 * jas_oracle.c -- CPU oracle for the fixed-order, batch-invariant row softmax
 * and its backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP kernels are checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * constant with the HIP library, and the HIP library never calls it.
 *
 * Sources (the web pages this implementation is written from):
 *   [P1] RL-Kernel PR #453, "[WS1][kernels] Add fixed-order joint-attention
 *        softmax for Qwen-Image", section Summary: "Fixed-order online
 *        softmax" and "Fixed-order backward".
 *   [P2] ROCm TransformerEngine PR #678, "Add softmax sink (learnable
 *        off-by-one) support for the ROCm/CK fused attention backend",
 *        title and Description (sink added to the denominator, one value per
 *        head, d_sink per head).
 *   [P3] RL-Kernel PR #240, "Batch-invariant attention (standard softmax --
 *        cuda version)", sections "Fixed Reduction Contract / Softmax and
 *        LSE" (power-of-two tree whose shape depends on nothing but the tile;
 *        the row's log-sum-exp as a second output) and "Path Status" (fully
 *        masked rows; FP16 and BF16 dtypes).
 *
 * Arithmetic model.  Every floating-point operation below is one IEEE-754
 * binary32 operation rounded to nearest-even: the file is compiled with
 * -ffp-contract=off and without fast-math (no FMA, no reassociation), on
 * x86-64 where float arithmetic uses SSE, with the MXCSR forced to
 * round-to-nearest and no flush-to-zero / denormals-are-zero.
 *
 * The per-row routines are written in the order the pages give the steps:
 *   forward  : split the keys into 256-key tiles, left to right; per tile a
 *              fixed tree for the max and for the sum of exponentials; merge
 *              the tile states in tile order; optional sink merged last;
 *              one conversion to the output dtype at the write.
 *   backward : delta = fixed-order sum of P*dP over the same tiles, then
 *              dS = P*(dP - delta); one conversion at the write.
 *   d_sink   : per head, a fixed-order sum of -p_sink*delta over that head's
 *              rows (no atomics).
 */
#if !defined(_DEFAULT_SOURCE)
#define _DEFAULT_SOURCE
#endif
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#if defined(__x86_64__)
#include <xmmintrin.h>
#endif

#if defined(__FAST_MATH__) || (defined(__FINITE_MATH_ONLY__) && __FINITE_MATH_ONLY__)
#error "the oracle must be compiled without fast-math"
#endif

#define TILE 256          /* [P1] Benchmark: TILE_K = 256, fixed, never tuned */

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

static size_t elem_size(int dt) { return dt == DT_F32 ? 4 : 2; }

/* ------------------------------------------------------------------------ */
/* Floating-point environment                                               */
/* ------------------------------------------------------------------------ */

/* Round to nearest-even, keep subnormals (no FTZ, no DAZ).  Called in every
   thread that runs oracle arithmetic. */
static void ieee_env(void) {
#if defined(__x86_64__)
  unsigned csr = _mm_getcsr();
  csr &= ~(0x8000u | 0x0040u | 0x6000u); /* FTZ, DAZ, rounding-control bits */
  _mm_setcsr(csr);
#endif
}

/* ------------------------------------------------------------------------ */
/* Element conversions                                                      */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Narrow binary32 -> bf16, round to nearest, ties to even ([P1]: one dtype
   conversion at the final write).  bf16 keeps the binary32 sign and exponent
   and the top 7 fraction bits, so the two bf16 neighbours of a finite x are
   its truncation `lo` and the next value away from zero `lo + 1` (the carry
   into the exponent field is the correct next value, up to infinity).  The
   16 dropped bits say which neighbour is nearer; exactly half-way picks the
   one whose last kept bit is 0.  NaN stays NaN (quiet, sign kept). */
static uint16_t f32_to_bf16(float x) {
  uint32_t u = bits_from_f32(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lo = u >> 16;          /* truncation toward zero */
  uint32_t rest = u & 0xffffu;    /* dropped bits */
  if (rest > 0x8000u || (rest == 0x8000u && (lo & 1u)))
    lo += 1u;                     /* nearer to (or tie with odd) the next value */
  return (uint16_t)lo;
}

/* IEEE binary16 -> binary32, exact.  Fields: sign, 5 exponent bits (bias
   15), 10 fraction bits.  Exponent 0 holds zero and the subnormals
   (fraction * 2^-24), exponent 31 infinity and NaN. */
static float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t ex = (h >> 10) & 0x1fu;
  uint32_t fr = h & 0x3ffu;
  if (ex == 0x1fu) return f32_from_bits(sign | 0x7f800000u | (fr << 13));
  if (ex == 0) {
    float v = (float)fr * 0x1p-24f;  /* exact: fr < 2^10 */
    return sign ? -v : v;
  }
  return f32_from_bits(sign | ((ex + 112u) << 23) | (fr << 13));
}

/* Narrow binary32 -> binary16, round to nearest, ties to even ([P3] lists
   FP16 beside BF16; one conversion at the final write).  A finite x is
   first written as an integer count of its binary16 unit: 2^(e-25) for the
   normal range (e = x's unbiased exponent + 15), 2^-24 below it; the bits
   below that unit are the rounding remainder.  Rounding up can carry into
   the exponent field, which is the correct next value; magnitudes from
   65520 (half-way past the largest finite 65504, a tie that goes to the
   even neighbour, infinity) round to infinity.  NaN stays NaN (quiet, sign
   kept). */
static uint16_t f32_to_f16(float x) {
  uint32_t u = bits_from_f32(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu));
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);   /* >= 65520: infinity */
  uint32_t e = a >> 23;                  /* biased binary32 exponent */
  uint32_t mant = (a & 0x7fffffu) | (e ? 0x800000u : 0u);
  uint32_t shift, q, rest, half;
  if (e >= 113) {                        /* binary16 normal range: >= 2^-14 */
    shift = 13;
    q = (((e - 112u) << 10) | ((a >> 13) & 0x3ffu));
    rest = a & 0x1fffu;
  } else {                               /* subnormal or zero: unit 2^-24 */
    shift = 126u - e;                    /* x = mant * 2^(e-150) = (mant >> shift) units */
    if (e == 0 || shift > 24) return sign;   /* below 2^-25: rounds to zero */
    q = mant >> shift;
    rest = mant & ((1u << shift) - 1u);
  }
  half = 1u << (shift - 1);
  if (rest > half || (rest == half && (q & 1u))) q += 1u;
  return (uint16_t)(sign | q);
}

static float load_elem(int dt, const void *base, int64_t idx) {
  if (dt == DT_BF16) return bf16_to_f32(((const uint16_t *)base)[idx]);
  if (dt == DT_F16) return f16_to_f32(((const uint16_t *)base)[idx]);
  return ((const float *)base)[idx];
}

static void store_elem(int dt, void *base, int64_t idx, float v) {
  if (dt == DT_BF16) ((uint16_t *)base)[idx] = f32_to_bf16(v);
  else if (dt == DT_F16) ((uint16_t *)base)[idx] = f32_to_f16(v);
  else ((float *)base)[idx] = v;
}

/* ------------------------------------------------------------------------ */
/* The exponential                                                          */
/* ------------------------------------------------------------------------ */

/* The binary32 nearest to log2(e); 1/ln(2) in double is within 2^-53
   relative of log2(e), far from a binary32 rounding boundary. */
static float log2e_f32(void) { return (float)(1.0 / log(2.0)); }

/* exp_(y) for y <= 0 or -inf.  [P1] says every backend shares one
   exponential approximation without naming it; the reading taken here is
   exp(y) = 2^(y*log2 e), with the product rounded to binary32 and 2^u
   rounded to the nearest binary32 (exp2 evaluated in double, then rounded).
   Results below 2^-126 are flushed to +0 so that no subnormal e enters the
   sums; -inf gives +0. */
static float exp_(float y) {
  if (y == -INFINITY) return 0.0f;
  float u = y * log2e_f32();
  if (u < -126.0f) return 0.0f;
  return (float)exp2((double)u);
}

/* ------------------------------------------------------------------------ */
/* Fixed reduction trees over one 256-key tile                              */
/* ------------------------------------------------------------------------ */

/* Balanced pairwise tree over the 256 positions of a tile, in key order:
   level 0 adds keys (0,1), (2,3), ...; level 1 adds those pair sums two by
   two; and so on, 8 levels.  The tree is defined by key position alone
   ([P1] fixed reduction tree per tile; [P3] power-of-two tree that does not
   depend on batch, length or launch).  `v` is overwritten. */
static float tree_sum256(float *v) {
  for (int width = TILE; width > 1; width /= 2)
    for (int i = 0; i < width / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

static float max2(float a, float b) { return (a >= b) ? a : b; }

/* Same tree shape with max; max is exact, so any shape gives the same value
   up to the sign of a zero. */
static float tree_max256(float *v) {
  for (int width = TILE; width > 1; width /= 2)
    for (int i = 0; i < width / 2; ++i) v[i] = max2(v[2 * i], v[2 * i + 1]);
  return v[0];
}

/* ------------------------------------------------------------------------ */
/* Online-softmax state merge                                               */
/* ------------------------------------------------------------------------ */

/* Merge the running state (M, L) with a tile state (m, l): rescale both to
   the larger max and add, each product and the sum rounded once.  A -inf
   max contributes nothing ([P1] online softmax states merged in a fixed
   order; [P3] fully masked rows are handled). */
static void merge(float *M, float *L, float m, float l) {
  float Mn = max2(*M, m);
  if (Mn == -INFINITY) { *M = -INFINITY; *L = 0.0f; return; }
  float a = (*M == -INFINITY) ? 0.0f : exp_(*M - Mn);
  float b = (m == -INFINITY) ? 0.0f : exp_(m - Mn);
  float La = *L * a;
  float lb = l * b;
  *M = Mn;
  *L = La + lb;
}

/* ------------------------------------------------------------------------ */
/* Forward, one row                                                         */
/* ------------------------------------------------------------------------ */

/* One row of N keys.  `s` is the row of scores (dtype dt), `a` the additive
   mask row (binary32, may be NULL), `sigma` the head's sink logit when
   has_sink.  Keys at or past `kend` are excluded (causal or key-length
   exclusion): they count as a score of -inf and are not read.  Writes the
   row of probabilities, with a sink the sink's own probability, and when
   `lse` is given the row's log-sum-exp.  Scratch buffers are supplied by
   the caller. */
static void fwd_row(int dt, int64_t N, int64_t kend, const void *s, const float *a,
                    int has_sink, float sigma, void *P, float *p_sink, float *lse,
                    float *x, float *e, float *m, float *l) {
  const int64_t T = (N + TILE - 1) / TILE;
  float buf[TILE];

  /* scores to binary32 (exact), then the additive mask, one rounding */
  for (int64_t j = 0; j < N; ++j) {
    if (j >= kend) {
      x[j] = -INFINITY;
      continue;
    }
    x[j] = load_elem(dt, s, j);
    if (a) x[j] = x[j] + a[j];
  }

  /* per tile: max tree, exponentials relative to the tile max, sum tree.
     Positions past the end of the row are -inf for the max and 0 for the sum. */
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < TILE; ++i) {
      int64_t j = t * TILE + i;
      buf[i] = (j < N) ? x[j] : -INFINITY;
    }
    m[t] = tree_max256(buf);
    for (int i = 0; i < TILE; ++i) {
      int64_t j = t * TILE + i;
      float ej = 0.0f;
      if (j < N) {
        ej = (m[t] == -INFINITY) ? 0.0f : exp_(x[j] - m[t]);
        e[j] = ej;
      }
      buf[i] = ej;
    }
    l[t] = tree_sum256(buf);
  }

  /* tile states merged strictly left to right; the sink, a state with
     max sigma and sum 1, is merged after the last tile */
  float M = -INFINITY, L = 0.0f;
  for (int64_t t = 0; t < T; ++t) merge(&M, &L, m[t], l[t]);
  if (has_sink) merge(&M, &L, sigma, 1.0f);

  float invL = (L == 0.0f) ? 0.0f : 1.0f / L;

  /* each tile's e is rescaled from its own max to the row max and
     normalised; one conversion at the write */
  for (int64_t t = 0; t < T; ++t) {
    float c = (m[t] == -INFINITY) ? 0.0f : exp_(m[t] - M) * invL;
    for (int i = 0; i < TILE; ++i) {
      int64_t j = t * TILE + i;
      if (j < N) store_elem(dt, P, j, e[j] * c);
    }
  }
  if (has_sink)
    *p_sink = (sigma == -INFINITY) ? 0.0f : exp_(sigma - M) * invL;

  /* the row's log-sum-exp ([P3] Softmax and LSE), from the final state:
     the exponentials summed in L are relative to M, so
     ln(sum exp) = M + ln(L), the sink included when there is one.  Taken
     here as that value rounded once to binary32 (ln in double); a row with
     nothing to sum gets -inf. */
  if (lse) *lse = (L == 0.0f) ? -INFINITY : (float)((double)M + log((double)L));
}

/* ------------------------------------------------------------------------ */
/* Backward, one row                                                        */
/* ------------------------------------------------------------------------ */

/* One row: delta is the fixed-order sum of P*dP (same tiles and tree as the
   forward, tiles folded left to right starting from the first tile's sum),
   then dS = P * (dP - delta) ([P1] Fixed-order backward).  Keys at or past
   `kend` are excluded keys, whose probability the forward wrote as +0: P is
   taken as +0 there without being read (dP still is, so dS keeps its signed
   zero).  With a sink the row's share of d_sink, -p_sink*delta, is written
   to *v. */
static float p_at(int dt, const void *P, int64_t j, int64_t kend) {
  return (j < kend) ? load_elem(dt, P, j) : 0.0f;
}

static void bwd_row(int dt, int64_t N, int64_t kend, const void *P, const void *dP,
                    int has_sink, float ps, void *dS, float *v) {
  const int64_t T = (N + TILE - 1) / TILE;
  float buf[TILE];
  float delta = 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    for (int i = 0; i < TILE; ++i) {
      int64_t j = t * TILE + i;
      buf[i] = (j < N) ? p_at(dt, P, j, kend) * load_elem(dt, dP, j) : 0.0f;
    }
    float d = tree_sum256(buf);
    delta = (t == 0) ? d : delta + d;
  }
  for (int64_t j = 0; j < N; ++j) {
    float p = p_at(dt, P, j, kend);
    float g = load_elem(dt, dP, j);
    store_elem(dt, dS, j, p * (g - delta));
  }
  if (has_sink && v) *v = -(ps * delta);
}

/* Valid key prefix of row (b, q): all N keys, cut by the causal condition
   key <= N - Sq + q ([P3] Prefill / Decode: key_index <= Skv - Sq +
   query_index) and by the batch entry's valid key length (key padding,
   [P3] Path Status), clamped to [0, N]. */
static int64_t row_kend(int64_t N, int64_t Sq, int64_t b, int64_t q, int causal,
                        const int32_t *key_len) {
  int64_t kend = N;
  if (causal) {
    int64_t c = q + (N - Sq) + 1;
    if (c < kend) kend = c;
  }
  if (key_len) {
    int64_t k = key_len[b];
    if (k < kend) kend = k;
  }
  return kend < 0 ? 0 : kend;
}

/* ------------------------------------------------------------------------ */
/* Row drivers (threads over contiguous row ranges; rows are independent)   */
/* ------------------------------------------------------------------------ */

typedef struct {
  int dt;
  int64_t B, H, Sq, N, ld;
  const void *in0;      /* fwd: scores      bwd: P       */
  const void *in1;      /* fwd: (unused)    bwd: dP      */
  const float *mask;    /* fwd only, may be NULL */
  int64_t msb, msh, msq;
  const float *sink;    /* fwd: [H] sink logits     bwd: [rows] p_sink */
  int causal;           /* exclude keys past the causal condition */
  const int32_t *key_len; /* [B] valid keys per batch entry, or NULL */
  void *out;            /* fwd: P           bwd: dS      */
  float *out_row;       /* fwd: p_sink[rows]  bwd: v[rows] (may be NULL) */
  float *lse;           /* fwd: [rows] log-sum-exp, or NULL */
  int64_t r0, r1;
  int status;
} job_t;

static void *fwd_worker(void *arg) {
  job_t *j = (job_t *)arg;
  ieee_env();
  const int64_t N = j->N;
  const int64_t T = (N + TILE - 1) / TILE;
  float *x = (float *)malloc(sizeof(float) * (size_t)N);
  float *e = (float *)malloc(sizeof(float) * (size_t)N);
  float *m = (float *)malloc(sizeof(float) * (size_t)T);
  float *l = (float *)malloc(sizeof(float) * (size_t)T);
  if (!x || !e || !m || !l) { j->status = -1; free(x); free(e); free(m); free(l); return NULL; }
  const size_t es = elem_size(j->dt);
  for (int64_t r = j->r0; r < j->r1; ++r) {
    /* row r = (b*H + h)*Sq + q */
    int64_t q = r % j->Sq;
    int64_t h = (r / j->Sq) % j->H;
    int64_t b = r / (j->Sq * j->H);
    const char *srow = (const char *)j->in0 + (size_t)(r * j->ld) * es;
    char *prow = (char *)j->out + (size_t)(r * j->ld) * es;
    const float *arow = j->mask ? j->mask + b * j->msb + h * j->msh + q * j->msq : NULL;
    int has_sink = j->sink != NULL;
    float sigma = has_sink ? j->sink[h] : 0.0f;  /* one value per head ([P2]) */
    float *ps = has_sink ? &j->out_row[r] : NULL;
    int64_t kend = row_kend(N, j->Sq, b, q, j->causal, j->key_len);
    fwd_row(j->dt, N, kend, srow, arow, has_sink, sigma, prow, ps, j->lse ? &j->lse[r] : NULL,
            x, e, m, l);
  }
  free(x); free(e); free(m); free(l);
  j->status = 0;
  return NULL;
}

static void *bwd_worker(void *arg) {
  job_t *j = (job_t *)arg;
  ieee_env();
  const size_t es = elem_size(j->dt);
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t q = r % j->Sq;
    int64_t b = r / (j->Sq * j->H);
    int64_t kend = row_kend(j->N, j->Sq, b, q, j->causal, j->key_len);
    const char *prow = (const char *)j->in0 + (size_t)(r * j->ld) * es;
    const char *grow = (const char *)j->in1 + (size_t)(r * j->ld) * es;
    char *drow = (char *)j->out + (size_t)(r * j->ld) * es;
    int has_sink = j->sink != NULL;
    float ps = has_sink ? j->sink[r] : 0.0f;
    float *v = (has_sink && j->out_row) ? &j->out_row[r] : NULL;
    bwd_row(j->dt, j->N, kend, prow, grow, has_sink, ps, drow, v);
  }
  j->status = 0;
  return NULL;
}

static int run_jobs(job_t *proto, int64_t rows, int threads, void *(*fn)(void *)) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((int64_t)threads > rows) threads = (int)(rows > 0 ? rows : 1);
  job_t jobs[256];
  pthread_t tid[256];
  int started[256];
  int64_t per = rows / threads, extra = rows % threads, r = 0;
  for (int i = 0; i < threads; ++i) {
    jobs[i] = *proto;
    jobs[i].r0 = r;
    r += per + (i < extra ? 1 : 0);
    jobs[i].r1 = r;
    jobs[i].status = -1;
  }
  for (int i = 0; i < threads; ++i)
    started[i] = (i > 0) && pthread_create(&tid[i], NULL, fn, &jobs[i]) == 0;
  fn(&jobs[0]);
  for (int i = 1; i < threads; ++i) {
    if (started[i]) pthread_join(tid[i], NULL);
    else fn(&jobs[i]);  /* thread could not start: run it here */
  }
  for (int i = 0; i < threads; ++i)
    if (jobs[i].status != 0) return -1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Exported entry points                                                    */
/* ------------------------------------------------------------------------ */

/* Forward over scores [B, H, Sq, N] (row stride ld elements).  mask: binary32,
   element (b,h,q,k) at mask[b*msb + h*msh + q*msq + k], or NULL.  causal:
   exclude keys past the causal condition.  key_len: int32 [B] valid keys per
   batch entry, or NULL.  sink: binary32 [H] or NULL.  probs: same layout as
   scores.  p_sink: binary32 [B*H*Sq], written when sink is given.  lse:
   binary32 [B*H*Sq] row log-sum-exp, written when given.  Returns 0 on
   success. */
int jas_oracle_fwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t N, int64_t ld,
                   const void *scores, const float *mask, int64_t msb, int64_t msh,
                   int64_t msq, int causal, const int32_t *key_len, const float *sink,
                   void *probs, float *p_sink, float *lse, int threads) {
  if ((dtype != DT_F32 && dtype != DT_BF16 && dtype != DT_F16) || B < 0 || H < 0 || Sq < 0 ||
      N < 1 || ld < N)
    return -2;
  if (sink && !p_sink) return -3;
  int64_t rows = B * H * Sq;
  if (rows == 0) return 0;
  job_t j;
  memset(&j, 0, sizeof j);
  j.dt = dtype; j.B = B; j.H = H; j.Sq = Sq; j.N = N; j.ld = ld;
  j.in0 = scores; j.mask = mask; j.msb = msb; j.msh = msh; j.msq = msq;
  j.sink = sink; j.out = probs; j.out_row = p_sink; j.lse = lse;
  j.causal = causal; j.key_len = key_len;
  return run_jobs(&j, rows, threads, fwd_worker);
}

/* Backward over probs/dprobs [B, H, Sq, N] (row stride ld).  causal and
   key_len as for the forward (excluded keys: P taken as +0).  p_sink: [rows]
   or NULL.  dscores: same layout.  v: [rows] per-row d_sink share, written
   when p_sink and v are both given. */
int jas_oracle_bwd(int dtype, int64_t B, int64_t H, int64_t Sq, int64_t N, int64_t ld,
                   const void *probs, const void *dprobs, int causal, const int32_t *key_len,
                   const float *p_sink, void *dscores, float *v, int threads) {
  if ((dtype != DT_F32 && dtype != DT_BF16 && dtype != DT_F16) || B < 0 || H < 0 || Sq < 0 ||
      N < 1 || ld < N)
    return -2;
  int64_t rows = B * H * Sq;
  if (rows == 0) return 0;
  job_t j;
  memset(&j, 0, sizeof j);
  j.dt = dtype; j.B = B; j.H = H; j.Sq = Sq; j.N = N; j.ld = ld;
  j.in0 = probs; j.in1 = dprobs; j.sink = p_sink; j.out = dscores; j.out_row = v;
  j.causal = causal; j.key_len = key_len;
  return run_jobs(&j, rows, threads, bwd_worker);
}

/* d_sink[h] from the per-row shares v[B*H*Sq]: the rows of head h taken in
   (b, q) order, cut into 256-row chunks (the last padded with +0), each chunk
   summed with the balanced tree, chunk sums folded left to right starting
   from the first.  d_sink is overwritten, never accumulated ([P2] d_sink per
   head; here in a fixed order without atomics).  A head with no rows gets
   +0. */
int jas_oracle_dsink(int64_t B, int64_t H, int64_t Sq, const float *v, float *d_sink) {
  if (B < 0 || H < 0 || Sq < 0) return -2;
  ieee_env();
  const int64_t n = B * Sq;
  const int64_t chunks = (n + TILE - 1) / TILE;
  float buf[TILE];
  for (int64_t h = 0; h < H; ++h) {
    float D = 0.0f;
    for (int64_t k = 0; k < chunks; ++k) {
      for (int i = 0; i < TILE; ++i) {
        int64_t idx = k * TILE + i;          /* position in the head's row list */
        if (idx < n) {
          int64_t b = idx / Sq, q = idx % Sq;
          buf[i] = v[(b * H + h) * Sq + q];
        } else {
          buf[i] = 0.0f;
        }
      }
      float cs = tree_sum256(buf);
      D = (k == 0) ? cs : D + cs;
    }
    d_sink[h] = D;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Fixed-order attention forward: QK, this softmax, PV                      */
/* ------------------------------------------------------------------------ */

/* One query row of attention ([P3] Fixed Reduction Contract: every score
   has one writer and accumulates the head dimension in ascending order, the
   softmax is the fixed-order one above, every output element has one writer
   and accumulates the keys in ascending order; [P1] Summary: the softmax
   sits between the QK GEMM and the AV GEMM and rounds once, to the tensor
   dtype, when it writes P).
     s_j   = fl(scale * dot_j), dot_j = sum over d = 0..D-1 of fl(q_d*k_jd),
             added in that order
     P_j   = the row softmax of s (mask, exclusion, sink as in fwd_row),
             rounded to the tensor dtype
     out_d = sum over j = 0..N-1 of fl(P_j*v_jd), added in that order, then
             rounded to the tensor dtype
   Optional outputs: the scores s (binary32) and P (tensor dtype). */
typedef struct {
  int dt;
  int64_t B, H, Hkv, Sq, N, D;
  const void *q, *k, *v;
  float scale;
  const float *mask;
  int64_t msb, msh, msq;
  int causal;
  const int32_t *key_len;
  const float *sink;
  void *out;
  float *lse, *p_sink;
  void *probs;
  float *scores;
  int64_t r0, r1;
  int status;
} attn_job_t;

static void *attn_worker(void *arg) {
  attn_job_t *j = (attn_job_t *)arg;
  ieee_env();
  const int64_t N = j->N, D = j->D;
  const int64_t T = (N + TILE - 1) / TILE;
  const size_t es = elem_size(j->dt);
  float *s = (float *)malloc(sizeof(float) * (size_t)N);
  float *pf = (float *)malloc(sizeof(float) * (size_t)N);
  void *P = malloc(es * (size_t)N);
  float *x = (float *)malloc(sizeof(float) * (size_t)N);
  float *e = (float *)malloc(sizeof(float) * (size_t)N);
  float *m = (float *)malloc(sizeof(float) * (size_t)T);
  float *l = (float *)malloc(sizeof(float) * (size_t)T);
  if (!s || !pf || !P || !x || !e || !m || !l) {
    j->status = -1;
    free(s); free(pf); free(P); free(x); free(e); free(m); free(l);
    return NULL;
  }
  const int64_t group = j->H / j->Hkv;  /* query heads per key/value head */
  for (int64_t r = j->r0; r < j->r1; ++r) {
    const int64_t qi = r % j->Sq;
    const int64_t h = (r / j->Sq) % j->H;
    const int64_t b = r / (j->Sq * j->H);
    const int64_t hk = h / group;
    const int64_t qoff = r * D;
    const int64_t kvoff = (b * j->Hkv + hk) * N * D;
    for (int64_t kj = 0; kj < N; ++kj) {
      float dot = 0.0f;
      for (int64_t d = 0; d < D; ++d) {
        const float prod = load_elem(j->dt, j->q, qoff + d) * load_elem(j->dt, j->k, kvoff + kj * D + d);
        dot = dot + prod;
      }
      s[kj] = j->scale * dot;
    }
    if (j->scores) memcpy(j->scores + r * N, s, sizeof(float) * (size_t)N);
    const float *arow = j->mask ? j->mask + b * j->msb + h * j->msh + qi * j->msq : NULL;
    const int has_sink = j->sink != NULL;
    const float sigma = has_sink ? j->sink[h] : 0.0f;
    float ps = 0.0f, ls = 0.0f;
    const int64_t kend = row_kend(N, j->Sq, b, qi, j->causal, j->key_len);
    /* the softmax of the binary32 scores, rounded to the tensor dtype at the write */
    fwd_row(DT_F32, N, kend, s, arow, has_sink, sigma, pf, &ps, &ls, x, e, m, l);
    for (int64_t kj = 0; kj < N; ++kj) store_elem(j->dt, P, kj, pf[kj]);
    if (j->probs) memcpy((char *)j->probs + (size_t)(r * N) * es, P, es * (size_t)N);
    if (has_sink) j->p_sink[r] = ps;
    if (j->lse) j->lse[r] = ls;
    for (int64_t d = 0; d < D; ++d) {
      float acc = 0.0f;
      for (int64_t kj = 0; kj < N; ++kj) {
        const float prod = load_elem(j->dt, P, kj) * load_elem(j->dt, j->v, kvoff + kj * D + d);
        acc = acc + prod;
      }
      store_elem(j->dt, j->out, qoff + d, acc);
    }
  }
  free(s); free(pf); free(P); free(x); free(e); free(m); free(l);
  j->status = 0;
  return NULL;
}

/* Attention forward.  q, out [B, H, Sq, D]; k, v [B, Hkv, N, D] (H a
   multiple of Hkv; query head h reads key/value head h / (H / Hkv)); all
   contiguous, dtype bf16 or fp16.  mask / causal / key_len / sink as for
   jas_oracle_fwd.  lse, p_sink: [B*H*Sq] or NULL; probs [B, H, Sq, N]
   (dtype) and scores [B, H, Sq, N] (binary32) written when given. */
int jas_oracle_attn_fwd(int dtype, int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t N,
                        int64_t D, const void *q, const void *k, const void *v, float scale,
                        const float *mask, int64_t msb, int64_t msh, int64_t msq, int causal,
                        const int32_t *key_len, const float *sink, void *out, float *lse,
                        float *p_sink, void *probs, float *scores, int threads) {
  if ((dtype != DT_BF16 && dtype != DT_F16) || B < 0 || H < 1 || Hkv < 1 || H % Hkv ||
      Sq < 0 || N < 1 || D < 1)
    return -2;
  if (sink && !p_sink) return -3;
  const int64_t rows = B * H * Sq;
  if (rows == 0) return 0;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((int64_t)threads > rows) threads = (int)rows;
  attn_job_t jobs[256];
  pthread_t tid[256];
  int started[256];
  int64_t per = rows / threads, extra = rows % threads, r = 0;
  for (int i = 0; i < threads; ++i) {
    attn_job_t *a = &jobs[i];
    memset(a, 0, sizeof *a);
    a->dt = dtype; a->B = B; a->H = H; a->Hkv = Hkv; a->Sq = Sq; a->N = N; a->D = D;
    a->q = q; a->k = k; a->v = v; a->scale = scale;
    a->mask = mask; a->msb = msb; a->msh = msh; a->msq = msq;
    a->causal = causal; a->key_len = key_len; a->sink = sink;
    a->out = out; a->lse = lse; a->p_sink = p_sink; a->probs = probs; a->scores = scores;
    a->r0 = r;
    r += per + (i < extra ? 1 : 0);
    a->r1 = r;
    a->status = -1;
  }
  for (int i = 0; i < threads; ++i)
    started[i] = (i > 0) && pthread_create(&tid[i], NULL, attn_worker, &jobs[i]) == 0;
  attn_worker(&jobs[0]);
  for (int i = 1; i < threads; ++i) {
    if (started[i]) pthread_join(tid[i], NULL);
    else attn_worker(&jobs[i]);
  }
  for (int i = 0; i < threads; ++i)
    if (jobs[i].status != 0) return -1;
  return 0;
}

/* Small pieces exported for the pin tests. */
float jas_oracle_exp(float y) { ieee_env(); return exp_(y); }
float jas_oracle_log2e(void) { return log2e_f32(); }
uint16_t jas_oracle_bf16(float x) { return f32_to_bf16(x); }
void jas_oracle_f16_array(const float *x, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16(x[i]);
}
void jas_oracle_f16_decode_array(const uint16_t *h, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f32(h[i]);
}
float jas_oracle_tree_sum256(const float *v) {
  float buf[TILE];
  ieee_env();
  memcpy(buf, v, sizeof buf);
  return tree_sum256(buf);
}
