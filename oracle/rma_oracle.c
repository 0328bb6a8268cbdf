/*
 * RMA layer-step oracle: TEST INFRASTRUCTURE ONLY (see rma_oracle.h).
 *
 * Plain C, double arithmetic, OpenMP only over independent items: the
 * (sequence, group, head) reads of a token and the (sequence, group)
 * admits.  Written from the EdgeRock pages; each
 * function names the passage it follows.  Readings of points the pages
 * leave open are marked "Reading:".
 */
#include "rma_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 */

static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Exact round-to-nearest-even of a double to bf16: take the two bf16
 * neighbours of x and pick the closer one (even mantissa on a tie). */
uint16_t orc_round_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  if (isinf(x)) return x > 0 ? 0x7F80 : 0xFF80;
  float f = (float)x;
  /* force f toward zero of x so that it lies between the neighbours */
  if (fabs((double)f) > fabs(x)) f = nextafterf(f, 0.0f);
  uint32_t lo = float_bits(f) & 0xFFFF0000u;      /* toward zero */
  uint32_t hi = lo + 0x10000u;                    /* away from zero */
  /* past the largest finite bf16 the next grid point is 2^128, which
     rounds to infinity */
  const double vhi = ((hi & 0x7FFFFFFFu) == 0x7F800000u)
                         ? copysign(ldexp(1.0, 128), x)
                         : (double)bits_float(hi);
  double dlo = fabs(x - (double)bits_float(lo));
  double dhi = fabs(vhi - x);
  uint32_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = ((lo >> 16) & 1u) ? hi : lo;
  return (uint16_t)(pick >> 16);
}

void orc_round_bf16_array(const double* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_round_bf16(x[i]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------- indexing */

static size_t unit_index(const orc_state* st, int32_t l, int32_t b, int32_t g) {
  return ((size_t)l * st->B + b) * st->cfg.G + g;
}

static int cfg_ok(const orc_state* st) {
  if (!st) return 0;
  const orc_cfg* c = &st->cfg;
  if (c->L < 1 || c->H < 1 || c->G < 1 || c->H % c->G || c->d < 1) return 0;
  if (c->R < 1 || c->N < 1 || c->C < 1 || st->B < 1) return 0;
  return 1;
}

/* --------------------------------------------------------- attention read */

/* Softmax attention of one query over `nk` keys:
 *   o = sum_j softmax_j(scale * <q, K_j>) V_j,
 * with the maximum subtracted before exponentiation (same value, no
 * overflow).  keys[j] / vals[j] point at d bf16 values. */
static void attend(int d, double scale, const double* q, int nk,
                   const uint16_t* const* keys, const uint16_t* const* vals,
                   double* s, double* o) {
  double m = -INFINITY;
  for (int j = 0; j < nk; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += q[i] * bf16_to_double(keys[j][i]);
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double z = 0.0;
  for (int j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  for (int i = 0; i < d; ++i) o[i] = 0.0;
  for (int j = 0; j < nk; ++j) {
    double w = s[j] / z;
    for (int i = 0; i < d; ++i) o[i] += w * bf16_to_double(vals[j][i]);
  }
}

/* Output of one token at position t for sequence b, query head hh of
 * group g of a layer.
 *
 * Retrieve (ai-primer, three-operation list, item 3; model card "How Rock
 * Memory Anchors work"): queries read the committed bank; a
 * query-dependent signed gate combines the retrieved information with
 * attention over the local window.
 *   - local window: 1,024 positions = the ring's 1,023 preceding
 *     positions plus the current token (model card, persistent-history
 *     table note; ai-primer memory section).
 *     Reading: positions max(0, t-R) .. t-1 from ring slot p mod R, plus
 *     the current (k_t, v_t); no padding keys while t < R.
 *   - anchor read: committed bank slots 0 .. n-1 of the query's group.
 *     Reading: n == 0 gives a zero anchor read.
 *   - Reading (gate form, fixed for this build): out = o_local +
 *     tanh(<qa_h, w_g[h]>) * o_anchor, two separately normalised reads,
 *     where qa is the query of the anchor read.
 *   - Reading: the anchor read and the gate use their own query qa (the
 *     card's "separate RMA modules" and "query-dependent read"); when no
 *     such query is given, qa = q, the attention query of the head.
 *   - Reading: heads h = g*(H/G) ... g*(H/G)+H/G-1 share group g.
 *   - Reading (per-group gate, cfg.gate_group; the separate RMA modules of
 *     the models page and the tpsreport "How it works" paragraph, which
 *     select per KV group): one gate per (token, group),
 *     tanh(<mean of the group's anchor queries, w_g[g]>), one weight
 *     vector per group; every head of the group uses it.
 */
static void token_output(const orc_state* st, int32_t layer, int32_t b, int32_t g,
                         int32_t hh, int64_t t, const uint16_t* qtok /*[H][d]*/,
                         const uint16_t* qatok /*[H][d]*/,
                         const uint16_t* kcur, const uint16_t* vcur,
                         const float* w_g /*[H][d]*/, double* out /*[H][d]*/) {
  const orc_cfg* c = &st->cfg;
  const int d = c->d, R = c->R, N = c->N, hpg = c->H / c->G;
  const size_t u = unit_index(st, layer, b, g);
  const uint16_t* ringk = st->ring_k + u * (size_t)R * d;
  const uint16_t* ringv = st->ring_v + u * (size_t)R * d;
  const uint16_t* bankk = st->bank_k + u * (size_t)N * d;
  const uint16_t* bankv = st->bank_v + u * (size_t)N * d;
  const int n = st->bank_n[u];

  /* local keys: the preceding positions still in the ring, then the
     current token */
  const int64_t first = t - R > 0 ? t - R : 0;
  const int nloc = (int)(t - first) + 1;
  const uint16_t** lk = (const uint16_t**)malloc(sizeof(void*) * nloc);
  const uint16_t** lv = (const uint16_t**)malloc(sizeof(void*) * nloc);
  int j = 0;
  for (int64_t p = first; p < t; ++p, ++j) {
    const size_t slot = (size_t)(p % R);
    lk[j] = ringk + slot * d;
    lv[j] = ringv + slot * d;
  }
  lk[j] = kcur;
  lv[j] = vcur;

  /* anchor keys: committed slots 0 .. n-1 */
  const int nb = n > 0 ? n : 1;
  const uint16_t** ak = (const uint16_t**)malloc(sizeof(void*) * nb);
  const uint16_t** av = (const uint16_t**)malloc(sizeof(void*) * nb);
  for (int i = 0; i < n; ++i) {
    ak[i] = bankk + (size_t)i * d;
    av[i] = bankv + (size_t)i * d;
  }

  const int ns = nloc > n ? nloc : n;
  double* s = (double*)malloc(sizeof(double) * ns);
  double* q = (double*)malloc(sizeof(double) * d);
  double* qa = (double*)malloc(sizeof(double) * d);
  double* oloc = (double*)malloc(sizeof(double) * d);
  double* oanc = (double*)malloc(sizeof(double) * d);

  const int h = g * hpg + hh;
  for (int i = 0; i < d; ++i) q[i] = bf16_to_double(qtok[(size_t)h * d + i]);
  for (int i = 0; i < d; ++i) qa[i] = bf16_to_double(qatok[(size_t)h * d + i]);

  attend(d, c->scale, q, nloc, lk, lv, s, oloc);
  if (n > 0) {
    attend(d, c->scale, qa, n, ak, av, s, oanc);
  } else {
    for (int i = 0; i < d; ++i) oanc[i] = 0.0;
  }

  double zg = 0.0;
  if (c->gate_group) {
    /* the mean of the group's anchor queries against the group's weights */
    double* qm = (double*)calloc((size_t)d, sizeof(double));
    for (int h2 = g * hpg; h2 < (g + 1) * hpg; ++h2)
      for (int i = 0; i < d; ++i) qm[i] += bf16_to_double(qatok[(size_t)h2 * d + i]);
    for (int i = 0; i < d; ++i) zg += (qm[i] / hpg) * (double)w_g[(size_t)g * d + i];
    free(qm);
  } else {
    for (int i = 0; i < d; ++i) zg += qa[i] * (double)w_g[(size_t)h * d + i];
  }
  const double gate = tanh(zg);
  for (int i = 0; i < d; ++i) out[(size_t)h * d + i] = oloc[i] + gate * oanc[i];
  free(lk); free(lv); free(ak); free(av); free(s); free(q); free(qa); free(oloc); free(oanc);
}

/* Write (ai-primer list item 1; tpsreport "How it works"): the current
 * token's K/V enters the ring, replacing position t - R (the ring keeps
 * the 1,023 preceding positions), and the writer's candidate record and
 * its score go to pending slot t mod C (a fixed 256-position buffer).
 * Reading: one fp32 score per (token, layer, group). */
static void token_write(const orc_state* st, int32_t layer, int32_t b, int32_t g,
                        int64_t t, const uint16_t* kcur, const uint16_t* vcur,
                        const uint16_t* ckc, const uint16_t* cvc, float csc) {
  const orc_cfg* c = &st->cfg;
  const int d = c->d;
  const size_t u = unit_index(st, layer, b, g);
  const size_t rs = (size_t)(t % c->R), ps = (size_t)(t % c->C);
  memcpy(st->ring_k + (u * c->R + rs) * d, kcur, sizeof(uint16_t) * d);
  memcpy(st->ring_v + (u * c->R + rs) * d, vcur, sizeof(uint16_t) * d);
  memcpy(st->pend_k + (u * c->C + ps) * d, ckc, sizeof(uint16_t) * d);
  memcpy(st->pend_v + (u * c->C + ps) * d, cvc, sizeof(uint16_t) * d);
  st->pscore[u * c->C + ps] = csc;
}

int orc_decode_step(const orc_state* st, int32_t layer,
                    const uint16_t* q, const uint16_t* q_anchor, const uint16_t* k,
                    const uint16_t* v, const uint16_t* ck, const uint16_t* cv,
                    const float* cs, const float* w_g, double* out, int32_t compute_out) {
  if (!cfg_ok(st) || layer < 0 || layer >= st->cfg.L) return ORC_E_ARG;
  const orc_cfg* c = &st->cfg;
  const int64_t t = st->t[layer];
  if (t < 0) return ORC_E_ARG;
  /* a full pending buffer must be admitted before the next token */
  if (st->pend_n[layer] >= c->C) return ORC_E_PENDING_FULL;
  const int B = st->B, G = c->G, H = c->H, d = c->d;
  if (compute_out) {
    if (!out) return ORC_E_ARG;
    const int hpg = H / G;
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < G; ++g)
        for (int hh = 0; hh < hpg; ++hh)
          token_output(st, layer, b, g, hh, t, q + (size_t)b * H * d,
                       (q_anchor ? q_anchor : q) + (size_t)b * H * d,
                       k + ((size_t)b * G + g) * d, v + ((size_t)b * G + g) * d,
                       w_g, out + (size_t)b * H * d);
  }
  /* writes only after every read of this token (slot t mod R is still
     inside this token's window) */
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < G; ++g) {
      const size_t o = ((size_t)b * G + g) * d;
      token_write(st, layer, b, g, t, k + o, v + o, ck + o, cv + o, cs[(size_t)b * G + g]);
    }
  st->t[layer] = t + 1;
  st->pend_n[layer] += 1;
  return ORC_OK;
}

/* ------------------------------------------------------------------ admit */

typedef struct {
  float score;
  int32_t gidx;   /* anchors: slot; candidates: N + pending slot */
} pool_entry;

/* Score order.  Reading: higher score first; -0.0 and +0.0 are equal;
 * every NaN is equal to every other NaN and ranks below -inf. */
static int score_before(float a, float b) {
  if (isnan(a)) return 0;
  if (isnan(b)) return 1;
  return a > b;
}

/* Total order of the pool: score descending, then global index ascending
 * (an incumbent anchor beats a candidate of equal score; earlier slots
 * and earlier candidates win ties). */
static int pool_cmp(const void* pa, const void* pb) {
  const pool_entry* a = (const pool_entry*)pa;
  const pool_entry* b = (const pool_entry*)pb;
  if (score_before(a->score, b->score)) return -1;
  if (score_before(b->score, a->score)) return 1;
  return (a->gidx > b->gidx) - (a->gidx < b->gidx);
}

/* Admit (ai-primer list item 2; tpsreport "How it works"; model card
 * "How Rock Memory Anchors work"): every 256 tokens the existing anchors
 * and the new candidates compete, per KV group, for at most 1,024
 * records; the highest-priority ones are kept; retained records stay
 * where they are, unchanged.
 * Reading: keep the first K = min(N, n + C) of the pool in the order
 * above.  Evicted anchor slots, in ascending order, receive the admitted
 * candidates in ascending pending order; the rest are appended at
 * n, n+1, ...; score and source position travel with the record. */
static int admit_group(const orc_state* st, int32_t layer, int32_t b, int32_t g,
                       int64_t block_start) {
  const orc_cfg* c = &st->cfg;
  const int d = c->d, N = c->N, C = c->C;
  const size_t u = unit_index(st, layer, b, g);
  const int n = st->bank_n[u];
  const int P = n + C;
  const int K = N < P ? N : P;
  pool_entry* pool = (pool_entry*)malloc(sizeof(pool_entry) * P);
  unsigned char* kept = (unsigned char*)calloc(P, 1);  /* by pool position */
  int* evicted = (int*)malloc(sizeof(int) * (n > 0 ? n : 1));
  int* admitted = (int*)malloc(sizeof(int) * C);

  for (int i = 0; i < n; ++i) {
    pool[i].score = st->bscore[u * N + i];
    pool[i].gidx = i;
  }
  for (int j = 0; j < C; ++j) {
    pool[n + j].score = st->pscore[u * C + j];
    pool[n + j].gidx = N + j;
  }
  qsort(pool, P, sizeof(pool_entry), pool_cmp);
  for (int r = 0; r < K; ++r) {
    const int gi = pool[r].gidx;
    kept[gi < N ? gi : n + (gi - N)] = 1;
  }
  int ne = 0, na = 0;
  for (int i = 0; i < n; ++i)
    if (!kept[i]) evicted[ne++] = i;
  for (int j = 0; j < C; ++j)
    if (kept[n + j]) admitted[na++] = j;

  for (int a = 0; a < na; ++a) {
    const int j = admitted[a];
    const int dst = a < ne ? evicted[a] : n + (a - ne);
    memcpy(st->bank_k + (u * N + dst) * d, st->pend_k + (u * C + j) * d, sizeof(uint16_t) * d);
    memcpy(st->bank_v + (u * N + dst) * d, st->pend_v + (u * C + j) * d, sizeof(uint16_t) * d);
    st->bscore[u * N + dst] = st->pscore[u * C + j];
    st->bsrc[u * N + dst] = (int32_t)(block_start + j);
  }
  st->bank_n[u] = K;
  free(pool); free(kept); free(evicted); free(admitted);
  return na;
}

int orc_admit(const orc_state* st, int32_t layer, int32_t* moved) {
  if (!cfg_ok(st) || layer < 0 || layer >= st->cfg.L) return ORC_E_ARG;
  const int64_t t = st->t[layer];
  const int C = st->cfg.C;
  /* Reading: blocks are [C*i, C*i + C) from position 0; admit runs once
     the block's C candidates are pending. */
  if (st->pend_n[layer] != C || t % C != 0) return ORC_E_NOT_BOUNDARY;
  const int B = st->B, G = st->cfg.G;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < G; ++g) {
      const int na = admit_group(st, layer, b, g, t - C);
      if (moved) moved[(size_t)b * G + g] = na;
    }
  st->pend_n[layer] = 0;
  return ORC_OK;
}

/* ---------------------------------------------------------------- prefill */

/* A block of the prompt is the same computation as its tokens decoded in
 * order: reads use the committed bank (new records become visible only in
 * the next block, model card "How Rock Memory Anchors work"), and admit
 * waits for the block's end. */
int orc_prefill_block(const orc_state* st, int32_t layer, int32_t n,
                      const uint16_t* q, const uint16_t* q_anchor, const uint16_t* k,
                      const uint16_t* v, const uint16_t* ck, const uint16_t* cv,
                      const float* cs, const float* w_g, double* out) {
  if (!cfg_ok(st) || layer < 0 || layer >= st->cfg.L) return ORC_E_ARG;
  const orc_cfg* c = &st->cfg;
  if (n < 1 || n > c->C) return ORC_E_ARG;
  if (st->pend_n[layer] != 0 || st->t[layer] % c->C != 0) return ORC_E_NOT_BOUNDARY;
  const int B = st->B, G = c->G, H = c->H, d = c->d;
  uint16_t* tq = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * H * d);
  uint16_t* tqa = q_anchor ? (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * H * d) : NULL;
  uint16_t* tk = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * G * d);
  uint16_t* tv = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * G * d);
  uint16_t* tck = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * G * d);
  uint16_t* tcv = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * G * d);
  float* tcs = (float*)malloc(sizeof(float) * (size_t)B * G);
  double* tout = (double*)malloc(sizeof(double) * (size_t)B * H * d);
  int rc = ORC_OK;
  for (int i = 0; i < n && rc == ORC_OK; ++i) {
    for (int b = 0; b < B; ++b) {
      memcpy(tq + (size_t)b * H * d, q + ((size_t)b * n + i) * H * d, sizeof(uint16_t) * H * d);
      if (tqa)
        memcpy(tqa + (size_t)b * H * d, q_anchor + ((size_t)b * n + i) * H * d,
               sizeof(uint16_t) * H * d);
      memcpy(tk + (size_t)b * G * d, k + ((size_t)b * n + i) * G * d, sizeof(uint16_t) * G * d);
      memcpy(tv + (size_t)b * G * d, v + ((size_t)b * n + i) * G * d, sizeof(uint16_t) * G * d);
      memcpy(tck + (size_t)b * G * d, ck + ((size_t)b * n + i) * G * d, sizeof(uint16_t) * G * d);
      memcpy(tcv + (size_t)b * G * d, cv + ((size_t)b * n + i) * G * d, sizeof(uint16_t) * G * d);
      memcpy(tcs + (size_t)b * G, cs + ((size_t)b * n + i) * G, sizeof(float) * G);
    }
    rc = orc_decode_step(st, layer, tq, tqa, tk, tv, tck, tcv, tcs, w_g, tout, out != NULL);
    if (out)
      for (int b = 0; b < B; ++b)
        memcpy(out + ((size_t)b * n + i) * H * d, tout + (size_t)b * H * d, sizeof(double) * H * d);
  }
  free(tq); free(tqa); free(tk); free(tv); free(tck); free(tcv); free(tcs); free(tout);
  return rc;
}
