/*
 * librma.so driven through its C ABI alone (include/rma.h), with no Python
 * in the loop, and checked against the C oracle (oracle/rma_oracle.h).
 * Test infrastructure: it links the oracle.
 *
 * A small geometry (1 layer, 3 sequences, 2 KV groups of 4 query heads,
 * head_dim 256, window 40 = ring 39, bank 24, commit 8) from an empty
 * history:
 *   - 24 lockstep decode tokens (rma_decode_step), with rma_admit at each
 *     of the three block ends;
 *   - one full prompt block (rma_prefill_block) and its admit;
 * every output against the oracle's within the decode tolerance (2e-2
 * max-abs on bf16 outputs), then the whole device history, decoded through
 * rma_state_layout, bit for bit against the oracle's state.  Inputs come
 * from a seeded xorshift generator of this file (values ~N(0,1)/16 rounded
 * to bf16, as the library's workloads draw them).  Exit status 0 on
 * success; the first failure is printed.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rma.h"
#include "rma_oracle.h"

enum { L = 1, B = 3, G = 2, H = 8, D = 256, WINDOW = 40, R = WINDOW - 1, N = 24, C = 8 };
static const double kTol = 2e-2;

#define HIP_OK(x)                                                        \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #x);            \
      exit(2);                                                           \
    }                                                                    \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform01(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0);
}
/* approximately N(0,1): the sum of 12 uniforms minus 6 */
static double normal(void) {
  double s = 0.0;
  for (int i = 0; i < 12; ++i) s += uniform01();
  return s - 6.0;
}
/* bf16 bits of a float, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static void fill_bf16(uint16_t* p, size_t n, double std) {
  for (size_t i = 0; i < n; ++i) p[i] = to_bf16((float)(normal() * std));
}
static void fill_f32(float* p, size_t n, double std) {
  for (size_t i = 0; i < n; ++i) p[i] = (float)(normal() * std);
}
static void* dev_copy(const void* h, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes));
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}
static void fail(const char* what) {
  fprintf(stderr, "FAIL: %s\n", what);
  exit(1);
}

/* outputs [rows][D] bf16 from the device against the oracle's doubles */
static double max_err(const uint16_t* got, const double* ref, size_t n) {
  double e = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double x = fabs((double)from_bf16(got[i]) - ref[i]);
    if (!(x <= e)) e = x; /* a NaN output makes e NaN and fails below */
  }
  return e;
}

/* a chunk-major K plane (chunk c of slot s at 16-byte index c*slots + s)
 * against natural [slots_used][D] rows */
static int k_plane_equal(const uint16_t* plane, int slots, const uint16_t* rows, int used) {
  for (int s = 0; s < used; ++s)
    for (int c = 0; c < D / 8; ++c)
      if (memcmp(plane + ((size_t)c * slots + s) * 8, rows + (size_t)s * D + 8 * c, 16) != 0)
        return 0;
  return 1;
}

int main(void) {
  rma_config cfg;
  if (rma_config_default(&cfg) != RMA_OK) fail("rma_config_default");
  cfg.layers = L;
  cfg.q_heads = H;
  cfg.kv_groups = G;
  cfg.window = WINDOW;
  cfg.bank_cap = N;
  cfg.commit = C;
  rma_layout lay;
  if (rma_state_layout(&cfg, B, &lay) != RMA_OK) fail("rma_state_layout");
  const size_t bytes = rma_state_bytes(&cfg, B);
  if (bytes != lay.total_bytes) fail("rma_state_bytes disagrees with the layout");

  void* dbuf = NULL;
  HIP_OK(hipMalloc(&dbuf, bytes));
  HIP_OK(hipMemset(dbuf, 0, bytes));
  rma_state st;
  memset(&st, 0, sizeof(st));
  if (rma_state_init(&st, &cfg, B, dbuf, bytes, 0, 0, NULL) != RMA_OK) fail("rma_state_init");

  /* the oracle's state, natural layout, empty history */
  const size_t units = (size_t)L * B * G;
  orc_state o;
  memset(&o, 0, sizeof(o));
  o.cfg.L = L;
  o.cfg.H = H;
  o.cfg.G = G;
  o.cfg.d = D;
  o.cfg.R = R;
  o.cfg.N = N;
  o.cfg.C = C;
  o.cfg.scale = cfg.scale;
  o.cfg.gate_group = 0;
  o.B = B;
  o.ring_k = calloc(units * R * D, 2);
  o.ring_v = calloc(units * R * D, 2);
  o.bank_k = calloc(units * N * D, 2);
  o.bank_v = calloc(units * N * D, 2);
  o.bscore = calloc(units * N, 4);
  o.bsrc = calloc(units * N, 4);
  o.bank_n = calloc(units, 4);
  o.pend_k = calloc(units * C * D, 2);
  o.pend_v = calloc(units * C * D, 2);
  o.pscore = calloc(units * C, 4);
  o.t = calloc(L, 8);
  o.pend_n = calloc(L, 4);

  float* wg = malloc(sizeof(float) * H * D);
  fill_f32(wg, (size_t)H * D, 1.0 / 16);
  void* d_wg = dev_copy(wg, sizeof(float) * H * D);

  /* decode: three blocks, admit at each block end */
  const size_t qn = (size_t)B * H * D, kn = (size_t)B * G * D, sn = (size_t)B * G;
  uint16_t *q = malloc(2 * qn), *k = malloc(2 * kn), *v = malloc(2 * kn), *ck = malloc(2 * kn),
           *cv = malloc(2 * kn), *out = malloc(2 * qn);
  float* cs = malloc(4 * sn);
  double* ref = malloc(8 * qn);
  void *d_q, *d_k, *d_v, *d_ck, *d_cv, *d_cs, *d_out;
  HIP_OK(hipMalloc(&d_q, 2 * qn));
  HIP_OK(hipMalloc(&d_k, 2 * kn));
  HIP_OK(hipMalloc(&d_v, 2 * kn));
  HIP_OK(hipMalloc(&d_ck, 2 * kn));
  HIP_OK(hipMalloc(&d_cv, 2 * kn));
  HIP_OK(hipMalloc(&d_cs, 4 * sn));
  HIP_OK(hipMalloc(&d_out, 2 * qn));
  double worst = 0.0;
  int admits = 0;
  for (int step = 0; step < 3 * C; ++step) {
    fill_bf16(q, qn, 1.0 / 16);
    fill_bf16(k, kn, 1.0 / 16);
    fill_bf16(v, kn, 1.0 / 16);
    fill_bf16(ck, kn, 1.0 / 16);
    fill_bf16(cv, kn, 1.0 / 16);
    fill_f32(cs, sn, 1.0);
    HIP_OK(hipMemcpy(d_q, q, 2 * qn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_k, k, 2 * kn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_v, v, 2 * kn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_ck, ck, 2 * kn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cv, cv, 2 * kn, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_cs, cs, 4 * sn, hipMemcpyHostToDevice));
    if (rma_decode_step(&st, 0, d_q, d_k, d_v, d_ck, d_cv, d_cs, d_wg, d_out, NULL) != RMA_OK)
      fail("rma_decode_step");
    HIP_OK(hipMemcpy(out, d_out, 2 * qn, hipMemcpyDeviceToHost));
    if (orc_decode_step(&o, 0, q, NULL, k, v, ck, cv, cs, wg, ref, 1) != ORC_OK)
      fail("orc_decode_step");
    const double e = max_err(out, ref, qn);
    if (!(e <= kTol)) {
      fprintf(stderr, "decode step %d: max error %.3e\n", step, e);
      fail("decode output");
    }
    if (e > worst) worst = e;
    if (st.pend_n[0] == C) {
      if (rma_admit(&st, 0, NULL) != RMA_OK) fail("rma_admit");
      if (orc_admit(&o, 0, NULL) != ORC_OK) fail("orc_admit");
      ++admits;
    }
  }
  if (admits != 3 || st.t[0] != 3 * C || o.t[0] != 3 * C) fail("block ends");

  /* one full prompt block, then its admit */
  const size_t pq = (size_t)C * qn, pk = (size_t)C * kn, ps = (size_t)C * sn;
  uint16_t *bq = malloc(2 * pq), *bk = malloc(2 * pk), *bv = malloc(2 * pk), *bck = malloc(2 * pk),
           *bcv = malloc(2 * pk), *bout = malloc(2 * pq);
  float* bcs = malloc(4 * ps);
  double* bref = malloc(8 * pq);
  fill_bf16(bq, pq, 1.0 / 16);
  fill_bf16(bk, pk, 1.0 / 16);
  fill_bf16(bv, pk, 1.0 / 16);
  fill_bf16(bck, pk, 1.0 / 16);
  fill_bf16(bcv, pk, 1.0 / 16);
  fill_f32(bcs, ps, 1.0);
  void *e_q = dev_copy(bq, 2 * pq), *e_k = dev_copy(bk, 2 * pk), *e_v = dev_copy(bv, 2 * pk),
       *e_ck = dev_copy(bck, 2 * pk), *e_cv = dev_copy(bcv, 2 * pk), *e_cs = dev_copy(bcs, 4 * ps);
  void* e_out = NULL;
  HIP_OK(hipMalloc(&e_out, 2 * pq));
  if (rma_prefill_block(&st, 0, C, e_q, e_k, e_v, e_ck, e_cv, e_cs, d_wg, e_out, NULL) != RMA_OK)
    fail("rma_prefill_block");
  if (rma_admit(&st, 0, NULL) != RMA_OK) fail("rma_admit after the block");
  HIP_OK(hipMemcpy(bout, e_out, 2 * pq, hipMemcpyDeviceToHost));
  if (orc_prefill_block(&o, 0, C, bq, NULL, bk, bv, bck, bcv, bcs, wg, bref) != ORC_OK)
    fail("orc_prefill_block");
  if (orc_admit(&o, 0, NULL) != ORC_OK) fail("orc_admit after the block");
  const double eb = max_err(bout, bref, pq);
  if (!(eb <= kTol)) {
    fprintf(stderr, "prefill block: max error %.3e\n", eb);
    fail("prefill output");
  }

  /* the whole device history against the oracle's, bit for bit */
  unsigned char* h = malloc(bytes);
  HIP_OK(hipMemcpy(h, dbuf, bytes, hipMemcpyDeviceToHost));
  const int Rk = (int)lay.ring_k_slots;
  for (size_t u = 0; u < units; ++u) {
    const uint16_t* rk = (const uint16_t*)(h + lay.ring_k) + u * (size_t)Rk * D;
    const uint16_t* bkp = (const uint16_t*)(h + lay.bank_k) + u * (size_t)N * D;
    if (!k_plane_equal(rk, Rk, o.ring_k + u * R * D, R)) fail("ring K");
    if (!k_plane_equal(bkp, N, o.bank_k + u * N * D, N)) fail("bank K");
  }
  if (memcmp(h + lay.ring_v, o.ring_v, units * R * D * 2) != 0) fail("ring V");
  if (memcmp(h + lay.bank_v, o.bank_v, units * N * D * 2) != 0) fail("bank V");
  if (memcmp(h + lay.pend_k, o.pend_k, units * C * D * 2) != 0) fail("pending K");
  if (memcmp(h + lay.pend_v, o.pend_v, units * C * D * 2) != 0) fail("pending V");
  if (memcmp(h + lay.bscore, o.bscore, units * N * 4) != 0) fail("bank scores");
  if (memcmp(h + lay.bsrc, o.bsrc, units * N * 4) != 0) fail("bank source positions");
  if (memcmp(h + lay.pscore, o.pscore, units * C * 4) != 0) fail("pending scores");
  if (memcmp(h + lay.bank_n, o.bank_n, units * 4) != 0) fail("bank counts");
  if (st.t[0] != o.t[0] || st.pend_n[0] != o.pend_n[0]) fail("host counters");
  if (o.bank_n[0] != N) fail("the bank should be full after four blocks");

  printf("c abi parity ok: %d decode tokens (max error %.3e), %d-token prompt block "
         "(max error %.3e), 4 admits, history bit-exact\n",
         3 * C, worst, C, eb);
  return 0;
}
