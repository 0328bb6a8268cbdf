/*
 * RMA layer-step oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of what the Rock Memory Anchors (RMA)
 * attention-layer step computes, written from the EdgeRock pages:
 *   - EdgeRock model card (ModelScope), "How Rock Memory Anchors work"
 *     (history-component table and the paragraph after it), and
 *     "Constant history and GPU memory" (persistent-history table);
 *   - "EdgeRock-4B fixes its attention KV cache at 72 MiB" (ai-primer),
 *     the Write / Admit / Retrieve list and the memory table;
 *   - "EdgeRock-4B holds KV cache at 72 MiB ..." (tpsreport), "How it works".
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
 * load this library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code with it.
 *
 * Arithmetic: every float is widened exactly to double; dot products,
 * softmax, tanh and the gate are done in double.  bf16 values are raw
 * uint16 bit patterns.  No blocking, no reordering beyond the definition.
 *
 * State layout here is the natural one (independent of the GPU layout):
 *   ring_k, ring_v : [L][B][G][R][d]   bf16 bits
 *   bank_k, bank_v : [L][B][G][N][d]   bf16 bits
 *   bscore         : [L][B][G][N]      float
 *   bsrc           : [L][B][G][N]      int32 (source position of the record)
 *   bank_n         : [L][B][G]         int32 (committed records, dense prefix)
 *   pend_k, pend_v : [L][B][G][C][d]   bf16 bits
 *   pscore         : [L][B][G][C]      float
 *   t              : [L]               int64 (position of the next token)
 *   pend_n         : [L]               int32 (candidates pending, 0..C)
 * All buffers are owned by the caller.
 */
#ifndef RMA_ORACLE_H
#define RMA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t L;      /* RMA layers                                  */
  int32_t H;      /* query heads                                 */
  int32_t G;      /* KV groups; heads h share group h / (H/G)    */
  int32_t d;      /* head dimension                              */
  int32_t R;      /* ring slots (local window minus the current) */
  int32_t N;      /* anchor-bank capacity per group              */
  int32_t C;      /* pending slots = commit interval             */
  double scale;   /* softmax scale applied to q.k                */
  int32_t gate_group; /* 0: one gate per (token, head), w_g [H][d];
                         1: one gate per (token, KV group), w_g [G][d] */
} orc_cfg;

typedef struct {
  orc_cfg cfg;
  int32_t B;
  uint16_t *ring_k, *ring_v;
  uint16_t *bank_k, *bank_v;
  float *bscore;
  int32_t *bsrc;
  int32_t *bank_n;
  uint16_t *pend_k, *pend_v;
  float *pscore;
  int64_t *t;
  int32_t *pend_n;
} orc_state;

/* Return codes. */
#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_PENDING_FULL (-2)
#define ORC_E_NOT_BOUNDARY (-3)

/* One decode token for every sequence of layer `layer`.
 *   q     [B][H][d] bf16 (query of the local read)
 *   q_anchor [B][H][d] bf16 (query of the anchor read and the gate), or
 *         NULL: q
 *   k, v  [B][G][d] bf16 (current token)
 *   ck,cv [B][G][d] bf16 (candidate record)   cs [B][G] float (its score)
 *   w_g   [H][d] float (gate weights of this layer), or [G][d] with
 *         cfg.gate_group
 *   out   [B][H][d] double (unrounded output), may be NULL when
 *         compute_out == 0 (state update only).
 * Reads come first; then the ring write, the pending append, t += 1.
 * Returns ORC_E_PENDING_FULL when C candidates wait for an admit. */
int orc_decode_step(const orc_state* st, int32_t layer,
                    const uint16_t* q, const uint16_t* q_anchor, const uint16_t* k,
                    const uint16_t* v, const uint16_t* ck, const uint16_t* cv,
                    const float* cs, const float* w_g, double* out, int32_t compute_out);

/* Admit for layer `layer`; requires a full pending buffer (pend_n == C,
 * which happens at t % C == 0), else ORC_E_NOT_BOUNDARY.  `moved` [B][G] (may be NULL) receives the number of candidate
 * records copied into the bank per group. */
int orc_admit(const orc_state* st, int32_t layer, int32_t* moved);

/* A prefill block of n tokens (1..C) starting at a block boundary
 * (pend_n == 0, else ORC_E_NOT_BOUNDARY):
 * the tokens are decoded in order against the committed bank, with no
 * admit inside the block.  Shapes as orc_decode_step with a token axis
 * after the batch axis: q, q_anchor [B][n][H][d], k [B][n][G][d],
 * cs [B][n][G], out [B][n][H][d]. */
int orc_prefill_block(const orc_state* st, int32_t layer, int32_t n,
                      const uint16_t* q, const uint16_t* q_anchor, const uint16_t* k,
                      const uint16_t* v, const uint16_t* ck, const uint16_t* cv,
                      const float* cs, const float* w_g, double* out);

/* bf16 (round to nearest, ties to even) of a double, computed exactly. */
uint16_t orc_round_bf16(double x);
void orc_round_bf16_array(const double* x, uint16_t* y, int64_t n);

/* Threads OpenMP will use for the parallel loops. */
int orc_num_threads(void);
/* Threads for later parallel loops (n > 0; used to time the oracle on one
 * core).  Results do not depend on it. */
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
