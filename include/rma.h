/*
 * rma.h - C ABI of librma.so, the Rock Memory Anchors (RMA) attention-layer
 * step on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (EdgeRock model card on ModelScope, section
 * "How Rock Memory Anchors work" and its history-component table; the
 * ai-primer story "EdgeRock-4B fixes its attention KV cache at 72 MiB",
 * list of the three operations Write / Admit / Retrieve):
 *
 *   per sequence, per RMA layer, per KV group g, a fixed-capacity history:
 *     ring     : the K/V of the R = window-1 preceding positions
 *     bank     : up to N committed anchor records (K, V, score, source pos)
 *     pending  : the C candidate records of the current block (K, V, score)
 *
 *   decode of the token at position t, query head h of group g:
 *     o_local  = softmax attention over ring positions max(0,t-R) .. t-1
 *                plus the current token (the local window of R+1 positions)
 *     o_anchor = softmax attention over committed bank slots 0 .. n-1
 *                (zero when n == 0)
 *     out      = o_local + tanh(q_h . w_g[h]) * o_anchor
 *   then the token's K/V replaces ring slot t mod R and its candidate
 *   record and score go to pending slot t mod C.
 *
 *   admit, once C candidates are pending: the n anchors and C candidates
 *   of each (sequence, layer, group) compete; the first min(N, n + C) in
 *   the order (score descending, then global index ascending; anchors have
 *   global index = slot, candidates N + pending slot; -0.0 == +0.0; NaN
 *   below -inf) are kept.  Evicted anchor slots, ascending, receive the
 *   admitted candidates in ascending pending order; the remainder is
 *   appended after slot n-1.  Retained records are not touched.  Reads of
 *   the bank see an admitted record only from the next block on.
 *
 * The gate form, the tie-break and the compaction order are readings of
 * the pages: they name a query-dependent signed gate, keep the records of
 * highest priority and leave kept records as they are, without fixing
 * these details (model card, "How Rock Memory Anchors work").
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as `const void*` to 16-bit IEEE bfloat16
 *     values; fp32 as `float*`.  All tensor pointers are DEVICE pointers,
 *     16-byte aligned, C-contiguous, owned by the caller, and must stay
 *     valid until the work on `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *     work and return; nothing is synchronous.  Device-side conditions are
 *     never reported back; argument and sequencing errors are detected on
 *     the host before anything is enqueued, and leave the state unchanged.
 *   - The library allocates no memory.  The caller owns the rma_state
 *     struct and one device buffer holding the whole state (its size from
 *     rma_state_bytes).
 *   - Calls on one state must be ordered: issue them from one host
 *     thread, on one stream (or order the streams with events).  They
 *     share the state's scratch region and the host mirror in rma_state,
 *     so calls on one state that overlap race.  Distinct states are
 *     independent.
 *   - The lockstep calls (rma_decode_step, rma_prefill_block, rma_admit)
 *     move a batch together: all sequences of a layer share the position
 *     t, which the host mirrors in rma_state.  The per-sequence calls
 *     (the _at calls below) take each sequence's position from device
 *     memory instead.
 *   - Kernels support head_dim 256 and 4 query heads per KV group (the
 *     EdgeRock geometry); other shapes return RMA_E_UNSUPPORTED.
 */
#ifndef RMA_H
#define RMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMA_MAX_LAYERS 64

/* Status codes. */
#define RMA_OK 0
#define RMA_E_ARG (-1)          /* null/misaligned pointer, bad size or index */
#define RMA_E_PENDING_FULL (-2) /* decode with C candidates pending, no admit */
#define RMA_E_NOT_BOUNDARY (-3) /* admit with < C pending; prefill off a block start */
#define RMA_E_HIP (-4)          /* a HIP launch failed; code in rma_state.hip_error */
#define RMA_E_UNSUPPORTED (-5)  /* geometry the kernels are not built for */
#define RMA_E_SCRATCH (-6)      /* partials beyond RMA_STATIC_SCRATCH_BYTES */

/* Layer geometry.  EdgeRock values (rma_config_default): 8 layers,
 * 16 query heads, 4 KV groups, head_dim 256, window 1024 (ring 1023),
 * bank_cap 1024, commit 256, scale 1/16 (model card history-component
 * table; Rock Matrix models page spec list; head_dim from the card's
 * persistent-history MiB table), gate per head.  Limits: 1 <= layers <= RMA_MAX_LAYERS,
 * q_heads == 4 * kv_groups, head_dim == 256, 2 <= window <= 4097,
 * 1 <= bank_cap, 1 <= commit <= 256, commit <= window - 1 (a block's
 * tokens take distinct ring slots), bank_cap + commit <= 2048. */
typedef struct {
  int32_t layers;
  int32_t q_heads;
  int32_t kv_groups;
  int32_t head_dim;
  int32_t window;    /* local window incl. the current token; ring = window-1 */
  int32_t bank_cap;  /* N: committed anchors per (sequence, layer, group) */
  int32_t commit;    /* C: pending slots = tokens between admits */
  float scale;       /* softmax scale on q.k, normally 1/sqrt(head_dim) */
  int32_t gate;      /* RMA_GATE_HEAD or RMA_GATE_GROUP (below) */
} rma_config;

/* Gate granularity (rma_config.gate).  RMA_GATE_HEAD: one gate per (token,
 * query head), tanh(qa_h . w_g[h]), w_g [q_heads][head_dim].
 * RMA_GATE_GROUP: one gate per (token, KV group) shared by the group's
 * heads, tanh(mean of the group's qa_h . w_g[g]), w_g [kv_groups][head_dim]
 * (a reading of the models page's and tpsreport's "separate RMA modules",
 * whose selection is per KV group; the pages fix no gate form).  qa is the
 * anchor query where a call takes one, else q. */
#define RMA_GATE_HEAD 0
#define RMA_GATE_GROUP 1

/* Byte offsets of the regions inside the state buffer.  Every region is
 * indexed by unit u = (layer * batch + b) * kv_groups + g first, and is
 * 256-byte aligned.  R = window-1, N = bank_cap, C = commit, d = head_dim.
 *
 *   ring_k  [units][d/8][Rk][8] bf16  K, split in 16-byte chunks of 8 dims,
 *                                     chunk-major: chunk c of slot s is at
 *                                     uint4 index c*Rk + s of the unit's
 *                                     plane; Rk = R rounded up to a multiple
 *                                     of 64 (ring_k_slots below; slots R ..
 *                                     Rk-1 are alignment padding, never read
 *                                     or written)
 *   ring_v  [units][R][d]      bf16   V rows
 *   bank_k  [units][d/8][N][8] bf16   as ring_k with N slots
 *   bank_v  [units][N][d]      bf16
 *   pend_k  [units][C][d]      bf16   K rows of pending candidates
 *   pend_v  [units][C][d]      bf16
 *   bscore  [units][N]         f32    score of each committed anchor
 *   bsrc    [units][N]         i32    source position of each anchor
 *   pscore  [units][C]         f32    score of each pending candidate
 *   bank_n  [units]            i32    committed anchors (dense prefix)
 *   scratch                           split-K partials of the decode and of the
 *                                     small-batch prefill, library-private
 */
typedef struct {
  uint64_t ring_k, ring_v, bank_k, bank_v, pend_k, pend_v;
  uint64_t bscore, bsrc, pscore, bank_n, scratch;
  uint64_t scratch_bytes;
  uint64_t total_bytes;
  uint64_t ring_bytes, bank_bytes, pend_bytes, meta_bytes; /* K+V+metadata totals
                                                             (records, without padding) */
  uint64_t ring_k_slots;        /* Rk: slots of a ring K plane */
} rma_layout;

/* Caller-owned state handle.  Plain data; copy it to snapshot the host
 * counters (together with a copy of the device buffer).  Fields are read
 * by the library and updated only by the calls below. */
typedef struct {
  rma_config cfg;
  int32_t batch;
  int32_t hip_error;            /* last HIP error code seen (0 = none) */
  void* base;                   /* device state buffer */
  uint64_t bytes;               /* its size */
  rma_layout layout;
  int64_t t[RMA_MAX_LAYERS];    /* next position per layer */
  int32_t bank_n[RMA_MAX_LAYERS]; /* committed anchors per layer (same in
                                     every sequence and group) */
  int32_t pend_n[RMA_MAX_LAYERS]; /* pending candidates per layer */
} rma_state;

/* Fill *cfg with the EdgeRock geometry.  Returns RMA_OK, or RMA_E_ARG for
 * a null pointer. */
int rma_config_default(rma_config* cfg);

/* Bytes of device memory a state for `batch` sequences needs (capacity
 * planning before inference starts; the model card's FAQ and the
 * tpsreport "What this means" paragraph note that fixed per-sequence
 * memory can be computed up front).  Returns 0 for an invalid config or
 * batch < 1. */
size_t rma_state_bytes(const rma_config* cfg, int32_t batch);

/* Region offsets for `batch` sequences: where the ring, bank, pending and
 * metadata records of every (layer, sequence, group) sit in the state
 * buffer (the record sizes are those of the model card's persistent-history
 * table, section "Constant history and GPU memory": 31.97 MiB of local KV,
 * 32.00 MiB of anchors, 8.00 MiB of pending candidates per sequence, plus
 * metadata).  Fills *out; the caller owns it.  Returns RMA_OK, RMA_E_ARG
 * (null out, batch < 1) or RMA_E_UNSUPPORTED; *out is unspecified on
 * error. */
int rma_state_layout(const rma_config* cfg, int32_t batch, rma_layout* out);

/* Token positions run from 0 to RMA_MAX_POS: source positions are kept as
 * int32 (bsrc), and the per-sequence calls take int32 positions. */
#define RMA_MAX_POS ((int64_t)2147483647)

/* Bind `dev_buf` (at least rma_state_bytes bytes, 256-byte aligned) to
 * *st and start every layer at position `start_pos` (0 .. RMA_MAX_POS)
 * with `bank_n`
 * committed anchors (0 <= bank_n <= bank_cap) and start_pos % commit
 * pending candidates.  The history's memory is fixed before inference and
 * allocated once (tpsreport, "What this means"): this call takes the
 * caller's buffer and nothing is allocated later.  Enqueues a write of the
 * device bank counts; record contents, scores and source positions are
 * left as they are (the caller fills them through the layout, or starts
 * from an empty history).  The caller keeps ownership of dev_buf and *st.
 * Returns RMA_OK, RMA_E_ARG (null pointer, misaligned or short buffer,
 * bad position or bank count; *st unchanged), RMA_E_UNSUPPORTED, or
 * RMA_E_HIP (the count write failed to launch; st->hip_error set). */
int rma_state_init(rma_state* st, const rma_config* cfg, int32_t batch,
                   void* dev_buf, size_t bytes, int64_t start_pos,
                   int32_t bank_n, void* stream);

/* Decode one token of layer `layer` for all sequences (Retrieve, then
 * Write; ai-primer three-operation list, items 1 and 3):
 *   q          [batch][q_heads][head_dim]   bf16  query of the token
 *   k, v       [batch][kv_groups][head_dim] bf16  the token's own K/V
 *   cand_k/v   [batch][kv_groups][head_dim] bf16  its candidate record
 *   cand_score [batch][kv_groups]           f32   the candidate's score
 *   w_g        [q_heads][head_dim]          f32   gate weights of the layer
 *                                                 ([kv_groups][head_dim] with
 *                                                 cfg.gate == RMA_GATE_GROUP)
 *   out        [batch][q_heads][head_dim]   bf16  result
 * Returns RMA_E_PENDING_FULL (state unchanged) when C candidates are
 * pending; call rma_admit first; RMA_E_ARG (state unchanged) when the
 * token's position would pass RMA_MAX_POS. */
int rma_decode_step(rma_state* st, int32_t layer, const void* q, const void* k,
                    const void* v, const void* cand_k, const void* cand_v,
                    const float* cand_score, const float* w_g, void* out,
                    void* stream);

/* A chunked-prefill block of `n_tokens` (1 .. commit) consecutive tokens
 * of layer `layer`, starting at a block boundary (no candidates pending).
 * Same result as that many rma_decode_step calls: each query attends to
 * its causal local window over the ring and the earlier tokens of the
 * block, and to the bank committed before the block; the block's own
 * candidates are readable only after the admit at its end (model card,
 * "How Rock Memory Anchors work": reads use the committed bank, and new
 * selections become visible in the next block).  Shapes as in
 * rma_decode_step with a token axis after the batch axis:
 *   q [batch][n][q_heads][d], k/v/cand_k/cand_v [batch][n][kv_groups][d],
 *   cand_score [batch][n][kv_groups], out [batch][n][q_heads][d].
 * Returns RMA_E_NOT_BOUNDARY when t % commit != 0 or candidates pend;
 * RMA_E_ARG when the block's last position would pass RMA_MAX_POS. */
int rma_prefill_block(rma_state* st, int32_t layer, int32_t n_tokens,
                      const void* q, const void* k, const void* v,
                      const void* cand_k, const void* cand_v,
                      const float* cand_score, const float* w_g, void* out,
                      void* stream);

/* Admit for layer `layer`, or for every layer when layer == -1 (Admit;
 * ai-primer list item 2, tpsreport "How it works").  Every selected
 * layer must hold exactly C pending candidates, else RMA_E_NOT_BOUNDARY
 * and nothing is enqueued. */
int rma_admit(rma_state* st, int32_t layer, void* stream);

/* ---- Per-sequence positions ------------------------------------------
 * The calls above move a batch in lockstep, with the positions mirrored on
 * the host.  The three calls below serve batches whose sequences stand at
 * different positions (continuous batching: a sequence joins, idles or
 * leaves without the others), and need no host bookkeeping per call, so a
 * whole token step can be captured once in a HIP graph and replayed (the
 * EdgeRock model card, section "Inference efficiency", credits CUDA Graphs
 * for part of its decode speed).  Each sequence follows the same method as above; only
 * where the positions live differs:
 *   pos  [batch] int32, DEVICE memory, 4-byte aligned, read when the work
 *        runs (so a graph replays with whatever pos holds then).
 *        pos[b] >= 0: sequence b takes part, at that position;
 *        pos[b] <  0: sequence b is left out: nothing of its state is read
 *        or written and its rows of `out` are not written.
 * A sequence's block is admitted by the call that writes its last
 * candidate (the token at a position p with (p + 1) % commit == 0), after
 * that call's reads, exactly as rma_admit would.  These calls neither read
 * nor update the host counters t, pend_n and bank_n of rma_state: the
 * device bank counts are the truth, and the caller owns the positions
 * (advancing pos by one after each token, e.g. with a kernel captured in
 * the same graph).  Mixing them with the lockstep calls on one state is
 * the caller's business: the lockstep calls trust the host counters.
 * A sequence that starts at a position that is not a multiple of commit
 * finds pending slots below it as they are in the buffer (as after
 * rma_state_init).  Device-side conditions are not reported; a position
 * the kernels cannot honour leaves the sequence out as documented per
 * call. */

/* Decode one token for every sequence b with pos[b] >= 0, at position
 * pos[b]; tensors as in rma_decode_step.  Then admits the blocks these
 * tokens complete.
 *   q_anchor  [batch][q_heads][head_dim] bf16, or NULL.  A separate query
 *             for the anchor read and the gate: o_anchor attends with
 *             q_anchor[h] and the gate is tanh(q_anchor[h] . w_g[h]); the
 *             local read keeps q.  NULL: q serves both reads, as in
 *             rma_decode_step.  (Reading of the model card's "separate RMA
 *             modules" and query-dependent read, section "How Rock Memory
 *             Anchors work"; the pages fix neither the query's source nor
 *             the gate's input.)
 * Returns RMA_OK, RMA_E_ARG or RMA_E_HIP. */
int rma_decode_step_at(rma_state* st, int32_t layer, const int32_t* pos, const void* q,
                       const void* q_anchor, const void* k, const void* v, const void* cand_k,
                       const void* cand_v, const float* cand_score, const float* w_g, void* out,
                       void* stream);

/* A prefill block of n_tokens (1 .. commit) for every sequence b whose
 * pos[b] is >= 0 and a multiple of commit (the block's first position);
 * other sequences are left out.  Tensors as in rma_prefill_block;
 * q_anchor [batch][n][q_heads][head_dim] or NULL, as in
 * rma_decode_step_at.  A full block (n_tokens == commit) is admitted by
 * the same call.  Returns RMA_OK, RMA_E_ARG or RMA_E_HIP. */
int rma_prefill_block_at(rma_state* st, int32_t layer, int32_t n_tokens, const int32_t* pos,
                         const void* q, const void* q_anchor, const void* k, const void* v,
                         const void* cand_k, const void* cand_v, const float* cand_score,
                         const float* w_g, void* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * rma_decode_step_at with the same arguments, results and admits, whose
 * split-K partials (the small-batch launches) go to a static device array
 * of RMA_STATIC_SCRATCH_BYTES instead of the state's scratch region.  The
 * library holds one such array on every GPU it runs on, from the first
 * call on that GPU until the process ends; the call itself allocates
 * nothing.  Every call on a GPU shares that GPU's array, so calls that
 * overlap on one GPU (other streams, other states) race: order them.  The
 * kernels write every partial before reading it; nothing needs clearing.
 * Returns RMA_E_SCRATCH, before anything is enqueued, when the batch's
 * partials would exceed the array; otherwise as rma_decode_step_at.  On
 * MI355X the array holds the partials of every configuration and batch
 * the library accepts: a split launch covers fewer than 640 units, at
 * most 32 partials of 4,128 B each, and the largest need, 76.6 MiB, is
 * the EdgeRock geometry's at batch 152 (and at 408, 664, ..., whose
 * second launch is that batch).  The check guards the bound. */
#define RMA_STATIC_SCRATCH_BYTES ((size_t)80 << 20)
int rma_decode_step_at_static(rma_state* st, int32_t layer, const int32_t* pos, const void* q,
                              const void* q_anchor, const void* k, const void* v,
                              const void* cand_k, const void* cand_v, const float* cand_score,
                              const float* w_g, void* out, void* stream);

/* Give sequences first .. first+count-1 (every layer and group) a bank of
 * `bank_n` committed anchors (0 for a new sequence in a reused batch slot;
 * a new sequence's ring needs no clearing, the position decides which
 * slots are read).  Enqueued on `stream`.  Returns RMA_OK, RMA_E_ARG or
 * RMA_E_HIP. */
int rma_seq_reset(rma_state* st, int32_t first, int32_t count, int32_t bank_n, void* stream);

/* Static text for a status code. */
const char* rma_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* RMA_H */
