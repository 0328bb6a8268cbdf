// Host side of librma.so: the C ABI declared in include/rma.h.
//
// Everything here is argument checking, state bookkeeping (for the
// lockstep calls the position, pending and bank counters of every layer
// are mirrored on the host; the per-sequence calls keep no host state) and
// kernel launches.  No arithmetic of the layer runs on the host.
#include "rma.h"

#include <cmath>
#include <cstring>

#include "rma_kernels.h"

namespace {

using rma::kD;
using rma::kHpg;
using rma::kMaxSplits;
using rma::kPart;
using rma::kTile;

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// RMA_OK, RMA_E_ARG (nonsense) or RMA_E_UNSUPPORTED (valid, not built for).
int check_config(const rma_config* c) {
  if (!c) return RMA_E_ARG;
  if (c->layers < 1 || c->layers > RMA_MAX_LAYERS || c->q_heads < 1 || c->kv_groups < 1 ||
      c->head_dim < 1 || c->window < 2 || c->bank_cap < 1 || c->commit < 1 ||
      !std::isfinite(c->scale) || c->q_heads % c->kv_groups != 0 ||
      (c->gate != RMA_GATE_HEAD && c->gate != RMA_GATE_GROUP))
    return RMA_E_ARG;
  if (c->head_dim != kD || c->q_heads != kHpg * c->kv_groups) return RMA_E_UNSUPPORTED;
  if (c->window > 4097 || c->commit > 256 || c->bank_cap + c->commit > 2048)
    return RMA_E_UNSUPPORTED;
  // A block's tokens must land in distinct ring slots, and each query of a
  // prefill block must have its whole local window inside the ring plus
  // the block's earlier tokens: the block is at most window - 1 tokens.
  if (c->commit > c->window - 1) return RMA_E_UNSUPPORTED;
  return RMA_OK;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }
int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K policy: every read (ring, bank) of a (sequence, group) unit is
// cut into s parts of whole 64-key tiles for the persistent attention
// kernel, whose 1,024 waves (256 CUs) take the parts round by round.  The
// split s (a power of two) minimises rounds x tiles per part, the time of
// the launch if every part costs its tiles; ties go to the smaller s (fewer
// partials to merge) except as noted below.  A function of the batch
// only, so that the scratch size is known before the first call.
struct Splits {
  int ring, bank, tiles_ring, tiles_bank;
};

Splits split_of(int tr, int tb, int s) {
  Splits r;
  r.tiles_ring = ceil_div(tr, s);
  r.tiles_bank = ceil_div(tb, s);
  // no part starts past the last tile
  r.ring = ceil_div(tr, r.tiles_ring);
  r.bank = ceil_div(tb, r.tiles_bank);
  return r;
}

Splits choose_splits(const rma_config* c, int32_t batch) {
  constexpr int64_t kWavesPerLaunch = 1024;
  const int64_t units = (int64_t)batch * c->kv_groups;
  const int tr = ceil_div(c->window - 1, kTile);
  const int tb = ceil_div(c->bank_cap, kTile);
  const int tmax = tr > tb ? tr : tb;
  Splits best = split_of(tr, tb, 1);
  int64_t best_cost = -1;
  for (int s = 1;; s *= 2) {
    const Splits r = split_of(tr, tb, s);
    const int64_t rounds = ceil_div64(units * (r.ring + r.bank), kWavesPerLaunch);
    const int64_t cost = rounds * (r.tiles_ring > r.tiles_bank ? r.tiles_ring : r.tiles_bank);
    // on a tie, one-tile parts (the small-batch part kernel) win while they
    // fill at most 4 rounds of 1,024 (measured faster up to 128 units, 2%
    // faster at 192, 6% slower at 256); otherwise the smaller split does
    const bool one_tile = r.tiles_ring == 1 && r.tiles_bank == 1 &&
                          units * (r.ring + r.bank) <= 4 * kWavesPerLaunch;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && one_tile)) {
      best = r;
      best_cost = cost;
    }
    if (s >= kMaxSplits || s >= tmax) break;
  }
  return best;
}

// Sequences left to the split launch when a hybrid decode launch gives
// the full rounds of 1,024 resident waves whole units (the rule of
// rma::decode_whole_prefix with MI355X's 1,024 waves), or 0.  The layout
// sizes its scratch for them; on a device with another wave count the
// launch checks the need against the scratch it has.
int32_t rest_batch(const rma_config* c, int32_t batch) {
  constexpr int64_t kWavesPerLaunch = 1024;
  const int64_t units = (int64_t)batch * c->kv_groups;
  if (units <= kWavesPerLaunch) return 0;
  const int64_t rounds = ceil_div64(units, kWavesPerLaunch);
  const int64_t last = units - (rounds - 1) * kWavesPerLaunch;
  if (last * 8 >= kWavesPerLaunch * 5) return 0;
  int64_t k = (rounds - 1) * kWavesPerLaunch;
  k -= k % c->kv_groups;
  return (int32_t)(batch - k / c->kv_groups);
}

int make_layout(const rma_config* c, int32_t batch, rma_layout* L) {
  std::memset(L, 0, sizeof(*L));
  const uint64_t units = (uint64_t)c->layers * batch * c->kv_groups;
  const uint64_t R = c->window - 1, N = c->bank_cap, C = c->commit, d = c->head_dim;
  const uint64_t rec_half = d * 2;  // bytes of K (or V) of one record
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L->ring_k = take(units * (uint64_t)rma::ring_k_slots((int)R) * rec_half);
  L->ring_v = take(units * R * rec_half);
  L->bank_k = take(units * N * rec_half);
  L->bank_v = take(units * N * rec_half);
  L->pend_k = take(units * C * rec_half);
  L->pend_v = take(units * C * rec_half);
  L->bscore = take(units * N * 4);
  L->bsrc = take(units * N * 4);
  L->pscore = take(units * C * 4);
  L->bank_n = take(units * 4);
  const Splits sp = choose_splits(c, batch);
  // split-K partials of the decode launch and, for small batches, of the
  // split prefill launch (never both at once: calls on a state are ordered)
  L->scratch_bytes = (uint64_t)batch * c->kv_groups * (sp.ring + sp.bank) * kPart * 4;
  // ... and of the split launch of the sequences a hybrid decode launch
  // leaves after its whole-unit rounds (rest_batch)
  const int32_t rb = rest_batch(c, batch);
  if (rb > 0) {
    const Splits sr = choose_splits(c, rb);
    const uint64_t r = (uint64_t)rb * c->kv_groups * (sr.ring + sr.bank) * kPart * 4;
    L->scratch_bytes = r > L->scratch_bytes ? r : L->scratch_bytes;
  }
  const rma::PrefillPlan pp = rma::prefill_plan(batch, c->kv_groups);
  if (pp.split()) {
    const uint64_t pf = (uint64_t)batch * c->commit * c->q_heads * pp.parts() * rma::kPfPart * 4;
    L->scratch_bytes = pf > L->scratch_bytes ? pf : L->scratch_bytes;
  }
  L->scratch = take(L->scratch_bytes);
  L->total_bytes = off;
  L->ring_k_slots = (uint64_t)rma::ring_k_slots((int)R);
  L->ring_bytes = units * R * rec_half * 2;
  L->bank_bytes = units * N * rec_half * 2;
  L->pend_bytes = units * C * rec_half * 2;
  L->meta_bytes = units * (N * 8 + C * 4 + 4);
  return RMA_OK;
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

int check_state(const rma_state* st, int32_t layer) {
  if (!st || !st->base) return RMA_E_ARG;
  const int rc = check_config(&st->cfg);
  if (rc != RMA_OK) return rc;
  if (layer < 0 || layer >= st->cfg.layers || st->batch < 1) return RMA_E_ARG;
  return RMA_OK;
}

template <typename T>
T* region(const rma_state* st, uint64_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(st->base) + off);
}

int hip_fail(rma_state* st, hipError_t e) {
  st->hip_error = (int32_t)e;
  return RMA_E_HIP;
}

// Fill the launch arguments of one token (or one token of a block) of a
// layer.  Token inputs are [B][...] slices with the given batch strides.
rma::DecodeArgs decode_args(const rma_state* st, int32_t layer, int64_t t, const void* q,
                            const void* k, const void* v, const void* ck, const void* cv,
                            const float* cs, const float* w_g, void* out, int64_t q_bs,
                            int64_t kv_bs, int64_t cs_bs, int64_t out_bs) {
  const rma_config& c = st->cfg;
  const rma_layout& L = st->layout;
  const int B = st->batch, G = c.kv_groups;
  const int R = c.window - 1, N = c.bank_cap, C = c.commit;
  const uint64_t unit0 = (uint64_t)layer * B * G;
  const Splits sp = choose_splits(&c, B);
  rma::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.qa = nullptr;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.ck = static_cast<const uint16_t*>(ck);
  a.cv = static_cast<const uint16_t*>(cv);
  a.cs = cs;
  a.w_g = w_g;
  a.out = static_cast<uint16_t*>(out);
  a.ring_k = region<uint16_t>(st, L.ring_k) + unit0 * rma::ring_k_slots(R) * kD;
  a.ring_v = region<uint16_t>(st, L.ring_v) + unit0 * R * kD;
  a.bank_k = region<uint16_t>(st, L.bank_k) + unit0 * N * kD;
  a.bank_v = region<uint16_t>(st, L.bank_v) + unit0 * N * kD;
  a.bank_n = region<int32_t>(st, L.bank_n) + unit0;
  a.bscore = region<float>(st, L.bscore) + unit0 * N;
  a.bsrc = region<int32_t>(st, L.bsrc) + unit0 * N;
  a.pend_k = region<uint16_t>(st, L.pend_k) + unit0 * C * kD;
  a.pend_v = region<uint16_t>(st, L.pend_v) + unit0 * C * kD;
  a.pscore = region<float>(st, L.pscore) + unit0 * C;
  a.part = region<float>(st, L.scratch);
  a.pos = nullptr;
  a.q_bs = q_bs;
  a.kv_bs = kv_bs;
  a.cs_bs = cs_bs;
  a.out_bs = out_bs;
  a.units = B * G;
  a.G = G;
  a.H = c.q_heads;
  a.R = R;
  a.Rk = rma::ring_k_slots(R);
  a.N = N;
  a.C = C;
  a.ring_count = (int)(t < R ? t : R);
  a.ring_slot = (int)(t % R);
  a.pend_slot = (int)(t % C);
  a.splits_ring = sp.ring;
  a.splits_bank = sp.bank;
  a.tiles_ring = sp.tiles_ring;
  a.tiles_bank = sp.tiles_bank;
  a.gate_group = c.gate == RMA_GATE_GROUP;
  a.sl2e = (float)((double)c.scale * 1.4426950408889634);
  return a;
}

// The decode of one layer's token as one or two launch_decode calls.  A
// batch whose whole units would leave a later round of the resident waves
// less than 5/8 full (rma::decode_whole_prefix) is decoded in two parts
// on the stream, one after the other: the sequences of the full rounds
// with the whole-unit launch (one unit per wave and round, nothing to
// merge), then the remaining sequences with the launch shape and split
// plan of their own batch.  The two parts touch disjoint units.  Where
// the remaining part's partials would exceed `scratch_cap`, the whole
// batch takes the single launch.
struct DecodePlan {
  rma::DecodeArgs head, rest;
  bool two;
};

DecodePlan plan_decode(const rma_state* st, const rma::DecodeArgs& a, uint64_t scratch_cap) {
  DecodePlan p;
  p.head = a;
  p.rest = a;
  p.two = false;
  const int k = rma::decode_whole_prefix(a);
  if (k <= 0 || k >= a.units) return p;
  const rma_config& c = st->cfg;
  const int G = a.G, b0 = k / G;
  const int64_t R = a.R, N = a.N, C = a.C, Rk = a.Rk;
  rma::DecodeArgs r = a;
  r.q += b0 * a.q_bs;
  if (r.qa) r.qa += b0 * a.q_bs;
  r.k += b0 * a.kv_bs;
  r.v += b0 * a.kv_bs;
  r.ck += b0 * a.kv_bs;
  r.cv += b0 * a.kv_bs;
  r.cs += b0 * a.cs_bs;
  r.out += b0 * a.out_bs;
  r.ring_k += (int64_t)k * Rk * kD;
  r.ring_v += (int64_t)k * R * kD;
  r.bank_k += (int64_t)k * N * kD;
  r.bank_v += (int64_t)k * N * kD;
  r.bank_n += k;
  r.bscore += (int64_t)k * N;
  r.bsrc += (int64_t)k * N;
  r.pend_k += (int64_t)k * C * kD;
  r.pend_v += (int64_t)k * C * kD;
  r.pscore += (int64_t)k * C;
  if (r.pos) r.pos += b0;
  r.units = a.units - k;
  const Splits sp = choose_splits(&c, r.units / G);
  r.splits_ring = sp.ring;
  r.splits_bank = sp.bank;
  r.tiles_ring = sp.tiles_ring;
  r.tiles_bank = sp.tiles_bank;
  if (rma::decode_scratch_bytes(r) > scratch_cap) return p;
  p.head.units = k;
  p.rest = r;
  p.two = true;
  return p;
}

// Partials the plan writes (the whole-unit head writes none).
uint64_t plan_scratch_bytes(const DecodePlan& p) {
  return p.two ? rma::decode_scratch_bytes(p.rest) : rma::decode_scratch_bytes(p.head);
}

hipError_t launch_plan(const DecodePlan& p, hipStream_t s) {
  const hipError_t e = rma::launch_decode(p.head, s);
  if (e != hipSuccess || !p.two) return e;
  return rma::launch_decode(p.rest, s);
}

rma::PrefillArgs prefill_args(const rma_state* st, int32_t layer, int32_t n_tokens, int64_t P,
                              const int32_t* pos, const void* q, const void* k, const void* v,
                              const void* ck, const void* cv, const float* cs,
                              const float* w_g, void* out) {
  const rma_config& c = st->cfg;
  const rma_layout& L = st->layout;
  const int B = st->batch, G = c.kv_groups;
  const int R = c.window - 1, N = c.bank_cap, C = c.commit;
  const uint64_t unit0 = (uint64_t)layer * B * G;
  rma::PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.qa = nullptr;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.ck = static_cast<const uint16_t*>(ck);
  a.cv = static_cast<const uint16_t*>(cv);
  a.cs = cs;
  a.w_g = w_g;
  a.out = static_cast<uint16_t*>(out);
  a.ring_k = region<uint16_t>(st, L.ring_k) + unit0 * rma::ring_k_slots(R) * kD;
  a.ring_v = region<uint16_t>(st, L.ring_v) + unit0 * R * kD;
  a.bank_k = region<uint16_t>(st, L.bank_k) + unit0 * N * kD;
  a.bank_v = region<uint16_t>(st, L.bank_v) + unit0 * N * kD;
  a.bank_n = region<int32_t>(st, L.bank_n) + unit0;
  a.pend_k = region<uint16_t>(st, L.pend_k) + unit0 * C * kD;
  a.pend_v = region<uint16_t>(st, L.pend_v) + unit0 * C * kD;
  a.pscore = region<float>(st, L.pscore) + unit0 * C;
  a.part = region<float>(st, L.scratch);
  a.pos = pos;
  const rma::PrefillPlan plan = rma::prefill_plan(B, G);
  a.pf_loc = plan.loc;
  a.pf_bank = plan.bank;
  a.B = B;
  a.G = G;
  a.H = c.q_heads;
  a.R = R;
  a.Rk = rma::ring_k_slots(R);
  a.N = N;
  a.C = C;
  a.n = n_tokens;
  a.P = P;
  a.gate_group = c.gate == RMA_GATE_GROUP;
  a.sl2e = (float)((double)c.scale * 1.4426950408889634);
  return a;
}

rma::AdmitArgs admit_args(const rma_state* st) {
  const rma_config& c = st->cfg;
  const rma_layout& L = st->layout;
  rma::AdmitArgs a;
  a.bank_k = region<uint16_t>(st, L.bank_k);
  a.bank_v = region<uint16_t>(st, L.bank_v);
  a.bscore = region<float>(st, L.bscore);
  a.bsrc = region<int32_t>(st, L.bsrc);
  a.bank_n = region<int32_t>(st, L.bank_n);
  a.pend_k = region<const uint16_t>(st, L.pend_k);
  a.pend_v = region<const uint16_t>(st, L.pend_v);
  a.pscore = region<const float>(st, L.pscore);
  a.N = c.bank_cap;
  a.C = c.commit;
  a.unit0 = 0;
  a.units = 0;
  a.block_start = 0;
  a.pos = nullptr;
  a.G = c.kv_groups;
  a.pos_add = 0;
  a.aligned_only = 0;
  return a;
}

// The admit launch of the per-sequence calls: every unit of the layer
// whose sequence's last written token (pos[b] + pos_add) completes a block.
hipError_t admit_at(const rma_state* st, int32_t layer, const int32_t* pos, int pos_add,
                    int aligned_only, hipStream_t s) {
  rma::AdmitArgs a = admit_args(st);
  const int BG = st->batch * st->cfg.kv_groups;
  a.unit0 = layer * BG;
  a.units = BG;
  a.pos = pos;
  a.pos_add = pos_add;
  a.aligned_only = aligned_only;
  return rma::launch_admit(a, s);
}

bool aligned4(const void* p) { return p && ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" {

int rma_config_default(rma_config* cfg) {
  if (!cfg) return RMA_E_ARG;
  cfg->layers = 8;
  cfg->q_heads = 16;
  cfg->kv_groups = 4;
  cfg->head_dim = 256;
  cfg->window = 1024;
  cfg->bank_cap = 1024;
  cfg->commit = 256;
  cfg->scale = 0.0625f;
  cfg->gate = RMA_GATE_HEAD;
  return RMA_OK;
}

size_t rma_state_bytes(const rma_config* cfg, int32_t batch) {
  if (check_config(cfg) != RMA_OK || batch < 1) return 0;
  rma_layout L;
  make_layout(cfg, batch, &L);
  return (size_t)L.total_bytes;
}

int rma_state_layout(const rma_config* cfg, int32_t batch, rma_layout* out) {
  if (!out || batch < 1) return RMA_E_ARG;
  const int rc = check_config(cfg);
  if (rc != RMA_OK) return rc;
  return make_layout(cfg, batch, out);
}

int rma_state_init(rma_state* st, const rma_config* cfg, int32_t batch, void* dev_buf,
                   size_t bytes, int64_t start_pos, int32_t bank_n, void* stream) {
  if (!st || !dev_buf || batch < 1 || start_pos < 0 || start_pos > RMA_MAX_POS) return RMA_E_ARG;
  const int rc = check_config(cfg);
  if (rc != RMA_OK) return rc;
  if (((uintptr_t)dev_buf % kAlign) != 0) return RMA_E_ARG;
  if (bank_n < 0 || bank_n > cfg->bank_cap) return RMA_E_ARG;
  rma_layout L;
  make_layout(cfg, batch, &L);
  if (bytes < L.total_bytes) return RMA_E_ARG;
  rma_state s;
  std::memset(&s, 0, sizeof(s));
  s.cfg = *cfg;
  s.batch = batch;
  s.base = dev_buf;
  s.bytes = bytes;
  s.layout = L;
  for (int l = 0; l < cfg->layers; ++l) {
    s.t[l] = start_pos;
    s.bank_n[l] = bank_n;
    s.pend_n[l] = (int32_t)(start_pos % cfg->commit);
  }
  const int64_t units = (int64_t)cfg->layers * batch * cfg->kv_groups;
  const hipError_t e = rma::launch_fill_i32(region<int32_t>(&s, L.bank_n), bank_n, units,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    st->hip_error = (int32_t)e;
    return RMA_E_HIP;
  }
  *st = s;
  return RMA_OK;
}

int rma_decode_step(rma_state* st, int32_t layer, const void* q, const void* k, const void* v,
                    const void* cand_k, const void* cand_v, const float* cand_score,
                    const float* w_g, void* out, void* stream) {
  int rc = check_state(st, layer);
  if (rc != RMA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cand_k) ||
      !aligned16(cand_v) || !cand_score || !w_g || !aligned16(out))
    return RMA_E_ARG;
  const rma_config& c = st->cfg;
  if (st->pend_n[layer] >= c.commit) return RMA_E_PENDING_FULL;
  const int64_t t = st->t[layer];
  if (t > RMA_MAX_POS) return RMA_E_ARG;
  const int64_t H = c.q_heads, G = c.kv_groups;
  const rma::DecodeArgs a = decode_args(st, layer, t, q, k, v, cand_k, cand_v, cand_score, w_g,
                                        out, H * kD, G * kD, G, H * kD);
  const hipError_t e =
      launch_plan(plan_decode(st, a, st->layout.scratch_bytes), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e);
  st->t[layer] = t + 1;
  st->pend_n[layer] += 1;
  return RMA_OK;
}

int rma_prefill_block(rma_state* st, int32_t layer, int32_t n_tokens, const void* q,
                      const void* k, const void* v, const void* cand_k, const void* cand_v,
                      const float* cand_score, const float* w_g, void* out, void* stream) {
  int rc = check_state(st, layer);
  if (rc != RMA_OK) return rc;
  const rma_config& c = st->cfg;
  if (n_tokens < 1 || n_tokens > c.commit) return RMA_E_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cand_k) ||
      !aligned16(cand_v) || !cand_score || !w_g || !aligned16(out))
    return RMA_E_ARG;
  const int64_t t0 = st->t[layer];
  if (st->pend_n[layer] != 0 || t0 % c.commit != 0) return RMA_E_NOT_BOUNDARY;
  if (t0 + n_tokens - 1 > RMA_MAX_POS) return RMA_E_ARG;
  const rma::PrefillArgs a = prefill_args(st, layer, n_tokens, t0, nullptr, q, k, v, cand_k,
                                          cand_v, cand_score, w_g, out);
  const hipError_t e = rma::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e);
  st->t[layer] = t0 + n_tokens;
  st->pend_n[layer] = n_tokens;
  return RMA_OK;
}

int rma_admit(rma_state* st, int32_t layer, void* stream) {
  if (!st) return RMA_E_ARG;
  const int lo = layer == -1 ? 0 : layer;
  const int hi = layer == -1 ? st->cfg.layers : layer + 1;
  int rc = check_state(st, lo);
  if (rc != RMA_OK) return rc;
  if (layer < -1 || hi > st->cfg.layers) return RMA_E_ARG;
  const rma_config& c = st->cfg;
  for (int l = lo; l < hi; ++l)
    if (st->pend_n[l] != c.commit || st->t[l] % c.commit != 0) return RMA_E_NOT_BOUNDARY;
  const int BG = st->batch * c.kv_groups;
  rma::AdmitArgs a = admit_args(st);
  // one launch over consecutive layers at the same position
  int l = lo;
  while (l < hi) {
    int e_end = l + 1;
    while (e_end < hi && st->t[e_end] == st->t[l]) ++e_end;
    a.unit0 = l * BG;
    a.units = (e_end - l) * BG;
    a.block_start = st->t[l] - c.commit;
    const hipError_t e = rma::launch_admit(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(st, e);
    for (int x = l; x < e_end; ++x) {
      const int nn = st->bank_n[x] + c.commit;
      st->bank_n[x] = nn < c.bank_cap ? nn : c.bank_cap;
      st->pend_n[x] = 0;
    }
    l = e_end;
  }
  return RMA_OK;
}

int rma_decode_step_at(rma_state* st, int32_t layer, const int32_t* pos, const void* q,
                       const void* q_anchor, const void* k, const void* v, const void* cand_k,
                       const void* cand_v, const float* cand_score, const float* w_g, void* out,
                       void* stream) {
  int rc = check_state(st, layer);
  if (rc != RMA_OK) return rc;
  if (!aligned4(pos) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cand_k) ||
      !aligned16(cand_v) || !cand_score || !w_g || !aligned16(out) ||
      (q_anchor && !aligned16(q_anchor)))
    return RMA_E_ARG;
  const rma_config& c = st->cfg;
  const int64_t H = c.q_heads, G = c.kv_groups;
  rma::DecodeArgs a = decode_args(st, layer, 0, q, k, v, cand_k, cand_v, cand_score, w_g, out,
                                  H * kD, G * kD, G, H * kD);
  a.pos = pos;
  a.qa = static_cast<const uint16_t*>(q_anchor);
  const hipError_t e =
      launch_plan(plan_decode(st, a, st->layout.scratch_bytes), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e);
  return RMA_OK;
}

int rma_decode_step_at_static(rma_state* st, int32_t layer, const int32_t* pos, const void* q,
                              const void* q_anchor, const void* k, const void* v,
                              const void* cand_k, const void* cand_v, const float* cand_score,
                              const float* w_g, void* out, void* stream) {
  int rc = check_state(st, layer);
  if (rc != RMA_OK) return rc;
  if (!aligned4(pos) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cand_k) ||
      !aligned16(cand_v) || !cand_score || !w_g || !aligned16(out) ||
      (q_anchor && !aligned16(q_anchor)))
    return RMA_E_ARG;
  const rma_config& c = st->cfg;
  const int64_t H = c.q_heads, G = c.kv_groups;
  rma::DecodeArgs a = decode_args(st, layer, 0, q, k, v, cand_k, cand_v, cand_score, w_g, out,
                                  H * kD, G * kD, G, H * kD);
  a.pos = pos;
  a.qa = static_cast<const uint16_t*>(q_anchor);
  // the partials go to the library's static array of the state's device
  // instead of the state's scratch region; nothing is allocated
  DecodePlan p = plan_decode(st, a, rma::kStaticScratchBytes);
  if (plan_scratch_bytes(p) > rma::kStaticScratchBytes) return RMA_E_SCRATCH;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, st->base);
  if (e != hipSuccess) return hip_fail(st, e);
  float* part = nullptr;
  e = rma::static_scratch(attr.device, &part);
  if (e != hipSuccess) return hip_fail(st, e);
  p.head.part = part;
  p.rest.part = part;
  e = launch_plan(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e);
  return RMA_OK;
}

int rma_prefill_block_at(rma_state* st, int32_t layer, int32_t n_tokens, const int32_t* pos,
                         const void* q, const void* q_anchor, const void* k, const void* v,
                         const void* cand_k, const void* cand_v, const float* cand_score,
                         const float* w_g, void* out, void* stream) {
  int rc = check_state(st, layer);
  if (rc != RMA_OK) return rc;
  const rma_config& c = st->cfg;
  if (n_tokens < 1 || n_tokens > c.commit) return RMA_E_ARG;
  if (!aligned4(pos) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(cand_k) ||
      !aligned16(cand_v) || !cand_score || !w_g || !aligned16(out) ||
      (q_anchor && !aligned16(q_anchor)))
    return RMA_E_ARG;
  rma::PrefillArgs a = prefill_args(st, layer, n_tokens, 0, pos, q, k, v, cand_k, cand_v,
                                    cand_score, w_g, out);
  a.qa = static_cast<const uint16_t*>(q_anchor);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = rma::launch_prefill(a, s);
  // only a full block can complete one (its start is a multiple of C)
  if (e == hipSuccess && n_tokens == c.commit) e = admit_at(st, layer, pos, n_tokens - 1, 1, s);
  if (e != hipSuccess) return hip_fail(st, e);
  return RMA_OK;
}

int rma_seq_reset(rma_state* st, int32_t first, int32_t count, int32_t bank_n, void* stream) {
  int rc = check_state(st, 0);
  if (rc != RMA_OK) return rc;
  if (first < 0 || count < 1 || first > st->batch - count || bank_n < 0 ||
      bank_n > st->cfg.bank_cap)
    return RMA_E_ARG;
  const hipError_t e = rma::launch_seq_bank_n(region<int32_t>(st, st->layout.bank_n),
                                              st->cfg.layers, st->batch, st->cfg.kv_groups,
                                              first, count, bank_n,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(st, e);
  return RMA_OK;
}

const char* rma_strerror(int status) {
  switch (status) {
    case RMA_OK: return "ok";
    case RMA_E_ARG: return "invalid argument (null or misaligned pointer, bad size or index)";
    case RMA_E_PENDING_FULL: return "pending buffer full: admit before the next decode step";
    case RMA_E_NOT_BOUNDARY: return "not at a block boundary";
    case RMA_E_HIP: return "HIP launch failed";
    case RMA_E_UNSUPPORTED: return "geometry not supported by the kernels";
    case RMA_E_SCRATCH:
      return "the call's split-K partials exceed the library's static scratch array "
             "(RMA_STATIC_SCRATCH_BYTES); use rma_decode_step_at";
    default: return "unknown status";
  }
}

}  // extern "C"
