// Chunked prefill of the RMA layer on gfx950: a block of n <= 256 tokens
// starting at a block boundary P, every query against its causal local
// window (ring positions P-R .. P-1 and the block's earlier tokens) and the
// bank committed before the block, merged by the signed gate; then the
// block's ring writes and pending fill.
//
// Semantics: EdgeRock model card (ModelScope), "How Rock Memory Anchors
// work" (1,024-position local window; reads use the committed bank, newly
// selected records become visible in the next block) and the
// persistent-history table note (ring of 1,023 preceding positions plus the
// current token).  Reading: the block gives the same result as decoding
// its tokens one by one, since admission waits for the block's end.
//
// The block is a dense contraction, so it runs on MFMA:
// v_mfma_f32_16x16x32_bf16 (A: lane l holds row l%16, k = 8*(l/16)+j;
// B: column l%16, same k; D: register i holds row 4*(l/16)+i, column l%16).
// One 8-wave workgroup per (sequence, group, tile of 32 tokens); each wave
// owns 16 queries (4 tokens x 4 heads), one per MFMA column, so a lane
// holds one query throughout.
//  * Scores are computed transposed, S^T = K Q^T (A = 16 keys x 32 dims of
//    the staged K tile, B = the wave's Q^T in registers), which leaves each
//    lane's probabilities exactly where the B operand of O^T = V^T P^T
//    wants them: P never leaves registers.
//  * Every 32-key tile of K and V is staged once per workgroup in LDS
//    (double-buffered, rows padded against bank conflicts); the V^T operand is read
//    with ds_read_b64_tr_b16, the gfx950 LDS transpose read, straight from
//    the row-major V rows.
//  * Online softmax in the log2 domain; local and anchor reads separately
//    normalised, then out = o_local + tanh(q . w_g) * o_anchor.
//  * Small batches (batch * groups <= 16, where the query tiles alone fill
//    at most half the CUs): each query tile's local and anchor reads are
//    cut into slices of their tiles (prefill_plan), one workgroup per
//    slice, and prefill_merge_kernel merges the slices' partials by their
//    running maxima and applies the gate.
#include "rma_kernels.h"

namespace rma {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

constexpr int kPT = 32;          // keys per tile
// Largest lead (log2 units) of a tile's score over a row's reference
// maximum before the reference moves (conditional rescaling).
constexpr float kLazyLog2 = 8.f;
// Bytes per staged row (padding against LDS bank conflicts).  Chosen by
// measurement of the batch-8 prefill over 16-byte multiples: K rows 544
// (136 dwords) and V rows 544 ran fastest (K rows of 528: +5%, 576: +10%;
// V rows of 528 or 560: +2-4%).
constexpr int kRowK = 544;
constexpr int kRowV = 544;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// A 16-byte store with the non-temporal hint, for the ring and pending
// records the block commits: their next reader is the decode's
// non-temporal stream (batch-8 block 1-2 us faster).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Max / sum of the values of lanes l and l ^ 16 (resp. l ^ 32), in every
// lane: v_permlane16_swap / v_permlane32_swap with the value in both
// operands leave the lane's own value in one result and its partner's in
// the other (which is which depends on the lane; max and + do not care).
// VALU only, no LDS round trip.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t swap16(float x) {
  const unsigned u = __float_as_uint(x);
  return __builtin_amdgcn_permlane16_swap(u, u, false, false);
}
__device__ __forceinline__ u32x2_t swap32(float x) {
  const unsigned u = __float_as_uint(x);
  return __builtin_amdgcn_permlane32_swap(u, u, false, false);
}
__device__ __forceinline__ float max16(float x) {
  const u32x2_t r = swap16(x);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float max32(float x) {
  const u32x2_t r = swap32(x);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float sum16(float x) {
  const u32x2_t r = swap16(x);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}
__device__ __forceinline__ float sum32(float x) {
  const u32x2_t r = swap32(x);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt 0, expcnt and lgkmcnt left
// at their maxima (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;

// Key source of one segment (ring, block, bank).
enum : int { kSegRing = 0, kSegBlock = 1, kSegBank = 2 };

// Key slot order of a 32-key tile in the k dimension of the P.V product:
// k slot 8 lg + j holds key 4 lg + j (j < 4, first 16-key sub-tile) or key
// 16 + 4 lg + (j - 4) (second sub-tile), which is where the S^T accumulator
// of lane group lg keeps them; the V^T operand is read in the same order.
// kSplit (small batches): the workgroup reads one slice of one read, part
// pr of a.pf_loc + a.pf_bank (the local read cut in a.pf_loc slices of its
// tiles, the anchor read in a.pf_bank), and writes its unnormalised partial
// (o, running max, sum) per query row to a.part for prefill_merge_kernel.
template <int kWaves, bool kSplit>
__global__ __launch_bounds__(64 * kWaves) void prefill_attn_kernel(PrefillArgs a) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kTokWG = 4 * kWaves;                     // 4 tokens (16 query rows) per wave
  constexpr int kStage = 2 * kPT * kChunks / kThreads;   // K and V chunks staged per thread
  // Workgroup -> (query tile, sequence, group[, part]).  The hardware hands
  // workgroup w to XCD w mod 8, each XCD with its own L2; all query tiles of
  // one (sequence, group[, part]) read the same K/V tiles, so when the
  // number of such units is a multiple of 8 they are all placed on one XCD
  // (w mod 8 fixed) and share its L2.
  const int nqt = (a.n + kTokWG - 1) / kTokWG;
  const int parts = kSplit ? a.pf_loc + a.pf_bank : 1;
  const int units = a.B * a.G * parts;
  const int w = blockIdx.x;
  int qt, vu;
  if ((units & 7) == 0) {
    const int r = w >> 3;
    qt = r % nqt;
    vu = (w & 7) + 8 * (r / nqt);
  } else {
    qt = w % nqt;
    vu = w / nqt;
  }
  const int u = kSplit ? vu / parts : vu;
  const int pr = kSplit ? vu - u * parts : 0;  // part (kSplit)
  const bool anchor_part = kSplit && pr >= a.pf_loc;
  const int b = u / a.G, g = u - b * a.G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;  // MFMA column / k-group
  const int n = a.n;
  const int tok0 = qt * kTokWG + wave * 4;    // first token of this wave
  const int q_tok = tok0 + (l16 >> 2);        // this lane's query: token q_tok, head q_head
  const int q_head = l16 & 3;

  // [buffer][32 keys][kRowK bytes] and [buffer][32 keys][kRowV bytes]
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][kPT * kRowK];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2][kPT * kRowV];

  // Q^T as B-operands (column = query): 8 k-steps of 32 dims; with a
  // separate anchor query (a.qa) the bank tiles and the gate use its rows
  uint4 qa[8];
  auto load_q = [&](const uint16_t* src) {
    const bool ok = q_tok < n;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        src + (((size_t)b * n + (ok ? q_tok : 0)) * a.H + g * kHpg + q_head) * kD);
#pragma unroll
    for (int st = 0; st < 8; ++st) qa[st] = ok ? qrow[st * 4 + lg] : make_uint4(0, 0, 0, 0);
  };
  load_q(anchor_part && a.qa != nullptr ? a.qa : a.q);

  const int R = a.R;
  int64_t P = a.P;
  if (a.pos != nullptr) {  // per-sequence block start (uniform per workgroup)
    const int p = a.pos[b];
    if (p < 0 || p % a.C != 0) return;
    P = p;
  }
  const int ring_valid = (int)(P < R ? P : R);
  const int t_ring = (ring_valid + kPT - 1) / kPT;
  // block keys a query tile can see: tokens 0 .. last token of the tile
  int last_tok = qt * kTokWG + kTokWG - 1;
  last_tok = last_tok < n - 1 ? last_tok : n - 1;
  const int t_blk = last_tok / kPT + 1;
  const int nb = a.bank_n[u];
  const int t_bank = (nb + kPT - 1) / kPT;
  const int t_loc = t_ring + t_blk;
  const int t_all = t_loc + t_bank;
  // tiles of this workgroup: all, or the slice of its part
  int ta = 0, tb = t_all;
  if (kSplit) {
    if (anchor_part) {
      const int i = pr - a.pf_loc;
      ta = t_loc + i * t_bank / a.pf_bank;
      tb = t_loc + (i + 1) * t_bank / a.pf_bank;
    } else {
      ta = pr * t_loc / a.pf_loc;
      tb = (pr + 1) * t_loc / a.pf_loc;
    }
  }
  // ring age threshold: slot s holds position P - R + age(s), age(s) =
  // (s - P) mod R; it exists iff age >= R - P
  const int min_age = (int)(R - P > 0 ? R - P : 0);
  const int p_mod = (int)(P % R);

  const uint16_t* ring_k = a.ring_k + (size_t)u * a.Rk * kD;
  const uint16_t* ring_v = a.ring_v + (size_t)u * R * kD;
  const uint16_t* bank_k = a.bank_k + (size_t)u * a.N * kD;
  const uint16_t* bank_v = a.bank_v + (size_t)u * a.N * kD;

  // segment and in-segment tile of combined tile index t
  auto seg_of = [&](int t, int& seg, int& ti) {
    if (t < t_ring) { seg = kSegRing; ti = t; }
    else if (t < t_loc) { seg = kSegBlock; ti = t - t_ring; }
    else { seg = kSegBank; ti = t - t_loc; }
  };
  auto seg_count = [&](int seg) { return seg == kSegRing ? ring_valid : (seg == kSegBlock ? n : nb); };

  // Uniform (scalar) source of tile t: base, key stride and chunk stride in
  // 16-byte units for K; base and key stride for V rows.  Ring and bank K
  // planes are chunk-major (key stride 1, chunk stride = slots); the
  // block's K and V are rows of the [B][n][G][D] inputs.
  struct Src {
    const uint4* k;
    const uint4* v;
    int kks, kcs, vks, cnt, ti;
  };
  auto src_of = [&](int t) {
    Src sr;
    int seg, ti;
    seg_of(t, seg, ti);
    const uint4* kblk = reinterpret_cast<const uint4*>(a.k + ((size_t)b * n * a.G + g) * kD);
    const uint4* vblk = reinterpret_cast<const uint4*>(a.v + ((size_t)b * n * a.G + g) * kD);
    const bool ring = seg == kSegRing, blk = seg == kSegBlock;
    sr.k = ring ? reinterpret_cast<const uint4*>(ring_k)
                : (blk ? kblk : reinterpret_cast<const uint4*>(bank_k));
    sr.v = ring ? reinterpret_cast<const uint4*>(ring_v)
                : (blk ? vblk : reinterpret_cast<const uint4*>(bank_v));
    sr.kks = blk ? a.G * kChunks : 1;
    sr.kcs = ring ? a.Rk : (blk ? 1 : a.N);
    sr.vks = blk ? a.G * kChunks : kChunks;
    sr.cnt = seg_count(seg);
    sr.ti = ti;
    return sr;
  };

  // Cooperative staging of one tile: 32 keys x 32 chunks of K and of V.
  // A stage is 2 K and 2 V chunks per thread (8-wave workgroups take one
  // per tile, 4-wave ones two): chunk x = tid + kThreads * (2 part + m) of
  // a plane.  K: key x % 32, chunk x / 32 (consecutive lanes read
  // consecutive slots of one chunk plane); V: key x / 32, chunk x % 32 (32
  // lanes per row).  Keys past the count re-read the last valid key.
  // Named registers, no arrays: the stage must stay out of scratch.
  constexpr int kParts = kStage / 4;
  struct Stage {
    uint4 k0, k1, v0, v1;
  };
  auto stage_load = [&](int t, int part) {
    const Src sr = src_of(t);
    // offsets in 16-byte units fit 32 bits (< 2^16 within one unit's plane)
    auto kload = [&](int m) {
      const int x = tid + kThreads * (2 * part + m);
      int kk = sr.ti * kPT + (x & 31);
      kk = kk < sr.cnt ? kk : sr.cnt - 1;
      return sr.k[(uint32_t)(kk * sr.kks + (x >> 5) * sr.kcs)];
    };
    auto vload = [&](int m) {
      const int x = tid + kThreads * (2 * part + m);
      int kv = sr.ti * kPT + (x >> 5);
      kv = kv < sr.cnt ? kv : sr.cnt - 1;
      return sr.v[(uint32_t)(kv * sr.vks + (x & 31))];
    };
    Stage sg;
    sg.k0 = kload(0);
    sg.k1 = kload(1);
    sg.v0 = vload(0);
    sg.v1 = vload(1);
    return sg;
  };
  auto stage_store = [&](int buf, int part, const Stage& sg) {
    const int x0 = tid + kThreads * (2 * part), x1 = x0 + kThreads;
    *reinterpret_cast<uint4*>(&k_lds[buf][(x0 & 31) * kRowK + (x0 >> 5) * 16]) = sg.k0;
    *reinterpret_cast<uint4*>(&k_lds[buf][(x1 & 31) * kRowK + (x1 >> 5) * 16]) = sg.k1;
    *reinterpret_cast<uint4*>(&v_lds[buf][(x0 >> 5) * kRowV + (x0 & 31) * 16]) = sg.v0;
    *reinterpret_cast<uint4*>(&v_lds[buf][(x1 >> 5) * kRowV + (x1 & 31) * 16]) = sg.v1;
  };

  f32x4_t o[16];    // running read O^T: register i of lane (lg, l16) = dim 16 dt + 4 lg + i, query l16
  f32x4_t oloc[16]; // the finished local read
  float m_run, l_run;
  auto reset = [&]() {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  };
  reset();

  // kSplit: the part's partial of this lane's query row (an empty slice:
  // m = -inf, l = 0, o = 0)
  auto write_part = [&](bool empty) {
    if (q_tok < n) {
      float* dst = a.part + ((((size_t)b * n + q_tok) * a.H + g * kHpg + q_head) * parts + pr) *
                                kPfPart;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        *reinterpret_cast<float4*>(dst + 16 * dt + 4 * lg) =
            empty ? make_float4(0.f, 0.f, 0.f, 0.f)
                  : make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (lg == 0) {
        dst[kD] = empty ? -INFINITY : m_run;
        dst[kD + 1] = empty ? 0.f : l_run;
      }
    }
  };
  if (kSplit && ta >= tb) {
    write_part(true);
    return;
  }

  // tile ta into LDS; tile ta + 1 in registers (each tile's loads are
  // issued two tiles ahead of its use, so they have two tiles of work to
  // land)
  stage_store(ta & 1, 0, stage_load(ta, 0));
  if (kParts == 2) stage_store(ta & 1, 1, stage_load(ta, 1));
  const int t1 = ta + 1 < tb ? ta + 1 : ta;
  Stage x0 = stage_load(t1, 0), x1 = x0, y0 = x0, y1 = x0;
  if (kParts == 2) x1 = stage_load(t1, 1);
  __syncthreads();

  // One tile: LDS buffer t & 1 holds tile t, registers `cur` hold tile
  // t + 1, and tile t + 2 is loaded into `nxt`.  Two register sets that
  // swap roles from one tile to the next (the loop below takes two tiles
  // per turn) mean no register copy of loads in flight, which would make
  // the compiler wait for them at the end of every tile.
  auto tile_step = [&](int t, const Stage& cur0, const Stage& cur1, Stage& nxt0, Stage& nxt1)
                       __attribute__((always_inline)) {
    int seg, ti;
    seg_of(t, seg, ti);
    const int cnt = seg_count(seg);
    if (!kSplit && a.qa != nullptr && t == t_loc) {  // first bank tile: the anchor query
      load_q(a.qa);
      // wait for these loads here, on this one tile: left pending, they
      // make the compiler guard the scores of every tile with a wait on
      // all outstanding loads, the prefetches included
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    // prefetch of tile t + 2, without branches: past the last tile, reload
    // the last one
    const int tn = t + 2 < tb ? t + 2 : tb - 1;
    nxt0 = stage_load(tn, 0);
    if (kParts == 2) nxt1 = stage_load(tn, 1);

    const unsigned char* kl = k_lds[t & 1];
    const unsigned char* vl = v_lds[t & 1];

    // S^T = K Q^T for the tile's two 16-key sub-tiles: A = 16 keys x 32
    // dims (lane: key l16, chunk 4 st + lg), B = Q^T
    // (two accumulators per sub-tile, even and odd k-steps: four independent
    // MFMA chains instead of two)
    f32x4_t s4[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) s4[sub][0] = s4[sub][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&kl[(sub * 16 + l16) * kRowK +
                                                              (st * 4 + lg) * 16]);
        s4[sub][st & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(ka), as_bf16x8(qa[st]), s4[sub][st & 1], 0, 0, 0);
      }
    }
    const f32x4_t s[2] = {s4[0][0] + s4[0][1], s4[1][0] + s4[1][1]};

    // Mask.  A tile every key of which is visible to every query of the
    // wave (most ring and bank tiles) skips it; the test is wave-uniform.
    //   ring: slot kk holds age (kk - P) mod R; query token q sees ages
    //         >= max(min_age, q); the tile's least age is 0 if it holds
    //         slot P mod R, else that of its first slot
    //   block: keys up to the query's own token
    //   bank: all committed keys
    const int kt0 = ti * kPT;
    bool full = kt0 + kPT <= cnt;
    if (seg == kSegRing) {
      int a0 = kt0 - p_mod;
      a0 += a0 < 0 ? R : 0;
      const int amin = (p_mod >= kt0 && p_mod < kt0 + kPT) ? 0 : a0;
      const int need = min_age > tok0 + 3 ? min_age : tok0 + 3;
      full = full && amin >= need;
    } else if (seg == kSegBlock) {
      full = full && kt0 + kPT - 1 <= tok0;
    }
    float sv[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[sub][i] = s[sub][i];
    if (!full) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kt0 + sub * 16 + lg * 4 + i;
          bool vis = kk < cnt && q_tok < n;
          if (seg == kSegRing) {
            int age = kk - p_mod;
            age += age < 0 ? R : 0;
            vis = vis && age >= min_age && age >= q_tok;
          } else if (seg == kSegBlock) {
            vis = vis && kk <= q_tok;
          }
          sv[sub][i] = vis ? sv[sub][i] : -INFINITY;
        }
      }
    }

    // online softmax of this lane's query (log2 domain, scale folded into
    // the exponent): the tile's 32 keys are this lane's 8 values and those
    // of lanes l16 + 16, + 32, + 48
    float mt = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                     fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
    mt = max32(max16(mt));
    // Conditional rescaling: a row's reference maximum moves only when the
    // tile's maximum passes it by more than kLazyLog2, so the rescale of o
    // below runs on few tiles.  Probabilities are then at most 2^kLazyLog2
    // (exact in fp32 and in bf16's range), and the normalisation by the sum
    // of the same probabilities cancels the reference: only rounding differs
    // from rescaling on every new maximum.
    const float mt2 = mt * a.sl2e;
    const float mn = mt2 > m_run + kLazyLog2 ? mt2 : m_run;  // from -inf: any finite maximum
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float al = __builtin_amdgcn_exp2f(m_run - mref);   // exactly 1 where mn == m_run
    float pr[2][4];
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[sub][i] = __builtin_amdgcn_exp2f(fmaf(sv[sub][i], a.sl2e, -mref));
        ps += pr[sub][i];
      }
    ps = sum32(sum16(ps));
    l_run = l_run * al + ps;
    // rescale only if some lane's reference moved (elsewhere al == 1 exactly)
    if (__any(mn != m_run)) {
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] *= al;
    }
    m_run = mn;

    // P^T B-operand straight from registers (k slot order above), bf16
    uint4 pb;
    pb.x = pack_bf16(pr[0][0], pr[0][1]);
    pb.y = pack_bf16(pr[0][2], pr[0][3]);
    pb.z = pack_bf16(pr[1][0], pr[1][1]);
    pb.w = pack_bf16(pr[1][2], pr[1][3]);

    // O^T += V^T P^T.  A = V^T rows 16 dt .. 16 dt + 15 in k slot order,
    // read transposed from the row-major V tile: in each 16-lane group,
    // ds_read_b64_tr_b16 gives lane 4a + b element b of the 4 elements
    // read by lanes a, a + 4, a + 8, a + 12; so lane l16 of group lg
    // addresses key 16 h + 4 lg + l16 / 4, dims 16 dt + 4 (l16 % 4) .. + 3
    // (h = 0: k slots 0-3 of the group, h = 1: slots 4-7).
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const unsigned char* v0 = &vl[(4 * lg + (l16 >> 2)) * kRowV + (16 * dt + 4 * (l16 & 3)) * 2];
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(v0));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(v0 + 16 * kRowV));
      const bf16x8_t va = __builtin_bit_cast(
          bf16x8_t, (v8i16_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_bf16x8(pb), o[dt], 0, 0, 0);
    }

    // end of the local read: normalise and keep it
    if (!kSplit && t == t_loc - 1) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) oloc[dt] = o[dt] * inv;
      reset();
    }
    stage_store((t + 1) & 1, 0, cur0);  // tile t + 1
    if (kParts == 2) stage_store((t + 1) & 1, 1, cur1);
    __syncthreads();
  };
  int t = ta;
  for (; t + 1 < tb; t += 2) {
    tile_step(t, x0, x1, y0, y1);
    tile_step(t + 1, y0, y1, x0, x1);
  }
  if (t < tb) tile_step(t, x0, x1, y0, y1);
  if (kSplit) {
    write_part(false);
    return;
  }
  if (t_loc == 0) {
    // no visible local key is impossible for a real token (it sees itself)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) oloc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // anchor read (zero for an empty bank)
  const float inv_b = (t_bank > 0 && l_run > 0.f) ? 1.f / l_run : 0.f;

  // gate argument qa . w_g of this lane's query (qa = the anchor query if
  // given, else q), summed over the 4 k-groups
  if (a.qa != nullptr && t_bank == 0) load_q(a.qa);
  float z = 0.f;
  {
    const float* wrow = a.w_g + (size_t)(a.gate_group ? g : g * kHpg + q_head) * kD;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const float4 w0 = reinterpret_cast<const float4*>(wrow + st * 32 + lg * 8)[0];
      const float4 w1 = reinterpret_cast<const float4*>(wrow + st * 32 + lg * 8)[1];
      const uint4 qv = qa[st];
      z = fmaf(__uint_as_float(qv.x << 16), w0.x, z);
      z = fmaf(__uint_as_float(qv.x & 0xffff0000u), w0.y, z);
      z = fmaf(__uint_as_float(qv.y << 16), w0.z, z);
      z = fmaf(__uint_as_float(qv.y & 0xffff0000u), w0.w, z);
      z = fmaf(__uint_as_float(qv.z << 16), w1.x, z);
      z = fmaf(__uint_as_float(qv.z & 0xffff0000u), w1.y, z);
      z = fmaf(__uint_as_float(qv.w << 16), w1.z, z);
      z = fmaf(__uint_as_float(qv.w & 0xffff0000u), w1.w, z);
    }
    z += __shfl_xor(z, 16, 64);
    z += __shfl_xor(z, 32, 64);
    if (a.gate_group) {  // the token's 4 heads sit in lanes 4j .. 4j+3 of a row
      z += __shfl_xor(z, 1, 64);
      z += __shfl_xor(z, 2, 64);
      z *= 1.f / kHpg;
    }
  }
  const float gate = tanhf(z);

  if (q_tok < n) {
    uint16_t* orow = a.out + (((size_t)b * n + q_tok) * a.H + g * kHpg + q_head) * kD;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = fmaf(gate, o[dt][i] * inv_b, oloc[dt][i]);
      *reinterpret_cast<uint2*>(orow + 16 * dt + 4 * lg) =
          make_uint2(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]));
    }
  }
}

// The block's writes, after every query of the block has read the ring:
// token j goes to ring slot (P + j) mod R and pending slot (P + j) mod C.
// Workgroup (bx, u) of (ceil(n / 8), units): 256 threads, 8 tokens of one unit.  V,
// pending and score rows are row-contiguous and copied directly; ring K is
// chunk-major, so the 8 K rows pass through LDS and each chunk plane gets
// 8 consecutive slots (128 bytes, contiguous up to the wrap at R) per
// store instead of 16-byte pieces from separate workgroups.  (64 tokens per
// workgroup left too few workgroups at small batches.)
constexpr int kCommitTok = 8;
__device__ __forceinline__ void commit_tokens(const PrefillArgs& a, int bx, int u) {
  const int j0 = bx * kCommitTok;
  const int b = u / a.G, g = u - b * a.G;
  const int tid = threadIdx.x;
  int64_t P = a.P;
  if (a.pos != nullptr) {
    const int p = a.pos[b];
    if (p < 0 || p % a.C != 0) return;
    P = p;
  }
  const int nt = a.n - j0 < kCommitTok ? a.n - j0 : kCommitTok;
  __shared__ uint4 kt[kCommitTok][kChunks + 1];  // K rows, one chunk of padding each
  // thread x = tid + 256 i: token x / 32, chunk x % 32 (rows read whole)
#pragma unroll
  for (int i = 0; i < kCommitTok * kChunks / 256; ++i) {
    const int x = tid + 256 * i, jj = x >> 5, c = x & 31;
    if (jj < nt) {
      const int j = j0 + jj;
      const size_t src = (((size_t)b * a.n + j) * a.G + g) * kD;
      const int rs = (int)((P + j) % a.R), ps = (int)((P + j) % a.C);
      kt[jj][c] = reinterpret_cast<const uint4*>(a.k + src)[c];
      store16_nt(reinterpret_cast<uint4*>(a.ring_v + ((size_t)u * a.R + rs) * kD) + c,
                 reinterpret_cast<const uint4*>(a.v + src)[c]);
      store16_nt(reinterpret_cast<uint4*>(a.pend_k + ((size_t)u * a.C + ps) * kD) + c,
                 reinterpret_cast<const uint4*>(a.ck + src)[c]);
      store16_nt(reinterpret_cast<uint4*>(a.pend_v + ((size_t)u * a.C + ps) * kD) + c,
                 reinterpret_cast<const uint4*>(a.cv + src)[c]);
      if (c == 0) a.pscore[(size_t)u * a.C + ps] = a.cs[((size_t)b * a.n + j) * a.G + g];
    }
  }
  __syncthreads();
  // ring K: thread x: chunk x / 64, token x % 64 (consecutive lanes write
  // consecutive slots of one chunk plane)
  uint4* rk = reinterpret_cast<uint4*>(a.ring_k + (size_t)u * a.Rk * kD);
#pragma unroll
  for (int i = 0; i < kCommitTok * kChunks / 256; ++i) {
    const int x = tid + 256 * i, c = x / kCommitTok, jj = x % kCommitTok;
    if (jj < nt) store16_nt(&rk[k_chunk_index((int)((P + j0 + jj) % a.R), c, a.Rk)], kt[jj][c]);
  }
}

__global__ __launch_bounds__(256) void prefill_commit_kernel(PrefillArgs a) {
  commit_tokens(a, blockIdx.x, blockIdx.y);
}

// Merge of the split launch, workgroup bx of ceil(B n H / 4): 4 waves, one
// query row (sequence, token, head) per wave, lane = dims 4 lane ..
// 4 lane + 3.  The local slices and the anchor slices are each merged by
// their running maxima, then out = o_local + tanh(qa . w_g) * o_anchor (an
// empty bank reads as zero).
__device__ __forceinline__ void merge_rows(const PrefillArgs& a, int bx) {
  const int row = bx * 4 + (threadIdx.x >> 6);  // (b, token, head)
  const int lane = threadIdx.x & 63;
  const int rows = a.B * a.n * a.H;
  if (row >= rows) return;
  const int b = row / (a.n * a.H);
  if (a.pos != nullptr) {  // left-out sequences: no partials, no output
    const int p = a.pos[b];
    if (p < 0 || p % a.C != 0) return;
  }
  const int hq = row % a.H;
  const int parts = a.pf_loc + a.pf_bank;
  const float* pp = a.part + (size_t)row * parts * kPfPart;
  // every slice's partial is loaded before any is used (one memory round
  // trip); slices past `parts` read as empty
  float4 o[kPfMaxSplits];
  float m[kPfMaxSplits], l[kPfMaxSplits];
#pragma unroll
  for (int i = 0; i < kPfMaxSplits; ++i) {
    const bool on = i < parts;
    const float* pi = pp + (on ? i : 0) * kPfPart;
    o[i] = *reinterpret_cast<const float4*>(pi + 4 * lane);
    m[i] = on ? pi[kD] : -INFINITY;
    l[i] = on ? pi[kD + 1] : 0.f;
  }
  const uint16_t* qsrc = a.qa != nullptr ? a.qa : a.q;
  float z;
  if (a.gate_group) {  // the mean of the token's group of anchor queries . w_g[g]
    const int h0 = hq - hq % kHpg;
    const float4 wv = *reinterpret_cast<const float4*>(a.w_g + (size_t)(h0 / kHpg) * kD + 4 * lane);
    float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll
    for (int hh = 0; hh < kHpg; ++hh) {
      const uint2 x = *reinterpret_cast<const uint2*>(qsrc + (size_t)(row - hq + h0 + hh) * kD +
                                                       4 * lane);
      m0 += __uint_as_float(x.x << 16);
      m1 += __uint_as_float(x.x & 0xffff0000u);
      m2 += __uint_as_float(x.y << 16);
      m3 += __uint_as_float(x.y & 0xffff0000u);
    }
    z = m0 * wv.x;
    z = fmaf(m1, wv.y, z);
    z = fmaf(m2, wv.z, z);
    z = fmaf(m3, wv.w, z);
    z *= 1.f / kHpg;
  } else {
    const uint2 qv = *reinterpret_cast<const uint2*>(qsrc + (size_t)row * kD + 4 * lane);
    const float4 wv = *reinterpret_cast<const float4*>(a.w_g + (size_t)hq * kD + 4 * lane);
    z = __uint_as_float(qv.x << 16) * wv.x;
    z = fmaf(__uint_as_float(qv.x & 0xffff0000u), wv.y, z);
    z = fmaf(__uint_as_float(qv.y << 16), wv.z, z);
    z = fmaf(__uint_as_float(qv.y & 0xffff0000u), wv.w, z);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  const float gate = tanhf(z);

  // slices [i0, i1) of one read -> (sum of e_i o_i) / (sum of e_i l_i)
  auto merge = [&](int i0, int i1) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPfMaxSplits; ++i)
      if (i >= i0 && i < i1) M = fmaxf(M, m[i]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kPfMaxSplits; ++i) {
      if (i < i0 || i >= i1) continue;
      const float e = m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[i] - M);
      acc.x = fmaf(e, o[i].x, acc.x);
      acc.y = fmaf(e, o[i].y, acc.y);
      acc.z = fmaf(e, o[i].z, acc.z);
      acc.w = fmaf(e, o[i].w, acc.w);
      L = fmaf(e, l[i], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    return make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  };
  const float4 ol = merge(0, a.pf_loc);
  const float4 oa = merge(a.pf_loc, parts);
  uint16_t* orow = a.out + (size_t)row * kD + 4 * lane;
  *reinterpret_cast<uint2*>(orow) = make_uint2(pack_bf16(fmaf(gate, oa.x, ol.x), fmaf(gate, oa.y, ol.y)),
                                               pack_bf16(fmaf(gate, oa.z, ol.z), fmaf(gate, oa.w, ol.w)));
}

// After the split attention kernel, one launch for both: workgroups
// [0, merge_wgs) merge query rows, the rest commit the block's tokens (the
// two touch disjoint memory, and both must follow every read of the ring).
__global__ __launch_bounds__(256) void prefill_merge_commit_kernel(PrefillArgs a, int merge_wgs,
                                                                   int commit_x) {
  const int w = blockIdx.x;
  if (w < merge_wgs) {
    merge_rows(a, w);
  } else {
    const int c = w - merge_wgs;
    commit_tokens(a, c % commit_x, c / commit_x);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  // 8-wave workgroups (32 tokens: twice the reuse of every staged tile);
  // small batches split each query tile's reads into slices (a.pf_loc,
  // a.pf_bank from prefill_plan)
  const int units = a.B * a.G;
  const int tiles8 = (a.n + 31) / 32;
  if (a.pf_loc > 0) {
    hipLaunchKernelGGL((prefill_attn_kernel<8, true>),
                       dim3(tiles8 * units * (a.pf_loc + a.pf_bank)), dim3(512), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int merge_wgs = (a.B * a.n * a.H + 3) / 4;
    const int commit_x = (a.n + kCommitTok - 1) / kCommitTok;
    hipLaunchKernelGGL(prefill_merge_commit_kernel, dim3(merge_wgs + commit_x * units), dim3(256),
                       0, s, a, merge_wgs, commit_x);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_attn_kernel<8, false>), dim3(tiles8 * units), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_commit_kernel, dim3((a.n + kCommitTok - 1) / kCommitTok, units),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rma
