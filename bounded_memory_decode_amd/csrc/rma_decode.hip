// Decode step of the RMA layer on gfx950: attention of each query head over
// the local ring and over the committed anchor bank, the signed gate that
// merges the two reads, the ring write and the pending append.
//
// Three launch shapes (launch_decode picks one per batch):
//   * whole-unit (with 4 KV groups: batch 160-256 and 416-512, where
//     the units fill at least 5/8 of the resident waves in their last
//     round): a wave of the persistent,
//     wave-pipelined attention kernel owns a (sequence, group) unit, reads
//     its ring then its bank, and finishes the token in-wave (current
//     token, gate, output, ring write, pending append): one launch;
//   * split, multi-tile parts (batch 33-159): reads are cut into parts
//     of whole 64-key tiles taken by the same persistent kernel; partials
//     go to scratch and a combine kernel finishes the token;
//   * split, one-tile parts (batch 1-32): one four-wave workgroup per
//     64-key tile in decode_part_kernel (all loads at once, a 16-key block
//     per wave, scores on MFMA), then the combine kernel.
// A batch whose whole units would leave a later round less than 5/8 full
// (batch 257-415) goes through two of these in turn (decode_whole_prefix):
// the whole-unit launch for the sequences of the full rounds, then the
// shape of the remaining batch for the rest.
// Positions come from the lockstep arguments or, per sequence, from a
// device array (TokPos); with per-sequence positions a completed block is
// admitted right after the token (in the combine workgroup, or by an admit
// launch after the whole-unit kernel).  kQA instantiates the whole-unit
// kernel for a separate anchor query (the anchor read and the gate use it).
//
// Semantics: EdgeRock model card (ModelScope), "How Rock Memory Anchors
// work" (local window of 1,024 positions, committed-bank reads, signed gate)
// and the persistent-history table note (ring of 1,023 preceding positions
// plus the current token); ai-primer "EdgeRock-4B fixes its attention KV
// cache at 72 MiB", three-operation list (Write, Retrieve).  Gate reading:
// out = o_local + tanh(qa . w_g) * o_anchor, qa = the anchor query if one
// is given, else q.
//
// Data layout (owned by this library, see include/rma.h): K planes are
// chunk-major (16-byte chunks of 8 dims), so that one load of a score
// MFMA's A operand (16 consecutive slots x 4 consecutive chunks) reads four
// contiguous 256-byte runs; V planes are row-major so that a half-wave
// loads one 512-byte row.  Neither read needs an LDS transpose.
#include "rma_admit_unit.h"

#include <atomic>

namespace rma {
namespace {

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform read of memory no kernel of this launch writes, through
// the constant address space: a scalar load, so it never waits on the
// vector-memory counter (and never drains the load pipeline).
__device__ __forceinline__ int32_t scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Reductions over a 16-lane row with DPP moves (swap neighbours, swap
// pairs, mirror within 8, mirror within 16; no LDS round trip), then over
// the 4 rows with lane reads.  The result is wave-uniform.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float wave_sum_u(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
}

__device__ __forceinline__ float wave_max_u(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)),
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48))));
}

// Max / sum over lanes l and l ^ 16 (resp. l ^ 32), in every lane:
// v_permlane16_swap / v_permlane32_swap with the value in both operands
// leave the lane's own value in one result and its partner's in the other.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float max16(float x) {
  const unsigned u = __float_as_uint(x);
  const u32x2_t r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float max32(float x) {
  const unsigned u = __float_as_uint(x);
  const u32x2_t r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float sum16(float x) {
  const unsigned u = __float_as_uint(x);
  const u32x2_t r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}
__device__ __forceinline__ float sum32(float x) {
  const unsigned u = __float_as_uint(x);
  const u32x2_t r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// One of two wave-uniform pointers, chosen per lane.  The pointers go
// through readfirstlane first: a per-lane select between two fields of the
// kernel-argument struct otherwise becomes a dynamically indexed private
// copy of the struct (scratch memory, and a scratch load plus a full
// vector-memory wait wherever it is read).
template <typename T>
__device__ __forceinline__ T* pick(bool first, T* p0, T* p1) {
  const uint64_t u0 = reinterpret_cast<uint64_t>(p0), u1 = reinterpret_cast<uint64_t>(p1);
  const uint64_t v0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u0 >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u0);
  const uint64_t v1 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u1 >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u1);
  return reinterpret_cast<T*>(first ? v0 : v1);
}

// 16-byte accesses through the global address space: a generic (flat)
// access could also reach LDS, and the compiler then waits for every
// outstanding vector-memory access at its next wait instead of for the one
// it needs.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16(void* p, uint4 v) {
  *(__attribute__((address_space(1))) u32x4_t*)p = u32x4_t{v.x, v.y, v.z, v.w};
}
// The same store with the non-temporal hint, for the ring and pending
// records the finish and the combine write: the next read of them is the
// decode's own non-temporal stream (about 1 us per launch at batch 512).
__device__ __forceinline__ void store16_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                              (__attribute__((address_space(1))) u32x4_t*)p);
}
__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// fp32 -> bf16, round to nearest, ties to even.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int kWaves = 4;  // waves per workgroup of the split launch's persistent kernel

// Where the token of sequence b sits: the valid ring slots (positions
// max(0, t-R) .. t-1), the ring slot and pending slot it writes, and
// whether the sequence takes part in this call (per-sequence positions:
// a negative position leaves it out).  Wave-uniform; scalar arithmetic.
struct TokPos {
  int pos;  // per-sequence positions only
  int ring_count, ring_slot, pend_slot;
  bool live;
};

__device__ __forceinline__ TokPos tok_pos(const DecodeArgs& a, int b) {
  TokPos tp;
  if (a.pos == nullptr) {
    tp.pos = 0;
    tp.ring_count = a.ring_count;
    tp.ring_slot = a.ring_slot;
    tp.pend_slot = a.pend_slot;
    tp.live = true;
    return tp;
  }
  const int p = scalar_load(a.pos + b);
  const int pp = p > 0 ? p : 0;
  tp.pos = pp;
  tp.live = p >= 0;
  tp.ring_count = tp.live ? (pp < a.R ? pp : a.R) : 0;
  tp.ring_slot = pp % a.R;
  tp.pend_slot = pp % a.C;
  return tp;
}

// A segment: one contiguous range of 64-key tiles of one read (ring or
// bank) of one (sequence, group) unit.
struct Seg {
  const uint4* K4;  // K plane of the unit (chunk-major, `slots` slots)
  const uint4* V4;  // V rows of the unit
  const uint4* q4;  // the unit's 4 query rows (2 KiB)
  int slots, count, ta, tb;
};

__device__ __forceinline__ Seg make_seg(const DecodeArgs& a, int u, bool ring, int t0,
                                        int tiles) {
  const int b = u / a.G, g = u - b * a.G;
  const TokPos tp = tok_pos(a, b);
  Seg sg;
  if (ring) {
    sg.count = tp.ring_count;
    sg.slots = a.Rk;
    sg.K4 = reinterpret_cast<const uint4*>(a.ring_k + (size_t)u * a.Rk * kD);
    sg.V4 = reinterpret_cast<const uint4*>(a.ring_v + (size_t)u * a.R * kD);
  } else {
    sg.count = tp.live ? scalar_load(a.bank_n + u) : 0;
    sg.slots = a.N;
    sg.K4 = reinterpret_cast<const uint4*>(a.bank_k + (size_t)u * a.N * kD);
    sg.V4 = reinterpret_cast<const uint4*>(a.bank_v + (size_t)u * a.N * kD);
  }
  const uint16_t* qsrc = (ring || a.qa == nullptr) ? a.q : a.qa;  // the anchor read's query
  sg.q4 = reinterpret_cast<const uint4*>(qsrc + (size_t)b * a.q_bs + (size_t)g * kHpg * kD);
  const int ntiles = (sg.count + kTile - 1) / kTile;
  int t1 = t0 + tiles;
  t1 = t1 < ntiles ? t1 : ntiles;
  sg.ta = t0 < t1 ? t0 : t1;
  sg.tb = t1;
  return sg;
}

// Segment `sub` of work item `item`.
//   whole-unit: item = unit, sub 0 = the ring, sub 1 = the bank;
//   split: item = u * S + r, a single segment (part r of the ring for
//   r < splits_ring, else part r - splits_ring of the bank).
template <bool kWhole>
__device__ __forceinline__ Seg seg_of(const DecodeArgs& a, int item, int sub) {
  if (kWhole) return make_seg(a, item, sub == 0, 0, 1 << 20);
  const int S = a.splits_ring + a.splits_bank;
  const int u = item / S, r = item - u * S;
  if (r < a.splits_ring) return make_seg(a, u, true, r * a.tiles_ring, a.tiles_ring);
  return make_seg(a, u, false, (r - a.splits_ring) * a.tiles_bank, a.tiles_bank);
}

// Finish one token of unit u inside one wave (whole-unit launch): the
// local read is the ring result (mr, lr, o_r in LDS) plus the current
// token, the anchor read is the bank result (lb, accb in lanes 0-31); then
// out = o_local + tanh(q . w_g) * o_anchor, the ring write and the pending
// append.  Every read of the unit's ring by this launch is already done:
// only this wave reads it.
// Operands of the in-wave finish of one unit, loaded ahead (with the last
// bank tile's prefetch) so that the finish never waits on the vector-memory
// counter: lanes 0-31 / 32-63 hold 16-byte chunk c32 of the current K / V
// (k_or_v) and of the candidate K / V (ck_or_cv).
struct FinOps {
  uint4 k_or_v, ck_or_cv;
};

// Sources of the two auxiliary loads issued when a wave moves to segment
// `nsub` of the next item: the segment's query rows, except that a
// whole-unit wave entering the bank segment of the unit it is on (`item`)
// keeps its query rows and fetches that unit's finish operands instead
// (with a separate anchor query, kQA, it fetches the anchor query rows and
// the finish loads its own operands).
struct AuxPtrs {
  const uint4* p0;
  const uint4* p1;
};

template <bool kWhole, bool kQA>
__device__ __forceinline__ AuxPtrs aux_ptrs(const DecodeArgs& a, const Seg& nxt, int nsub,
                                            int item, int lane) {
  AuxPtrs ap;
  ap.p0 = nxt.q4 + 2 * lane;
  ap.p1 = nxt.q4 + 2 * lane + 1;
  if (kWhole && !kQA) {
    const int b = item / a.G, g = item - b * a.G;
    const size_t kvo = (size_t)b * a.kv_bs + (size_t)g * kD;
    const int c32 = lane & 31;
    const uint4* fk = reinterpret_cast<const uint4*>(pick(lane < 32, a.k, a.v) + kvo) + c32;
    const uint4* fc = reinterpret_cast<const uint4*>(pick(lane < 32, a.ck, a.cv) + kvo) + c32;
    ap.p0 = nsub == 1 ? fk : ap.p0;
    ap.p1 = nsub == 1 ? fc : ap.p1;
  }
  return ap;
}

// Finish one token of unit u inside one wave (whole-unit launch): the
// local read is the ring result (mr, lr, o_r in LDS) plus the current
// token, the anchor read is the bank result (lb, accb in lanes 0-31); then
// out = o_local + tanh(q . w_g) * o_anchor, the ring write and the pending
// append.  Every read of the unit's ring by this launch is already done:
// only this wave reads it.
template <bool kQA, bool kGG>
__device__ __forceinline__ void finish_unit(const DecodeArgs& a, int u, int lane,
                                            const uint4* q_w, const uint4* qa_w,
                                            const float* o_r, const float* mr,
                                            const float* lr, const float* lb,
                                            float accb[kHpg][8], FinOps f) {
  const int b = u / a.G, g = u - b * a.G;
  const TokPos tp = tok_pos(a, b);
  if (!tp.live) return;
  const int c32 = lane & 31;
  if (kQA) {  // operands not delivered by the pipeline in this mode
    const size_t kvo = (size_t)b * a.kv_bs + (size_t)g * kD;
    f.k_or_v = load16(reinterpret_cast<const uint4*>(pick(lane < 32, a.k, a.v) + kvo) + c32);
    f.ck_or_cv = load16(reinterpret_cast<const uint4*>(pick(lane < 32, a.ck, a.cv) + kvo) + c32);
  }
  // the current K (lanes 0-31, 8 dims each) and V (lanes 32-63)
  const uint4 kv = f.k_or_v;
  // q . k_t over 8 dims in lanes 0-31; q . w_g over 4 dims in all lanes
  float sc[kHpg], z[kHpg];
#pragma unroll
  for (int h = 0; h < kHpg; ++h) {
    const uint4 q8 = q_w[h * kChunks + c32];
    float ds = bf_lo(q8.x) * bf_lo(kv.x);
    ds = fmaf(bf_hi(q8.x), bf_hi(kv.x), ds);
    ds = fmaf(bf_lo(q8.y), bf_lo(kv.y), ds);
    ds = fmaf(bf_hi(q8.y), bf_hi(kv.y), ds);
    ds = fmaf(bf_lo(q8.z), bf_lo(kv.z), ds);
    ds = fmaf(bf_hi(q8.z), bf_hi(kv.z), ds);
    ds = fmaf(bf_lo(q8.w), bf_lo(kv.w), ds);
    ds = fmaf(bf_hi(q8.w), bf_hi(kv.w), ds);
    ds = lane < 32 ? ds : 0.f;
    const uint2 q2 = reinterpret_cast<const uint2*>((kQA ? qa_w : q_w) + h * kChunks)[lane];
    const float4 w4 =
        reinterpret_cast<const float4*>(a.w_g + (size_t)(kGG ? g : g * kHpg + h) * kD)[lane];
    float dz = bf_lo(q2.x) * w4.x;
    dz = fmaf(bf_hi(q2.x), w4.y, dz);
    dz = fmaf(bf_lo(q2.y), w4.z, dz);
    dz = fmaf(bf_hi(q2.y), w4.w, dz);
    sc[h] = wave_sum_u(ds) * a.sl2e;
    z[h] = wave_sum_u(dz);
  }
  if (kGG) {  // one gate for the group: its mean anchor query . w_g[g]
    const float zm = ((z[0] + z[1]) + (z[2] + z[3])) * (1.f / kHpg);
#pragma unroll
    for (int h = 0; h < kHpg; ++h) z[h] = zm;
  }
  // the current V: lanes 32-63 hold it; bring chunk c32 to lane c32
  uint4 v4;
  v4.x = __shfl_xor(kv.x, 32, 64);
  v4.y = __shfl_xor(kv.y, 32, 64);
  v4.z = __shfl_xor(kv.z, 32, 64);
  v4.w = __shfl_xor(kv.w, 32, 64);
  if (lane < 32) {
    const float vf[8] = {bf_lo(v4.x), bf_hi(v4.x), bf_lo(v4.y), bf_hi(v4.y),
                         bf_lo(v4.z), bf_hi(v4.z), bf_lo(v4.w), bf_hi(v4.w)};
    uint16_t* outp = a.out + (size_t)b * a.out_bs + (size_t)g * kHpg * kD + 8 * c32;
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
      const float M = fmaxf(mr[h], sc[h]);
      const float er = fast_exp2(mr[h] - M);  // ring empty: mr = -inf -> 0
      const float ec = fast_exp2(sc[h] - M);
      const float inv_l = 1.f / (lr[h] * er + ec);
      const float inv_b = lb[h] > 0.f ? 1.f / lb[h] : 0.f;  // empty bank reads as zero
      const float gate = tanhf(z[h]);
      const float4 r0 = reinterpret_cast<const float4*>(o_r + h * kD + 8 * c32)[0];
      const float4 r1 = reinterpret_cast<const float4*>(o_r + h * kD + 8 * c32)[1];
      const float orr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      uint16_t o16[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float oloc = fmaf(orr[i], er, ec * vf[i]) * inv_l;
        o16[i] = to_bf16(fmaf(gate, accb[h][i] * inv_b, oloc));
      }
      uint4 pk;
      pk.x = (uint32_t)o16[0] | ((uint32_t)o16[1] << 16);
      pk.y = (uint32_t)o16[2] | ((uint32_t)o16[3] << 16);
      pk.z = (uint32_t)o16[4] | ((uint32_t)o16[5] << 16);
      pk.w = (uint32_t)o16[6] | ((uint32_t)o16[7] << 16);
      store16(outp + (size_t)h * kD, pk);
    }
  }
  // Write: ring slot t mod R (K chunks from lanes 0-31, the V row from
  // lanes 32-63), pending slot t mod C likewise.
  {
    const bool kside = lane < 32;
    const size_t ro = kside ? (size_t)u * a.Rk * kChunks + k_chunk_index(tp.ring_slot, c32, a.Rk)
                            : ((size_t)u * a.R + tp.ring_slot) * kChunks + c32;
    store16_nt(reinterpret_cast<uint4*>(pick(kside, a.ring_k, a.ring_v)) + ro, kv);
    const size_t po = ((size_t)u * a.C + tp.pend_slot) * kChunks + c32;
    store16_nt(reinterpret_cast<uint4*>(pick(kside, a.pend_k, a.pend_v)) + po, f.ck_or_cv);
  }
  if (lane == 0) {
    const float cs = *(const __attribute__((address_space(4))) float*)(a.cs + (size_t)b * a.cs_bs + g);
    *(__attribute__((address_space(1))) float*)(a.pscore + (size_t)u * a.C + tp.pend_slot) = cs;
  }
}

// Raw buffer loads: a wave-uniform descriptor per plane, one 32-bit offset
// register per lane, and the rest of each address in the scalar and
// immediate offsets (so a tile's 64 loads need no 64-bit addresses).  The
// descriptor's byte bound applies to the whole offset (vector + scalar +
// immediate) on gfx950: past it a load returns zeros.
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same with the non-temporal hint (cache policy bit nt): for state
// streamed once per token.  A plain streaming-read probe on MI355X reaches
// about 7.1 TB/s with it and 6.0-6.3 TB/s without; the whole-unit decode
// launch at batch 512 went from 702 to 674 us.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kBufWord3 = 0x00020000;  // descriptor word 3 for gfx9-family raw buffers

// K of one 64-key tile for decode_attn_kernel, as the A operands of its
// score MFMAs: kr[8 kb + st] = chunk 4 st + l / 16 of key 64 tile + 16 kb +
// l % 16 of a chunk-major plane of `slots` slots; a key past `hi` re-reads
// key hi, so every load stays inside the plane.  Raw buffer loads: the
// plane's descriptor, one offset register per 16-key block, the k-step in
// the scalar offset.  With `idle` (nothing left to fetch) the descriptor's
// range is empty: the loads are still issued, so the loop has no
// conditional loads, but they touch no memory and return zeros.
__device__ __forceinline__ void load_k_tile(const uint4* base, int slots, int hi, int tile,
                                            int lane, bool idle, uint4 (&kr)[kChunks]) {
  // the descriptor and the scalar offset are wave-uniform; readfirstlane
  // tells the compiler so (else it wraps each load in a waterfall loop)
  const uint64_t bp = reinterpret_cast<uint64_t>(base);
  // (the builtin returns int: each word goes back through uint32_t, or the
  // low word's bit 31 would sign-extend over the high word)
  const uint32_t bp_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
  const uint32_t bp_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32));
  const uint64_t bu = ((uint64_t)bp_hi << 32) | bp_lo;
  const uint32_t bytes =
      (uint32_t)__builtin_amdgcn_readfirstlane(idle ? 0 : slots * kChunks * 16);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(bu), (short)0, bytes, kBufWord3);
  uint32_t vo[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int key = tile * kTile + 16 * kb + (lane & 15);
    vo[kb] = idle ? 0u : (uint32_t)(((lane >> 4) * slots + (key < hi ? key : hi)) * 16);
  }
  const uint32_t sst = (uint32_t)__builtin_amdgcn_readfirstlane(idle ? 0 : 4 * slots * 16);
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) kr[8 * kb + st] = buf_load16_nt(r, vo[kb], st * sst);
}

// Persistent attention kernel.  grid: at most the resident workgroups;
// block: 256 = 4 independent waves.  Wave gw takes items gw, gw + W, ...
// (W = all waves) and walks their segments.  Per tile i, in issue order:
//   V(i) loads -> QK(i) on K(i) already in registers -> softmax ->
//   query rows + K(i+1) loads of the next tile, or of the next segment's
//   first tile -> P.V(i).
// The vector-memory counter retires loads in order, so QK(i) never waits
// for V(i) and P.V(i) never waits for K(i+1): a wave keeps ~64 16-byte
// loads in flight across tile, segment and item boundaries.  No
// workgroup barrier: each wave owns its LDS slices.
// QK runs on the matrix cores (v_mfma_f32_16x16x32_bf16, K as loaded by
// load_k_tile as the A operand, the 4 query rows as B columns, repeated
// over the 16 columns); P.V runs on the vector ALU, a half-wave per key
// and 8 dims per lane, on V rows as stored.
template <bool kWhole, bool kQA, int kW, bool kGG = false>
__global__ __launch_bounds__(64 * kW) void decode_attn_kernel(DecodeArgs a, int items) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * kW;
  int item = blockIdx.x * kW + wave;
  if (item >= items) return;
  int sub = 0;

  __shared__ uint4 q_s[kW][kHpg * kChunks];  // each wave's 4 query rows
  __shared__ uint4 qa_s[kQA ? kW : 1][kHpg * kChunks];  // anchor query rows (kQA)
  // per-key probabilities of the 4 heads, then a pad that takes the stores
  // of the lanes that hold copies (no branch)
  __shared__ float4 p_s[kW][2 * kTile];
  __shared__ float or_s[kWhole ? kW : 1][kHpg * kD];  // ring result

  const int half = lane >> 5, c32 = lane & 31;
  const int l16 = lane & 15, lg = lane >> 4;
  uint4 qb[8];  // B operands of the score MFMAs (the segment's query rows)
  uint4 kr[kChunks];
  uint4 vr[kTile / 2];
  uint4 qn0, qn1;  // auxiliary loads for the next segment (2 x 16 B per lane)
  FinOps fin;      // whole-unit: operands of the unit's finish
  float mr[kHpg], lr[kHpg];  // whole-unit: the ring result

  Seg cur = seg_of<kWhole>(a, item, sub);
  qn0 = cur.q4[2 * lane];
  qn1 = cur.q4[2 * lane + 1];
  load_k_tile(cur.K4, cur.slots, cur.count > 0 ? cur.count - 1 : 0, cur.ta, lane, false, kr);

  for (;;) {
    if (!kWhole || sub == 0) {
      q_s[wave][2 * lane] = qn0;
      q_s[wave][2 * lane + 1] = qn1;
    } else if (kQA) {
      qa_s[kQA ? wave : 0][2 * lane] = qn0;
      qa_s[kQA ? wave : 0][2 * lane + 1] = qn1;
    } else {
      fin.k_or_v = qn0;
      fin.ck_or_cv = qn1;
    }
    // query rows of this segment's scores
    const uint4* qrows = (kWhole && kQA && sub == 1) ? qa_s[kQA ? wave : 0] : q_s[wave];
    __builtin_amdgcn_wave_barrier();
    // B operand of k-step st: column n takes query row n mod 4, chunk
    // 4 st + l / 16 (columns 4-15 repeat rows 0-3)
#pragma unroll
    for (int st = 0; st < 8; ++st) qb[st] = qrows[(lane & 3) * kChunks + 4 * st + lg];

    int nitem = item, nsub = sub + 1;
    if (!kWhole || nsub == 2) {
      nitem = item + W;
      nsub = 0;
    }
    const bool has_next = nitem < items;
    const Seg nxt = seg_of<kWhole>(a, has_next ? nitem : item, has_next ? nsub : sub);

    float m[kHpg], l[kHpg], acc[kHpg][8];
#pragma unroll
    for (int h = 0; h < kHpg; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    float mq = -INFINITY, lq = 0.f;  // running max and sum of head lane % 4

    for (int tile = cur.ta; tile < cur.tb; ++tile) {
      const int tbase = tile * kTile;

      // V of the tile, non-temporal (streamed once per token, as K)
#pragma unroll
      for (int j = 0; j < kTile / 2; ++j) {
        const int k2 = tbase + 2 * j + half;
        const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            cur.V4 + (size_t)(k2 < cur.count ? k2 : cur.count - 1) * kChunks + c32));
        vr[j] = make_uint4(x.x, x.y, x.z, x.w);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the V loads ahead of QK

      // Scores on the matrix cores, per 16-key block kb: S^T (16 keys x 16
      // columns) = K Q^T with v_mfma_f32_16x16x32_bf16 over the 8 k-steps;
      // register r of lane l then holds key 16 kb + 4 (l / 16) + r against
      // head l mod 4 (lanes l, l ^ 4, l ^ 8, l ^ 12 hold the same scores).
      f32x4_t d[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) d[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          d[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[8 * kb + st]),
                                                          as_bf16x8(qb[st]), d[kb], 0, 0, 0);

      // online softmax update of head lane mod 4 (log2 domain): the max over
      // the lane's 16 keys, then over lanes l ^ 16 and l ^ 32
      const int k0 = tbase + 4 * lg;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          d[kb][r] = k0 + 16 * kb + r < cur.count ? d[kb][r] * a.sl2e : -INFINITY;
          mx = fmaxf(mx, d[kb][r]);
        }
      mx = max32(max16(mx));
      const float mn = fmaxf(mq, mx);
      const float al = fast_exp2(mq - mn);
      float ps = 0.f;
      float* pw = reinterpret_cast<float*>(&p_s[wave][(l16 < kHpg ? 0 : kTile) + 4 * lg]) +
                  (lane & 3);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(d[kb][r] - mn);
          ps += p;
          pw[4 * (16 * kb + r)] = p;
        }
      lq = lq * al + ps;
      mq = mn;
      // rescale the P.V accumulators of every head (lane h holds head h)
#pragma unroll
      for (int h = 0; h < kHpg; ++h) {
        const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), h));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= ah;
      }
      __builtin_amdgcn_wave_barrier();

      // prefetch: the next tile of this segment, else the next segment's
      // first tile and query rows.  Loads with nothing to fetch are still
      // issued, so the loop stays free of branches: the query-row loads
      // while the segment continues re-read the V row this lane loaded
      // above (a cache hit), and K after the last segment goes through an
      // empty descriptor range.  Bases and strides are selected on the
      // scalar unit.
      {
        const bool more = tile + 1 < cur.tb;
        const bool go_next = !more && has_next;
        const bool idle = !more && !has_next;
        const int vrow = tbase + half < cur.count ? tbase + half : cur.count - 1;
        const int voff = vrow * kChunks + c32;
        // two auxiliary loads first (the segment switch then waits for
        // them alone): the next segment's query rows; or, whole-unit, when
        // the ring segment of a unit hands over to its bank segment (same
        // query rows), the operands of the unit's finish
        const uint4* vrow_p = cur.V4 + voff;
        const AuxPtrs ap = aux_ptrs<kWhole, kQA>(a, nxt, nsub, item, lane);
        qn0 = load16(go_next ? ap.p0 : vrow_p);
        qn1 = load16(go_next ? ap.p1 : vrow_p);
        const int ktile = more ? tile + 1 : nxt.ta;
        const int kcount = more ? cur.count : nxt.count;
        load_k_tile(more ? cur.K4 : nxt.K4, more ? cur.slots : nxt.slots,
                    kcount > 0 ? kcount - 1 : 0, ktile, lane, idle, kr);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of P.V

      // P.V: a half-wave per key, 8 dims per lane
#pragma unroll
      for (int j = 0; j < kTile / 2; ++j) {
        const uint4 vv = vr[j];
        const float4 pp = p_s[wave][2 * j + half];
        const float x[8] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y),
                            bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[0][i] = fmaf(pp.x, x[i], acc[0][i]);
          acc[1][i] = fmaf(pp.y, x[i], acc[1][i]);
          acc[2][i] = fmaf(pp.z, x[i], acc[2][i]);
          acc[3][i] = fmaf(pp.w, x[i], acc[3][i]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    // segment result: m and l of each head (l summed over lanes l, l ^ 16,
    // l ^ 32, l ^ 48; lane h holds head h), o over the two half-waves
    lq = sum32(sum16(lq));
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
      m[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mq), h));
      l[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lq), h));
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] += __shfl_xor(acc[h][i], 32, 64);
    }
    if (!kWhole) {
      // the item's partial (m, l, o[4][256]) for the combine kernel
      float* P = a.part + (size_t)item * kPart;
      if (lane < 32) {
#pragma unroll
        for (int h = 0; h < kHpg; ++h) {
          float4* dst = reinterpret_cast<float4*>(P + h * kD + 8 * c32);
          dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
          dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        }
      }
      if (lane < kHpg) {
        float mm = m[0], ll = l[0];
#pragma unroll
        for (int h = 1; h < kHpg; ++h) {
          mm = lane == h ? m[h] : mm;
          ll = lane == h ? l[h] : ll;
        }
        P[kHpg * kD + lane] = mm;
        P[kHpg * kD + kHpg + lane] = ll;
      }
    } else if (sub == 0) {
      // ring result: m, l stay in registers, o goes to this wave's LDS
#pragma unroll
      for (int h = 0; h < kHpg; ++h) {
        mr[h] = m[h];
        lr[h] = l[h];
      }
      if (lane < 32) {
#pragma unroll
        for (int h = 0; h < kHpg; ++h) {
          float4* dst = reinterpret_cast<float4*>(&or_s[kWhole ? wave : 0][h * kD + 8 * c32]);
          dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
          dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    } else {
      finish_unit<kQA, kGG>(a, item, lane, q_s[wave], qa_s[kQA ? wave : 0],
                            or_s[kWhole ? wave : 0], mr, lr, l, acc, fin);
      __builtin_amdgcn_wave_barrier();
    }

    if (!has_next) break;
    if (cur.ta == cur.tb) {  // empty segment: nothing was prefetched for nxt
      const AuxPtrs ap = aux_ptrs<kWhole, kQA>(a, nxt, nsub, item, lane);
      qn0 = load16(ap.p0);
      qn1 = load16(ap.p1);
      load_k_tile(nxt.K4, nxt.slots, nxt.count > 0 ? nxt.count - 1 : 0, nxt.ta, lane, false, kr);
    }
    cur = nxt;
    item = nitem;
    sub = nsub;
  }
}


// Attention of the split launch when every part is one 64-key tile
// (small batches).  grid: items; block: 256 = 4 waves, one part (item =
// unit * S + r: tile r of the unit's ring for r < splits_ring, else tile
// r - splits_ring of its bank), writing the part's partial (o[4][256],
// m[4], l[4]) for the combine kernel.
//
// Latency first: wave w takes the part's 16-key block w, loads its query
// rows, its K and its V rows all at once (one memory round trip; raw
// buffer loads: a wave-uniform descriptor per plane, the k-step or row in
// the immediate and scalar offsets, and the descriptor's byte bound, which
// on gfx950 applies to the whole offset, returns zeros for V rows past the
// count), then computes that block's scores, softmax and P.V; the four
// blocks' (m, l, o) are merged in LDS into the part's partial.  Scores on
// the matrix cores: S^T (16 keys x 16 columns) = K Q^T with
// v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims (lane l: key l % 16,
// chunk 4 st + l / 16 of k-step st), B = Q^T (lane l: query row
// (l % 16) mod 4, same chunk; columns 4-15 repeat rows 0-3 and are
// ignored).  P.V on the vector ALU as in the whole-unit kernel: a half-wave
// per key, 8 dims per lane, on V rows as stored.  Four waves per part
// rather than one take a quarter of the loads and of the P.V each, which
// shortens the part's chain (batch 1: 91 against 102 us per 8-layer token
// as a graph replay).  kNT: non-temporal loads, used at batch 1 only
// (88 against 91 us per token there; at batches 16 and 32 they cost 15%).
template <bool kNT>
__global__ __launch_bounds__(256) void decode_part_kernel(DecodeArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 16-key block of the tile
  const int item = blockIdx.x;
  __shared__ float4 p_s[4][20];            // per wave: 16 keys' probabilities, then a pad
  __shared__ float o_s[4][kHpg * kD];      // per wave: its block's o
  __shared__ float ml_s[4][2 * kHpg];      // per wave: its block's m and l of each head
  const Seg sg = seg_of<false>(a, item, 0);
  const int l16 = lane & 15, lg = lane >> 4;
  const int half = lane >> 5, c32 = lane & 31;
  float* P = a.part + (size_t)item * kPart;

  if (sg.ta == sg.tb) {  // nothing to read: m = -inf, l = 0, o = 0
    const int h = w;
    reinterpret_cast<float4*>(P + h * kD)[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0) {
      P[kHpg * kD + h] = -INFINITY;
      P[kHpg * kD + kHpg + h] = 0.f;
    }
    return;
  }
  const int tile = sg.ta;

  uint4 qb[8];  // B operands (Q^T), k-step st
  uint4 kr[8];  // A operands of block w, k-step st
  uint4 vr[8];  // V rows: key 16 w + 2 j + half, chunk c32
#pragma unroll
  for (int st = 0; st < 8; ++st) qb[st] = sg.q4[(l16 & 3) * kChunks + 4 * st + lg];
  {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)sg.K4, (short)0, sg.slots * kChunks * 16, kBufWord3);
    const uint32_t v0 = (uint32_t)((lg * sg.slots + tile * kTile + 16 * w + l16) * 16);
#pragma unroll
    for (int st = 0; st < 8; ++st)
      kr[st] = kNT ? buf_load16_nt(r, v0, (uint32_t)(4 * st * sg.slots * 16))
                   : buf_load16(r, v0, (uint32_t)(4 * st * sg.slots * 16));
  }
  {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)sg.V4, (short)0, sg.count * kChunks * 16, kBufWord3);
    const uint32_t v0 = (uint32_t)(((tile * kTile + 16 * w + half) * kChunks + c32) * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vr[j] = kNT ? buf_load16_nt(r, v0 + j * 1024, 0u) : buf_load16(r, v0 + j * 1024, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);

  // scores: register r of lane l holds key 16 w + 4 (l / 16) + r for query
  // l % 16 (columns 4-15 repeat rows 0-3)
  f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 8; ++st)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[st]), as_bf16x8(qb[st]), sc, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);

  // the block's softmax (log2 domain); a block past the count has m = -inf
  const int kbase = tile * kTile + 16 * w + 4 * lg;
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = kbase + r < sg.count ? sc[r] * a.sl2e : -INFINITY;
    mt = fmaxf(mt, sc[r]);
  }
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mref = mt == -INFINITY ? 0.f : mt;
  float ps = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = fast_exp2(sc[r] - mref);
    ps += p;
    const int key = l16 < kHpg ? 4 * lg + r : 16;
    reinterpret_cast<float*>(&p_s[w][key])[l16 & 3] = p;
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  __builtin_amdgcn_wave_barrier();

  float acc[kHpg][8];
#pragma unroll
  for (int h = 0; h < kHpg; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 vv = vr[j];
    const float4 pp = p_s[w][2 * j + half];
    const float x[8] = {bf_lo(vv.x), bf_hi(vv.x), bf_lo(vv.y), bf_hi(vv.y),
                        bf_lo(vv.z), bf_hi(vv.z), bf_lo(vv.w), bf_hi(vv.w)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[0][i] = fmaf(pp.x, x[i], acc[0][i]);
      acc[1][i] = fmaf(pp.y, x[i], acc[1][i]);
      acc[2][i] = fmaf(pp.z, x[i], acc[2][i]);
      acc[3][i] = fmaf(pp.w, x[i], acc[3][i]);
    }
  }
#pragma unroll
  for (int h = 0; h < kHpg; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] += __shfl_xor(acc[h][i], 32, 64);
  if (lane < 32) {
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
      float4* dst = reinterpret_cast<float4*>(&o_s[w][h * kD + 8 * c32]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (lane < kHpg) {  // lane h holds head h's m and l
    ml_s[w][lane] = mt;
    ml_s[w][kHpg + lane] = ps;
  }
  __syncthreads();

  // merge of the four blocks: wave h takes head h, lane dims 4 lane .. 4 lane + 3
  const int h = w;
  float mb[4], M = -INFINITY;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    mb[b] = ml_s[b][h];
    M = fmaxf(M, mb[b]);
  }
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float e = mb[b] == -INFINITY ? 0.f : fast_exp2(mb[b] - M);
    const float4 ob = reinterpret_cast<const float4*>(&o_s[b][h * kD])[lane];
    o.x = fmaf(e, ob.x, o.x);
    o.y = fmaf(e, ob.y, o.y);
    o.z = fmaf(e, ob.z, o.z);
    o.w = fmaf(e, ob.w, o.w);
    L = fmaf(e, ml_s[b][kHpg + h], L);
  }
  reinterpret_cast<float4*>(P + h * kD)[lane] = o;
  if (lane == 0) {
    P[kHpg * kD + h] = M;
    P[kHpg * kD + kHpg + h] = L;
  }
}

// Finish of the split launch.  grid: units; block: 256 = 4 waves, wave h
// = query head h of the unit's group, lane = dims 4 lane .. 4 lane + 3.
// Merges the parts of the local read (ring parts plus the current token)
// and of the anchor read (bank parts), applies the gate, writes the
// output, the ring slot and the pending slot; with per-sequence positions,
// a token that completes its block is followed by the unit's admit in this
// same workgroup.  Each wave merges its head alone: lane p holds part p's
// (m, l), the weights come out of wave reductions, and every part's o for
// the lane's dims is loaded before any is used (one memory round trip, no
// barrier).
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int u = blockIdx.x;
  const int b = u / a.G, g = u - b * a.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TokPos tp = tok_pos(a, b);
  if (!tp.live) return;  // the whole block: no barrier is skipped
  __shared__ AdmitShared sh;

  const int sr = a.splits_ring, S = a.splits_ring + a.splits_bank;
  const float* P = a.part + (size_t)u * S * kPart;
  // o of every part for this head and the lane's 4 dims (parts past S
  // re-read part S-1; their weight is 0); (m, l) of part `lane`
  float4 po[2 * kMaxSplits];
#pragma unroll
  for (int sp = 0; sp < 2 * kMaxSplits; ++sp) {
    const int sc = sp < S ? sp : S - 1;
    po[sp] = *reinterpret_cast<const float4*>(P + (size_t)sc * kPart + h * kD + 4 * lane);
  }
  const bool have = lane < S;
  const float mp = have ? P[(size_t)lane * kPart + kHpg * kD + h] : -INFINITY;
  const float lp = have ? P[(size_t)lane * kPart + kHpg * kD + kHpg + h] : 0.f;

  // current token and gate operands for the lane's dims
  const size_t kvo = (size_t)b * a.kv_bs + (size_t)g * kD;
  const size_t qo = (size_t)b * a.q_bs + (size_t)(g * kHpg + h) * kD + 4 * lane;
  const uint2 qv = *reinterpret_cast<const uint2*>(a.q + qo);
  const uint2 qav = *reinterpret_cast<const uint2*>((a.qa ? a.qa : a.q) + qo);
  const uint2 kv = *reinterpret_cast<const uint2*>(a.k + kvo + 4 * lane);
  const uint2 vv = *reinterpret_cast<const uint2*>(a.v + kvo + 4 * lane);
  const float4 wv = *reinterpret_cast<const float4*>(
      a.w_g + (size_t)(a.gate_group ? g : g * kHpg + h) * kD + 4 * lane);
  const int n = scalar_load(a.bank_n + u);

  // q.k_t (current-token score) and qa.w_g (gate argument)
  float dk = bf_lo(qv.x) * bf_lo(kv.x);
  dk = fmaf(bf_hi(qv.x), bf_hi(kv.x), dk);
  dk = fmaf(bf_lo(qv.y), bf_lo(kv.y), dk);
  dk = fmaf(bf_hi(qv.y), bf_hi(kv.y), dk);
  float dz;
  if (a.gate_group) {  // the mean of the group's anchor queries . w_g[g]
    const uint16_t* qs = (a.qa ? a.qa : a.q) + (size_t)b * a.q_bs + (size_t)g * kHpg * kD +
                         4 * lane;
    float m0 = 0.f, m1 = 0.f, m2 = 0.f, m3 = 0.f;
#pragma unroll
    for (int hh = 0; hh < kHpg; ++hh) {
      const uint2 x = *reinterpret_cast<const uint2*>(qs + (size_t)hh * kD);
      m0 += bf_lo(x.x);
      m1 += bf_hi(x.x);
      m2 += bf_lo(x.y);
      m3 += bf_hi(x.y);
    }
    dz = m0 * wv.x;
    dz = fmaf(m1, wv.y, dz);
    dz = fmaf(m2, wv.z, dz);
    dz = fmaf(m3, wv.w, dz);
    dz *= 1.f / kHpg;
  } else {
    dz = bf_lo(qav.x) * wv.x;
    dz = fmaf(bf_hi(qav.x), wv.y, dz);
    dz = fmaf(bf_lo(qav.y), wv.z, dz);
    dz = fmaf(bf_hi(qav.y), wv.w, dz);
  }
  const float sc = wave_sum_u(dk) * a.sl2e;
  dz = wave_sum_u(dz);

  // weights: local read = ring parts 0 .. sr-1 plus the current token;
  // anchor read = bank parts sr .. S-1 (an empty bank reads as zero), the
  // gate folded into its weights
  const bool ring = lane < sr, bank = have && !ring;
  const float M = fmaxf(wave_max_u(ring ? mp : -INFINITY), sc);
  const float fr = ring ? fast_exp2(mp - M) : 0.f;  // m = -inf -> 0
  const float fc = fast_exp2(sc - M);
  const float L = wave_sum_u(lp * fr) + fc;
  const float M2 = wave_max_u(bank ? mp : -INFINITY);
  const float fb = (bank && mp != -INFINITY) ? fast_exp2(mp - M2) : 0.f;
  const float L2 = wave_sum_u(lp * fb);
  const float il = 1.f / L;
  const float ga = (n > 0 && L2 > 0.f) ? tanhf(dz) / L2 : 0.f;
  const float w = ring ? fr * il : fb * ga;  // weight of part `lane`
  const float wc = fc * il;

  float o[4] = {wc * bf_lo(vv.x), wc * bf_hi(vv.x), wc * bf_lo(vv.y), wc * bf_hi(vv.y)};
#pragma unroll
  for (int sp = 0; sp < 2 * kMaxSplits; ++sp) {
    const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp));
    o[0] = fmaf(po[sp].x, ws, o[0]);
    o[1] = fmaf(po[sp].y, ws, o[1]);
    o[2] = fmaf(po[sp].z, ws, o[2]);
    o[3] = fmaf(po[sp].w, ws, o[3]);
  }
  uint16_t* outp = a.out + (size_t)b * a.out_bs + (size_t)(g * kHpg + h) * kD + 4 * lane;
  *reinterpret_cast<uint2*>(outp) =
      make_uint2((uint32_t)to_bf16(o[0]) | ((uint32_t)to_bf16(o[1]) << 16),
                 (uint32_t)to_bf16(o[2]) | ((uint32_t)to_bf16(o[3]) << 16));

  // Write: ring slot t mod R takes the current K/V (after every read of
  // this step, which all finished in the attention kernel), and pending
  // slot t mod C takes the candidate record and score; one wave each.
  if (lane < 32) {
    if (h == 0) {
      uint4* rk = reinterpret_cast<uint4*>(a.ring_k + (size_t)u * a.Rk * kD);
      store16_nt(&rk[k_chunk_index(tp.ring_slot, lane, a.Rk)], reinterpret_cast<const uint4*>(a.k + kvo)[lane]);
    } else if (h == 1) {
      uint4* rv = reinterpret_cast<uint4*>(a.ring_v + ((size_t)u * a.R + tp.ring_slot) * kD);
      store16_nt(&rv[lane], reinterpret_cast<const uint4*>(a.v + kvo)[lane]);
    } else if (h == 2) {
      uint4* pk = reinterpret_cast<uint4*>(a.pend_k + ((size_t)u * a.C + tp.pend_slot) * kD);
      store16_nt(&pk[lane], reinterpret_cast<const uint4*>(a.ck + kvo)[lane]);
    } else {
      uint4* pv = reinterpret_cast<uint4*>(a.pend_v + ((size_t)u * a.C + tp.pend_slot) * kD);
      store16_nt(&pv[lane], reinterpret_cast<const uint4*>(a.cv + kvo)[lane]);
      if (lane == 0) a.pscore[(size_t)u * a.C + tp.pend_slot] = a.cs[(size_t)b * a.cs_bs + g];
    }
  }

  // per-sequence positions: the token completes its block -> admit now
  // (the stores above are complete and visible to the block after the
  // barrier; no other workgroup touches this unit)
  if (a.pos != nullptr && ((int64_t)tp.pos + 1) % a.C == 0) {  // 64-bit: pos may be 2^31 - 1
    __syncthreads();
    AdmitUnit au;
    au.bank_k = a.bank_k + (size_t)u * a.N * kD;
    au.bank_v = a.bank_v + (size_t)u * a.N * kD;
    au.bscore = a.bscore + (size_t)u * a.N;
    au.bsrc = a.bsrc + (size_t)u * a.N;
    au.bank_n = a.bank_n + u;
    au.pend_k = a.pend_k + (size_t)u * a.C * kD;
    au.pend_v = a.pend_v + (size_t)u * a.C * kD;
    au.pscore = a.pscore + (size_t)u * a.C;
    au.N = a.N;
    au.C = a.C;
    au.block_start = (int64_t)tp.pos + 1 - a.C;
    admit_unit(au, sh);
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t value, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// bank_n of units (l * B + b) * G + g for b in [first, first + count):
// thread i -> layer i / (count * G), offset i mod (count * G).
__global__ void seq_bank_n_kernel(int32_t* bank_n, int L, int B, int G, int first, int count,
                                  int32_t value) {
  const int per = count * G;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= L * per) return;
  const int l = i / per, r = i - l * per;
  bank_n[((size_t)l * B + first) * G + r] = value;
}


// Workgroups of a kernel that are resident at once on the current device
// (CUs x workgroups per CU), computed once per device (host threads may
// race to fill an entry: each computes and stores the same value).
template <bool kWhole, bool kQA, int kW, bool kGG = false>
int resident_workgroups() {
  static std::atomic<int> cached[64];  // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int r = cached[dev].load(std::memory_order_relaxed);
  if (r == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu,
                                                     decode_attn_kernel<kWhole, kQA, kW, kGG>,
                                                     64 * kW, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    r = cus * per_cu;
    cached[dev].store(r, std::memory_order_relaxed);
  }
  return r;
}

template <bool kQA, int kW, bool kGG>
hipError_t launch_whole(const DecodeArgs& a, hipStream_t s) {
  int grid = (a.units + kW - 1) / kW;
  const int res = resident_workgroups<true, kQA, kW, kGG>();
  if (grid > res) grid = res;
  hipLaunchKernelGGL((decode_attn_kernel<true, kQA, kW, kGG>), dim3(grid), dim3(64 * kW), 0, s, a,
                     a.units);
  return hipGetLastError();
}

// The whole-unit launch with its template choices: a separate anchor
// query (kQA), one-wave or four-wave workgroups, and the per-group gate
// (kGG, a separate instantiation so that the default finish keeps its
// code: a runtime test there cost 4 us per launch at batch 512).
template <bool kQA>
hipError_t launch_whole_gate(const DecodeArgs& a, bool one, hipStream_t s) {
  if (a.gate_group)
    return one ? launch_whole<kQA, 1, true>(a, s) : launch_whole<kQA, kWaves, true>(a, s);
  return one ? launch_whole<kQA, 1, false>(a, s) : launch_whole<kQA, kWaves, false>(a, s);
}

// The launch rule below: true for a whole-unit launch (and *one: one-wave
// workgroups), false for the split launch.
bool whole_unit_launch(const DecodeArgs& a, bool* one) {
  const bool qa = a.qa != nullptr;
  const int waves = kWaves * (qa ? resident_workgroups<true, true, kWaves>()
                                 : resident_workgroups<true, false, kWaves>());
  const int rounds = (a.units + waves - 1) / waves;
  const int last = a.units - (rounds - 1) * waves;
  const bool wide = (int64_t)last * 8 >= (int64_t)waves * 5;  // last round >= 5/8 of the waves
  const bool mid = rounds > 1 && (int64_t)last * 8 >= (int64_t)waves * 3;  // later round >= 3/8
  // one-wave workgroups with at least one unit per wave; four-wave ones
  // for a single round (5/8 of the waves or more)
  *one = a.units >= waves || !wide;
  return wide || mid;
}

// Split-K partials for the allocation-free entry point: a static device
// array, one per GPU the library runs on, held until the process ends.
// Host code never names it directly (its name there is a host stand-in,
// not a device address); it uses the address from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

}  // namespace

int decode_whole_prefix(const DecodeArgs& a) {
  const bool qa = a.qa != nullptr;
  const int waves = kWaves * (qa ? resident_workgroups<true, true, kWaves>()
                                 : resident_workgroups<true, false, kWaves>());
  if (waves <= 0 || a.units <= waves) return 0;
  const int rounds = (a.units + waves - 1) / waves;
  const int last = a.units - (rounds - 1) * waves;
  if ((int64_t)last * 8 >= (int64_t)waves * 5) return 0;  // whole units fill the last round
  const int k = (rounds - 1) * waves;
  return k - k % a.G;  // whole sequences
}

size_t decode_scratch_bytes(const DecodeArgs& a) {
  bool one = false;
  if (whole_unit_launch(a, &one)) return 0;
  return (size_t)a.units * (a.splits_ring + a.splits_bank) * kPart * sizeof(float);
}

hipError_t static_scratch(int device, float** out) {
  static std::atomic<float*> cached[64];  // per device, zero-initialised
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  float* p = cached[device].load(std::memory_order_acquire);
  if (p == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    cached[device].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  // Whole-unit launch when the last round of units occupies at least 5/8
  // of the waves, or 3/8 when it follows full rounds; else the split
  // launch.  Measured on MI355X
  // (1,024 waves, 1 layer, per token, non-temporal loads, padded ring K
  // planes): whole-unit wins from batch 160 (640 units) up to 255 and at
  // batch 448 (a last round of 768: 594 against 673 us); the split wins
  // below 160 (at 96: 142 against 153 us; at 128: 178 against 190; at 112
  // whole units win by 3%) and at 288-320 (last rounds of 128-256 units:
  // 455 against 466 us at 320); at 352 (a last round of 384 after a full
  // one) whole units win, 491 against 518 us.  (Callers hand a batch
  // with a later round under 5/8 full to this function in two parts, see
  // decode_whole_prefix; the 3/8 rule remains for the whole batch when the
  // remainder's partials would not fit the scratch.)  With at least one unit per wave, one-wave
  // workgroups (704 against 713 us per launch at batch 512, 637 against
  // 651 at 448); for a single round of 5/8 or more, four-wave ones, which
  // fill fewer CUs completely (237 against 241 us at batch 160, 272
  // against 281 at 192); below 5/8, one-wave ones again (232 against 240
  // at 144).
  const bool qa = a.qa != nullptr;
  bool one = false;
  if (whole_unit_launch(a, &one)) {
    hipError_t e = qa ? launch_whole_gate<true>(a, one, s) : launch_whole_gate<false>(a, one, s);
    if (e != hipSuccess || a.pos == nullptr) return e;
    // per-sequence positions: admit the units whose block this token ends
    AdmitArgs ad;
    ad.bank_k = a.bank_k;
    ad.bank_v = a.bank_v;
    ad.bscore = a.bscore;
    ad.bsrc = a.bsrc;
    ad.bank_n = a.bank_n;
    ad.pend_k = a.pend_k;
    ad.pend_v = a.pend_v;
    ad.pscore = a.pscore;
    ad.unit0 = 0;  // the pointers are already the layer's
    ad.units = a.units;
    ad.N = a.N;
    ad.C = a.C;
    ad.block_start = 0;
    ad.pos = a.pos;
    ad.G = a.G;
    ad.pos_add = 0;
    ad.aligned_only = 0;
    return launch_admit(ad, s);
  }
  const int S = a.splits_ring + a.splits_bank;
  const int items = a.units * S;
  if (a.tiles_ring == 1 && a.tiles_bank == 1) {  // one tile per part
    if (a.units <= 4)
      hipLaunchKernelGGL(decode_part_kernel<true>, dim3(items), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(decode_part_kernel<false>, dim3(items), dim3(256), 0, s, a);
  } else {
    int grid = (items + kWaves - 1) / kWaves;
    const int res = resident_workgroups<false, false, kWaves>();
    if (grid > res) grid = res;
    hipLaunchKernelGGL((decode_attn_kernel<false, false, kWaves>), dim3(grid), dim3(64 * kWaves), 0,
                       s, a, items);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.units), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_seq_bank_n(int32_t* bank_n, int L, int B, int G, int first, int count,
                             int32_t value, hipStream_t s) {
  const int n = L * count * G;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(seq_bank_n_kernel, dim3((n + 255) / 256), dim3(256), 0, s, bank_n, L, B, G,
                     first, count, value);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

}  // namespace rma
