// Internal launcher interface between the C-ABI host code (rma_host.cpp)
// and the gfx950 kernels.  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rma.h"

namespace rma {

constexpr int kD = 256;       // head dimension the kernels are built for
constexpr int kHpg = 4;       // query heads per KV group
constexpr int kTile = 64;     // keys per wave tile
constexpr int kChunks = kD / 8;  // 16-byte chunks per K/V row
constexpr int kPart = kHpg * kD + 2 * kHpg;  // floats per split partial
constexpr int kMaxSplits = 16;  // split-K parts per read (ring, bank)

// K planes are chunk-major: the 16-byte chunk c (dims 8c .. 8c+7) of slot
// s of a plane with `slots` slots lives at uint4 index c * slots + s.  A
// tile's K then spreads over 32 regions of the plane, one 1 KiB run per
// chunk (measured faster on MI355X than a contiguous 32 KiB tile block,
// which concentrates a wave's loads on fewer channels).
__host__ __device__ inline size_t k_chunk_index(int slot, int c, int slots) {
  return (size_t)c * slots + slot;
}

// Slots of a ring K plane: the ring's R slots rounded up to a multiple of
// 64, so that every chunk plane starts on a 1 KiB boundary and a tile's
// 1 KiB chunk run does not straddle cache lines (R = 1,023: 1,024 slots,
// one padding slot that is never read or written).  Measured on MI355X at
// batch 512: 660 us per decode launch against 673 with a 1,023-slot stride.
__host__ __device__ inline int ring_k_slots(int R) { return (R + 63) / 64 * 64; }

// One decode token of one layer.
struct DecodeArgs {
  const uint16_t* q;       // [B][H][D]
  const uint16_t* qa;      // [B][H][D] query of the anchor read and the gate, or null: q
  const uint16_t* k;       // [B][G][D]
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  const float* cs;         // [B][G]
  const float* w_g;        // [H][D], or [G][D] with gate_group
  uint16_t* out;           // [B][H][D]
  uint16_t* ring_k;        // layer base, unit stride Rk*D
  uint16_t* ring_v;
  uint16_t* bank_k;        // layer base, unit stride N*D (written only by
  uint16_t* bank_v;        // the per-sequence admit)
  int32_t* bank_n;         // [B*G] of this layer
  float* bscore;           // layer base, unit stride N
  int32_t* bsrc;
  uint16_t* pend_k;        // layer base, unit stride C*D
  uint16_t* pend_v;
  float* pscore;           // layer base, unit stride C
  float* part;             // scratch: [units][splits][kPart]
  const int32_t* pos;      // [B] position of each sequence's token (< 0: the
                           // sequence is left out), or null: every sequence
                           // at the lockstep position below
  int64_t q_bs;            // elements between sequences in q
  int64_t kv_bs;           // ... in k, v, ck, cv
  int64_t cs_bs;           // ... in cs
  int64_t out_bs;          // ... in out
  int units;               // B*G
  int G, H, R, N, C;
  int Rk;                  // ring K plane slots (ring_k_slots(R))
  int ring_count;          // lockstep: valid ring slots, min(t, R)
  int ring_slot;           // lockstep: t mod R
  int pend_slot;           // lockstep: t mod C
  int splits_ring, splits_bank;
  int tiles_ring, tiles_bank;  // tiles per split
  int gate_group;          // 1: one gate per (token, group) from the mean anchor query
  float sl2e;              // scale * log2(e)
};

// The decode of one token; with per-sequence positions (a.pos), also the
// admit of every unit whose block the token completes.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Units of a batch that the hybrid launch gives the whole-unit kernel:
// its full rounds of resident waves, in whole sequences, when a
// whole-unit launch of the batch would fill less than 5/8 of the waves in
// a later round; 0 for a batch of one round or a well-filled last round.
// The caller decodes those sequences with launch_decode on their own,
// then the rest with their own split plan.
int decode_whole_prefix(const DecodeArgs& a);

// Bytes of split-K partials (a.part) launch_decode(a) writes and reads on
// the current device: 0 when it takes the whole-unit launch.
size_t decode_scratch_bytes(const DecodeArgs& a);

// Size of the library's static device scratch array (the partials of the
// allocation-free decode call), and its address on `device`, looked up
// once per device with hipGetSymbolAddress and cached.
constexpr size_t kStaticScratchBytes = RMA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(int device, float** out);

// A chunked-prefill block of one layer.
struct PrefillArgs {
  const uint16_t* q;       // [B][n][H][D]
  const uint16_t* qa;      // [B][n][H][D] query of the anchor read and the gate, or null: q
  const uint16_t* k;       // [B][n][G][D]
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  const float* cs;         // [B][n][G]
  const float* w_g;        // [H][D], or [G][D] with gate_group
  uint16_t* out;           // [B][n][H][D]
  uint16_t* ring_k;        // layer bases as in DecodeArgs
  uint16_t* ring_v;
  const uint16_t* bank_k;
  const uint16_t* bank_v;
  const int32_t* bank_n;
  uint16_t* pend_k;
  uint16_t* pend_v;
  float* pscore;
  const int32_t* pos;      // [B] block start of each sequence (a sequence
                           // whose entry is < 0 or not a multiple of C is
                           // left out), or null: every sequence at P
  float* part;             // scratch of the split launch (small batches):
                           // [B][n][H][pf_loc + pf_bank][kPfPart]
  int pf_loc, pf_bank;     // split launch: slices of the local and anchor reads
  int B, G, H, R, N, C;
  int Rk;                  // ring K plane slots (ring_k_slots(R))
  int n;                   // tokens in the block (1 .. C)
  int64_t P;               // lockstep: position of the block's first token
  int gate_group;          // 1: one gate per (token, group) from the mean anchor query
  float sl2e;              // scale * log2(e)
};

// Launch plan of a prefill block.  A full block of one (sequence, group)
// is 8 query tiles of 32 tokens (one 8-wave workgroup each); when the batch
// gives fewer than 256 such workgroups (one per CU), each query tile's
// local read is cut in `loc` slices of its tiles and its anchor read in
// `bank`, one workgroup per slice, whose partials (o[D], m, l) are merged
// by a second kernel.  A function of the batch only, so that the scratch
// size is known at layout time.
constexpr int kPfMaxSplits = 8;
constexpr int kPfPart = kD + 4;  // floats per partial: o[D], m, l, padding
struct PrefillPlan {
  int loc, bank;  // slices of the local and anchor reads; 0, 0: no split
  int parts() const { return loc + bank; }
  bool split() const { return loc > 0; }
};
inline PrefillPlan prefill_plan(int batch, int groups) {
  const int units = batch * groups;
  if (units <= 4) return {4, 4};
  if (units <= 8) return {2, 2};
  if (units <= 16) return {1, 1};
  return {0, 0};
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// Admit of one or more layers.
struct AdmitArgs {
  uint16_t* bank_k;        // region base (unit 0)
  uint16_t* bank_v;
  float* bscore;
  int32_t* bsrc;
  int32_t* bank_n;
  const uint16_t* pend_k;
  const uint16_t* pend_v;
  const float* pscore;
  int unit0;               // first unit (layer * B * G)
  int units;               // units to admit
  int N, C;
  int64_t block_start;     // lockstep: position of pending slot 0
  // Per-sequence mode (pos != null, one layer, unit0 + i = unit of
  // sequence i / G): sequence b's last written token is pos[b] + pos_add;
  // its units are admitted iff pos[b] >= 0 (and, if aligned_only, pos[b]
  // is a multiple of C) and that token completes a block.
  const int32_t* pos;
  int G;
  int pos_add;
  int aligned_only;
};

hipError_t launch_admit(const AdmitArgs& a, hipStream_t s);

// Fill an int32 array on the device.
hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);

// Set the bank counts of sequences first .. first+count-1 in every layer
// (bank_n region base; units (layer * B + b) * G + g).
hipError_t launch_seq_bank_n(int32_t* bank_n, int L, int B, int G, int first, int count,
                             int32_t value, hipStream_t s);

}  // namespace rma
