// Admit of one (sequence, layer, group) unit by one 256-thread workgroup:
// the device code shared by the admit kernel (lockstep and per-sequence
// admits of whole layers) and the small-batch decode combine kernel (which
// admits a unit's block in the same workgroup that wrote its last
// candidate).  Internal; not part of the public ABI.
//
// Semantics: EdgeRock model card (ModelScope), "How Rock Memory Anchors
// work" (every 256 tokens admission keeps the highest-priority records per
// KV group; retained records stay separate and unchanged); ai-primer
// three-operation list, item 2; tpsreport "How it works" (top 1,024 of
// anchors plus 256 candidates, independently in each group).
// Readings: order = score descending then global index ascending (anchor
// slot i has index i, pending slot j has index N + j); -0.0 equals +0.0;
// every NaN ranks below -inf; evicted slots (ascending) take admitted
// candidates (ascending j); the remainder is appended at n, n+1, ...
//
// Selection by rank: each pool entry becomes the 64-bit key
//   (order-preserving image of the score) << 32 | (0xFFFFFFFF - index),
// so that the order above is the descending order of distinct integers;
// an entry is kept iff fewer than K = min(N, n + C) keys exceed it.  Every
// thread counts, for the keys it owns, the keys above them in one pass
// over the pool in LDS (broadcast reads), so there is no sort and no
// barrier inside the selection.
#pragma once
#include "rma_kernels.h"

namespace rma {

constexpr int kMaxPool = 2048;  // N + C
constexpr int kAdmitThreads = 256;

// One unit's records and counts.
struct AdmitUnit {
  uint16_t* bank_k;        // the unit's K plane (chunk-major, N slots)
  uint16_t* bank_v;        // the unit's V rows
  float* bscore;           // [N]
  int32_t* bsrc;           // [N]
  int32_t* bank_n;         // the unit's count
  const uint16_t* pend_k;  // [C][D]
  const uint16_t* pend_v;
  const float* pscore;     // [C]
  int N, C;
  int64_t block_start;     // position of pending slot 0
};

struct AdmitShared {
  alignas(16) uint64_t key[kMaxPool + 2];  // + padding for pairwise reads
  int evicted[256];
  int admitted[256];
  int lds4[4];
};

// Order-preserving map of fp32 to uint32 (larger float -> larger key),
// with NaN -> 0 (below -inf, whose image is 0x007FFFFF) and -0 -> +0.
__device__ __forceinline__ uint32_t admit_score_key(float f) {
  uint32_t u = __float_as_uint(f);
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0u;
  if (mag == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Every real key is >= 0xFFFFFFFF - 2047 > 0, so 0 pads without counting.
__device__ __forceinline__ uint64_t admit_pool_key(float score, uint32_t gidx) {
  return ((uint64_t)admit_score_key(score) << 32) | (uint64_t)(0xffffffffu - gidx);
}

// Exclusive prefix sum over the 256 threads of the block; returns the sum
// of the threads before this one and writes the total to *total.
__device__ __forceinline__ int admit_block_scan(int v, int* total, int* lds4) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds4[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += lds4[w];
    all += lds4[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// ranks of keys tid, tid + 256, ... (kR of them): keys of the pool greater
// than each, counted over key[0 .. P) (key[P], key[P+1] are 0).
template <int kR>
__device__ __forceinline__ void admit_ranks(const uint64_t* key, int P, int* rank) {
  const int tid = threadIdx.x;
  uint64_t mine[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int i = r * kAdmitThreads + tid;
    mine[r] = i < P ? key[i] : ~0ull;  // past the pool: never counted as kept
    rank[r] = 0;
  }
  const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(key);
#pragma unroll 8
  for (int j = 0; j < (P + 1) / 2; ++j) {
    const ulonglong2 kk = k2[j];
#pragma unroll
    for (int r = 0; r < kR; ++r) rank[r] += (int)(kk.x > mine[r]) + (int)(kk.y > mine[r]);
  }
}

__device__ inline void admit_unit(const AdmitUnit& a, AdmitShared& sh) {
  const int tid = threadIdx.x;
  const int N = a.N, C = a.C;
  const int n = *a.bank_n;
  const int P = n + C;
  const int K = P < N ? P : N;
  const int R = (P + kAdmitThreads - 1) / kAdmitThreads;  // keys per thread, <= 8

  // rank of every pool entry (P <= N: everything is kept, no ranking)
  int rank[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rank[r] = 0;
  if (P > N) {
    // all score loads first (one memory round trip): entry i = r*256 + tid
    // (past the pool: a clamped re-read, replaced by the padding key 0)
    float sv[9];
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      const int i = r * kAdmitThreads + tid;
      const int ia = i < n ? i : n - 1;
      const int ic = i - n < C ? (i - n > 0 ? i - n : 0) : C - 1;
      sv[r] = i < n ? a.bscore[ia > 0 ? ia : 0] : a.pscore[ic];
    }
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      const int i = r * kAdmitThreads + tid;
      if (i < P + 2)
        sh.key[i] = i < n ? admit_pool_key(sv[r], (uint32_t)i)
                          : (i < P ? admit_pool_key(sv[r], (uint32_t)(N + (i - n))) : 0ull);
    }
    __syncthreads();
    switch (R) {
      case 1: admit_ranks<1>(sh.key, P, rank); break;
      case 2: admit_ranks<2>(sh.key, P, rank); break;
      case 3: admit_ranks<3>(sh.key, P, rank); break;
      case 4: admit_ranks<4>(sh.key, P, rank); break;
      case 5: admit_ranks<5>(sh.key, P, rank); break;
      case 6: admit_ranks<6>(sh.key, P, rank); break;
      case 7: admit_ranks<7>(sh.key, P, rank); break;
      default: admit_ranks<8>(sh.key, P, rank); break;
    }
  }

  // evicted anchors and admitted candidates, both ascending: pool entry
  // i = r * 256 + tid, round by round, through block scans (the two
  // counts share one scan: each is < 2^16)
  int ne = 0, na = 0;
  for (int r = 0; r < R; ++r) {
    const int i = r * kAdmitThreads + tid;
    int rr = rank[0];
#pragma unroll
    for (int x = 1; x < 8; ++x) rr = r == x ? rank[x] : rr;
    const bool kept = rr < K;
    const int ev = (i < n && !kept) ? 1 : 0;
    const int ad = (i >= n && i < P && kept) ? 1 : 0;
    int tot = 0;
    const int before = admit_block_scan(ev | (ad << 16), &tot, sh.lds4);
    if (ev) sh.evicted[ne + (before & 0xffff)] = i;
    if (ad) sh.admitted[na + (before >> 16)] = i - n;
    ne += tot & 0xffff;
    na += tot >> 16;
  }
  __syncthreads();

  // move the admitted records: chunk c of record r is one K and one V
  // copy; 8 chunks per thread per round, all 16 loads issued before the
  // first store (a lone unit's admit is latency-bound; named registers
  // rather than an array keep the batch out of scratch).  Past the end, a
  // lane repeats the last chunk's copy (same value, same place), so the
  // batch has no branch.
  uint4* bk = reinterpret_cast<uint4*>(a.bank_k);
  uint4* bv = reinterpret_cast<uint4*>(a.bank_v);
  const uint4* pk = reinterpret_cast<const uint4*>(a.pend_k);
  const uint4* pv = reinterpret_cast<const uint4*>(a.pend_v);
  const int total = na * kChunks;
  // source and destination of copy x of the round at `base`
  auto src_of = [&](int w) {
    const int wc = w < total ? w : total - 1;
    return (size_t)sh.admitted[wc / kChunks] * kChunks + (wc % kChunks);
  };
  auto put = [&](int w, const uint4& kx, const uint4& vx) {
    const int wc = w < total ? w : total - 1;
    const int r = wc / kChunks, c = wc % kChunks;
    const int dst = r < ne ? sh.evicted[r] : n + (r - ne);
    bk[k_chunk_index(dst, c, N)] = kx;
    bv[(size_t)dst * kChunks + c] = vx;
  };
  for (int base = tid; base < total; base += 8 * kAdmitThreads) {
    constexpr int T = kAdmitThreads;
    const size_t o0 = src_of(base), o1 = src_of(base + T), o2 = src_of(base + 2 * T),
                 o3 = src_of(base + 3 * T), o4 = src_of(base + 4 * T), o5 = src_of(base + 5 * T),
                 o6 = src_of(base + 6 * T), o7 = src_of(base + 7 * T);
    const uint4 k0 = pk[o0], k1 = pk[o1], k2 = pk[o2], k3 = pk[o3], k4 = pk[o4], k5 = pk[o5],
                k6 = pk[o6], k7 = pk[o7];
    const uint4 v0 = pv[o0], v1 = pv[o1], v2 = pv[o2], v3 = pv[o3], v4 = pv[o4], v5 = pv[o5],
                v6 = pv[o6], v7 = pv[o7];
    put(base, k0, v0);
    put(base + T, k1, v1);
    put(base + 2 * T, k2, v2);
    put(base + 3 * T, k3, v3);
    put(base + 4 * T, k4, v4);
    put(base + 5 * T, k5, v5);
    put(base + 6 * T, k6, v6);
    put(base + 7 * T, k7, v7);
  }
  for (int r = tid; r < na; r += kAdmitThreads) {
    const int j = sh.admitted[r];
    const int dst = r < ne ? sh.evicted[r] : n + (r - ne);
    a.bscore[dst] = a.pscore[j];
    a.bsrc[dst] = (int32_t)(a.block_start + j);
  }
  __syncthreads();  // every thread has read n before it changes
  if (tid == 0) *a.bank_n = K;
}

}  // namespace rma
