// Admit of one (sequence, layer, group) unit by one 256-thread workgroup:
// the device code shared by the admit kernel (lockstep and per-sequence
// admits of whole layers) and the small-batch decode combine kernel (which
// admits a unit's block in the same workgroup that wrote its last
// candidate).  Internal; not part of the public ABI.
//
// Semantics: EdgeRock model card (ModelScope), "How Rock Memory Anchors
// work" (every 256 tokens admission keeps the highest-priority records per
// KV group; a kept record is neither merged with others nor modified); ai-primer
// three-operation list, item 2; tpsreport "How it works" (top 1,024 of
// anchors plus 256 candidates, independently in each group).
// Readings: order = score descending then global index ascending (anchor
// slot i has index i, pending slot j has index N + j); -0.0 equals +0.0;
// every NaN ranks below -inf; evicted slots (ascending) take admitted
// candidates (ascending j); the remainder is appended at n, n+1, ...
//
// Selection by threshold: each pool entry becomes the 64-bit key
//   (order-preserving image of the score) << 32 | (0xFFFFFFFF - index),
// so that the order above is the descending order of distinct integers;
// an entry is kept iff its key is at least the K-th largest key,
// K = min(N, n + C).  The K-th largest key comes from a radix select,
// most-significant 8-bit digit first: a 256-bin LDS histogram of the keys
// that still match the chosen digits, a block scan to find the digit whose
// bin holds the K-th, until that bin holds a single key (at most 8
// passes).  No sort and no all-pairs comparison.
#pragma once
#include "rma_kernels.h"

namespace rma {

constexpr int kMaxPool = 2048;  // N + C (the configuration check enforces it)
constexpr int kAdmitThreads = 256;
static_assert(9 * kAdmitThreads >= kMaxPool, "each thread holds at most 9 pool entries");

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
  int hist[256];      // radix-select histogram
  int sel[3];         // chosen digit, keys above it, keys in its bin
  uint64_t kth;       // the K-th largest key, once found
  int evicted[256];
  int admitted[256];
  int lds4[4];
};

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte store with the non-temporal hint: the moved records are
// written once and next read by the decode's non-temporal stream.  With
// the hint the stress round of scattered 16-byte K pieces takes 3.7
// instead of 4.3 ms.
__device__ __forceinline__ void admit_store_nt(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

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
// of the threads before this one and writes the total to *total.  kSync:
// end with a barrier, so that lds4 may be written again at once (a caller
// that meets a barrier before its next scan passes false).
template <bool kSync = true>
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
  if (kSync) __syncthreads();
  *total = all;
  return before + x - v;
}

// Pool entries per thread: thread tid holds entries tid * kPool ..
// tid * kPool + kPool - 1 (bank_cap + commit <= 2,048 = 256 x 8).
constexpr int kPool = 8;

// The k-th largest (1 <= k <= valid keys) of the keys kv[r] held by the
// block's threads (entry i = tid * kPool + r, valid iff i < P; keys are
// distinct), by a radix select over 8-bit digits, most significant first.
// Four barriers per pass: after the histogram, inside the scan, after the
// digit is chosen, and one that both orders the reads of the choice before
// the next pass and publishes the next pass's cleared histogram.
__device__ inline uint64_t admit_kth_largest(const uint64_t (&kv)[kPool], int P, int k,
                                             AdmitShared& sh) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;  // the digits chosen so far
  sh.hist[tid] = 0;
  __syncthreads();
  for (int shift = 56; shift >= 0; shift -= 8) {
    const uint64_t above_mask = shift == 56 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
    for (int r = 0; r < kPool; ++r) {
      const int i = tid * kPool + r;
      if (i < P && (kv[r] & above_mask) == prefix)
        atomicAdd(&sh.hist[(int)((kv[r] >> shift) & 255u)], 1);
    }
    __syncthreads();
    // bins in descending digit order: thread tid holds digit 255 - tid
    // (the scan's lds4 is next written after two more barriers)
    const int cnt = sh.hist[255 - tid];
    int tot = 0;
    const int above = admit_block_scan<false>(cnt, &tot, sh.lds4);  // keys with a larger digit
    if (above < k && k <= above + cnt) {
      sh.sel[0] = 255 - tid;
      sh.sel[1] = above;
      sh.sel[2] = cnt;
    }
    __syncthreads();  // the choice is visible; every bin has been read
    k -= sh.sel[1];
    prefix |= (uint64_t)sh.sel[0] << shift;
    if (sh.sel[2] == 1) {  // one key left with these digits: it is the k-th
      const uint64_t mask = ~0ull << shift;
#pragma unroll
      for (int r = 0; r < kPool; ++r) {
        const int i = tid * kPool + r;
        if (i < P && (kv[r] & mask) == prefix) sh.kth = kv[r];
      }
      __syncthreads();
      const uint64_t t = sh.kth;
      __syncthreads();  // every thread has read sel and kth before they change
      return t;
    }
    sh.hist[tid] = 0;  // the next pass's histogram
    __syncthreads();   // ... and every thread has read sel before it is written again
  }
  return prefix;
}

__device__ inline void admit_unit(const AdmitUnit& a, AdmitShared& sh) {
  const int tid = threadIdx.x;
  const int N = a.N, C = a.C;
  const int n = *a.bank_n;
  const int P = n + C;
  const int K = P < N ? P : N;
  static_assert(kAdmitThreads * kPool >= 2048, "the largest pool (bank_cap + commit)");

  // the pool's keys, entry i = tid * kPool + r (past the pool: 0, below
  // every real key); P <= N keeps everything, with no selection
  uint64_t kv[kPool];
  uint64_t thr = 0;  // kept iff key >= thr
  if (P > N) {
    // all score loads first (one memory round trip); past the pool: a
    // clamped re-read, replaced by the key 0
    float sv[kPool];
#pragma unroll
    for (int r = 0; r < kPool; ++r) {
      const int i = tid * kPool + r;
      const int ia = i < n ? i : n - 1;
      const int ic = i - n < C ? (i - n > 0 ? i - n : 0) : C - 1;
      sv[r] = i < n ? a.bscore[ia > 0 ? ia : 0] : a.pscore[ic];
    }
#pragma unroll
    for (int r = 0; r < kPool; ++r) {
      const int i = tid * kPool + r;
      kv[r] = i < n ? admit_pool_key(sv[r], (uint32_t)i)
                    : (i < P ? admit_pool_key(sv[r], (uint32_t)(N + (i - n))) : 0ull);
    }
    thr = admit_kth_largest(kv, P, K, sh);
  } else {
#pragma unroll
    for (int r = 0; r < kPool; ++r) kv[r] = 0;
  }

  // evicted anchors and admitted candidates, both ascending: each thread
  // holds a contiguous run of the pool, so one block scan of the threads'
  // counts places every entry (the two counts share the scan: each is
  // < 2^16)
  uint32_t evm = 0, adm = 0;  // bit r: entry tid * kPool + r is evicted / admitted
#pragma unroll
  for (int r = 0; r < kPool; ++r) {
    const int i = tid * kPool + r;
    const bool kept = kv[r] >= thr;
    evm |= (i < n && !kept) ? 1u << r : 0u;
    adm |= (i >= n && i < P && kept) ? 1u << r : 0u;
  }
  int tot = 0;
  const int before =
      admit_block_scan(__builtin_popcount(evm) | (__builtin_popcount(adm) << 16), &tot, sh.lds4);
  {
    int pe = before & 0xffff, pa = before >> 16;
#pragma unroll
    for (int r = 0; r < kPool; ++r) {
      const int i = tid * kPool + r;
      if (evm & (1u << r)) sh.evicted[pe++] = i;
      if (adm & (1u << r)) sh.admitted[pa++] = i - n;
    }
  }
  const int ne = tot & 0xffff, na = tot >> 16;
  __syncthreads();

  // move the admitted records, K and V together in 4 batches, each with
  // all its loads issued before its first store (a lone unit's admit is a
  // chain of memory round trips: 4 of them instead of 8 with K and V in
  // separate loops).  K: thread r moves record r (na <= C <= 256 =
  // threads) chunk plane by chunk plane, 8 chunks (128 contiguous bytes of
  // its pending row) per batch; one store instruction then writes one
  // chunk plane for 64 consecutive records, whose destination slots ascend
  // (evicted slots in ascending order, then the appended ones), so records
  // whose slots share a cache line leave in one write request instead of
  // one each.  Threads past na load record 0's chunks and store nothing.
  // V: copy w moves chunk w % 32 of record w / 32 as rows (a record's V row
  // is one 512-byte run on both sides), 8 copies per thread per batch;
  // past the end a lane repeats the last copy (same value, same place).
  // Named registers rather than arrays keep the batches out of scratch;
  // the record stores carry the non-temporal hint.
  uint4* bk = reinterpret_cast<uint4*>(a.bank_k);
  uint4* bv = reinterpret_cast<uint4*>(a.bank_v);
  const uint4* pk = reinterpret_cast<const uint4*>(a.pend_k);
  const uint4* pv = reinterpret_cast<const uint4*>(a.pend_v);
  static_assert(kAdmitThreads >= 256, "one thread per admitted record (commit <= 256)");
  static_assert(kChunks == 32 && 4 * 8 * kAdmitThreads >= 256 * kChunks,
                "4 batches of 8 cover every K chunk and every V copy");
  const int total = na * kChunks;  // V copies
  constexpr int T = kAdmitThreads;
  const bool kmove = tid < na;
  // na > 0 (uniform): every clamped index below names a real admitted record
  for (int b = 0; na > 0 && b < kChunks / 8; ++b) {
    const uint4* ksrc = pk + (size_t)sh.admitted[kmove ? tid : 0] * kChunks;
    const int kdst = kmove ? (tid < ne ? sh.evicted[tid] : n + (tid - ne)) : 0;
    auto vsrc = [&](int w) -> size_t {
      const int wc = w < total ? w : total - 1;
      return (size_t)sh.admitted[wc / kChunks] * kChunks + (wc % kChunks);
    };
    auto vdst = [&](int w) -> size_t {
      const int wc = w < total ? w : total - 1;
      const int r = wc / kChunks, c = wc % kChunks;
      return (size_t)(r < ne ? sh.evicted[r] : n + (r - ne)) * kChunks + c;
    };
    const int base = tid + b * 8 * T;
    const int c0 = 8 * b;
    const uint4 k0 = ksrc[c0], k1 = ksrc[c0 + 1], k2 = ksrc[c0 + 2], k3 = ksrc[c0 + 3],
                k4 = ksrc[c0 + 4], k5 = ksrc[c0 + 5], k6 = ksrc[c0 + 6], k7 = ksrc[c0 + 7];
    const uint4 v0 = pv[vsrc(base)], v1 = pv[vsrc(base + T)], v2 = pv[vsrc(base + 2 * T)],
                v3 = pv[vsrc(base + 3 * T)], v4 = pv[vsrc(base + 4 * T)],
                v5 = pv[vsrc(base + 5 * T)], v6 = pv[vsrc(base + 6 * T)],
                v7 = pv[vsrc(base + 7 * T)];
    if (kmove) {
      admit_store_nt(&bk[k_chunk_index(kdst, c0, N)], k0);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 1, N)], k1);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 2, N)], k2);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 3, N)], k3);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 4, N)], k4);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 5, N)], k5);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 6, N)], k6);
      admit_store_nt(&bk[k_chunk_index(kdst, c0 + 7, N)], k7);
    }
    if (base < total) {
      admit_store_nt(&bv[vdst(base)], v0);
      admit_store_nt(&bv[vdst(base + T)], v1);
      admit_store_nt(&bv[vdst(base + 2 * T)], v2);
      admit_store_nt(&bv[vdst(base + 3 * T)], v3);
      admit_store_nt(&bv[vdst(base + 4 * T)], v4);
      admit_store_nt(&bv[vdst(base + 5 * T)], v5);
      admit_store_nt(&bv[vdst(base + 6 * T)], v6);
      admit_store_nt(&bv[vdst(base + 7 * T)], v7);
    }
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
