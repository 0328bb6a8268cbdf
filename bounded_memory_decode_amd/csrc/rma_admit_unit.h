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

// The k-th largest (1 <= k <= valid keys) of the keys kv[r] held by the
// block's threads (entry i = r * 256 + tid, valid iff i < P; keys are
// distinct), by a radix select over 8-bit digits, most significant first.
__device__ inline uint64_t admit_kth_largest(const uint64_t (&kv)[9], int P, int k,
                                             AdmitShared& sh) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;  // the digits chosen so far
  for (int shift = 56; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0;
    __syncthreads();
    const uint64_t above_mask = shift == 56 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
    for (int r = 0; r < 9; ++r) {
      const int i = r * kAdmitThreads + tid;
      if (i < P && (kv[r] & above_mask) == prefix)
        atomicAdd(&sh.hist[(int)((kv[r] >> shift) & 255u)], 1);
    }
    __syncthreads();
    // bins in descending digit order: thread tid holds digit 255 - tid
    const int cnt = sh.hist[255 - tid];
    int tot = 0;
    const int above = admit_block_scan(cnt, &tot, sh.lds4);  // keys with a larger digit
    if (above < k && k <= above + cnt) {
      sh.sel[0] = 255 - tid;
      sh.sel[1] = above;
      sh.sel[2] = cnt;
    }
    __syncthreads();
    k -= sh.sel[1];
    prefix |= (uint64_t)sh.sel[0] << shift;
    if (sh.sel[2] == 1) {  // one key left with these digits: it is the k-th
      const uint64_t mask = ~0ull << shift;
#pragma unroll
      for (int r = 0; r < 9; ++r) {
        const int i = r * kAdmitThreads + tid;
        if (i < P && (kv[r] & mask) == prefix) sh.kth = kv[r];
      }
      __syncthreads();
      const uint64_t t = sh.kth;
      __syncthreads();  // every thread has read sel and kth before they change
      return t;
    }
    __syncthreads();  // every thread has read sel before the next pass writes it
  }
  return prefix;
}

__device__ inline void admit_unit(const AdmitUnit& a, AdmitShared& sh) {
  const int tid = threadIdx.x;
  const int N = a.N, C = a.C;
  const int n = *a.bank_n;
  const int P = n + C;
  const int K = P < N ? P : N;
  const int R = (P + kAdmitThreads - 1) / kAdmitThreads;  // keys per thread, <= 8

  // the pool's keys, entry i = r * 256 + tid (past the pool: 0, below every
  // real key); P <= N keeps everything, with no selection
  uint64_t kv[9];
  uint64_t thr = 0;  // kept iff key >= thr
  if (P > N) {
    // all score loads first (one memory round trip); past the pool: a
    // clamped re-read, replaced by the key 0
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
      kv[r] = i < n ? admit_pool_key(sv[r], (uint32_t)i)
                    : (i < P ? admit_pool_key(sv[r], (uint32_t)(N + (i - n))) : 0ull);
    }
    thr = admit_kth_largest(kv, P, K, sh);
  } else {
#pragma unroll
    for (int r = 0; r < 9; ++r) kv[r] = 0;
  }

  // evicted anchors and admitted candidates, both ascending: pool entry
  // i = r * 256 + tid, round by round, through block scans (the two
  // counts share one scan: each is < 2^16)
  int ne = 0, na = 0;
  for (int r = 0; r < R; ++r) {
    const int i = r * kAdmitThreads + tid;
    uint64_t key = kv[0];
#pragma unroll
    for (int x = 1; x < 9; ++x) key = r == x ? kv[x] : key;
    const bool kept = key >= thr;
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
