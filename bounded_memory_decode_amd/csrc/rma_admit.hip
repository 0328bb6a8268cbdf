// Admit step of the RMA layer on gfx950: per (sequence, layer, group), the
// committed anchors and the pending candidates compete for the bank; the
// best min(N, n + C) stay; admitted candidates are copied into the evicted
// slots and then appended.
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
// One workgroup per unit.  The pool becomes 64-bit keys
//   (order-preserving image of the score) << 32 | (0xFFFFFFFF - index)
// so that a plain descending sort of distinct integers gives the order
// above; a bitonic network in LDS sorts them and the K-th key is the cut.
#include "rma_kernels.h"

namespace rma {
namespace {

constexpr int kMaxPool = 2048;

// Order-preserving map of fp32 to uint32 (larger float -> larger key),
// with NaN -> 0 (below -inf, whose image is 0x007FFFFF) and -0 -> +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0u;
  if (mag == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t pool_key(float score, uint32_t gidx) {
  return ((uint64_t)score_key(score) << 32) | (uint64_t)(0xffffffffu - gidx);
}

// Exclusive prefix sum over the 256 threads of the block; returns the sum
// of the threads before this one and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* total, int* lds4) {
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

__global__ __launch_bounds__(256) void admit_kernel(AdmitArgs a) {
  const int u = a.unit0 + blockIdx.x;
  const int tid = threadIdx.x;
  const int N = a.N, C = a.C;
  int64_t block_start = a.block_start;
  if (a.pos != nullptr) {  // per-sequence: admit only where a block just completed
    const int first = a.pos[blockIdx.x / a.G];
    if (first < 0 || (a.aligned_only && first % C != 0)) return;
    const int64_t last = (int64_t)first + a.pos_add;
    if ((last + 1) % C != 0) return;
    block_start = last + 1 - C;
  }

  __shared__ uint64_t key[kMaxPool];
  __shared__ int evicted[kMaxPool];
  __shared__ int admitted[256];
  __shared__ int lds4[4];

  const int n = a.bank_n[u];
  const int P = n + C;
  const int K = P < N ? P : N;
  const float* bs = a.bscore + (size_t)u * N;
  const float* ps = a.pscore + (size_t)u * C;

  // the cut: the K-th largest key (no selection when everything fits)
  uint64_t cut = 0;
  if (P > N) {
    int size = 64;
    while (size < P) size <<= 1;
    for (int i = tid; i < size; i += 256) {
      uint64_t k = 0;  // padding sorts last
      if (i < n) k = pool_key(bs[i], (uint32_t)i);
      else if (i < P) k = pool_key(ps[i - n], (uint32_t)(N + (i - n)));
      key[i] = k;
    }
    __syncthreads();
    for (int k2 = 2; k2 <= size; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < size; i += 256) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t x = key[i], y = key[ixj];
            const bool desc = (i & k2) == 0;
            if (desc ? (x < y) : (x > y)) {
              key[i] = y;
              key[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    cut = key[K - 1];
  }

  // evicted anchors, ascending: thread tid scans a contiguous slice
  const int per = (n + 255) / 256;
  const int lo = tid * per;
  const int hi = (lo + per < n) ? lo + per : n;
  int ne_local = 0;
  for (int i = lo; i < hi; ++i) ne_local += pool_key(bs[i], (uint32_t)i) < cut;
  int ne = 0;
  int pos = block_exclusive_scan(ne_local, &ne, lds4);
  for (int i = lo; i < hi; ++i)
    if (pool_key(bs[i], (uint32_t)i) < cut) evicted[pos++] = i;

  // admitted candidates, ascending: thread tid owns pending slot tid
  const int kept = (tid < C) && pool_key(ps[tid], (uint32_t)(N + tid)) >= cut;
  int na = 0;
  const int apos = block_exclusive_scan(kept, &na, lds4);
  if (kept) admitted[apos] = tid;
  __syncthreads();

  // move the admitted records: 32 K chunks and 32 V chunks each
  uint4* bk = reinterpret_cast<uint4*>(a.bank_k + (size_t)u * N * kD);
  uint4* bv = reinterpret_cast<uint4*>(a.bank_v + (size_t)u * N * kD);
  const uint4* pk = reinterpret_cast<const uint4*>(a.pend_k + (size_t)u * C * kD);
  const uint4* pv = reinterpret_cast<const uint4*>(a.pend_v + (size_t)u * C * kD);
  for (int w = tid; w < na * 2 * kChunks; w += 256) {
    const int r = w / (2 * kChunks);
    const int part = w - r * 2 * kChunks;
    const int j = admitted[r];
    const int dst = r < ne ? evicted[r] : n + (r - ne);
    if (part < kChunks) {
      bk[k_chunk_index(dst, part, N)] = pk[(size_t)j * kChunks + part];
    } else {
      const int c = part - kChunks;
      bv[(size_t)dst * kChunks + c] = pv[(size_t)j * kChunks + c];
    }
  }
  for (int r = tid; r < na; r += 256) {
    const int j = admitted[r];
    const int dst = r < ne ? evicted[r] : n + (r - ne);
    a.bscore[(size_t)u * N + dst] = ps[j];
    a.bsrc[(size_t)u * N + dst] = (int32_t)(block_start + j);
  }
  if (tid == 0) a.bank_n[u] = K;
}

}  // namespace

hipError_t launch_admit(const AdmitArgs& a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(admit_kernel, dim3(a.units), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rma
