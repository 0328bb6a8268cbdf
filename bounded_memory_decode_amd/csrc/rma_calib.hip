// Streaming-read probe: the HBM read bandwidth a plain kernel reaches on
// this part, the yardstick for the decode kernel's loads.  Every wave reads
// its own contiguous share of a buffer with 16-byte non-temporal loads
// (the cache policy the decode uses for its streamed K/V) and folds the
// words into one value that it stores, so no load can be dropped.
#include "rma_calib.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 16;  // loads in flight per lane per turn (swept: 8, 16, 32)

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ buf,
                                                          uint64_t per_wave, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const uint64_t wave = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const u32x4_t* p = buf + wave * per_wave;
  uint32_t acc = 0;
  uint64_t i = lane;
  // per_wave is a multiple of 64 * kUnroll (checked on the host): every
  // turn's loads are in bounds
  for (; i < per_wave; i += 64 * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + 64 * u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[wave] = acc;
}

}  // namespace

extern "C" int rma_calib_stream_read(const void* buf, size_t bytes, int32_t waves,
                                     uint32_t* sink, void* stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15u) || waves < 4 || waves % 4) return -1;
  const uint64_t per_turn = (uint64_t)waves * 64 * kUnroll * 16;  // bytes per turn of all waves
  if (bytes == 0 || bytes % per_turn) return -1;
  const uint64_t per_wave = bytes / 16 / (uint64_t)waves;
  hipLaunchKernelGGL(stream_read_kernel, dim3(waves / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf), per_wave,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
