// Admit kernel of the RMA layer on gfx950: one 256-thread workgroup per
// (sequence, layer, group) unit runs admit_unit (rma_admit_unit.h: the
// committed anchors and the pending candidates compete for the bank, the
// best min(N, n + C) stay, admitted candidates fill the evicted slots and
// then append).
//
// Lockstep: every unit of one or more layers, all at the same block end.
// Per-sequence positions: every unit of one layer whose sequence's last
// written token completes a block; the others exit at once.
#include "rma_admit_unit.h"

namespace rma {
namespace {

__global__ __launch_bounds__(kAdmitThreads) void admit_kernel(AdmitArgs a) {
  const int u = a.unit0 + blockIdx.x;
  const int N = a.N, C = a.C;
  int64_t block_start = a.block_start;
  if (a.pos != nullptr) {  // per-sequence: admit only where a block just completed
    const int first = a.pos[blockIdx.x / a.G];
    if (first < 0 || (a.aligned_only && first % C != 0)) return;
    const int64_t last = (int64_t)first + a.pos_add;
    if ((last + 1) % C != 0) return;
    block_start = last + 1 - C;
  }
  __shared__ AdmitShared sh;
  AdmitUnit au;
  au.bank_k = a.bank_k + (size_t)u * N * kD;
  au.bank_v = a.bank_v + (size_t)u * N * kD;
  au.bscore = a.bscore + (size_t)u * N;
  au.bsrc = a.bsrc + (size_t)u * N;
  au.bank_n = a.bank_n + u;
  au.pend_k = a.pend_k + (size_t)u * C * kD;
  au.pend_v = a.pend_v + (size_t)u * C * kD;
  au.pscore = a.pscore + (size_t)u * C;
  au.N = N;
  au.C = C;
  au.block_start = block_start;
  admit_unit(au, sh);
}

}  // namespace

hipError_t launch_admit(const AdmitArgs& a, hipStream_t s) {
  if (a.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(admit_kernel, dim3(a.units), dim3(kAdmitThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rma
