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
// One workgroup per (sequence, group, 16-token query tile); wave w owns 16
// query rows, row = token * 4 + head, so each accumulator lane holds the 4
// heads of one token and the mask (a function of the token) is per lane.
//  * QK: K B-operands come straight from the chunk-major K planes (16 keys
//    of one chunk are 256 contiguous bytes) or from the block's K rows.
//  * P.V: V tiles of 32 keys are staged in LDS (double-buffered, shared by
//    the 4 waves) and gathered as B-operands (8 keys of one dim per lane);
//    P goes from the accumulator layout to the A layout through a per-wave
//    LDS slice.
//  * Online softmax in the log2 domain; local and anchor reads separately
//    normalised, then out = o_local + tanh(q . w_g) * o_anchor.
#include "rma_kernels.h"

namespace rma {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPT = 32;          // keys per tile
constexpr int kVRow = 520;       // bytes per staged V row (8-aligned, conflict-free gathers)
constexpr int kTokPerWave = 4;
constexpr int kTokPerWG = 16;

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// All-reduce over each row of 16 lanes with DPP moves (single-cycle VALU
// operand swizzles, no LDS round trip): swap neighbours, swap pairs, then
// mirror within 8 and within 16 lanes.  After the first two steps the 4
// lanes of a quad agree, so each mirror combines two already-reduced
// groups.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kQuadSwap1>(x));
  x = fmaxf(x, dpp<kQuadSwap2>(x));
  x = fmaxf(x, dpp<kRowHalfMirror>(x));
  x = fmaxf(x, dpp<kRowMirror>(x));
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Key source of one segment (ring, block, bank).
enum : int { kSegRing = 0, kSegBlock = 1, kSegBank = 2 };

__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a) {
  const int qt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int u = b * a.G + g;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;  // MFMA column / k-group
  const int n = a.n;
  const int tok0 = qt * kTokPerWG + wave * kTokPerWave;  // first token of this wave
  const int my_tok = tok0 + lg;                          // token of this lane's D rows

  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2][kPT * kVRow];
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[4][16 * kPT];

  // Q as A-operands: 8 k-steps of 32 dims; row l16 -> token l16/4, head l16%4
  uint4 qa[8];
  {
    const int t = tok0 + (l16 >> 2), h = l16 & 3;
    const bool ok = t < n;
    const uint4* qrow = reinterpret_cast<const uint4*>(
        a.q + (((size_t)b * n + (ok ? t : 0)) * a.H + g * kHpg + h) * kD);
#pragma unroll
    for (int st = 0; st < 8; ++st) qa[st] = ok ? qrow[st * 4 + lg] : make_uint4(0, 0, 0, 0);
  }

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
  int last_tok = qt * kTokPerWG + kTokPerWG - 1;
  last_tok = last_tok < n - 1 ? last_tok : n - 1;
  const int t_blk = last_tok / kPT + 1;
  const int nb = a.bank_n[u];
  const int t_bank = (nb + kPT - 1) / kPT;
  const int t_loc = t_ring + t_blk;
  const int t_all = t_loc + t_bank;
  // ring age threshold: slot s holds position P - R + age(s), age(s) =
  // (s - P) mod R; it exists iff age >= R - P
  const int min_age = (int)(R - P > 0 ? R - P : 0);
  const int p_mod = (int)(P % R);

  const uint16_t* ring_k = a.ring_k + (size_t)u * R * kD;
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
    sr.kcs = ring ? R : (blk ? 1 : a.N);
    sr.vks = blk ? a.G * kChunks : kChunks;
    sr.cnt = seg_count(seg);
    sr.ti = ti;
    return sr;
  };

  // cooperative V tile load: 32 keys x 32 chunks, 4 chunks per thread
  uint4 vpre[4];
  auto load_v = [&](int t) {
    const Src sr = src_of(t);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int id = tid + 256 * m;
      const int key = id >> 5, c = id & 31;
      int kk = sr.ti * kPT + key;
      kk = kk < sr.cnt ? kk : sr.cnt - 1;
      vpre[m] = sr.v[(size_t)kk * sr.vks + c];
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int id = tid + 256 * m;
      const int key = id >> 5, c = id & 31;
      uint2* dst = reinterpret_cast<uint2*>(&v_lds[buf][key * kVRow + c * 16]);
      dst[0] = make_uint2(vpre[m].x, vpre[m].y);
      dst[1] = make_uint2(vpre[m].z, vpre[m].w);
    }
  };
  // K B-operands of a tile: 2 sub-tiles of 16 keys x 8 k-steps
  uint4 kb[2][8];
  auto load_k = [&](int t) {
    const Src sr = src_of(t);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      int kk = sr.ti * kPT + sub * 16 + l16;
      kk = kk < sr.cnt ? kk : sr.cnt - 1;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        kb[sub][st] = sr.k[(size_t)kk * sr.kks + (size_t)(st * 4 + lg) * sr.kcs];
    }
  };

  f32x4_t o[16];    // the running read: 16 dim sub-tiles of 16 rows x 16 dims
  f32x4_t oloc[16]; // the finished local read
  float m[4], l[4];
  auto reset = [&]() {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
  };
  reset();

  if (t_all > 0) {
    load_v(0);
    store_v(0);
    load_k(0);
  }
  __syncthreads();

  for (int t = 0; t < t_all; ++t) {
    int seg, ti;
    seg_of(t, seg, ti);
    const int cnt = seg_count(seg);
    const bool has_next = t + 1 < t_all;
    // prefetch without branches: past the last tile, reload the last one
    const int tn = has_next ? t + 1 : t;
    load_v(tn);

    // S = Q K^T for 32 keys
    f32x4_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st)
        s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[st]), as_bf16x8(kb[sub][st]),
                                                          s[sub], 0, 0, 0);
    }
    load_k(tn);

    // mask and scale: lane's token my_tok, key = column l16 of each sub-tile
    float sv[2][4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = ti * kPT + sub * 16 + l16;
      bool vis = kk < cnt && my_tok < n;
      if (seg == kSegRing) {
        int age = kk - p_mod;
        age += age < 0 ? R : 0;
        vis = vis && age >= min_age && age >= my_tok;
      } else if (seg == kSegBlock) {
        vis = vis && kk <= my_tok;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[sub][i] = vis ? s[sub][i] * a.sl2e : -INFINITY;
    }

    // online softmax per row (token my_tok, head i)
    float pb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mt = row16_max(fmaxf(sv[0][i], sv[1][i]));
      const float mn = fmaxf(m[i], mt);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m[i] - mref);
      pb[0][i] = __builtin_amdgcn_exp2f(sv[0][i] - mref);
      pb[1][i] = __builtin_amdgcn_exp2f(sv[1][i] - mref);
      l[i] = l[i] * al + row16_sum(pb[0][i] + pb[1][i]);
      m[i] = mn;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt][i] *= al;
    }
    // P (bf16) to the A layout through this wave's LDS slice
    uint16_t* ps = p_lds[wave];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[(lg * 4 + i) * kPT + sub * 16 + l16] = to_bf16(pb[sub][i]);
    __builtin_amdgcn_wave_barrier();
    const uint4 pa = *reinterpret_cast<const uint4*>(&ps[l16 * kPT + lg * 8]);

    // O += P V: B-operand = 8 keys (8*lg .. 8*lg+7) of dim 16*dt + l16
    const unsigned char* vt = v_lds[t & 1];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const int dim = dt * 16 + l16;
      uint16_t e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        e[j] = *reinterpret_cast<const uint16_t*>(&vt[(lg * 8 + j) * kVRow + dim * 2]);
      uint4 vb;
      vb.x = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
      vb.y = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
      vb.z = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
      vb.w = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), as_bf16x8(vb), o[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();

    // end of the local read: normalise and keep it
    if (t == t_loc - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) oloc[dt][i] = o[dt][i] * inv;
      }
      reset();
    }
    store_v((t + 1) & 1);
    __syncthreads();
  }
  if (t_loc == 0) {
    // no visible local key is impossible for a real token (it sees itself)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) oloc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // anchor read (zero for an empty bank)
  float inv_b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) inv_b[i] = (t_bank > 0 && l[i] > 0.f) ? 1.f / l[i] : 0.f;

  // gate argument q . w_g for row l16 (token l16/4, head l16%4), summed over
  // the 4 k-groups; then fetched for the D-layout rows (token lg, head i)
  float z = 0.f;
  {
    const int h = l16 & 3;
    const float* wrow = a.w_g + (size_t)(g * kHpg + h) * kD;
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
  }
  float gate[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) gate[i] = tanhf(__shfl(z, lg * 4 + i, 64));

  if (my_tok < n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* orow = a.out + (((size_t)b * n + my_tok) * a.H + g * kHpg + i) * kD;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
        orow[dt * 16 + l16] = to_bf16(fmaf(gate[i], o[dt][i] * inv_b[i], oloc[dt][i]));
    }
  }
}

// The block's writes, after every query of the block has read the ring:
// token j goes to ring slot (P + j) mod R and pending slot (P + j) mod C.
// grid: (n, units); block: 128.
__global__ __launch_bounds__(128) void prefill_commit_kernel(PrefillArgs a) {
  const int j = blockIdx.x, u = blockIdx.y;
  const int b = u / a.G, g = u - b * a.G;
  const int tid = threadIdx.x;
  int64_t P = a.P;
  if (a.pos != nullptr) {
    const int p = a.pos[b];
    if (p < 0 || p % a.C != 0) return;
    P = p;
  }
  const size_t src = (((size_t)b * a.n + j) * a.G + g) * kD;
  const int rs = (int)((P + j) % a.R), ps = (int)((P + j) % a.C);
  const int c = tid & 31;
  if (tid < 32) {
    uint4* rk = reinterpret_cast<uint4*>(a.ring_k + (size_t)u * a.R * kD);
    rk[k_chunk_index(rs, c, a.R)] = reinterpret_cast<const uint4*>(a.k + src)[c];
  } else if (tid < 64) {
    reinterpret_cast<uint4*>(a.ring_v + ((size_t)u * a.R + rs) * kD)[c] =
        reinterpret_cast<const uint4*>(a.v + src)[c];
  } else if (tid < 96) {
    reinterpret_cast<uint4*>(a.pend_k + ((size_t)u * a.C + ps) * kD)[c] =
        reinterpret_cast<const uint4*>(a.ck + src)[c];
  } else {
    reinterpret_cast<uint4*>(a.pend_v + ((size_t)u * a.C + ps) * kD)[c] =
        reinterpret_cast<const uint4*>(a.cv + src)[c];
    if (tid == 96) a.pscore[(size_t)u * a.C + ps] = a.cs[((size_t)b * a.n + j) * a.G + g];
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const int tiles = (a.n + kTokPerWG - 1) / kTokPerWG;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(tiles, a.G, a.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_commit_kernel, dim3(a.n, a.B * a.G), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace rma
