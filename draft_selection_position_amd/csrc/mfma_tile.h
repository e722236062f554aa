// One tile of C = A B^T on gfx950's matrix cores, both operands bf16 and
// K-contiguous ([rows, K] row-major), fp32 sums.
//
// Four waves in a WMW x WNW grid; each wave computes TM x TN tiles of 16 x 16
// (V_MFMA_F32_16X16X32_BF16), so the workgroup tile is BM = 16 WMW TM rows of A by
// BN = 16 WNW TN rows of B.  Per 64-wide k step the workgroup fetches BM (and BN)
// rows x 128 bytes with full-cache-line 16-byte buffer loads (eight lanes per row),
// issued kDepth steps ahead into registers, and stages them through a
// double-buffered LDS tile (row pitch 144 bytes: the 16 rows a fragment read
// touches fall on distinct bank groups); the waves then read their fragments from
// LDS.  One barrier per step.  Rows past the end of either operand read as zeros
// (buffer range check), so a ragged tile needs no masking in the loop.
#pragma once

#include "dfs_device.h"

namespace dfs {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
constexpr int kThreads = 256;                 // 4 waves
constexpr int kKStep = 64;                    // k per step: 128 bytes of every row
constexpr int kPitch = kKStep + 8;            // bf16 per LDS row

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer resource over `nrows` rows of length K starting at `p` (range-checked).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* p, int64_t nrows, int64_t K) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)(nrows * K * 2),
                                           kRawBufferWord3);
}

template <int WMW, int WNW, int TM, int TN>
struct Shape {
  static_assert(WMW * WNW == 4, "four waves");
  static constexpr int BM = 16 * WMW * TM;
  static constexpr int BN = 16 * WNW * TN;
  static constexpr int kStageA = BM * kPitch;  // bf16 per LDS stage
  static constexpr int kStageB = BN * kPitch;
  static constexpr int kLdsBytes = 2 * (kStageA + kStageB) * 2;
  // Accumulators: C[16 TM wm + 16 mt + 4 q + i][16 TN wn + 16 nt + r] = v[mt][nt][i]
  // for lane (r = lane & 15, q = lane >> 4) of wave (wm, wn) = (wave / WNW, wave % WNW).
  struct Acc {
    f32x4 v[TM][TN];
  };
};

// acc += A[0:BM, ks0*64 : ks1*64] * B[0:BN, same]^T for the resources' rows.
// lds: Shape::kLdsBytes of shared memory.  Every thread of the workgroup must call it.
template <int WMW, int WNW, int TM, int TN, int kDepth>
__device__ __forceinline__ void mma(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int64_t K,
                                    int ks0, int ks1, uint16_t* lds,
                                    typename Shape<WMW, WNW, TM, TN>::Acc& acc) {
  using S = Shape<WMW, WNW, TM, TN>;
  constexpr int BM = S::BM, BN = S::BN;
  constexpr int NA = BM >= 32 ? BM / 32 : 1;  // loads per thread per step
  constexpr int NB = BN >= 32 ? BN / 32 : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave / WNW, wn = wave % WNW;
  uint16_t* sA = lds;                   // [2][BM][kPitch]
  uint16_t* sB = lds + 2 * S::kStageA;  // [2][BN][kPitch]
  // loader: rows (tid >> 3) + 32 i, bytes 16 (tid & 7) of the step's 128
  const int lrow = tid >> 3, lchunk = tid & 7;
  const bool a_on = lrow < BM, b_on = lrow < BN;
  const uint32_t voff = (uint32_t)(((int64_t)lrow * K + 8 * lchunk) * 2);
  const uint32_t rstride = (uint32_t)(32 * K * 2);
  const int nsteps = ks1 - ks0;
  uint4 ga[kDepth][NA], gb[kDepth][NB];
  auto fetch = [&](int j, int s) {
    const uint32_t so = (uint32_t)(ks0 + s) * kKStep * 2;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (a_on) ga[j][i] = bload(ra, voff + i * rstride, so);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (b_on) gb[j][i] = bload(rb, voff + i * rstride, so);
  };
  auto stash = [&](int j, int st) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if (a_on) *reinterpret_cast<uint4*>(sA + st * S::kStageA + (lrow + 32 * i) * kPitch + 8 * lchunk) = ga[j][i];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (b_on) *reinterpret_cast<uint4*>(sB + st * S::kStageB + (lrow + 32 * i) * kPitch + 8 * lchunk) = gb[j][i];
  };
  auto compute = [&](int st) {
    const uint16_t* a = sA + st * S::kStageA + (16 * TM * wm + r) * kPitch + 8 * q;
    const uint16_t* b = sB + st * S::kStageB + (16 * TN * wn + r) * kPitch + 8 * q;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) af[t] = *reinterpret_cast<const bf16x8*>(a + 16 * t * kPitch + 32 * h);
#pragma unroll
      for (int t = 0; t < TN; ++t) bfr[t] = *reinterpret_cast<const bf16x8*>(b + 16 * t * kPitch + 32 * h);
#pragma unroll
      for (int mt = 0; mt < TM; ++mt)
#pragma unroll
        for (int nt = 0; nt < TN; ++nt)
          acc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc.v[mt][nt], 0, 0, 0);
    }
  };
  // prologue: steps 0 .. kDepth-1 in flight, step 0 staged
#pragma unroll
  for (int j = 0; j < kDepth; ++j) fetch(j, j < nsteps ? j : nsteps - 1);
  stash(0, 0);
  __syncthreads();
  // step s: refill the slot of step s with step s + kDepth, compute step s from LDS,
  // stage step s + 1 (fetched kDepth - 1 steps ago), one barrier
  int s = 0;
  for (; s + kDepth <= nsteps; s += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int cur = s + j;
      const int nxt = cur + kDepth < nsteps ? cur + kDepth : nsteps - 1;
      fetch(j, nxt);
      compute(cur & 1);
      if (cur + 1 < nsteps) stash((j + 1) % kDepth, (cur + 1) & 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j) {
    const int cur = s + j;
    if (cur < nsteps) {
      compute(cur & 1);
      if (cur + 1 < nsteps) stash((j + 1) % kDepth, (cur + 1) & 1);
      __syncthreads();
    }
  }
}

template <int WMW, int WNW, int TM, int TN>
__device__ __forceinline__ void zero(typename Shape<WMW, WNW, TM, TN>::Acc& acc) {
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace tile
}  // namespace dfs
