// Repacking of the gate weight W_h [d, 256] (bf16) for the matrix cores.
//
// The MFMA wants each lane's operand to be 8 consecutive k values of one output
// column, but W_h is row-major (columns contiguous).  The packed copy is
// Wp[kb][n][kk] = W_h[32 kb + kk][n] (zero past d): slab kb holds, per column, its
// 32 k values in a row.  One 256-thread workgroup packs one slab, reading W_h
// with 16-byte loads and writing Wp with 16-byte stores, transposed through LDS.
// The standalone gate launches it as its own kernel; the fused selector runs the
// same slab jobs as extra workgroups of the top-16 launch, in that pass's tail.
#pragma once

#include "dfs_device.h"
#include "dfs_internal.h"

namespace dfs {

constexpr int kPackK = 32;               // k rows per slab
constexpr int kPackPitch = kE + 8;       // uint16 per LDS row (+8: spread column reads over banks)
constexpr int kPackThreads = 256;
constexpr size_t kPackLdsBytes = (size_t)kPackK * kPackPitch * sizeof(uint16_t);

// Pack slab kb of W (d rows) into Wp; `tile` is kPackLdsBytes of LDS, all 256
// threads of the workgroup take part (it holds a workgroup barrier).
__device__ __forceinline__ void pack_w_slab(const uint16_t* __restrict__ W, int64_t d,
                                            uint16_t* __restrict__ Wp, int64_t kb, int tid,
                                            uint16_t (*tile)[kPackPitch]) {
  {
    const int kk = tid >> 3;        // 32 rows, 8 threads per row
    const int n0 = (tid & 7) * 32;  // 32 columns per thread
    const int64_t k = kb * kPackK + kk;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (k < d) v = *reinterpret_cast<const uint4*>(W + k * kE + n0 + 8 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[kk][n0 + 8 * c + 2 * e] = (uint16_t)(w[e] & 0xffffu);
        tile[kk][n0 + 8 * c + 2 * e + 1] = (uint16_t)(w[e] >> 16);
      }
    }
  }
  __syncthreads();
  const int n = tid;  // one output column (32 k values = 64 bytes) per thread
  uint4* dst = reinterpret_cast<uint4*>(Wp + (kb * kE + n) * kPackK);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * c + 2 * e][n] | ((uint32_t)tile[8 * c + 2 * e + 1][n] << 16);
    dst[c] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace dfs
