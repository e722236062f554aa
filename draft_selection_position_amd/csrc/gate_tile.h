// Gate tiles for few rows: Z = H W_h over one K split for a handful of block
// positions, written as K-split partial sums (or, unsplit, passed through the
// sigmoid).  The context gate of the score (blog post "DFlash 2: Keep Drafting
// Parallel", section "A Lightweight Path Selector") is H(h_t) = sigmoid(h_t W_h) in
// this library.  Each tile is one 256-thread workgroup that needs no barrier, so it
// runs as a kernel of its own (the standalone gate) or as extra workgroups of the
// top-16 launch (the fused selector on a pre-packed W_h), with the same bits either
// way.
#pragma once

#include "dfs_device.h"
#include "dfs_internal.h"

namespace dfs {

namespace gtile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKB = 32;                      // k per MFMA step (one packed slab)
constexpr int kRows16 = 16;                  // rows per row group of a bf16 tile
// Tiles for more than 64 rows: 32 rows, one k step in flight.  Riding in the top-16
// launch of the selector at 512 x 5120, 128 such tiles (8 K splits) took a call from
// 52.1 to 48.1 us against 256 tiles of 16 rows; 256 tall tiles, 64, 96, 112, 144 or 192, and
// 2 or 3 steps in flight were slower, and 64-row tiles hold too many registers for the
// launch's three waves per SIMD.
#ifndef DFS_GATE_TALL_GROUPS
#define DFS_GATE_TALL_GROUPS 2
#endif
constexpr int kTallGroups = DFS_GATE_TALL_GROUPS;  // 16-row groups of a tall tile
#ifndef DFS_GATE_TALL_DEPTH
#define DFS_GATE_TALL_DEPTH 1
#endif
constexpr int kTallDepth = DFS_GATE_TALL_DEPTH;  // its k steps in flight per lane
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
#ifndef DFS_GATE_TILE16_DEPTH
#define DFS_GATE_TILE16_DEPTH 4
#endif
constexpr int kDepth = DFS_GATE_TILE16_DEPTH;  // k steps in flight per lane

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Rows [m0, m0 + 16 RG) x all 256 columns of Z over k steps [kb0, kb1) (bf16 H [rows, d],
// W_h packed [ceil(d/32)][256][32], zero past d).  Wave w owns columns [64 w, + 64) of
// every row: RG x 4 V_MFMA_F32_16X16X32_BF16 tiles.  Lane (r, q) feeds H rows
// m0 + 16 g + r (g < RG), k 8q .. 8q + 7 of each step (zero past the last row: buffer
// range check; zero past d) and the packed column 64 w + 16 nt + r at the same k: the
// operand layout of every other gate GEMM here, so a K split adds up the same products
// in the same order, bit for bit, whatever RG is.  Both operands go straight from memory
// into a register ring kDepth steps deep; a taller tile (RG > 1) reads each W_h fragment
// once for more rows.  Results: the K split's partial sums [splits, rows, 256]
// (splits > 1) or the sigmoid (splits 1).
template <int RG, int kDepth>
__device__ __forceinline__ void tile_rows(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wp,
                                          int64_t rows, int64_t d, int64_t m0, int kb0, int kb1, int split,
                                          int splits, float* __restrict__ partial, float* __restrict__ out,
                                          int tid) {
  constexpr int TR = kRows16 * RG;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int KB = (int)((d + kKB - 1) / kKB);
  const int64_t trows = rows - m0 < TR ? rows - m0 : TR;
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(H + m0 * d), (short)0, (int)(trows * d * 2), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wp), (short)0, (int)((int64_t)KB * kE * kKB * 2), kRawBufferWord3);
  uint32_t hvoff[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) hvoff[g] = (uint32_t)(((int64_t)(16 * g + r) * d + 8 * q) * 2);
  uint32_t wvoff[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) wvoff[nt] = (uint32_t)(((64 * wave + 16 * nt + r) * kKB + 8 * q) * 2);

  f32x4 acc[RG][4];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[g][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra[kDepth][RG], rb[kDepth][4];
  auto fill = [&](int j, int kb) {
#pragma unroll
    for (int g = 0; g < RG; ++g) ra[j][g] = bload(hrs, hvoff[g], (uint32_t)kb * kKB * 2);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) rb[j][nt] = bload(wrs, wvoff[nt], (uint32_t)kb * kE * kKB * 2);
  };
  auto step = [&](int kb, const uint4 (&a)[RG], const uint4 (&b)[4]) {
    const uint32_t keep = (int64_t)kb * kKB + 8 * q < d ? 0xffffffffu : 0u;  // H past d is another row
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const bf16x8 af =
          __builtin_bit_cast(bf16x8, make_uint4(a[g].x & keep, a[g].y & keep, a[g].z & keep, a[g].w & keep));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[g][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, b[nt]), acc[g][nt], 0, 0, 0);
    }
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j) fill(j, kb0 + j < kb1 ? kb0 + j : kb1 - 1);
  int base = kb0;
  for (; base + kDepth <= kb1; base += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      step(base + j, ra[j], rb[j]);
      fill(j, base + j + kDepth < kb1 ? base + j + kDepth : kb1 - 1);
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (base + j < kb1) step(base + j, ra[j], rb[j]);

  // lane (r, q) holds Z[m0 + 16 g + 4q + i][64 w + 16 nt + r] in acc[g][nt][i]
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 16 * g + 4 * q + i;
      if (m < rows) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int col = 64 * wave + 16 * nt + r;
          if (splits == 1) {
            out[m * kE + col] = sigmoidf(acc[g][nt][i]);
          } else {
            partial[((int64_t)split * rows + m) * kE + col] = acc[g][nt][i];
          }
        }
      }
    }
}

// ---------------------------------------------------------------- fp32
constexpr int kF32Rows = 8;      // rows per workgroup
constexpr int kF32KBlock = 256;  // k staged in LDS at a time
constexpr int kF32Unroll = 16;   // W_h loads in flight per thread
constexpr size_t kF32LdsBytes = (size_t)kF32Rows * kF32KBlock * sizeof(float);

// Rows [m0, m0 + 8) x 256 columns over k in [k0, k1), fp32 H [rows, d] and W_h [d, 256]:
// one thread per output column; the H rows of each k block are staged in LDS (`sH`,
// kF32LdsBytes, read back as broadcasts); the W_h column values are loaded 16 ahead of
// the FMAs.  Accumulation in k order.  Holds workgroup barriers: all 256 threads call it.
__device__ __forceinline__ void tile_f32(const float* __restrict__ H, const float* __restrict__ W, int64_t rows,
                                         int64_t d, int64_t m0, int64_t k0, int64_t k1, int split, int splits,
                                         float* __restrict__ partial, float* __restrict__ out, int tid,
                                         float (*sH)[kF32KBlock]) {
  const int n = tid;
  float acc[kF32Rows];
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) acc[i] = 0.0f;
  for (int64_t kb = k0; kb < k1; kb += kF32KBlock) {
    const int kc = (int)(k1 - kb < kF32KBlock ? k1 - kb : kF32KBlock);
    __syncthreads();  // the previous block has been consumed
    for (int e = n; e < kF32Rows * kF32KBlock; e += kThreads) {
      const int i = e / kF32KBlock, kk = e % kF32KBlock;
      float v = 0.0f;
      if (kk < kc && m0 + i < rows) v = H[(m0 + i) * d + kb + kk];
      sH[i][kk] = v;
    }
    __syncthreads();
    int k = 0;
    for (; k + kF32Unroll <= kc; k += kF32Unroll) {
      float w[kF32Unroll];
#pragma unroll
      for (int u = 0; u < kF32Unroll; ++u) w[u] = W[(kb + k + u) * kE + n];
#pragma unroll
      for (int u = 0; u < kF32Unroll; ++u)
#pragma unroll
        for (int i = 0; i < kF32Rows; ++i) acc[i] = fmaf(sH[i][k + u], w[u], acc[i]);
    }
    for (; k < kc; ++k) {
      const float w = W[(kb + k) * kE + n];
#pragma unroll
      for (int i = 0; i < kF32Rows; ++i) acc[i] = fmaf(sH[i][k], w, acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) {
    const int64_t m = m0 + i;
    if (m < rows) {
      if (splits == 1) {
        out[m * kE + n] = sigmoidf(acc[i]);
      } else {
        partial[((int64_t)split * rows + m) * kE + n] = acc[i];
      }
    }
  }
}

}  // namespace gtile

// Job `j` of `g` (bf16 or fp32 per `bf16`).  `lds`: at least gtile::kF32LdsBytes of
// shared memory for the fp32 tile.  All 256 threads of the workgroup call it.
__device__ __forceinline__ void run_gate_job(const GateJobs& g, bool bf16, int64_t j, int tid, void* lds) {
  const int mt = (int)(j % g.mtiles);
  const int s = (int)(j / g.mtiles);
  if (bf16) {
    const int kps = (int)(g.kchunk / gtile::kKB);
    const int KB = (int)((g.d + gtile::kKB - 1) / gtile::kKB);
    const int kb0 = s * kps;
    const int kb1 = kb0 + kps < KB ? kb0 + kps : KB;
    const uint16_t* H = static_cast<const uint16_t*>(g.H);
    const uint16_t* W = static_cast<const uint16_t*>(g.W);
    const int64_t m0 = (int64_t)mt * gtile::kRows16 * g.rgroups;
    if (g.rgroups == 1) {
      gtile::tile_rows<1, gtile::kDepth>(H, W, g.rows, g.d, m0, kb0, kb1, s, g.splits, g.partial, g.out, tid);
    } else {
      gtile::tile_rows<gtile::kTallGroups, gtile::kTallDepth>(H, W, g.rows, g.d, m0, kb0, kb1, s, g.splits, g.partial, g.out, tid);
    }
  } else {
    const int64_t k0 = (int64_t)s * g.kchunk;
    const int64_t k1 = k0 + g.kchunk < g.d ? k0 + g.kchunk : g.d;
    gtile::tile_f32(static_cast<const float*>(g.H), static_cast<const float*>(g.W), g.rows, g.d,
                    (int64_t)mt * gtile::kF32Rows, k0, k1, s, g.splits, g.partial, g.out, tid,
                    reinterpret_cast<float(*)[gtile::kF32KBlock]>(lds));
  }
}

}  // namespace dfs
