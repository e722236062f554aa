// Two-tap dynamic depthwise convolution across the positions of a draft block.
//
// The post places a short convolution before and after each attention and
// feed-forward sublayer of the drafter (blog post "DFlash 2: Keep Drafting
// Parallel", section "A Lightweight Local Convolution"; equation in the
// twiscan.com and decomputer.nl translations):
//     y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}     (elementwise over channels)
// Each coefficient is a learned base kernel plus a correction computed from the
// current hidden state, one correction per 16 channels; position 0's
// predecessor is the last verified token's representation.  This library's
// reading: c_t = W_c x_t with W_c [D/16, 2, D] (row 2g + tap), and
//     k_{t,tap}[ch] = base[tap, ch] + c_t[2 (ch / 16) + tap].
//
// bf16 path: the correction is a [rows, D] x [D, D/8] product on the matrix cores
// (mfma_tile.h: 128 x 128 tiles staged through LDS); a workgroup's epilogue applies
// the convolution to exactly its 128 rows and 1024 channels, so the correction
// never leaves the chip.  W_c is K-contiguous, the operand order the tile wants: no
// repacking.  Shapes too small to fill the chip split K; an elementwise kernel then
// adds the split partial sums in split order and applies the convolution (a
// device-wide fence per workgroup to let the last split do it in place writes
// back the L2 of a multi-XCD part and measured three times slower).
// fp32 path (small shapes): the correction by wave dot products into workspace,
// then an elementwise kernel.
#include "dfs_device.h"
#include "dfs_internal.h"
#include "mfma_tile.h"

namespace dfs {
namespace {

using CT = tile::Shape<2, 2, 4, 4>;           // 128 x 128 tiles, 64 x 64 per wave
constexpr int kThreads = tile::kThreads;      // 4 waves
constexpr int kTileM = CT::BM;                // rows per workgroup
constexpr int kTileN = CT::BN;                // correction columns per workgroup (64 groups)
constexpr int kKStep = tile::kKStep;
constexpr int kPitchC = kTileN + 4;           // fp32 per LDS row of the correction tile
#ifndef DFS_CONV_DEPTH
#define DFS_CONV_DEPTH 2
#endif
#ifndef DFS_CONV_XCD
#define DFS_CONV_XCD 1
#endif
static_assert(kTileM * kPitchC * 4 <= CT::kLdsBytes, "the correction tile reuses the operand stages");

// fp32 -> bf16 bits, round to nearest, ties to even (finite and infinite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Eight channels: y = (b0 + c0) x + (b1 + c1) p, widened from bf16, rounded back.
__device__ __forceinline__ uint4 conv8(uint4 xv, uint4 pv, uint4 b0, uint4 b1, float c0, float c1) {
  const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
  const uint32_t ps[4] = {pv.x, pv.y, pv.z, pv.w};
  const uint32_t b0s[4] = {b0.x, b0.y, b0.z, b0.w};
  const uint32_t b1s[4] = {b1.x, b1.y, b1.z, b1.w};
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ylo = fmaf(bf16_lo(b0s[i]) + c0, bf16_lo(xs[i]), (bf16_lo(b1s[i]) + c1) * bf16_lo(ps[i]));
    const float yhi = fmaf(bf16_hi(b0s[i]) + c0, bf16_hi(xs[i]), (bf16_hi(b1s[i]) + c1) * bf16_hi(ps[i]));
    out[i] = bf16_rne(ylo) | (bf16_rne(yhi) << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Workgroup (row tile, column tile, K split): the correction tile on the matrix
// cores (mfma_tile.h), then either the convolution of the tile's rows over its
// 1024 channels (one split) or the split's partial sums to `partial`.
#ifndef DFS_CONV_WAVES_PER_EU
#define DFS_CONV_WAVES_PER_EU 2
#endif
__global__ __launch_bounds__(kThreads, DFS_CONV_WAVES_PER_EU) void conv2_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xprev,
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ Wc, int64_t rows, int L,
    int64_t D, int ntiles_n, int64_t mtiles, int splits, int ks_per_split,
    float* __restrict__ partial, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[CT::kLdsBytes / 2];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int split = (int)(blockIdx.x % (unsigned)splits);
  const unsigned p = blockIdx.x / (unsigned)splits;
#if DFS_CONV_XCD
  // Workgroups go to the 8 XCDs round-robin: XCD p % 8 takes the row tiles congruent
  // to it, all column tiles of each, so a row tile's x and the column tiles' W_c
  // slices are shared through that XCD's L2.
  const unsigned xcd = p % 8u, jj = p / 8u;
  const int n_tile = (int)(jj % (unsigned)ntiles_n);
  const int64_t mt = (int64_t)(jj / (unsigned)ntiles_n) * 8 + xcd;
  if (mt >= mtiles) return;
#else
  const int n_tile = (int)(p % (unsigned)ntiles_n);
  const int64_t mt = (int64_t)(p / (unsigned)ntiles_n);
#endif
  const int64_t m0 = mt * kTileM;
  const int64_t ncols_all = D / 8;
  const int64_t n0 = (int64_t)n_tile * kTileN;
  const int ncols = (int)(ncols_all - n0 < kTileN ? ncols_all - n0 : kTileN);  // a multiple of 32
  const int tile_rows = (int)(rows - m0 < kTileM ? rows - m0 : kTileM);
  const int KS = (int)(D / kKStep);
  const int ks0 = split * ks_per_split;
  const int ks1 = ks0 + ks_per_split < KS ? ks0 + ks_per_split : KS;

  CT::Acc acc;
  tile::zero<2, 2, 4, 4>(acc);
  tile::mma<2, 2, 4, 4, DFS_CONV_DEPTH>(tile::rows_rsrc(x + m0 * D, tile_rows, D),
                                        tile::rows_rsrc(Wc + n0 * D, ncols, D), D, ks0, ks1, lds, acc);

  float* sC = reinterpret_cast<float*>(lds);  // [kTileM][kPitchC], after the loop's last barrier
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sC[(64 * wm + 16 * a + 4 * q + i) * kPitchC + 64 * wn + 16 * b + r] = acc.v[a][b][i];
  __syncthreads();
  if (splits > 1) {  // this split's partial sums [rows, D/8] of the tile; the epilogue kernel adds them
    float* pp = partial + (int64_t)split * rows * ncols_all;
    const int nv = ncols / 4;
    for (int jb = tid; jb < tile_rows * nv; jb += kThreads) {
      const int rr = jb / nv;
      const int v = jb - rr * nv;
      *reinterpret_cast<float4*>(pp + (m0 + rr) * ncols_all + n0 + 4 * v) =
          *reinterpret_cast<const float4*>(&sC[rr * kPitchC + 4 * v]);
    }
    return;
  }

  // The convolution of this tile's rows over its 8 * ncols channels, eight channels
  // (16 bytes) per job; column 2g + tap of the tile is group g's correction.
  const int64_t ch0 = 8 * n0;
  const int jobs = tile_rows * ncols;
  for (int jb = tid; jb < jobs; jb += kThreads) {
    const int rr = jb / ncols;
    const int v = jb - rr * ncols;
    const int64_t m = m0 + rr;
    const int64_t ch = ch0 + 8 * v;
    const int64_t b = m / L;
    const int t = (int)(m - b * L);
    const float c0 = sC[rr * kPitchC + 2 * (v >> 1)];
    const float c1 = sC[rr * kPitchC + 2 * (v >> 1) + 1];
    const uint4 xv = *reinterpret_cast<const uint4*>(x + m * D + ch);
    const uint4 pv = t > 0 ? *reinterpret_cast<const uint4*>(x + (m - 1) * D + ch)
                           : *reinterpret_cast<const uint4*>(xprev + b * D + ch);
    const uint4 b0 = *reinterpret_cast<const uint4*>(base + ch);
    const uint4 b1 = *reinterpret_cast<const uint4*>(base + D + ch);
    *reinterpret_cast<uint4*>(y + m * D + ch) = conv8(xv, pv, b0, b1, c0, c1);
  }
}

// The convolution after a K-split correction: partial sums added in split order.
__global__ __launch_bounds__(kThreads) void conv2_split_epilogue_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xprev,
    const uint16_t* __restrict__ base, const float* __restrict__ partial, int splits, int64_t rows,
    int L, int64_t D, uint16_t* __restrict__ y) {
  const int64_t nvec = D / 8;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * nvec) return;
  const int64_t m = i / nvec;
  const int64_t ch = 8 * (i - m * nvec);
  const int64_t b = m / L;
  const int t = (int)(m - b * L);
  const int64_t col = m * nvec + 2 * (ch / 16);
  float c0 = 0.0f, c1 = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const float2 v = *reinterpret_cast<const float2*>(partial + s * rows * nvec + col);
    c0 += v.x;
    c1 += v.y;
  }
  const uint4 xv = *reinterpret_cast<const uint4*>(x + m * D + ch);
  const uint4 pv = t > 0 ? *reinterpret_cast<const uint4*>(x + (m - 1) * D + ch)
                         : *reinterpret_cast<const uint4*>(xprev + b * D + ch);
  const uint4 b0 = *reinterpret_cast<const uint4*>(base + ch);
  const uint4 b1 = *reinterpret_cast<const uint4*>(base + D + ch);
  *reinterpret_cast<uint4*>(y + m * D + ch) = conv8(xv, pv, b0, b1, c0, c1);
}

// ---------------------------------------------------------------- fp32 path
constexpr int kF32Rows = 8;  // rows per wave

// c[m, n] = sum_k x[m, k] W_c[n, k] for 8 rows and one column per wave: lanes
// stride k (coalesced), then a fixed-order reduction across the wave.
__global__ __launch_bounds__(kWave) void corr_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ Wc, int64_t rows,
                                                         int64_t D, float* __restrict__ c) {
  const int lane = threadIdx.x;
  const int64_t N = D / 8;
  const int64_t n = (int64_t)blockIdx.x % N;
  const int64_t m0 = (int64_t)blockIdx.x / N * kF32Rows;
  float acc[kF32Rows];
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) acc[i] = 0.0f;
  for (int64_t k = lane; k < D; k += kWave) {
    const float w = Wc[n * D + k];
#pragma unroll
    for (int i = 0; i < kF32Rows; ++i)
      if (m0 + i < rows) acc[i] = fmaf(x[(m0 + i) * D + k], w, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) {
    float v = acc[i];
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) v += __uint_as_float(xor_lanes(__float_as_uint(v), s, lane));
    if (lane == 0 && m0 + i < rows) c[(m0 + i) * N + n] = v;
  }
}

__global__ __launch_bounds__(kThreads) void conv2_apply_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ xprev, const float* __restrict__ base,
    const float* __restrict__ c, int64_t rows, int L, int64_t D, float* __restrict__ y) {
  const int64_t nvec = D / 4;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * nvec) return;
  const int64_t m = i / nvec;
  const int64_t ch = 4 * (i - m * nvec);
  const int64_t b = m / L;
  const int t = (int)(m - b * L);
  const int64_t g = ch / 16;
  const float c0 = c[m * (D / 8) + 2 * g];
  const float c1 = c[m * (D / 8) + 2 * g + 1];
  const float4 xv = *reinterpret_cast<const float4*>(x + m * D + ch);
  const float4 pv = t > 0 ? *reinterpret_cast<const float4*>(x + (m - 1) * D + ch)
                          : *reinterpret_cast<const float4*>(xprev + b * D + ch);
  const float4 b0 = *reinterpret_cast<const float4*>(base + ch);
  const float4 b1 = *reinterpret_cast<const float4*>(base + D + ch);
  float4 o;
  o.x = fmaf(b0.x + c0, xv.x, (b1.x + c1) * pv.x);
  o.y = fmaf(b0.y + c0, xv.y, (b1.y + c1) * pv.y);
  o.z = fmaf(b0.z + c0, xv.z, (b1.z + c1) * pv.z);
  o.w = fmaf(b0.w + c0, xv.w, (b1.w + c1) * pv.w);
  *reinterpret_cast<float4*>(y + m * D + ch) = o;
}

}  // namespace

int64_t conv2_max_f32_elems() { return (int64_t)1 << 34; }

#ifndef DFS_CONV_TARGET_WG
#define DFS_CONV_TARGET_WG 512
#endif
// K splits of the bf16 correction (enough workgroups for the chip, at least 8 k steps
// each) and k steps per split; every split gets at least one step.
struct ConvSplit {
  int splits, kps;
};
ConvSplit conv2_splits(int64_t rows, int64_t D) {
  const int64_t ks = D / kKStep;
#ifdef DFS_CONV_SPLITS
  (void)rows;
  int64_t s = DFS_CONV_SPLITS;
#else
  const int64_t tiles = cdiv(rows, kTileM) * cdiv(D / 8, kTileN);
  int64_t s = DFS_CONV_TARGET_WG / tiles;
#endif
  if (s > ks / 8) s = ks / 8;
  if (s < 1) s = 1;
  const int64_t kps = cdiv(ks, s);
  return ConvSplit{(int)cdiv(ks, kps), (int)kps};
}

size_t conv2_workspace_bytes(int64_t rows, int64_t D, bool bf16) {
  const int64_t splits = bf16 ? conv2_splits(rows, D).splits : 1;
  if (bf16 && splits == 1) return 0;
  return align_up((size_t)splits * (size_t)rows * (size_t)(D / 8) * sizeof(float), 256);
}

hipError_t launch_conv2(const void* x, const void* x_prev, const void* base, const void* W_c,
                        bool bf16, int64_t batch, int64_t L, int64_t D, void* y, void* ws,
                        hipStream_t stream) {
  const int64_t rows = batch * L;
  if (bf16) {
    const int ntn = (int)cdiv(D / 8, kTileN);
    const int64_t mtiles = cdiv(rows, kTileM);
    const ConvSplit sp = conv2_splits(rows, D);
    const int splits = sp.splits, kps = sp.kps;
    const dim3 grid((unsigned)((DFS_CONV_XCD ? cdiv(mtiles, 8) * 8 : mtiles) * ntn * splits));
    conv2_bf16_kernel<<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(x_prev),
        static_cast<const uint16_t*>(base), static_cast<const uint16_t*>(W_c), rows, (int)L, D, ntn,
        mtiles, splits, kps, static_cast<float*>(ws), static_cast<uint16_t*>(y));
    if (splits > 1) {
      conv2_split_epilogue_kernel<<<dim3((unsigned)cdiv(rows * (D / 8), kThreads)), kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(x_prev),
          static_cast<const uint16_t*>(base), static_cast<const float*>(ws), splits, rows, (int)L, D,
          static_cast<uint16_t*>(y));
    }
  } else {
    float* c = static_cast<float*>(ws);
    corr_f32_kernel<<<dim3((unsigned)(D / 8 * cdiv(rows, kF32Rows))), kWave, 0, stream>>>(
        static_cast<const float*>(x), static_cast<const float*>(W_c), rows, D, c);
    const int64_t jobs = rows * (D / 4);
    conv2_apply_f32_kernel<<<dim3((unsigned)cdiv(jobs, kThreads)), kThreads, 0, stream>>>(
        static_cast<const float*>(x), static_cast<const float*>(x_prev),
        static_cast<const float*>(base), c, rows, (int)L, D, static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace dfs
