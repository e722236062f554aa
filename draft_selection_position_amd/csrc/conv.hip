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
// (mfma_big.h: 128 x 128 tiles, operands loaded straight into LDS); a workgroup's
// epilogue applies the convolution to exactly its 128 rows and 1024 channels, so the
// correction never leaves the chip.  W_c is K-contiguous, the operand order the tile wants: no
// repacking.  Shapes too small to fill the chip split K; an elementwise kernel then
// adds the split partial sums in split order and applies the convolution (a
// device-wide fence per workgroup to let the last split do it in place writes
// back the L2 of a multi-XCD part and measured three times slower).
// fp32 path (small shapes): one kernel, each workgroup the correction of an 8-row by
// 8-column tile by vector dot products (K split over its four waves) and then the
// convolution of those rows over the 64 channels the columns serve.
#include "dfs_device.h"
#include "dfs_internal.h"
#include "mfma_big.h"
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
// The product's mainloop: the LDS-DMA double buffer of 64 k per step (mfma_big.h),
// or (DFS_CONV_BIG 0) the register-staged tile of mfma_tile.h.  Both add the k
// chunks in the same order.
#ifndef DFS_CONV_BIG
#define DFS_CONV_BIG 1
#endif
using ConvCfg = big::Cfg<4, 4, 2, 64>;
static_assert(ConvCfg::BM == kTileM && ConvCfg::BN == kTileN && ConvCfg::KK == kKStep, "same tile");
constexpr int kMainLds = DFS_CONV_BIG ? ConvCfg::kLdsBytes : CT::kLdsBytes;
constexpr int kConvLds = kMainLds > kTileM * kPitchC * 4 ? kMainLds : kTileM * kPitchC * 4;

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
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kConvLds / 2];
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

#if DFS_CONV_BIG
  ConvCfg::Acc acc;
  ConvCfg::zero(acc);
  big::mma<ConvCfg>(big::rows_operand(x + m0 * D, tile_rows, D, kKStep),
                    big::rows_operand(Wc + n0 * D, ncols, D, kKStep), ks0, ks1, reinterpret_cast<char*>(lds), acc);
#else
  CT::Acc acc;
  tile::zero<2, 2, 4, 4>(acc);
  tile::mma<2, 2, 4, 4, DFS_CONV_DEPTH>(tile::rows_rsrc(x + m0 * D, tile_rows, D),
                                        tile::rows_rsrc(Wc + n0 * D, ncols, D), D, ks0, ks1, lds, acc);
#endif

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
// One thread per 16-byte piece (8 channels) of kR consecutive positions of one
// sequence: each position's x piece is read once and serves as the next position's
// predecessor from registers (with kR = 1 the predecessor is read again), and the
// base kernel's two pieces are read once.  Per position, the group's two correction
// columns are read for every split and added in split order.  Every load of a run
// (its x pieces and, up to kSplitRegs splits, all its correction columns) is issued
// before the first sum, so a thread waits for memory once, not once per position.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_sum(const float* pc, int64_t sstride, int splits, float& c0, float& c1) {
  c0 = 0.0f;
  c1 = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const f32x2 v = *reinterpret_cast<const f32x2*>(pc + s * sstride);
    c0 += v.x;
    c1 += v.y;
  }
}

#ifndef DFS_CONV_EPI_SPLIT_REGS
#define DFS_CONV_EPI_SPLIT_REGS 4
#endif
constexpr int kSplitRegs = DFS_CONV_EPI_SPLIT_REGS;  // splits whose columns are loaded up front
// The output leaves with non-temporal stores (nothing here reads it back): at 4096 x 5120
// with three splits the epilogue's loads issued up front and these stores took a call
// from 66.4 to 65.0 us.
#ifndef DFS_CONV_EPI_NT
#define DFS_CONV_EPI_NT 1
#endif

template <typename Idx, int kR>
__global__ __launch_bounds__(kThreads) void conv2_split_epilogue_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xprev,
    const uint16_t* __restrict__ base, const float* __restrict__ partial, int splits, int64_t batch,
    int L, int64_t D, uint16_t* __restrict__ y) {
  const Idx P = (Idx)(D / 8);                 // pieces per row
  const Idx runs = (Idx)((L + kR - 1) / kR);  // runs of kR positions per sequence
  const Idx j = (Idx)blockIdx.x * kThreads + threadIdx.x;
  if ((int64_t)j >= batch * (int64_t)runs * (int64_t)P) return;
  const Idx run = j / P;                      // (sequence, run), pieces fastest
  const int64_t ch = 8 * (int64_t)(j - run * P);
  const Idx b = run / runs;
  const int t0 = (int)(run - b * runs) * kR;
  const int n = (t0 + kR < L ? t0 + kR : L) - t0;  // positions of this run, 1..kR
  const int64_t rows = batch * (int64_t)L;
  const int64_t nvec = D / 8;
  const int64_t sstride = rows * nvec;
  const uint4 b0 = *reinterpret_cast<const uint4*>(base + ch);
  const uint4 b1 = *reinterpret_cast<const uint4*>(base + D + ch);
  const int64_t m0 = (int64_t)b * L + t0;
  uint4 pv = t0 > 0 ? *reinterpret_cast<const uint4*>(x + (m0 - 1) * D + ch)
                    : *reinterpret_cast<const uint4*>(xprev + (int64_t)b * D + ch);
  uint4 xs[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i)
    xs[i] = i < n ? *reinterpret_cast<const uint4*>(x + (m0 + i) * D + ch) : make_uint4(0u, 0u, 0u, 0u);
  const float* pc = partial + m0 * nvec + 2 * (ch / 16);
  float c0[kR], c1[kR];
  if (splits <= kSplitRegs) {
    f32x2 v[kR][kSplitRegs];
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
      for (int s = 0; s < kSplitRegs; ++s)
        v[i][s] = (i < n && s < splits) ? *reinterpret_cast<const f32x2*>(pc + i * nvec + s * sstride)
                                        : f32x2{0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      c0[i] = 0.0f;
      c1[i] = 0.0f;
#pragma unroll
      for (int s = 0; s < kSplitRegs; ++s)
        if (s < splits) {
          c0[i] += v[i][s].x;
          c1[i] += v[i][s].y;
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kR; ++i)
      if (i < n) split_sum(pc + i * nvec, sstride, splits, c0[i], c1[i]);
  }
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (i < n) {
      const uint4 o = conv8(xs[i], pv, b0, b1, c0[i], c1[i]);
#if DFS_CONV_EPI_NT
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4_t*>(y + (m0 + i) * D + ch));
#else
      *reinterpret_cast<uint4*>(y + (m0 + i) * D + ch) = o;
#endif
      pv = xs[i];
    }
  }
}

// Positions per thread of the split epilogue: runs of 4 while that leaves enough
// threads to fill the chip, else one position per thread.
#ifndef DFS_CONV_EPI_RUN
#define DFS_CONV_EPI_RUN 4
#endif
#ifndef DFS_CONV_EPI_MIN_THREADS
#define DFS_CONV_EPI_MIN_THREADS (256 * 1024)
#endif

// ---------------------------------------------------------------- fp32 path
constexpr int kF32Rows = 8;  // rows of a workgroup
constexpr int kF32Cols = 8;  // correction columns of a workgroup: four groups, 64 channels

// Sum over the wave of v[lane] for each of 64 per-lane values, ending in lane j with
// the sum of everyone's v[j]: six exchange steps, each halving the values a lane
// keeps (63 exchanges in all, against 384 for 64 separate butterflies).  Fixed
// pairing, so the result does not depend on timing.
__device__ __forceinline__ float wave_transpose_sum(float (&v)[64], int lane) {
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int s = 32 >> st;  // partner distance, also the values kept after this step
    const bool up = (lane & s) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      const float keep = up ? v[i + s] : v[i];
      const float give = up ? v[i] : v[i + s];
      v[i] = keep + __uint_as_float(xor_lanes(__float_as_uint(give), s, lane));
    }
  }
  return v[0];
}

// One workgroup: the correction c[m0 .. m0+7, 8 cg .. 8 cg + 7] and the convolution
// of those 8 rows over the 64 channels those columns serve.  The four waves split K
// (wave w takes the 256-wide k slices w, w + 4, ...; a lane one float4 of each), sum
// their slice partials within the wave, then in a fixed order across waves in LDS.
// Rows past the end load the last row and are not written.
__global__ __launch_bounds__(kThreads) void conv2_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ xprev, const float* __restrict__ base,
    const float* __restrict__ Wc, int64_t rows, int L, int64_t D, float* __restrict__ y) {
  __shared__ float part[4][64];
  __shared__ float cs[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ncg = D / 8 / kF32Cols;
  const int64_t cg = (int64_t)blockIdx.x % ncg;
  const int64_t m0 = (int64_t)blockIdx.x / ncg * kF32Rows;
  const float* xr[kF32Rows];
#pragma unroll
  for (int r = 0; r < kF32Rows; ++r) xr[r] = x + (m0 + r < rows ? m0 + r : rows - 1) * D;
  const float* wr = Wc + kF32Cols * cg * D;
  float v[64];  // v[8 r + j]: partial of c[m0 + r, 8 cg + j]
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = 0.0f;
  for (int64_t k = 4 * lane + 256 * wave; k < D; k += 1024) {
    float4 w[kF32Cols], xv[kF32Rows];
#pragma unroll
    for (int j = 0; j < kF32Cols; ++j) w[j] = *reinterpret_cast<const float4*>(wr + j * D + k);
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r) xv[r] = *reinterpret_cast<const float4*>(xr[r] + k);
#pragma unroll
    for (int r = 0; r < kF32Rows; ++r)
#pragma unroll
      for (int j = 0; j < kF32Cols; ++j) {
        float a = v[8 * r + j];
        a = fmaf(xv[r].x, w[j].x, a);
        a = fmaf(xv[r].y, w[j].y, a);
        a = fmaf(xv[r].z, w[j].z, a);
        v[8 * r + j] = fmaf(xv[r].w, w[j].w, a);
      }
  }
  part[wave][lane] = wave_transpose_sum(v, lane);
  __syncthreads();
  if (wave == 0) cs[lane] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  __syncthreads();
  // the convolution: 8 rows x 64 channels, two per thread; cs[8 r + 2 g + tap]
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = tid + kThreads * h;
    const int r = e >> 6, cl = e & 63;
    const int64_t m = m0 + r;
    if (m >= rows) continue;
    const int64_t ch = 64 * cg + cl;
    const int64_t b = m / L;
    const int t = (int)(m - b * L);
    const float c0 = cs[8 * r + 2 * (cl >> 4)];
    const float c1 = cs[8 * r + 2 * (cl >> 4) + 1];
    const float xv = x[m * D + ch];
    const float pv = t > 0 ? x[(m - 1) * D + ch] : xprev[b * D + ch];
    y[m * D + ch] = fmaf(base[ch] + c0, xv, (base[D + ch] + c1) * pv);
  }
}

}  // namespace

// fp32 grid: batch * L * D / 512 workgroups of 256 threads, within 2^32 work-items.
int64_t conv2_max_f32_elems() { return (int64_t)1 << 32; }

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
  if (splits == 1) return 0;
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
      const int64_t runs4 = cdiv(L, DFS_CONV_EPI_RUN);
      const bool long_runs = DFS_CONV_EPI_RUN > 1 && batch * runs4 * (D / 8) >= DFS_CONV_EPI_MIN_THREADS;
      const int64_t jobs = batch * (long_runs ? runs4 : L) * (D / 8);
      const dim3 eg((unsigned)cdiv(jobs, kThreads));
      const uint16_t* xp = static_cast<const uint16_t*>(x);
      const uint16_t* pp = static_cast<const uint16_t*>(x_prev);
      const uint16_t* bp = static_cast<const uint16_t*>(base);
      const float* sp = static_cast<const float*>(ws);
      uint16_t* yp = static_cast<uint16_t*>(y);
      if (jobs < ((int64_t)1 << 31)) {
        if (long_runs)
          conv2_split_epilogue_kernel<uint32_t, DFS_CONV_EPI_RUN><<<eg, kThreads, 0, stream>>>(xp, pp, bp, sp, splits, batch, (int)L, D, yp);
        else
          conv2_split_epilogue_kernel<uint32_t, 1><<<eg, kThreads, 0, stream>>>(xp, pp, bp, sp, splits, batch, (int)L, D, yp);
      } else {
        if (long_runs)
          conv2_split_epilogue_kernel<uint64_t, DFS_CONV_EPI_RUN><<<eg, kThreads, 0, stream>>>(xp, pp, bp, sp, splits, batch, (int)L, D, yp);
        else
          conv2_split_epilogue_kernel<uint64_t, 1><<<eg, kThreads, 0, stream>>>(xp, pp, bp, sp, splits, batch, (int)L, D, yp);
      }
    }
  } else {
    conv2_f32_kernel<<<dim3((unsigned)(D / 8 / kF32Cols * cdiv(rows, kF32Rows))), kThreads, 0, stream>>>(
        static_cast<const float*>(x), static_cast<const float*>(x_prev),
        static_cast<const float*>(base), static_cast<const float*>(W_c), rows, (int)L, D,
        static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace dfs
