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
// bf16 path, one kernel: the correction is a [rows, D] x [D, D/8] product on the
// matrix cores (V_MFMA_F32_16X16X32_BF16); a workgroup computes 64 rows x 128
// correction columns (64 groups = 1024 channels), and its epilogue applies the
// convolution to exactly those rows and channels, so the correction never
// leaves the chip.  W_c is K-contiguous, which is the MFMA operand order already:
// no repacking.  Per 64-wide k step a lane holds 16 consecutive k of its row (two
// MFMAs, the same k permutation on both operands), so each W_c fragment is one
// full 128-byte line per column.
// fp32 path (small shapes): the correction by wave dot products into workspace,
// then an elementwise kernel.
#include "dfs_device.h"
#include "dfs_internal.h"

namespace dfs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
constexpr int kThreads = 256;                 // 4 waves, one per 32 correction columns
constexpr int kTileM = 64;                    // rows per workgroup
constexpr int kTileN = 128;                   // correction columns per workgroup
constexpr int kKStep = 64;                    // k per step (two MFMAs per tile)
constexpr int kDepth = 3;                     // k steps in flight per thread
constexpr int kPitchA = kKStep + 8;           // bf16 per LDS row of the x tile
constexpr int kPitchC = kTileN + 4;           // fp32 per LDS row of the correction tile

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

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

__global__ __launch_bounds__(kThreads) void conv2_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ xprev,
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ Wc, int64_t rows, int L,
    int64_t D, int ntiles_n, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileM][kPitchA];
  __shared__ __attribute__((aligned(16))) float sC[kTileM][kPitchC];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int n_tile = (int)(blockIdx.x % (unsigned)ntiles_n);
  const int64_t m0 = (int64_t)(blockIdx.x / (unsigned)ntiles_n) * kTileM;
  const int64_t ncols_all = D / 8;
  const int64_t n0 = (int64_t)n_tile * kTileN;
  const int ncols = (int)(ncols_all - n0 < kTileN ? ncols_all - n0 : kTileN);  // a multiple of 32
  const bool wave_on = 32 * wave < ncols;
  const int tile_rows = (int)(rows - m0 < kTileM ? rows - m0 : kTileM);

  // x rows [m0, m0 + tile_rows): rows past the end read as zeros (range check)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * D), (short)0, (int)((int64_t)tile_rows * D * 2), kRawBufferWord3);
  const uint32_t a_voff = (uint32_t)((((int64_t)(tid >> 2)) * D + 16 * (tid & 3)) * 2);
  // W_c rows [n0, n0 + ncols): this wave's are 32 wave + 16 nt + r
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wc + n0 * D), (short)0, (int)((int64_t)ncols * D * 2), kRawBufferWord3);
  const uint32_t b_voff0 = (uint32_t)(((int64_t)(32 * wave + r) * D + 16 * q) * 2);
  const uint32_t b_voff1 = b_voff0 + (uint32_t)(16 * D * 2);

  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KS = (int)(D / kKStep);
  uint4 ra[kDepth][2], rb[kDepth][2][2];
  auto fill = [&](int j, int ks) {
    const uint32_t so = (uint32_t)ks * kKStep * 2;
    ra[j][0] = bload(xr, a_voff, so);
    ra[j][1] = bload(xr, a_voff + 16, so);
    rb[j][0][0] = bload(wr, b_voff0, so);
    rb[j][0][1] = bload(wr, b_voff0 + 16, so);
    rb[j][1][0] = bload(wr, b_voff1, so);
    rb[j][1][1] = bload(wr, b_voff1 + 16, so);
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j) fill(j, j < KS ? j : KS - 1);

  auto step = [&](int ks, int j) {
    const int st = ks & 1;
    *reinterpret_cast<uint4*>(&sA[st][tid >> 2][16 * (tid & 3)]) = ra[j][0];
    *reinterpret_cast<uint4*>(&sA[st][tid >> 2][16 * (tid & 3) + 8]) = ra[j][1];
    __syncthreads();
    if (wave_on) {
      const bf16x8 b00 = __builtin_bit_cast(bf16x8, rb[j][0][0]), b01 = __builtin_bit_cast(bf16x8, rb[j][0][1]);
      const bf16x8 b10 = __builtin_bit_cast(bf16x8, rb[j][1][0]), b11 = __builtin_bit_cast(bf16x8, rb[j][1][1]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sA[st][16 * mt + r][16 * q]);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sA[st][16 * mt + r][16 * q + 8]);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b00, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b10, acc[mt][1], 0, 0, 0);
        acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b01, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b11, acc[mt][1], 0, 0, 0);
      }
    }
  };
  int ks = 0;
  for (; ks + kDepth <= KS; ks += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      step(ks + j, j);
      fill(j, ks + j + kDepth < KS ? ks + j + kDepth : KS - 1);
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (ks + j < KS) step(ks + j, j);

  if (wave_on) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sC[16 * mt + 4 * q + i][32 * wave + 16 * nt + r] = acc[mt][nt][i];
  }
  __syncthreads();

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
    const float c0 = sC[rr][2 * (v >> 1)];
    const float c1 = sC[rr][2 * (v >> 1) + 1];
    const uint4 xv = *reinterpret_cast<const uint4*>(x + m * D + ch);
    const uint4 pv = t > 0 ? *reinterpret_cast<const uint4*>(x + (m - 1) * D + ch)
                           : *reinterpret_cast<const uint4*>(xprev + b * D + ch);
    const uint4 b0 = *reinterpret_cast<const uint4*>(base + ch);
    const uint4 b1 = *reinterpret_cast<const uint4*>(base + D + ch);
    *reinterpret_cast<uint4*>(y + m * D + ch) = conv8(xv, pv, b0, b1, c0, c1);
  }
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

size_t conv2_workspace_bytes(int64_t rows, int64_t D, bool bf16) {
  return bf16 ? 0 : align_up((size_t)rows * (size_t)(D / 8) * sizeof(float), 256);
}

hipError_t launch_conv2(const void* x, const void* x_prev, const void* base, const void* W_c,
                        bool bf16, int64_t batch, int64_t L, int64_t D, void* y, void* ws,
                        hipStream_t stream) {
  const int64_t rows = batch * L;
  if (bf16) {
    const int ntn = (int)cdiv(D / 8, kTileN);
    const dim3 grid((unsigned)(cdiv(rows, kTileM) * ntn));
    conv2_bf16_kernel<<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(x_prev),
        static_cast<const uint16_t*>(base), static_cast<const uint16_t*>(W_c), rows, (int)L, D, ntn,
        static_cast<uint16_t*>(y));
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
