// Context gate H(h_t) = sigmoid(h_t W_h) for every block position.
//
// The post scores each candidate pair under a gate computed from the drafter's
// hidden state (blog post "DFlash 2: Keep Drafting Parallel", section "A
// Lightweight Path Selector"); the sigmoid of a [d, 256] linear map is this
// library's parameterisation of it.
//
// bf16 path (gfx950 matrix cores): Z[rows, 256] = H[rows, d] x W_h[d, 256] with
// V_MFMA_F32_16X16X32_BF16.  The MFMA wants every lane's operand to be 8
// consecutive k values, but W_h is n-contiguous, so W_h is first repacked once per
// call into [d/32][256][32] (2.6 MB at d = 5120, stays in L2) and both operands are
// then read straight from memory with 16-byte loads.  Each wave owns 64 output
// columns and 16 * MT rows; small row counts split K across workgroups and a
// finish kernel adds the partial sums in a fixed order and applies the sigmoid.
// fp32 path: plain FMA over a [8 rows x 256 columns] tile per workgroup.
#include "dfs_device.h"
#include "dfs_internal.h"

namespace dfs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKB = 32;          // k per MFMA step
constexpr int kTargetWG = 256;   // one workgroup per CU is enough for this small GEMM

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// Wp[kb][n][kk] = W[kb*32 + kk][n], zero past d.
__global__ __launch_bounds__(kThreads) void pack_w_kernel(const uint16_t* __restrict__ W,
                                                          int64_t d, uint16_t* __restrict__ Wp) {
  const int n = threadIdx.x;
  const int64_t kb = blockIdx.x >> 2;
  const int g = blockIdx.x & 3;  // which 8 of the 32 k values
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = kb * kKB + g * 8 + i;
    v[i] = k < d ? W[k * kE + n] : (uint16_t)0;
  }
  uint4 o;
  o.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
  o.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
  o.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
  o.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
  *reinterpret_cast<uint4*>(Wp + ((kb * kE + n) * kKB + g * 8)) = o;
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gate_mfma_kernel(const uint16_t* __restrict__ H,
                                                             const uint16_t* __restrict__ Wp,
                                                             int64_t rows, int64_t d,
                                                             int64_t kchunk, int splits,
                                                             float* __restrict__ partial,
                                                             float* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16 * MT;
  const int s = blockIdx.y;
  const int64_t kb0 = (int64_t)s * kchunk / kKB;
  int64_t kb1 = ((int64_t)s + 1) * kchunk / kKB;
  const int64_t KB = (d + kKB - 1) / kKB;
  if (kb1 > KB) kb1 = KB;

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    const int64_t k = kb * kKB + 8 * q;  // this lane's 8 k values; d % 8 == 0
    uint4 a[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m0 + 16 * mt + r;
      a[mt] = zero;
      if (m < rows && k < d) a[mt] = *reinterpret_cast<const uint4*>(H + m * d + k);
    }
    uint4 b[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = 64 * wave + 16 * nt + r;
      b[nt] = *reinterpret_cast<const uint4*>(Wp + (kb * kE + n) * kKB + 8 * q);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[mt]), __builtin_bit_cast(bf16x8, b[nt]), acc[mt][nt], 0, 0,
            0);
  }
  // lane holds D[4q + i][r] of each 16x16 tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 16 * mt + 4 * q + i;
        const int n = 64 * wave + 16 * nt + r;
        if (m < rows) {
          if (splits == 1) {
            out[m * kE + n] = sigmoidf(acc[mt][nt][i]);
          } else {
            partial[((int64_t)s * rows + m) * kE + n] = acc[mt][nt][i];
          }
        }
      }
}

constexpr int kF32Rows = 8;

__global__ __launch_bounds__(kThreads) void gate_f32_kernel(const float* __restrict__ H,
                                                            const float* __restrict__ W,
                                                            int64_t rows, int64_t d,
                                                            int64_t kchunk, int splits,
                                                            float* __restrict__ partial,
                                                            float* __restrict__ out) {
  const int n = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * kF32Rows;
  const int s = blockIdx.y;
  const int64_t k0 = (int64_t)s * kchunk;
  const int64_t k1 = k0 + kchunk < d ? k0 + kchunk : d;
  float acc[kF32Rows];
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) acc[i] = 0.0f;
  for (int64_t k = k0; k < k1; ++k) {
    const float w = W[k * kE + n];
#pragma unroll
    for (int i = 0; i < kF32Rows; ++i)
      if (m0 + i < rows) acc[i] = fmaf(H[(m0 + i) * d + k], w, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < kF32Rows; ++i) {
    const int64_t m = m0 + i;
    if (m < rows) {
      if (splits == 1) {
        out[m * kE + n] = sigmoidf(acc[i]);
      } else {
        partial[((int64_t)s * rows + m) * kE + n] = acc[i];
      }
    }
  }
}

// out[m, n] = sigmoid(sum over splits, in split order).
__global__ __launch_bounds__(kThreads) void gate_finish_kernel(const float* __restrict__ partial,
                                                               int64_t rows, int splits,
                                                               float* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int n = threadIdx.x;
  float z = 0.0f;
  for (int s = 0; s < splits; ++s) z += partial[((int64_t)s * rows + m) * kE + n];
  out[m * kE + n] = sigmoidf(z);
}

}  // namespace

GatePlan plan_gate(int64_t rows, int64_t d, bool bf16) {
  GatePlan p{};
  p.rows = rows;
  p.d = d;
  p.bf16 = bf16;
  size_t off = 0;
  if (bf16) {
    p.row_tiles = rows >= 2048 ? 4 : 1;
    const int64_t mtiles = cdiv(rows, 16 * p.row_tiles);
    const int64_t KB = cdiv(d, kKB);
    int64_t splits = cdiv(kTargetWG, mtiles);
    const int64_t max_splits = KB / 2 > 1 ? KB / 2 : 1;  // at least two k steps per split
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    const int64_t kb_per = cdiv(KB, splits);
    p.kchunk = kb_per * kKB;
    p.splits = (int)cdiv(KB, kb_per);
    p.packed_off = 0;
    p.packed_bytes = align_up((size_t)KB * kE * kKB * sizeof(uint16_t), 256);
    off = p.packed_bytes;
  } else {
    p.row_tiles = 0;
    const int64_t mtiles = cdiv(rows, kF32Rows);
    int64_t splits = cdiv(kTargetWG, mtiles);
    const int64_t max_splits = d / 64 > 1 ? d / 64 : 1;  // at least 64 k per split
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    p.kchunk = cdiv(d, splits);
    p.splits = (int)cdiv(d, p.kchunk);
    p.packed_off = 0;
    p.packed_bytes = 0;
  }
  p.partial_off = off;
  p.partial_bytes = p.splits > 1 ? align_up((size_t)p.splits * rows * kE * sizeof(float), 256) : 0;
  p.ws_bytes = p.partial_off + p.partial_bytes;
  return p;
}

hipError_t launch_gate(const GatePlan& p, const void* hidden, const void* W_h, float* out_gate,
                       void* ws, hipStream_t stream) {
  char* wsb = static_cast<char*>(ws);
  float* partial = p.splits > 1 ? reinterpret_cast<float*>(wsb + p.partial_off) : nullptr;
  if (p.bf16) {
    uint16_t* Wp = reinterpret_cast<uint16_t*>(wsb + p.packed_off);
    const int64_t KB = cdiv(p.d, kKB);
    pack_w_kernel<<<dim3((unsigned)(KB * 4)), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(W_h), p.d, Wp);
    const uint16_t* H = static_cast<const uint16_t*>(hidden);
    if (p.row_tiles == 4) {
      const dim3 grid((unsigned)cdiv(p.rows, 64), (unsigned)p.splits);
      gate_mfma_kernel<4><<<grid, kThreads, 0, stream>>>(H, Wp, p.rows, p.d, p.kchunk, p.splits,
                                                          partial, out_gate);
    } else {
      const dim3 grid((unsigned)cdiv(p.rows, 16), (unsigned)p.splits);
      gate_mfma_kernel<1><<<grid, kThreads, 0, stream>>>(H, Wp, p.rows, p.d, p.kchunk, p.splits,
                                                          partial, out_gate);
    }
  } else {
    const dim3 grid((unsigned)cdiv(p.rows, kF32Rows), (unsigned)p.splits);
    gate_f32_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const float*>(hidden),
                                                   static_cast<const float*>(W_h), p.rows, p.d,
                                                   p.kchunk, p.splits, partial, out_gate);
  }
  if (p.splits > 1) {
    gate_finish_kernel<<<dim3((unsigned)p.rows), kThreads, 0, stream>>>(partial, p.rows, p.splits,
                                                                        out_gate);
  }
  return hipGetLastError();
}

}  // namespace dfs
