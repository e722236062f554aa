// Context gate H(h_t) = sigmoid(h_t W_h) for every block position.
//
// The post scores each candidate pair under a gate computed from the drafter's
// hidden state (blog post "DFlash 2: Keep Drafting Parallel", section "A
// Lightweight Path Selector"); the sigmoid of a [d, 256] linear map is this
// library's parameterisation of it.
//
// bf16 path (gfx950 matrix cores): Z[rows, 256] = H[rows, d] x W_h[d, 256] with
// V_MFMA_F32_16X16X32_BF16.  The MFMA wants every lane's operand to be 8
// consecutive k values, but W_h is n-contiguous, so W_h is repacked into
// [ceil(d/32)][256][32] (gate_pack.h; 2.6 MB at d = 5120): by the caller once
// (dfs_gate_pack), or per call into the workspace.  Both operands are then read
// straight from memory with 16-byte loads.  Three tilings, one operand layout (so
// a K split adds the same products in the same order in each):
//   - up to 512 rows: 16-row x 256-column tiles of four waves (gate_tile.h), K split
//     across about 16 workgroups (up to 64 rows) or 256 (more); the same tiles ride in
//     the top-16 launch of the fused selector when W_h comes pre-packed, where that
//     pass leaves CU slots free (it runs one or two workgroups per CU at these sizes);
//   - from 512 rows (d a multiple of 64): 128 x 128 LDS-DMA tiles (gate_dma_kernel);
//   - otherwise: 64-row x 256-column tiles of eight waves sharing the H tile in LDS.
// Row counts too small to fill the chip split K; the partial sums are added in split
// order (by the finish kernel here, or by the pair kernel that reads the gate) before
// the sigmoid.
// fp32 path: plain FMA over [8 rows x 256 columns] tiles (gate_tile.h).
#include "dfs_device.h"
#include "dfs_internal.h"
#include "gate_pack.h"
#include "gate_tile.h"
#include "mfma_big.h"

namespace dfs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kKB = 32;          // k per MFMA step
static_assert(kKB == kPackK, "the GEMM steps through W_h one packed slab at a time");
#ifndef DFS_GATE_TARGET_WG
#define DFS_GATE_TARGET_WG 256
#endif
constexpr int kTargetWG = DFS_GATE_TARGET_WG;  // workgroups the K split aims for
// Independent tiles up to kGateTileRows rows: 16-row tiles over about DFS_GATE_SMALL_WG
// workgroups up to DFS_GATE_SMALL_ROWS rows (their partial sums are added on the
// critical path of a short call), tiles of 16 kTallGroups rows over about
// DFS_GATE_JOBS_WG beyond; at least this many k steps per split.
#ifndef DFS_GATE_SMALL_ROWS
#define DFS_GATE_SMALL_ROWS 64
#endif
#ifndef DFS_GATE_SMALL_WG
#define DFS_GATE_SMALL_WG 16
#endif
#ifndef DFS_GATE_JOBS_WG
#define DFS_GATE_JOBS_WG 128
#endif
#ifndef DFS_GATE_SMALL_MIN_STEPS
#define DFS_GATE_SMALL_MIN_STEPS 4
#endif
static_assert(kThreads == gtile::kThreads, "gate tiles are 256-thread workgroups");

__global__ __launch_bounds__(kPackThreads) void pack_w_kernel(const uint16_t* __restrict__ W,
                                                              int64_t d, uint16_t* __restrict__ Wp) {
  __shared__ uint16_t tile[kPackK][kPackPitch];
  pack_w_slab(W, d, Wp, blockIdx.x, threadIdx.x, tile);
}

#ifndef DFS_GATE_DEPTH
#define DFS_GATE_DEPTH 4
#endif
constexpr int kGemmThreads = 512;       // 8 waves, one per 32-column slice
constexpr int kTileM = 64;              // rows per workgroup
constexpr int kDepth = DFS_GATE_DEPTH;  // k steps in flight per thread (register ring)
constexpr int kOutPitch = kE + 4;       // fp32 per LDS row of the output tile

// Buffer loads (base and range in scalar registers, a fixed 32-bit offset per
// lane, the k step as a scalar offset): the per-step address work is scalar, and
// the hardware range check returns zeros for H rows past the end of the matrix.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Z tile [64 rows x 256 columns] of one K split.  Wave w owns columns
// [32 w, + 32) of all 64 rows: 8 MFMA tiles.  Per k step the H tile (64 x 32,
// shared by all waves) goes through one of two LDS buffers with one barrier, and
// each wave's W_h fragments (its own columns, fetched by no other wave) go straight
// from memory to registers; both are loaded kDepth steps ahead of use.  The result
// is transposed through LDS so that every row is stored as contiguous 16-byte pieces.
__global__ __launch_bounds__(kGemmThreads) void gate_mfma_kernel(const uint16_t* __restrict__ H,
                                                                 const uint16_t* __restrict__ Wp,
                                                                 int64_t rows, int64_t d,
                                                                 int64_t kchunk, int splits,
                                                                 float* __restrict__ partial,
                                                                 float* __restrict__ out) {
  constexpr int kPitch = kKB + 16;  // bf16 per LDS row of the H tile (+32 bytes: fewest bank conflicts)
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileM][kPitch];
  __shared__ __attribute__((aligned(16))) float sOut[kTileM][kOutPitch];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int s = (int)(blockIdx.x % (unsigned)splits);
  const int64_t m0 = (int64_t)(blockIdx.x / (unsigned)splits) * kTileM;
  const int KB = (int)((d + kKB - 1) / kKB);
  const int kb0 = s * (int)(kchunk / kKB);
  int kb1 = kb0 + (int)(kchunk / kKB);
  if (kb1 > KB) kb1 = KB;

  // H: rows [m0, rows) of this tile; thread tid < 256 holds row tid / 4, k 8 (tid % 4) of a step
  const int64_t tile_rows = rows - m0 < kTileM ? rows - m0 : kTileM;
  const __amdgpu_buffer_rsrc_t hrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(H + m0 * d), (short)0, (int)(tile_rows * d * 2), kRawBufferWord3);
  const int hk = 8 * (tid & 3);
  const uint32_t hvoff = (uint32_t)((((tid & 255) >> 2) * d + hk) * 2);
  const bool last_ok = (int64_t)(KB - 1) * kKB + hk < d;  // this piece of the last slab is inside d
  // W_h: packed slabs [KB][256][32]
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wp), (short)0, (int)((int64_t)KB * kE * kKB * 2), kRawBufferWord3);
  const int nb = 32 * wave + r;
  const uint32_t wvoff0 = (uint32_t)((nb * kKB + 8 * q) * 2);
  const uint32_t wvoff1 = wvoff0 + 16 * kKB * 2;

  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[kDepth], rb0[kDepth], rb1[kDepth];
  auto fill = [&](int j, int kb) {
    ra[j] = bload(hrs, hvoff, (uint32_t)kb * kKB * 2);
    rb0[j] = bload(wrs, wvoff0, (uint32_t)kb * kE * kKB * 2);
    rb1[j] = bload(wrs, wvoff1, (uint32_t)kb * kE * kKB * 2);
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j) fill(j, kb0 + j < kb1 ? kb0 + j : kb1 - 1);

  auto step = [&](int kb, uint4 a, uint4 b0, uint4 b1) {
    const int st = (kb - kb0) & 1;
    if (tid < 256) {
      const uint32_t keep = (kb < KB - 1 || last_ok) ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(&sA[st][tid >> 2][hk]) =
          make_uint4(a.x & keep, a.y & keep, a.z & keep, a.w & keep);
    }
    __syncthreads();
    const bf16x8 bfr[2] = {__builtin_bit_cast(bf16x8, b0), __builtin_bit_cast(bf16x8, b1)};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sA[st][16 * mt + r][8 * q]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[nt], acc[mt][nt], 0, 0, 0);
    }
  };
  int base = kb0;
  for (; base + kDepth <= kb1; base += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      step(base + j, ra[j], rb0[j], rb1[j]);
      fill(j, base + j + kDepth < kb1 ? base + j + kDepth : kb1 - 1);
    }
  }
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (base + j < kb1) step(base + j, ra[j], rb0[j], rb1[j]);

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sOut[16 * mt + 4 * q + i][32 * wave + 16 * nt + r] = acc[mt][nt][i];
  __syncthreads();
  const int c4 = tid & 63;
#pragma unroll
  for (int rr = tid >> 6; rr < kTileM; rr += kGemmThreads / 64) {
    const int64_t m = m0 + rr;
    if (m >= rows) break;
    float4 v = *reinterpret_cast<const float4*>(&sOut[rr][4 * c4]);
    if (splits == 1) {
      v = make_float4(sigmoidf(v.x), sigmoidf(v.y), sigmoidf(v.z), sigmoidf(v.w));
      *reinterpret_cast<float4*>(out + m * kE + 4 * c4) = v;
    } else {
      *reinterpret_cast<float4*>(partial + ((int64_t)s * rows + m) * kE + 4 * c4) = v;
    }
  }
}

// ---------------------------------------------------------------- many rows
// 128 x 128 tiles of Z on the LDS-DMA mainloop (mfma_big.h: four waves of 64 x 64,
// operands straight from memory into an S-stage LDS ring), for row counts that give
// enough tiles: W_h is read 128 rows at a time instead of 64, and no wave fetches
// operands another wave also fetches.  A ring step covers 64 k: whole 128-byte lines of
// the H rows, and two packed W_h slabs (row n of slab ks sits at ks * 256 * 64 + n * 64
// bytes, so the step's second 64 bytes of a row are one slab, 16 KB, further on).  The
// products are added in the same k order as 32-k steps.  Work items (K split, row tile,
// column half) are numbered column half fastest and cut into eight contiguous runs,
// one per XCD: an XCD holds one K slice of W_h in its L2, and the two column halves
// of a row tile read its H rows back to back (the second from L2).  K-split partial
// sums leave with non-temporal stores: another kernel reads them, mostly from another
// XCD, and dirty lines left in L2 would be written back at the end of this kernel.
#ifndef DFS_GATE_STAGES
#define DFS_GATE_STAGES 4
#endif
#ifndef DFS_GATE_DMA_ROWS
#define DFS_GATE_DMA_ROWS 512
#endif
#ifndef DFS_GATE_DMA_TM
#define DFS_GATE_DMA_TM 4  // 16 x 16 tiles per wave along the rows
#endif
#ifndef DFS_GATE_DMA_TN
#define DFS_GATE_DMA_TN 4  // and along the 256 columns
#endif
#ifndef DFS_GATE_DMA_WG_PER_CU
#define DFS_GATE_DMA_WG_PER_CU 1
#endif
#ifndef DFS_GATE_NT_PARTIALS
#define DFS_GATE_NT_PARTIALS 1  // partial sums bypass L2 on the way out (read by another kernel, often on another XCD)
#endif
#ifndef DFS_GATE_DMA_KK
#define DFS_GATE_DMA_KK 64  // k per ring step: two packed slabs, whole 128-byte H lines
#endif
using GC = big::Cfg<DFS_GATE_DMA_TM, DFS_GATE_DMA_TN, DFS_GATE_STAGES, DFS_GATE_DMA_KK>;
constexpr int kDmaSlabs = GC::KK / kKB;        // packed W_h slabs per ring step
constexpr int kDmaBM = GC::BM;                 // 128 rows
constexpr int kDmaBN = GC::BN;                 // 128 columns: two halves of the 256
constexpr int kDmaHalves = kE / kDmaBN;        // column tiles per row tile
static_assert(kDmaHalves * kDmaBN == kE, "column tiles cover the 256 columns");
constexpr int kDmaPitch = kDmaBN + 4;          // fp32 per LDS row of the output tile
constexpr int kDmaLds = GC::kLdsBytes > kDmaBM * kDmaPitch * 4 ? GC::kLdsBytes : kDmaBM * kDmaPitch * 4;

__global__ __launch_bounds__(kThreads, DFS_GATE_DMA_WG_PER_CU) void gate_dma_kernel(const uint16_t* __restrict__ H,
                                                               const uint16_t* __restrict__ Wp,
                                                               int64_t rows, int64_t d, int mtiles,
                                                               int splits, int kps, int per_xcd,
                                                               float* __restrict__ partial,
                                                               float* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds[kDmaLds];
  const int64_t t = (int64_t)(blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  if (t >= (int64_t)splits * mtiles * kDmaHalves) return;
  const int nh = (int)(t % kDmaHalves);
  const int mt = (int)((t / kDmaHalves) % mtiles);
  const int s = (int)((t / kDmaHalves) / mtiles);
  const int64_t m0 = (int64_t)mt * kDmaBM;
  const int tile_rows = (int)(rows - m0 < kDmaBM ? rows - m0 : kDmaBM);
  const int KB = (int)(d / GC::KK);  // ring steps over the whole K
  const int ks0 = s * kps;
  const int ks1 = ks0 + kps < KB ? ks0 + kps : KB;
  const big::Operand a = big::rows_operand(H + m0 * d, tile_rows, d, GC::KK);
  // row n of ring step ks: slab kDmaSlabs * ks (+ 1 for the second 64 bytes) at n * 64
  const big::Operand b = big::make_operand(Wp + nh * kDmaBN * kKB,
                                           (int64_t)(d / kKB) * kE * kKB * 2 - nh * kDmaBN * kKB * 2,
                                           (uint32_t)(kKB * 2), (uint32_t)(kDmaSlabs * kE * kKB * 2),
                                           (uint32_t)(kE * kKB * 2));
  GC::Acc acc;
  GC::zero(acc);
  big::mma<GC>(a, b, ks0, ks1, lds, acc);
  // the tile through LDS (rows of 128 fp32), then row-contiguous 16-byte stores
  float* sOut = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mt_ = 0; mt_ < GC::TM; ++mt_)
#pragma unroll
    for (int nt = 0; nt < GC::TN; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sOut[(16 * GC::TM * wm + 16 * mt_ + 4 * q + i) * kDmaPitch + 16 * GC::TN * wn + 16 * nt + r] =
            acc.v[mt_][nt][i];
  __syncthreads();
  constexpr int kRowF4 = kDmaBN / 4;  // float4 per row of the tile
  const int c4 = tid % kRowF4;
  for (int rr = tid / kRowF4; rr < tile_rows; rr += kThreads / kRowF4) {
    float4 v = *reinterpret_cast<const float4*>(&sOut[rr * kDmaPitch + 4 * c4]);
    const int64_t col = (int64_t)(m0 + rr) * kE + nh * kDmaBN + 4 * c4;
    if (splits == 1) {
      v = make_float4(sigmoidf(v.x), sigmoidf(v.y), sigmoidf(v.z), sigmoidf(v.w));
      *reinterpret_cast<float4*>(out + col) = v;
    } else {
#if DFS_GATE_NT_PARTIALS
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w},
                                  reinterpret_cast<f32x4_t*>(partial + (int64_t)s * rows * kE + col));
#else
      *reinterpret_cast<float4*>(partial + (int64_t)s * rows * kE + col) = v;
#endif
    }
  }
}

// ---------------------------------------------------------------- few rows, fp32
// Independent 256-thread tiles (gate_tile.h): bf16 16-row tiles on the packed W_h, or
// fp32 8-row tiles; workgroup j is job j.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void gate_jobs_kernel(GateJobs g) {
  __shared__ float sH[gtile::kF32Rows][gtile::kF32KBlock];
  run_gate_job(g, kBf16, blockIdx.x, threadIdx.x, sH);
}

// out[m, n] = sigmoid(sum over splits, in split order).  The loads are issued
// eight at a time ahead of the (ordered) additions.
__global__ __launch_bounds__(kThreads) void gate_finish_kernel(const float* __restrict__ partial,
                                                               int64_t rows, int splits,
                                                               float* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int n = threadIdx.x;
  const float* p = partial + m * kE + n;
  const int64_t stride = rows * kE;
  float z = 0.0f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(s + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) z += v[u];
  }
  for (; s < splits; ++s) z += p[(int64_t)s * stride];
  out[m * kE + n] = sigmoidf(z);
}

}  // namespace

GatePlan plan_gate(int64_t rows, int64_t d, bool bf16) {
  GatePlan p{};
  p.rows = rows;
  p.d = d;
  p.bf16 = bf16;
  p.rgroups = 1;
  size_t off = 0;
  if (bf16) {
    const int64_t KB = cdiv(d, kKB);
    int64_t splits, min_steps;
    if (rows <= kGateTileRows) {
      // 16-row tiles, K split over about DFS_GATE_SMALL_WG or DFS_GATE_JOBS_WG workgroups
      // (at least DFS_GATE_SMALL_MIN_STEPS k steps each, so that a tile's loads overlap)
      p.kind = GatePlan::kJobs;
      p.rgroups = rows <= DFS_GATE_SMALL_ROWS ? 1 : gtile::kTallGroups;
      p.mtiles = (int)cdiv(rows, (int64_t)gtile::kRows16 * p.rgroups);
      splits = cdiv(rows <= DFS_GATE_SMALL_ROWS ? DFS_GATE_SMALL_WG : DFS_GATE_JOBS_WG, p.mtiles);
      min_steps = DFS_GATE_SMALL_MIN_STEPS;
    } else if (rows >= DFS_GATE_DMA_ROWS && d % GC::KK == 0) {
      // one workgroup per CU; at least 256 k per split on the DMA ring, in whole ring steps
      p.kind = GatePlan::kDma;
      p.mtiles = (int)cdiv(rows, kDmaBM);
      splits = cdiv(kTargetWG, (int64_t)p.mtiles * kDmaHalves);
      min_steps = 8;
      const int64_t KS = d / GC::KK;
      const int64_t max_splits = KS * kDmaSlabs / min_steps > 1 ? KS * kDmaSlabs / min_steps : 1;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
      const int64_t ks_per = cdiv(KS, splits);
      p.kchunk = ks_per * GC::KK;
      p.splits = (int)cdiv(KS, ks_per);
      p.packed_off = 0;
      p.packed_bytes = gate_packed_bytes(d);
      off = p.packed_bytes;
    } else {
      p.kind = GatePlan::kTile64;
      p.mtiles = (int)cdiv(rows, kTileM);
      splits = cdiv(kTargetWG, p.mtiles);
      min_steps = 2;
    }
    if (p.kind != GatePlan::kDma) {
      const int64_t max_splits = KB / min_steps > 1 ? KB / min_steps : 1;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
      const int64_t kb_per = cdiv(KB, splits);
      p.kchunk = kb_per * kKB;
      p.splits = (int)cdiv(KB, kb_per);
      p.packed_off = 0;
      p.packed_bytes = gate_packed_bytes(d);
      off = p.packed_bytes;
    }
  } else {
    p.kind = GatePlan::kJobs;
    p.mtiles = (int)cdiv(rows, gtile::kF32Rows);
    int64_t splits = cdiv(kTargetWG, p.mtiles);
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

size_t gate_packed_bytes(int64_t d) { return align_up((size_t)cdiv(d, kKB) * kE * kKB * sizeof(uint16_t), 256); }

PackJob gate_pack_job(const GatePlan& p, const void* W_h, void* ws) {
  if (!p.bf16) return PackJob{nullptr, 0, nullptr, 0};
  return PackJob{static_cast<const uint16_t*>(W_h), p.d,
                 reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.packed_off),
                 (int)cdiv(p.d, kKB)};
}

const void* gate_packed_in_ws(const GatePlan& p, const void* ws) {
  return static_cast<const char*>(ws) + p.packed_off;
}

const float* gate_partials(const GatePlan& p, const void* ws) {
  return p.splits > 1 ? reinterpret_cast<const float*>(static_cast<const char*>(ws) + p.partial_off)
                      : nullptr;
}

GateJobs gate_jobs(const GatePlan& p, const void* hidden, const void* W, float* out_gate, void* ws) {
  if (p.kind != GatePlan::kJobs) return GateJobs{};
  float* partial = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.partial_off) : nullptr;
  return GateJobs{hidden, W, p.rows, p.d, p.kchunk, p.mtiles, p.splits, p.rgroups, partial, out_gate};
}

hipError_t launch_gate_gemm(const GatePlan& p, const void* hidden, const void* W, float* out_gate, void* ws,
                            hipStream_t stream) {
  char* wsb = static_cast<char*>(ws);
  float* partial = p.splits > 1 ? reinterpret_cast<float*>(wsb + p.partial_off) : nullptr;
  if (p.kind == GatePlan::kJobs) {
    GateJobs g = gate_jobs(p, hidden, W, out_gate, ws);
    if (p.bf16 && g.rgroups != 1) {
      // A launch of its own keeps 16-row tiles over the same K split (so the same bits):
      // the tall tiles pay off beside the top-16 pass, not alone (512 x 5120: 11.6 us
      // with 256 short tiles, 13.8 with 128 tall ones).
      g.rgroups = 1;
      g.mtiles = (int)cdiv(p.rows, (int64_t)gtile::kRows16);
    }
    const dim3 grid((unsigned)((int64_t)g.mtiles * g.splits));
    if (p.bf16) {
      gate_jobs_kernel<true><<<grid, kThreads, 0, stream>>>(g);
    } else {
      gate_jobs_kernel<false><<<grid, kThreads, 0, stream>>>(g);
    }
  } else {
    const uint16_t* Wp = static_cast<const uint16_t*>(W);
    const uint16_t* H = static_cast<const uint16_t*>(hidden);
    if (p.kind == GatePlan::kDma) {
      const int per_xcd = (int)cdiv((int64_t)p.splits * p.mtiles * kDmaHalves, 8);
      gate_dma_kernel<<<dim3((unsigned)(8 * per_xcd)), kThreads, 0, stream>>>(
          H, Wp, p.rows, p.d, p.mtiles, p.splits, (int)(p.kchunk / GC::KK), per_xcd, partial, out_gate);
    } else {
      const dim3 grid((unsigned)((int64_t)p.mtiles * p.splits));
      gate_mfma_kernel<<<grid, kGemmThreads, 0, stream>>>(H, Wp, p.rows, p.d, p.kchunk, p.splits, partial,
                                                           out_gate);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gate_finish(const GatePlan& p, float* out_gate, void* ws, hipStream_t stream) {
  if (p.splits > 1) {
    gate_finish_kernel<<<dim3((unsigned)p.rows), kThreads, 0, stream>>>(gate_partials(p, ws), p.rows,
                                                                        p.splits, out_gate);
  }
  return hipGetLastError();
}

hipError_t launch_gate_pack(const void* W_h, int64_t d, void* Wp, hipStream_t stream) {
  pack_w_kernel<<<dim3((unsigned)cdiv(d, kKB)), kPackThreads, 0, stream>>>(static_cast<const uint16_t*>(W_h), d,
                                                                        static_cast<uint16_t*>(Wp));
  return hipGetLastError();
}

hipError_t launch_gate(const GatePlan& p, const void* hidden, const void* W_h, bool prepacked, float* out_gate,
                       void* ws, hipStream_t stream) {
  const void* W = W_h;
  if (p.bf16 && !prepacked) {
    const PackJob job = gate_pack_job(p, W_h, ws);
    pack_w_kernel<<<dim3((unsigned)job.nslabs), kPackThreads, 0, stream>>>(job.W, job.d, job.Wp);
    W = job.Wp;
  }
  hipError_t e = launch_gate_gemm(p, hidden, W, out_gate, ws, stream);
  if (e != hipSuccess) return e;
  return launch_gate_finish(p, out_gate, ws, stream);
}

}  // namespace dfs
