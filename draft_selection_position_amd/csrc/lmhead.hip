// Top-16 candidates straight from the drafter's hidden state, through its LM head.
//
// The selector reads the drafter's vocabulary logits U_t and makes no extra LM-head
// pass (blog post "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path
// Selector"); the logits are the drafter's LM head applied to its hidden state.
// Here the head's product U = h W_lm^T (h [rows, d], W_lm [V, d], bf16, fp32 sums on
// the matrix cores) and the top-16 selection (section "The Right Tokens Are Already
// There") run in one kernel: each workgroup walks a stripe of column tiles of U and
// folds every tile into running per-row top-16 lists, so U never reaches HBM.  Keys
// and order are those of the top-16 pass (value descending, then the lower token
// id), on the fp32 sums.  A merge pass then combines the stripes' lists per row.
// The same product can be written out (lmhead_logits*_kernel): the fused result
// equals the top-16 pass run on those logits, bit for bit.
//
// Tiles (LDS-DMA mainloop of mfma_big.h): the fused kernel uses 128 x 128 (four waves of
// 64 x 64, two workgroups per CU, a double buffer of 64 k per step: whole 128-byte lines)
// at every size, so that one workgroup's fold overlaps the other's products; the
// written-out product switches to 256 x 256 (four waves of 128 x 128, one per CU, a
// four-stage ring of 32 k per step: a double buffer of 64 k leaves too little in flight)
// from 2048 rows.
// For at most 32 rows the product (16-row register-staged tiles, mfma_tile.h, runs of
// column tiles per workgroup: the pass streams W_lm and the matrix cores idle) is
// written to the workspace and the top-16 pass runs over it, which is faster there.
// Workgroups are numbered so that each XCD runs a group of row tiles x stripes at a
// time: the group's W_lm tiles and h rows are shared through the XCD's L2.

#include <type_traits>

#include "dfs_device.h"
#include "dfs_internal.h"
#include "mfma_big.h"
#include "mfma_tile.h"

namespace dfs {
namespace {

constexpr int kThreads = tile::kThreads;
#ifndef DFS_LM_BIG_ROWS
#define DFS_LM_BIG_ROWS 2048
#endif
#ifndef DFS_LM_BIG_TILE
#define DFS_LM_BIG_TILE 1
#endif
#ifndef DFS_LM_ROUNDS
#define DFS_LM_ROUNDS 1
#endif
#ifndef DFS_LM_GM
#define DFS_LM_GM 16  // row tiles per XCD group (the rest of the group: stripes); 16 measured 1.4% faster than 8 at 4096 rows, 4 and 32 slower
#endif
#ifndef DFS_LM_DEPTH
#define DFS_LM_DEPTH 2
#endif
// ring stages and k per step of the 256 x 256 and 128 x 128 tiles
#ifndef DFS_LM_BIG_STAGES
#define DFS_LM_BIG_STAGES 4
#endif
#ifndef DFS_LM_BIG_KK
#define DFS_LM_BIG_KK 32
#endif
#ifndef DFS_LM_MID_STAGES
#define DFS_LM_MID_STAGES 2
#endif
#ifndef DFS_LM_MID_KK
#define DFS_LM_MID_KK 64
#endif
using BigCfg = big::Cfg<8, 8, DFS_LM_BIG_STAGES, DFS_LM_BIG_KK>;
using MidCfg = big::Cfg<4, 4, DFS_LM_MID_STAGES, DFS_LM_MID_KK>;
constexpr int kMidWG = MidCfg::kLdsBytes <= 72 * 1024 ? 2 : 1;  // workgroups per CU the LDS allows

struct Grid {
  int64_t rows, V, d;
  int mtiles;
  int64_t ntiles;
  int nstripes, tps;   // stripes of tps column tiles
  int group;           // workgroups an XCD runs at a time
  int gm, gs;          // row tiles x stripes per group (gm * gs = group)
  int mgroups, groups; // groups along the rows, all groups
  int cand_cap;        // pending candidates a row can hold: one tile's columns + kMergeAt - 1
};

// Workgroup -> (row tile, stripe); false for the padding of the last round.
__device__ __forceinline__ bool place(const Grid& g, int& mt, int& stripe) {
  const unsigned xcd = blockIdx.x % 8u, j = blockIdx.x / 8u;
  const int gi = (int)(j / (unsigned)g.group) * 8 + (int)xcd;
  const int local = (int)(j % (unsigned)g.group);
  if (gi >= g.groups) return false;
  mt = (gi % g.mgroups) * g.gm + local % g.gm;
  stripe = (gi / g.mgroups) * g.gs + local / g.gm;
  return mt < g.mtiles && stripe < g.nstripes;
}

// Candidates pending per row before its list is merged (one 64-lane sort takes the
// list and 48 candidates).
constexpr int kMergeAt = 32;

// Fold one product tile into the running row lists, in two passes.
// Offers: the wave holding rows 16 TM wm + ... and columns 16 TN wn + ... of the
// tile offers every value whose key beats its row's 16th at the last merge (s_thr):
// the key is appended to the row's pending candidates in the workspace (`cand_row`,
// an LDS counter per row).  Every accumulator is read once, in one pass.
// Merges: a row with kMergeAt or more pending candidates (any, at the stripe's last
// tile) merges them into its list (kept in `partial`) by 64-lane sorts, always on
// wave row % 4 and lanes 0-15, so that each list slot is read back by the lane that
// wrote it.  A stale threshold only lets more candidates through; every value that
// can be in the top-16 is offered.
//
// 128 x 128 tiles (whose registers allow it) test a row's values against its threshold
// as floats first, a wave at a time (keys above the threshold have values at or above
// its value), and on a stripe's first tile raise each row's threshold to the smallest of
// its 16 lanes' largest values (16 distinct elements of the row are at or above it), so
// that the first tile offers tens of candidates per row instead of all of them.
template <int TM, int TN, int WNW, class CandRow>
__device__ __forceinline__ void fold_tile(const tile::f32x4 (&v)[TM][TN], int tile_rows, int64_t n0,
                                          int64_t ncols, bool first, bool last, uint64_t* s_thr, int* s_cnt,
                                          int* s_has, CandRow cand_row, uint64_t* plist, int64_t m0,
                                          int64_t row_stride) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave / WNW, wn = wave % WNW;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 16 * TM * wm + 16 * a + 4 * q + i;
      if constexpr (TM * TN <= 16) {
        // row lr is held by the 16 lanes of one DPP row (r = 0..15), TN values each
        const bool row_ok = lr < tile_rows;
        uint64_t thr = row_ok ? s_thr[lr] : ~0ull;
        float m = -INFINITY;  // this lane's largest value of the row (NaN never counts)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          if (16 * TN * wn + 16 * b + r < ncols) m = fmaxf(m, v[a][b][i]);
        if (first) {
          float bm = m;
#pragma unroll
          for (int j = 1; j < 16; j <<= 1) bm = fminf(bm, __uint_as_float(xor_lanes(__float_as_uint(bm), j, lane)));
          const uint64_t bkey = (uint64_t)mono32(bm) << 32;  // below every key of value bm
          thr = bkey > thr ? bkey : thr;
        }
        const float thrf = thr == 0 ? -INFINITY : unmono32((uint32_t)(thr >> 32));
        if (__ballot(row_ok && m >= thrf) == 0) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int lc = 16 * TN * wn + 16 * b + r;
          const float x = v[a][b][i];
          if (row_ok && lc < ncols && x >= thrf) {
            const uint64_t key = make_key(x, (uint32_t)(n0 + lc));
            if (key > thr) cand_row(lr)[atomicAdd(&s_cnt[lr], 1)] = key;
          }
        }
      } else {
        if (lr >= tile_rows) continue;
        const uint64_t thr = s_thr[lr];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int lc = 16 * TN * wn + 16 * b + r;
          if (lc >= ncols) continue;
          const uint64_t key = make_key(v[a][b][i], (uint32_t)(n0 + lc));
          if (key > thr) cand_row(lr)[atomicAdd(&s_cnt[lr], 1)] = key;
        }
      }
    }
    // a row block at a time: keeps the scheduler from hoisting every key of the
    // tile into registers at once
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  for (int lr = wave; lr < tile_rows; lr += 4) {
    const int cnt = s_cnt[lr];
    if (cnt == 0 || (cnt < kMergeAt && !last)) continue;
    uint64_t* gl = plist + (m0 + lr) * row_stride;
    const uint64_t* cr = cand_row(lr);
    uint64_t cur = 0;
    int c0 = 0;
    if (s_has[lr]) {
      if (lane < kK) cur = gl[lane];
    } else {  // the row's first merge: its first 64 candidates alone (no list yet)
      uint64_t x = lane < cnt ? cr[lane] : 0;
      x = wave_sort_desc(x, lane);
      cur = lane < kK ? x : 0;
      c0 = kWave;
    }
    for (; c0 < cnt; c0 += kWave - kK) {
      const int ci = c0 + lane - kK;
      uint64_t x = lane < kK ? cur : (ci < cnt ? cr[ci] : 0);
      x = wave_sort_desc(x, lane);
      cur = lane < kK ? x : 0;
    }
    if (lane < kK) gl[lane] = cur;
    const uint64_t thr = lane_u64(cur, kK - 1);
    if (lane == 0) {
      s_thr[lr] = thr;
      s_cnt[lr] = 0;
      s_has[lr] = 1;
    }
  }
  __syncthreads();
}

// Workgroup (row tile, stripe): the product tile by tile on the LDS-DMA mainloop of
// mfma_big.h (TM = TN = 4: 128 x 128, two workgroups per CU; 8: 256 x 256, one),
// each tile folded into the stripe's row lists.  cand: the pending candidates,
// [rows, nstripes, g.cand_cap] keys.
template <class C, int kMinWG>
__global__ __launch_bounds__(kThreads, kMinWG) void lmhead_topk_dma_kernel(const uint16_t* __restrict__ h,
                                                                           const uint16_t* __restrict__ W,
                                                                           Grid g,
                                                                           uint64_t* __restrict__ partial,
                                                                           uint64_t* __restrict__ cand) {
  constexpr int TM = C::TM, TN = C::TN;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) char lds[C::kLdsBytes];
  __shared__ uint64_t s_thr[BM];
  __shared__ int s_cnt[BM];
  __shared__ int s_has[BM];
  int mt, stripe;
  if (!place(g, mt, stripe)) return;
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)mt * BM;
  const int tile_rows = (int)(g.rows - m0 < BM ? g.rows - m0 : BM);
  for (int i = tid; i < BM; i += kThreads) {
    s_thr[i] = 0;
    s_cnt[i] = 0;
    s_has[i] = 0;
  }
  const int64_t row_stride = (int64_t)g.nstripes * kK;
  uint64_t* plist = partial + (int64_t)stripe * kK;
  const big::Operand ra = big::rows_operand(h + m0 * g.d, tile_rows, g.d, C::KK);
  const int KS = (int)(g.d / C::KK);
  const int64_t t0 = (int64_t)stripe * g.tps;
  const int64_t t1 = t0 + g.tps < g.ntiles ? t0 + g.tps : g.ntiles;
  auto cand_row = [&](int lr) { return cand + ((m0 + lr) * g.nstripes + stripe) * g.cand_cap; };
  for (int64_t nt_ = t0; nt_ < t1; ++nt_) {
    const int64_t n0 = nt_ * BN;
    const int64_t ncols = g.V - n0 < BN ? g.V - n0 : BN;
    typename C::Acc acc;
    C::zero(acc);
    big::mma<C>(ra, big::rows_operand(W + n0 * g.d, ncols, g.d, C::KK), 0, KS, lds, acc);
    fold_tile<TM, TN, 2>(acc.v, tile_rows, n0, ncols, nt_ == t0, nt_ + 1 == t1, s_thr, s_cnt, s_has, cand_row, plist,
                         m0, row_stride);
  }
}

// U [rows, V] fp32 written out: the same product, for checks and the unfused chain.
template <int WMW, int WNW, int TM, int TN>
__global__ __launch_bounds__(kThreads, (TM * TN > 16 ? 1 : 2)) void lmhead_logits_kernel(const uint16_t* __restrict__ h,
                                                                    const uint16_t* __restrict__ W,
                                                                    int64_t rows, int64_t V, int64_t d,
                                                                    int64_t ntiles, int64_t nwg_n,
                                                                    float* __restrict__ U) {
  using S = tile::Shape<WMW, WNW, TM, TN>;
  constexpr int BM = S::BM, BN = S::BN;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::kLdsBytes / 2];
  // workgroup (row tile, run of column tiles): the runs cut the column tiles evenly
  const int64_t wg_n = (int64_t)blockIdx.x % nwg_n;
  const int64_t m0 = (int64_t)blockIdx.x / nwg_n * BM;
  const int64_t t0 = wg_n * ntiles / nwg_n, t1 = (wg_n + 1) * ntiles / nwg_n;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave / WNW, wn = wave % WNW;
  const int tile_rows = (int)(rows - m0 < BM ? rows - m0 : BM);
  for (int64_t nt_ = t0; nt_ < t1; ++nt_) {
    const int64_t n0 = nt_ * BN;
    const int64_t ncols = V - n0 < BN ? V - n0 : BN;
    typename S::Acc acc;
    tile::zero<WMW, WNW, TM, TN>(acc);
    tile::mma<WMW, WNW, TM, TN, DFS_LM_DEPTH>(tile::rows_rsrc(h + m0 * d, tile_rows, d),
                                              tile::rows_rsrc(W + n0 * d, ncols, d), d, 0,
                                              (int)(d / tile::kKStep), lds, acc);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = 16 * TM * wm + 16 * a + 4 * q + i;
        if (lr >= tile_rows) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int lc = 16 * TN * wn + 16 * b + r;
          if (lc < ncols) U[(m0 + lr) * V + n0 + lc] = acc.v[a][b][i];
        }
      }
    __syncthreads();  // the next tile's loop reuses the LDS stages
  }
}

template <class C, int kMinWG>
__global__ __launch_bounds__(kThreads, kMinWG) void lmhead_logits_dma_kernel(const uint16_t* __restrict__ h,
                                                                             const uint16_t* __restrict__ W,
                                                                             int64_t rows, int64_t V, int64_t d,
                                                                             int64_t ntiles, float* __restrict__ U) {
  constexpr int TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(1024))) char lds[C::kLdsBytes];
  const int64_t nt_ = (int64_t)blockIdx.x % ntiles;
  const int64_t m0 = (int64_t)blockIdx.x / ntiles * C::BM;
  const int64_t n0 = nt_ * C::BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile_rows = (int)(rows - m0 < C::BM ? rows - m0 : C::BM);
  const int64_t ncols = V - n0 < C::BN ? V - n0 : C::BN;
  typename C::Acc acc;
  C::zero(acc);
  big::mma<C>(big::rows_operand(h + m0 * d, tile_rows, d, C::KK), big::rows_operand(W + n0 * d, ncols, d, C::KK),
              0, (int)(d / C::KK), lds, acc);
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 16 * TM * wm + 16 * a + 4 * q + i;
      if (lr >= tile_rows) continue;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int lc = 16 * TN * wn + 16 * b + r;
        if (lc < ncols) U[(m0 + lr) * V + n0 + lc] = acc.v[a][b][i];
      }
    }
}

// Tile shapes of the written-out product: few rows -> 16 x 256 (W_lm streamed once);
// below DFS_LM_BIG_ROWS -> 128 x 128; from there 256 x 256 (one workgroup per CU;
// measured faster from 4096 rows, slower at 1024).  The fused kernel keeps 128 x 128
// tiles at every size (below DFS_LM_FUSED_BIG_ROWS): with two workgroups per CU one
// folds its tile while the other keeps the matrix cores busy, where a lone 256 x 256
// workgroup stalls them for its whole fold (4096 x 151936 x 5120: 7.55-7.67 ms against
// 7.99 ms).
constexpr int64_t kSmallRows = 32;
enum TileKind { kSmallTile = 0, kMidTile = 1, kBigTile = 2 };
TileKind tile_kind(int64_t rows) {
  return rows <= kSmallRows ? kSmallTile : rows < DFS_LM_BIG_ROWS ? kMidTile : kBigTile;
}
#ifndef DFS_LM_FUSED_BIG_ROWS
#define DFS_LM_FUSED_BIG_ROWS INT64_MAX
#endif
TileKind fused_tile_kind(int64_t rows) {
  return rows <= kSmallRows ? kSmallTile : rows < (int64_t)DFS_LM_FUSED_BIG_ROWS ? kMidTile : kBigTile;
}

// The fused kernel's grid.
Grid make_grid(int64_t rows, int64_t V, int64_t d) {
  Grid g{};
  g.rows = rows;
  g.V = V;
  g.d = d;
  const TileKind kind = fused_tile_kind(rows);
  const bool big = kind == kBigTile && DFS_LM_BIG_TILE;
  const int BM = kind == kSmallTile ? 16 : big ? 256 : 128;
  const int BN = kind == kSmallTile || big ? 256 : 128;
  g.group = big ? 32 : 64;  // one or two workgroups per CU, 32 CUs per XCD
  g.mtiles = (int)cdiv(rows, BM);
  g.ntiles = cdiv(V, BN);
  // about four rounds of the chip's workgroup slots, at least two column tiles per
  // stripe where there are enough
  // one round of the chip's workgroup slots: long stripes, so that few tiles are a
  // stripe's first (whose fold sees every value as a candidate)
  int64_t ns = cdiv(DFS_LM_ROUNDS * 8 * g.group, g.mtiles);
  if (ns > g.ntiles / 2) ns = g.ntiles / 2;
  if (ns > 2048) ns = 2048;
  if (ns < 1) ns = 1;
  g.tps = (int)cdiv(g.ntiles, ns);
  g.nstripes = (int)cdiv(g.ntiles, g.tps);
  g.gm = g.mtiles < DFS_LM_GM ? g.mtiles : DFS_LM_GM;
  while (g.group % g.gm) --g.gm;
  g.gs = g.group / g.gm;
  g.mgroups = (int)cdiv(g.mtiles, g.gm);
  g.groups = g.mgroups * (int)cdiv(g.nstripes, g.gs);
  g.cand_cap = (int)align_up((size_t)(BN + kMergeAt - 1), 32);
  return g;
}

}  // namespace

// Few rows: the logits are small (at most 32 x V fp32) and writing them, then one
// top-16 pass over them, beats folding every tile of a one-tile stripe (the two
// kernels stream W_lm at the same rate); the logits then live in the workspace.
static bool lmhead_two_pass(int64_t rows) { return rows <= kSmallRows; }

static size_t lmhead_lists_bytes(const Grid& g) {
  return align_up((size_t)g.rows * g.nstripes * kK * sizeof(uint64_t), 256);
}

static size_t lmhead_logits_bytes(int64_t rows, int64_t V) {
  return align_up((size_t)rows * (size_t)V * sizeof(float), 256);
}

size_t lmhead_workspace_bytes(int64_t rows, int64_t V, int64_t d) {
  if (lmhead_two_pass(rows)) return lmhead_logits_bytes(rows, V) + plan_topk(rows, V, 4).ws_bytes;
  const Grid g = make_grid(rows, V, d);
  return lmhead_lists_bytes(g) + align_up((size_t)rows * g.nstripes * g.cand_cap * sizeof(uint64_t), 256);
}

hipError_t launch_lmhead_topk(const void* hidden, const void* W_lm, int64_t rows, int64_t V, int64_t d,
                              int32_t* out_idx, float* out_val, void* ws, hipStream_t stream) {
  if (lmhead_two_pass(rows)) {
    float* U = static_cast<float*>(ws);
    hipError_t e = launch_lmhead_logits(hidden, W_lm, rows, V, d, U, stream);
    if (e != hipSuccess) return e;
    const TopkPlan tp = plan_topk(rows, V, 4);
    return launch_topk(tp, U, false, out_idx, out_val, static_cast<char*>(ws) + lmhead_logits_bytes(rows, V),
                       stream);
  }
  const Grid g = make_grid(rows, V, d);
  uint64_t* partial = static_cast<uint64_t*>(ws);
  uint64_t* cand = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + lmhead_lists_bytes(g));
  const dim3 grid((unsigned)(8 * g.group * cdiv(g.groups, 8)));
  const uint16_t* hp = static_cast<const uint16_t*>(hidden);
  const uint16_t* wp = static_cast<const uint16_t*>(W_lm);
  switch (fused_tile_kind(rows)) {  // (few rows took the two-pass way above)
    case kMidTile:
      lmhead_topk_dma_kernel<MidCfg, kMidWG><<<grid, kThreads, 0, stream>>>(hp, wp, g, partial, cand);
      break;
    default:
#if DFS_LM_BIG_TILE
      lmhead_topk_dma_kernel<BigCfg, 1><<<grid, kThreads, 0, stream>>>(hp, wp, g, partial, cand);
#else
      lmhead_topk_dma_kernel<MidCfg, kMidWG><<<grid, kThreads, 0, stream>>>(hp, wp, g, partial, cand);
#endif
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(partial, rows, g.nstripes, out_idx, out_val, stream);
}

hipError_t launch_lmhead_logits(const void* hidden, const void* W_lm, int64_t rows, int64_t V, int64_t d,
                                float* out, hipStream_t stream) {
  const uint16_t* hp = static_cast<const uint16_t*>(hidden);
  const uint16_t* wp = static_cast<const uint16_t*>(W_lm);
  switch (tile_kind(rows)) {
    case kSmallTile: {
      // 16-row tiles, 128 columns (one row tile) or 64 (two), spread evenly over 512
      // workgroups (two per CU), each walking a run of column tiles: measured against one
      // workgroup per 256-column tile, 272 vs 287 us at 16 x 151936 x 5120 and 380 vs
      // 533 us at 32 rows
      constexpr int64_t kSmallWGs = 512;
      if (rows <= 16) {
        const int64_t nt = cdiv(V, 128);
        const int64_t nwg = nt < kSmallWGs ? nt : kSmallWGs;
        lmhead_logits_kernel<1, 4, 1, 2><<<dim3((unsigned)nwg), kThreads, 0, stream>>>(hp, wp, rows, V, d, nt, nwg,
                                                                                        out);
      } else {
        const int64_t nt = cdiv(V, 64);
        const int64_t nwg = nt < kSmallWGs ? nt : kSmallWGs;
        lmhead_logits_kernel<1, 4, 1, 1><<<dim3((unsigned)(cdiv(rows, 16) * nwg)), kThreads, 0, stream>>>(
            hp, wp, rows, V, d, nt, nwg, out);
      }
      break;
    }
    case kMidTile: {
      const int64_t nt = cdiv(V, 128);
      lmhead_logits_dma_kernel<MidCfg, kMidWG><<<dim3((unsigned)(cdiv(rows, 128) * nt)), kThreads, 0, stream>>>(
          hp, wp, rows, V, d, nt, out);
      break;
    }
    default: {
#if DFS_LM_BIG_TILE
      const int64_t nt = cdiv(V, 256);
      lmhead_logits_dma_kernel<BigCfg, 1><<<dim3((unsigned)(cdiv(rows, 256) * nt)), kThreads, 0, stream>>>(
          hp, wp, rows, V, d, nt, out);
#else
      const int64_t nt = cdiv(V, 128);
      lmhead_logits_dma_kernel<MidCfg, kMidWG><<<dim3((unsigned)(cdiv(rows, 128) * nt)), kThreads, 0, stream>>>(
          hp, wp, rows, V, d, nt, out);
#endif
    }
  }
  return hipGetLastError();
}

}  // namespace dfs
