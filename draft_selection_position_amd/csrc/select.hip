// Pair scores for every adjacent candidate pair, and the walk over them.
//
// Score (blog post "DFlash 2: Keep Drafting Parallel", section "A Lightweight Path
// Selector"; the equation is spelled out in the twiscan.com Chinese translation):
//     S_t(a, b) = U_t(b) + < A(a) (elementwise) H(h_t), B(b) >
// for predecessor a in the 16 candidates of position t-1 (the last verified token
// at t = 0) and candidate b in the 16 candidates of position t.  All pairs are
// scored at once; the walk is the only sequential step: from the last verified
// token, greedy takes the best successor, sampling draws from the same scores.
//
// Design (gfx950): one workgroup per sequence, one wave per block position.  A
// position's 16x16 score tile is exactly one 16x16 output of the matrix cores with
// K = 256.  The sum over the embedding index e is order-free, so the k slots of
// the MFMAs may be mapped to e freely, as long as both operands agree: MFMA step c
// gives lane group q = lane / 16 the eight values e = 64 (c / 2) + 16 q + 8 (c % 2)
// + 0..7.  Each lane then loads its predecessor-row and candidate-row fragments as
// 16-byte vectors straight from the tables (no LDS staging), and the four lane
// groups of a row cover one whole 128-byte line in two load instructions.  For
// bf16 tables the gated predecessor
// embedding A(a) * g (fp32) is split as hi + lo in bf16 and fed to two MFMAs, so
// the products are exact to ~2^-17 before fp32 accumulation.  Each wave reduces
// its tile to the successor of every predecessor slot; one lane then follows the
// chain through LDS.  With few rows (one or a few sequences) a workgroup per sequence
// would put all the gathers behind a handful of CUs, so pair_pos_kernel gives each
// position a workgroup of its own and lets the last of a sequence's workgroups (an
// atomic ticket after a device-wide release) run the walk.
#include "dfs_device.h"
#include "dfs_internal.h"
#include "philox.h"
#include "topk_merge.h"

namespace dfs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxL = 16;
// The pair kernels issue a position's 16 + 16 table-row gathers before they wait for its
// gate row (1) or after (0): the per-sequence kernel (1: 4096 rows 220.3 -> 219.9 us per
// dfs_select; it then sums the gate in rounds of four splits, to stay within its registers)
// and the per-position tile kernel (1: 512 rows 43.9 -> 43.3 us, 1024 x 262144 107.5 -> 106.6).
#ifndef DFS_PW_GATHER_FIRST
#define DFS_PW_GATHER_FIRST 1
#endif
#ifndef DFS_TILE_GATHER_FIRST
#define DFS_TILE_GATHER_FIRST 1
#endif
// The same for the few-row kernel's wave 0 (1: 16 x 151936 16.9 -> 16.6 us per dfs_select).
#ifndef DFS_POS_GATHER_FIRST
#define DFS_POS_GATHER_FIRST 1
#endif
// fp32 tables, few-row kernel: a tile's 32 row loads of a lane in one round (1) or two (0):
// 8 x 32000 fp32 15.5 -> 15.35 us per dfs_select.
#ifndef DFS_F32_TILE_ONE_ROUND
#define DFS_F32_TILE_ONE_ROUND 1
#endif

// Standard Gumbel noise for (sequence b, position t, slot j), fp64:
// u = ((x >> 9) + 1/2) 2^-23 in (0, 1), g = -log(-log u).
__device__ __forceinline__ double gumbel_noise(uint64_t seed, uint32_t b, uint32_t t, uint32_t j) {
  uint32_t w[4];
  philox4x32_10(j, t, b, 0u, (uint32_t)seed, (uint32_t)(seed >> 32), w);
  const uint32_t x = w[0];
  const double u = uniform23(x);
  return -log(-log(u));
}

// The walk, split in two.  First, for every position t and predecessor slot a,
// the successor slot the walk would take from a: an argmax over the 16 candidate
// slots of the score tile, lowest slot on ties (greedy), or of
// S_t(a, j) / temperature + g(seed, b, t, j) in fp64 (Gumbel-max), computed for
// all a and t at once.  The tile of position t is held by one wave as lane
// (q, r) = (lane / 16, lane % 16) with s[i] = S_t(4q + i, r), so the argmax over
// j = r is a reduction inside one 16-lane row (DPP, no LDS).  Second, the chain
// itself: from slot 0 at t = 0 (every row of position 0 is the verified token's
// row) follow the successor table, one dependent LDS read per step.
struct WalkTables {
  int32_t next[kMaxL][kK];  // successor slot of (t, a); best-path walk: best predecessor of (t, j)
  float best[kMaxL][kK];    // S_t(a, next) (the score without noise)
  int32_t cand[kMaxL][kK];  // token id of (t, slot)
  int32_t slot[kMaxL];      // the walk's slot at each position
};

__device__ __forceinline__ void successors(const float (&s)[4], int t, int lane, int mode,
                                           double temperature, uint64_t seed, int64_t b,
                                           WalkTables& w) {
  const int r = lane & 15;
  const int q = lane >> 4;
  if (mode == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = s[i];
      int j = r;
#pragma unroll
      for (int m = 1; m < kK; m <<= 1) {
        const float ov = __uint_as_float(xor_lanes(__float_as_uint(v), m, lane));
        const int oj = (int)xor_lanes((uint32_t)j, m, lane);
        const bool take = ov > v || (ov == v && oj < j);
        v = take ? ov : v;
        j = take ? oj : j;
      }
      if (r == i) {
        w.next[t][4 * q + i] = j;
        w.best[t][4 * q + i] = v;
      }
    }
  } else {
    const double g = gumbel_noise(seed, (uint32_t)b, (uint32_t)t, (uint32_t)r);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double v = (double)s[i] / temperature + g;
      float raw = s[i];
      int j = r;
#pragma unroll
      for (int m = 1; m < kK; m <<= 1) {
        const uint64_t bits = (uint64_t)__double_as_longlong(v);
        const uint32_t lo = xor_lanes((uint32_t)bits, m, lane);
        const uint32_t hi = xor_lanes((uint32_t)(bits >> 32), m, lane);
        const double ov = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
        const float oraw = __uint_as_float(xor_lanes(__float_as_uint(raw), m, lane));
        const int oj = (int)xor_lanes((uint32_t)j, m, lane);
        const bool take = ov > v || (ov == v && oj < j);
        v = take ? ov : v;
        raw = take ? oraw : raw;
        j = take ? oj : j;
      }
      if (r == i) {
        w.next[t][4 * q + i] = j;
        w.best[t][4 * q + i] = raw;
      }
    }
  }
}

// The path of largest summed score (walk mode 2), by dynamic programming over
// the whole [L, 16, 16] score tensor `sS` (in LDS), run by one wave: lane j keeps
// best[j], the largest total of a path ending in slot j; a step takes
// best[i] + S_t(i, j) over i with the lowest i among equal values (best[i] comes
// from lane i through a scalar read) and stores the choice in `back`.  The last
// slot is the lowest j of largest best (a DPP row reduction); one lane then reads
// the path back.
__device__ __forceinline__ void viterbi_walk(const float (*sS)[kK][kK], int32_t (*back)[kK],
                                             const int32_t (*cand)[kK], int32_t* slot_out, int64_t b,
                                             int L, int lane, int32_t* __restrict__ out_path,
                                             float* __restrict__ out_scores) {
  const int j = lane & 15;
  float v = sS[0][0][j];
  for (int t = 1; t < L; ++t) {
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) + sS[t][0][j];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < kK; ++i) {
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i)) + sS[t][i][j];
      if (c > bv) {
        bv = c;
        bi = i;
      }
    }
    if (lane < kK) back[t][j] = bi;
    v = bv;
  }
  int fj = j;
#pragma unroll
  for (int m = 1; m < kK; m <<= 1) {
    const float ov = __uint_as_float(xor_lanes(__float_as_uint(v), m, lane));
    const int oj = (int)xor_lanes((uint32_t)fj, m, lane);
    const bool take = ov > v || (ov == v && oj < fj);
    v = take ? ov : v;
    fj = take ? oj : fj;
  }
  // the back pointers were written by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    int a = fj;
    for (int t = L - 1; t >= 0; --t) {
      const int pa = t > 0 ? back[t][a] : 0;
      slot_out[t] = a;
      out_path[b * L + t] = cand[t][a];
      out_scores[b * L + t] = sS[t][pa][a];
      a = pa;
    }
  }
}

// The chain, run by one whole wave: lanes 0..15 hold the successor column of their
// slot for every position (independent LDS reads), and each step picks the next slot
// with a lane read indexed by the current one, so the L dependent steps cost a few
// cycles each instead of an LDS round trip.  Lane t keeps position t's slot and
// predecessor slot and writes that position's outputs.
__device__ __forceinline__ void chase(WalkTables& w, int64_t b, int L, int lane,
                                      int32_t* __restrict__ out_path,
                                      float* __restrict__ out_scores) {
  const int l = lane & (kK - 1);
  int nx[kMaxL];
#pragma unroll
  for (int t = 0; t < kMaxL; ++t) nx[t] = t < L ? w.next[t][l] : 0;
  int a = 0, slot = 0, pred = 0;
#pragma unroll
  for (int t = 0; t < kMaxL; ++t) {
    if (t < L) {
      const int j = __builtin_amdgcn_readlane(nx[t], a);
      if (lane == t) {
        pred = a;
        slot = j;
      }
      a = j;
    }
  }
  if (lane < L) {
    w.slot[lane] = slot;
    out_path[b * L + lane] = w.cand[lane][slot];
    out_scores[b * L + lane] = w.best[lane][pred];
  }
}

// The draft distribution of position t given the walk's own predecessor: q =
// softmax(S_t(slot[t-1], .) / T) over the 16 candidates (slot[-1] = 0, the verified
// token's row), the distribution the Gumbel-max walk draws from; with the
// candidate ids it is what speculative-sampling verification needs from the
// drafter.  One wave per position; the 16 lanes of each DPP row hold the 16
// candidates (all four rows the same), the row maximum and the sum are row
// reductions, and every lane divides by lane 0's sum so the row is normalised
// once.
__device__ __forceinline__ void draft_q(const float (*sS)[kK][kK], const WalkTables& w, int t,
                                        int lane, double temperature, int64_t row,
                                        float* __restrict__ out_q, int32_t* __restrict__ out_cand) {
  const int prev = t > 0 ? w.slot[t - 1] : 0;
  const int j = lane & 15;
  const float x = (float)((double)sS[t][prev][j] / temperature);
  float m = x;
#pragma unroll
  for (int k = 1; k < kK; k <<= 1) m = fmaxf(m, __uint_as_float(xor_lanes(__float_as_uint(m), k, lane)));
  const float e = expf(x - m);
  float sum = e;
#pragma unroll
  for (int k = 1; k < kK; k <<= 1) sum += __uint_as_float(xor_lanes(__float_as_uint(sum), k, lane));
  sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), 0));
  if (lane < kK) {
    out_q[row * kK + j] = e / sum;
    out_cand[row * kK + j] = w.cand[t][j];
  }
}

// The gate row of a position, one 16-byte piece [4 lane, + 4) per lane: the finished
// gate (splits == 1), or the K-split partial sums [splits, rows, 256] (row stride
// `stride` between splits) added in split order from zero, exactly as the gate's finish
// kernel adds them, then passed through the sigmoid.  gate_issue puts the first round
// of loads (up to 16 splits) in flight without waiting for any; gate_finish adds them
// up, loading any further rounds.  The guards are wave-uniform branches, not predicated
// loads.
constexpr int kGateRound = 16;
template <int N = kGateRound>
struct GateRegs {
  float4 v[N];
};

template <int N>
__device__ __forceinline__ void gate_load_round(const float* p, int s0, int splits, int64_t stride, GateRegs<N>& g) {
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (s0 + u < splits) g.v[u] = *reinterpret_cast<const float4*>(p + (int64_t)(s0 + u) * stride);
}

template <int N>
__device__ __forceinline__ void gate_issue(const float* __restrict__ gate, int splits, int64_t stride,
                                           int64_t row, int lane, GateRegs<N>& g) {
  gate_load_round(gate + row * kE + 4 * lane, 0, splits, stride, g);
}

// Rounds of N splits; the sums run in split order whatever N is, so every N gives the same bits.
template <int N>
__device__ __forceinline__ float4 gate_finish(const float* __restrict__ gate, int splits, int64_t stride,
                                              int64_t row, int lane, GateRegs<N>& g) {
  if (splits == 1) return g.v[0];
  float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float* p = gate + row * kE + 4 * lane;
  for (int s0 = 0; s0 < splits; s0 += N) {
    if (s0 > 0) gate_load_round(p, s0, splits, stride, g);
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (s0 + u < splits) {
        z.x += g.v[u].x;
        z.y += g.v[u].y;
        z.z += g.v[u].z;
        z.w += g.v[u].w;
      }
    }
  }
  return make_float4(sigmoidf(z.x), sigmoidf(z.y), sigmoidf(z.z), sigmoidf(z.w));
}

// The 16 x 16 score tile of one position on the matrix cores, K = 256: lane (q, r) =
// (lane / 16, lane % 16) feeds predecessor row `pred` (A operand row r) and candidate row
// `cand` (B operand column r), and gets S(4q + i, r) = u_r + <A(pred_{4q+i}) * g, B(cand_r)>
// in sc[i], u = this lane's candidate logit (lanes r of every group hold the same u_r).
// gp: this lane's 16-byte piece [4 lane, + 4) of the gate row; sGr: 256 floats of LDS for
// that row, read back by other lanes of the wave only.  The gathers are all in flight
// before the gate row is parked in LDS (scheduling barriers keep that order).  Every
// kernel that scores pairs calls this, so their scores agree bit for bit.
// The bf16 tables' fragments of one tile, loaded by tile_rows_issue and consumed by
// score_tile_rows: a caller may issue them before it waits for the gate row.
struct TileRows {
  bf16x8 av[8], bv[8];
};
__device__ __forceinline__ void tile_rows_issue(const void* __restrict__ A_, const void* __restrict__ B_, int64_t pred,
                                                int64_t cand, int lane, TileRows& tr) {
  const int q = lane >> 4;
  // fragment c of this lane: elements [64 (c / 2) + 16 q + 8 (c % 2), + 8)
  const bf16x8* Ap = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(A_) + pred * kE + 16 * q);
  const bf16x8* Bp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(B_) + cand * kE + 16 * q);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    tr.av[c] = Ap[8 * (c >> 1) + (c & 1)];
    tr.bv[c] = Bp[8 * (c >> 1) + (c & 1)];
  }
}
__device__ __forceinline__ void score_tile_rows(const TileRows& tr, float u, float4 gp, float* sGr, int lane,
                                                float (&sc)[4]) {
  const int q = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  *reinterpret_cast<float4*>(&sGr[4 * lane]) = gp;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float g[8];
    const float4 g0 = *reinterpret_cast<const float4*>(&sGr[64 * (c >> 1) + 16 * q + 8 * (c & 1)]);
    const float4 g1 = *reinterpret_cast<const float4*>(&sGr[64 * (c >> 1) + 16 * q + 8 * (c & 1) + 4]);
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
    g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
    bf16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ag = (float)tr.av[c][e] * g[e];
      hi[e] = (__bf16)ag;
      lo[e] = (__bf16)(ag - (float)hi[e]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, tr.bv[c], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, tr.bv[c], acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = acc[i] + u;
}

// kOneRound (fp32 tables): every row piece of the lane in flight before the first product
// (32 float4 registers: for kernels with the registers to spare).
template <bool kBf16Tables, bool kOneRound = false>
__device__ __forceinline__ void score_tile(const void* __restrict__ A_, const void* __restrict__ B_, int64_t pred,
                                           int64_t cand, float u, float4 gp, float* sGr, int lane, float (&sc)[4]) {
  const int q = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kBf16Tables) {
    TileRows tr;
    tile_rows_issue(A_, B_, pred, cand, lane, tr);
    __builtin_amdgcn_sched_barrier(0);
    score_tile_rows(tr, u, gp, sGr, lane, sc);
    return;
  } else {
    // fp32 (one k slot per lane and step): step 4 c + s gives lane group q the value
    // e = 16 c + 4 q + s, so a lane reads e = 16 c + 4 q + 0..3 as one float4 and
    // feeds it to four consecutive steps (same mapping for A, gate and B).
    const float4* Ap = reinterpret_cast<const float4*>(static_cast<const float*>(A_) + pred * kE +
                                                       4 * q);
    const float4* Bp = reinterpret_cast<const float4*>(static_cast<const float*>(B_) + cand * kE +
                                                       4 * q);
    if constexpr (kOneRound) {
      float4 a[16], bb[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        a[c] = Ap[4 * c];
        bb[c] = Bp[4 * c];
      }
      __builtin_amdgcn_sched_barrier(0);
      *reinterpret_cast<float4*>(&sGr[4 * lane]) = gp;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float4 g = *reinterpret_cast<const float4*>(&sGr[16 * c + 4 * q]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].x * g.x, bb[c].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].y * g.y, bb[c].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].z * g.z, bb[c].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c].w * g.w, bb[c].w, acc, 0, 0, 0);
      }
    } else {
      *reinterpret_cast<float4*>(&sGr[4 * lane]) = gp;
      __builtin_amdgcn_wave_barrier();
#pragma unroll 8
      for (int c = 0; c < 16; ++c) {  // two rounds of 8 + 8 row loads in flight
        const float4 a = Ap[4 * c], bb = Bp[4 * c];
        const float4 g = *reinterpret_cast<const float4*>(&sGr[16 * c + 4 * q]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x * g.x, bb.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y * g.y, bb.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z * g.z, bb.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w * g.w, bb.w, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = acc[i] + u;
}

// One workgroup of 16 waves per CU is all a launch of <= 256 sequences gives, so
// registers are not rationed for a second one: every load of a wave can be in
// flight at once.
template <bool kBf16Tables, bool kWritePair, bool kWalk>
__global__ __launch_bounds__(kWave * kMaxL) __attribute__((amdgpu_waves_per_eu(4, 4))) void pair_walk_kernel(
    const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_val,
    const uint64_t* __restrict__ partial, int parts,
    const int32_t* __restrict__ prev_token, const float* __restrict__ gate, int gate_splits,
    int64_t gate_stride, const void* __restrict__ A_, const void* __restrict__ B_, int L,
    int64_t V, float* __restrict__ out_pair, int mode, double temperature, uint64_t seed,
    int32_t* __restrict__ out_path, float* __restrict__ out_scores, float* __restrict__ out_q,
    int32_t* __restrict__ out_cand) {
  __shared__ WalkTables sW;
  __shared__ __attribute__((aligned(16))) float sG[kMaxL][kE];  // gate row of each position
  __shared__ float sS[kWalk ? kMaxL : 1][kK][kK];                // whole tiles (best-path walk)
  __shared__ int32_t sC[kMaxL][kK];                              // merged candidates: ids
  __shared__ float sU[kMaxL][kK];                                //   and their logits
  __shared__ uint64_t sMerge[kMaxL][kMergeScratch];                // merge buffers, one per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int t = threadIdx.x / kWave;  // block position of this wave
  const int64_t b = blockIdx.x;
  const int r = lane & 15;  // predecessor slot (A operand row) and candidate slot (B column)
  const int q = lane >> 4;  // embedding quarter [64q, 64q + 64)
  const int64_t row = b * L + t;

  int32_t pred_id, cand_id;
  float u;
  // with the gathers issued first, rounds of four gate splits keep both within the
  // 128 registers of a 16-wave workgroup
  GateRegs<DFS_PW_GATHER_FIRST ? 4 : kGateRound> gr;
  if (parts <= 1) {
    // The candidates are final lists (cand_idx / cand_val).  The gate row does not
    // depend on them: its loads go out right after the id loads (a pointer select, not a
    // branch: no load has to wait for another).
    const int32_t* pred_p = t == 0 ? prev_token + b : cand_idx + (row - 1) * kK + r;
    pred_id = *pred_p;
    cand_id = cand_idx[row * kK + r];
    u = cand_val[row * kK + r];
    // Every wave's id loads go out before any wave's gate loads: the ids gate the table
    // gathers, and behind the workgroup's 64 KB of gate partial sums the last wave's ids
    // took 3.5 us to arrive (a bare barrier: it orders the issue, it waits for no load).
    __builtin_amdgcn_s_barrier();
    gate_issue(gate, gate_splits, gate_stride, row, lane, gr);
  } else {
    // The top-16 pass left `parts` sorted partial lists per row: each wave merges its
    // own row's, with the gate loads in flight meanwhile, and the merged lists meet in
    // LDS (position t needs the candidates of position t - 1 as predecessors).
    MergeRegs mr;
    merge_load(partial + row * parts * kK, parts, lane, mr);
    const int32_t prev = prev_token[b];
    gate_issue(gate, gate_splits, gate_stride, row, lane, gr);
    const uint64_t key = merge_keys(mr, parts, lane, sMerge[t]);
    if (lane < kK) {
      sC[t][lane] = (int32_t)key_index(key);
      sU[t][lane] = key_value(key);
    }
    __syncthreads();
    pred_id = t == 0 ? prev : sC[t - 1][r];
    cand_id = sC[t][r];
    u = sU[t][r];
  }
  // Ids outside [0, V) break the caller's contract; clamp them so that no gather
  // leaves the tables.
  const int64_t pred = pred_id < 0 ? 0 : (pred_id >= V ? V - 1 : pred_id);
  const int64_t cand = cand_id < 0 ? 0 : (cand_id >= V ? V - 1 : cand_id);

  // The gate row is parked in LDS before the table-row fragments are loaded, so that
  // all of them can be in flight at once; the scheduling barriers keep that order.  The
  // row is read back by other lanes of the same wave only.
  float sc[4];
  if constexpr (kBf16Tables && DFS_PW_GATHER_FIRST) {
    TileRows tr;
    tile_rows_issue(A_, B_, pred, cand, lane, tr);
    const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
    __builtin_amdgcn_sched_barrier(0);
    score_tile_rows(tr, u, gp, sG[t], lane, sc);
  } else {
    const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
    __builtin_amdgcn_sched_barrier(0);
    score_tile<kBf16Tables>(A_, B_, pred, cand, u, gp, sG[t], lane, sc);
  }
  if (kWalk && lane < kK) sW.cand[t][lane] = cand_id;
  // lane holds S_t(predecessor slot 4q + i, candidate slot r) in sc[i]
  if constexpr (kWritePair) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out_pair[(row * kK + 4 * q + i) * kK + r] = sc[i];
  }
  if constexpr (kWalk) {
    if (mode == 2 || out_q != nullptr) {  // whole tiles kept for the best path or the draft rows
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[t][4 * q + i][r] = sc[i];
    }
    if (mode == 2) {
      __syncthreads();
      if (t == 0) viterbi_walk(sS, sW.next, sW.cand, sW.slot, b, L, lane, out_path, out_scores);
    } else {
      successors(sc, t, lane, mode, temperature, seed, b, sW);
      __syncthreads();
      if (t == 0) chase(sW, b, L, lane, out_path, out_scores);
    }
    if (out_q != nullptr) {
      __syncthreads();
      draft_q(sS, sW, t, lane, temperature, row, out_q, out_cand);
    }
  }
}

// ---------------------------------------------------------------- mid-size batches
// A workgroup per sequence puts the gathers of a batch of a few dozen sequences on as
// many CUs.  Here each (sequence, position) is a workgroup of one wave that scores
// its 16 x 16 tile with score_tile into a pair tensor [rows, 16, 16]; walk_kernel then
// walks every sequence over it.  The tile and the walk are the fused kernel's own
// functions, so the path and the scores are the same bits.  Final candidate lists only
// (rows not split by the top-16 pass).
constexpr int kTileWaves = 1;  // positions per workgroup: 1 measured 0.5 us faster than 4 at 512 rows, 8 slower

template <bool kBf16Tables>
__global__ __launch_bounds__(kWave * kTileWaves) void pair_tile_kernel(
    const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_val, const int32_t* __restrict__ prev_token,
    const float* __restrict__ gate, int gate_splits, int64_t gate_stride, const void* __restrict__ A_,
    const void* __restrict__ B_, int L, int64_t V, int64_t rows, float* __restrict__ out_pair) {
  __shared__ __attribute__((aligned(16))) float sG[kTileWaves][kE];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int64_t row = (int64_t)blockIdx.x * kTileWaves + w;
  if (row >= rows) return;  // wave-uniform; only wave-level barriers follow
  const int64_t b = row / L;
  const int t = (int)(row % L);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int32_t* pred_p = t == 0 ? prev_token + b : cand_idx + (row - 1) * kK + r;
  const int32_t pred_id = *pred_p;
  const int32_t cand_id = cand_idx[row * kK + r];
  const float u = cand_val[row * kK + r];
  GateRegs<> gr;
  gate_issue(gate, gate_splits, gate_stride, row, lane, gr);
  // ids outside [0, V) break the caller's contract; clamped so no gather leaves the tables
  const int64_t pred = pred_id < 0 ? 0 : (pred_id >= V ? V - 1 : pred_id);
  const int64_t cand = cand_id < 0 ? 0 : (cand_id >= V ? V - 1 : cand_id);
  float sc[4];
  if constexpr (kBf16Tables && DFS_TILE_GATHER_FIRST) {
    TileRows tr;
    tile_rows_issue(A_, B_, pred, cand, lane, tr);
    const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
    __builtin_amdgcn_sched_barrier(0);
    score_tile_rows(tr, u, gp, sG[w], lane, sc);
  } else {
    const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
    __builtin_amdgcn_sched_barrier(0);
    score_tile<kBf16Tables>(A_, B_, pred, cand, u, gp, sG[w], lane, sc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out_pair[(row * kK + 4 * q + i) * kK + r] = sc[i];
}

// ---------------------------------------------------------------- few rows
// With few rows one workgroup per sequence would pull every position's gate partial sums
// and table rows through a single CU; instead each (sequence, position) gets a workgroup
// of eight waves: waves 0-3 merge position t's split top-16 lists, waves 4-7 position
// t - 1's (the predecessors), four lists per wave and then the four waves' lists, each
// a merge of four sorted runs; wave 0 then scores the tile and computes its successor
// table exactly as pair_walk_kernel does, and leaves them in `tiles`.  The last
// workgroup of a sequence to finish (an agent-scope release before an atomic count,
// acquire after it; the count wraps back to zero, and the launch before this one zeroes
// it as well) reads all L positions back and walks them with the same code.
constexpr int kPosThreads = 8 * kWave;

template <bool kBf16Tables>
__global__ __launch_bounds__(kPosThreads) void pair_pos_kernel(
    const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_val,
    const uint64_t* __restrict__ partial, int parts, const int32_t* __restrict__ prev_token,
    const float* __restrict__ gate, int gate_splits, int64_t gate_stride, const void* __restrict__ A_,
    const void* __restrict__ B_, int L, int64_t V, int mode, double temperature, uint64_t seed,
    int32_t* __restrict__ out_path, float* __restrict__ out_scores, float* __restrict__ out_q,
    int32_t* __restrict__ out_cand, PosTile* __restrict__ tiles, uint32_t* __restrict__ counters) {
  __shared__ int32_t sC[2][kK];  // [0]: position t - 1, [1]: position t
  __shared__ float sU[2][kK];
  __shared__ uint64_t sLists[2][4 * kK];  // the four waves' lists of each row
  __shared__ __attribute__((aligned(16))) float sG[kE];
  __shared__ WalkTables sW;
  __shared__ float sS[kMaxL][kK][kK];
  __shared__ int s_last;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  const int q = lane >> 4;
  const int64_t b = blockIdx.x / L;
  const int t = (int)(blockIdx.x % L);
  const int64_t row = b * L + t;

  int32_t pred_id = 0, cand_id = 0;
  float u = 0.0f;
  GateRegs<> gr;
  if (parts <= 1) {
    if (wave == 0) {
      const int32_t* pred_p = t == 0 ? prev_token + b : cand_idx + (row - 1) * kK + r;
      pred_id = *pred_p;
      cand_id = cand_idx[row * kK + r];
      u = cand_val[row * kK + r];
      gate_issue(gate, gate_splits, gate_stride, row, lane, gr);
    }
  } else {
    const int group = wave / 4, w4 = wave % 4;  // group 0: position t, 1: position t - 1
    const bool live = group == 0 || t > 0;       // wave-uniform
    Merge4Regs mr;
    if (live) merge4_load(partial + (row - group) * parts * kK, parts, w4, lane, mr);
    int32_t prev = 0;
    if (wave == 0) {
      prev = prev_token[b];
      gate_issue(gate, gate_splits, gate_stride, row, lane, gr);
    }
    const uint64_t list = live ? merge4_wave(mr, parts, w4, lane) : 0;
    if (lane < kK) sLists[group][w4 * kK + lane] = list;
    __syncthreads();
    if (live && w4 == 0) {
      const uint64_t key = wave_merge_runs16(sLists[group][lane], lane);
      if (lane < kK) {
        sC[1 - group][lane] = (int32_t)key_index(key);
        sU[1 - group][lane] = key_value(key);
      }
    }
    __syncthreads();
    if (wave == 0) {
      pred_id = t == 0 ? prev : sC[0][r];
      cand_id = sC[1][r];
      u = sU[1][r];
    }
  }
  PosTile* pt = tiles + row;
  if (wave == 0) {
    const int64_t pred = pred_id < 0 ? 0 : (pred_id >= V ? V - 1 : pred_id);
    const int64_t cand = cand_id < 0 ? 0 : (cand_id >= V ? V - 1 : cand_id);
    float sc[4];
    if constexpr (kBf16Tables && DFS_POS_GATHER_FIRST) {
      TileRows tr;
      tile_rows_issue(A_, B_, pred, cand, lane, tr);
      const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
      __builtin_amdgcn_sched_barrier(0);
      score_tile_rows(tr, u, gp, sG, lane, sc);
    } else {
      const float4 gp = gate_finish(gate, gate_splits, gate_stride, row, lane, gr);
      __builtin_amdgcn_sched_barrier(0);
      score_tile<kBf16Tables, DFS_F32_TILE_ONE_ROUND>(A_, B_, pred, cand, u, gp, sG, lane, sc);
    }
    if (mode == 2 || out_q != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pt->tile[4 * q + i][r] = sc[i];
    }
    if (mode != 2) {
      successors(sc, t, lane, mode, temperature, seed, b, sW);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (lane < kK) {
        pt->next[lane] = sW.next[t][lane];
        pt->best[lane] = sW.best[t][lane];
      }
    }
    if (lane < kK) pt->cand[lane] = cand_id;
    // publish this position, then count it; the last of the sequence walks
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) s_last = atomicInc(counters + b, (unsigned)(L - 1)) == (unsigned)(L - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const PosTile* seq = tiles + b * L;
  const bool need_tiles = mode == 2 || out_q != nullptr;
  for (int i = threadIdx.x; i < L * kK; i += kPosThreads) {
    const int tt = i / kK, j = i % kK;
    sW.cand[tt][j] = seq[tt].cand[j];
    if (mode != 2) {
      sW.next[tt][j] = seq[tt].next[j];
      sW.best[tt][j] = seq[tt].best[j];
    }
  }
  if (need_tiles) {
    for (int i = threadIdx.x; i < L * kK * kK; i += kPosThreads) {
      const int tt = i / (kK * kK), e = i % (kK * kK);
      sS[tt][e / kK][e % kK] = seq[tt].tile[e / kK][e % kK];
    }
  }
  __syncthreads();
  if (mode == 2) {
    if (wave == 0) viterbi_walk(sS, sW.next, sW.cand, sW.slot, b, L, lane, out_path, out_scores);
  } else if (wave == 0) {
    chase(sW, b, L, lane, out_path, out_scores);
  }
  if (out_q != nullptr) {
    __syncthreads();
    for (int tt = wave; tt < L; tt += kPosThreads / kWave) draft_q(sS, sW, tt, lane, temperature, b * L + tt, out_q, out_cand);
  }
}

// Walk over a pair tensor in memory: one workgroup per sequence, one wave per
// position, each wave reading its score tile in the lane layout of the matrix-core
// result above, so both walks run the same code on the same values.
__global__ __launch_bounds__(kWave * kMaxL) void walk_kernel(const float* __restrict__ pair,
                                                            const int32_t* __restrict__ cand_idx,
                                                            int L, int mode, double temperature,
                                                            uint64_t seed,
                                                            int32_t* __restrict__ out_path,
                                                            float* __restrict__ out_scores) {
  __shared__ WalkTables sW;
  __shared__ float sS[kMaxL][kK][kK];
  const int lane = threadIdx.x & (kWave - 1);
  const int t = threadIdx.x / kWave;
  const int64_t b = blockIdx.x;
  const int64_t row = b * L + t;
  const int r = lane & 15;
  const int q = lane >> 4;
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = pair[(row * kK + 4 * q + i) * kK + r];
  if (lane < kK) sW.cand[t][lane] = cand_idx[row * kK + lane];
  if (mode == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sS[t][4 * q + i][r] = sc[i];
    __syncthreads();
    if (t == 0) viterbi_walk(sS, sW.next, sW.cand, sW.slot, b, L, lane, out_path, out_scores);
  } else {
    successors(sc, t, lane, mode, temperature, seed, b, sW);
    __syncthreads();
    if (t == 0) chase(sW, b, L, lane, out_path, out_scores);
  }
}

template <bool kBf16, bool kWritePair, bool kWalk>
void launch_pw(int64_t batch, int64_t L, int64_t V, const CandSrc& c, const int32_t* prev_token,
               const GateSrc& g, const void* A, const void* B, float* out_pair, const WalkArgs* w,
               int32_t* out_path, float* out_scores, hipStream_t stream) {
  pair_walk_kernel<kBf16, kWritePair, kWalk><<<dim3((unsigned)batch), dim3((unsigned)(kWave * L)),
                                                0, stream>>>(
      c.idx, c.val, c.partial, c.parts, prev_token, g.gate, g.splits, g.stride, A, B, (int)L, V, out_pair,
      w ? w->mode : 0, w ? w->temperature : 1.0, w ? w->seed : 0ull, out_path, out_scores,
      w ? w->out_q : nullptr, w ? w->out_cand : nullptr);
}

}  // namespace

hipError_t launch_pair_walk(const CandSrc& cand, const int32_t* prev_token, const GateSrc& gate,
                            const void* A, const void* B, bool bf16_tables, int64_t batch, int64_t L,
                            int64_t V, float* out_pair, const WalkArgs* walk, int32_t* out_path,
                            float* out_scores, hipStream_t stream) {
  if (gate.splits < 1) return hipErrorInvalidValue;
  if (cand.parts > kMaxMergeParts || (cand.parts > 1 && cand.partial == nullptr)) return hipErrorInvalidValue;
  const bool wp = out_pair != nullptr;
  const bool wk = walk != nullptr;
#define DFS_PW(BF, WP, WK) \
  launch_pw<BF, WP, WK>(batch, L, V, cand, prev_token, gate, A, B, out_pair, walk, out_path, out_scores, stream)
  if (bf16_tables) {
    if (wp && wk) DFS_PW(true, true, true);
    else if (wp) DFS_PW(true, true, false);
    else DFS_PW(true, false, true);
  } else {
    if (wp && wk) DFS_PW(false, true, true);
    else if (wp) DFS_PW(false, true, false);
    else DFS_PW(false, false, true);
  }
#undef DFS_PW
  return hipGetLastError();
}

hipError_t launch_pair_pos(const CandSrc& c, const int32_t* prev_token, const GateSrc& g, const void* A,
                           const void* B, bool bf16_tables, int64_t batch, int64_t L, int64_t V, const WalkArgs& w,
                           int32_t* out_path, float* out_scores, PosTile* tiles, uint32_t* counters,
                           hipStream_t stream) {
  if (g.splits < 1) return hipErrorInvalidValue;
  if (c.parts > kMaxMergeParts || (c.parts > 1 && c.partial == nullptr)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(batch * L));
#define DFS_PP(BF)                                                                                                  \
  pair_pos_kernel<BF><<<grid, kPosThreads, 0, stream>>>(c.idx, c.val, c.partial, c.parts, prev_token, g.gate, g.splits, \
                                                        g.stride, A, B, (int)L, V, w.mode, w.temperature, w.seed,     \
                                                        out_path, out_scores, w.out_q, w.out_cand, tiles, counters)
  if (bf16_tables) {
    DFS_PP(true);
  } else {
    DFS_PP(false);
  }
#undef DFS_PP
  return hipGetLastError();
}

hipError_t launch_pair_tiles(const int32_t* cand_idx, const float* cand_val, const int32_t* prev_token,
                             const GateSrc& g, const void* A, const void* B, bool bf16_tables, int64_t batch,
                             int64_t L, int64_t V, float* out_pair, hipStream_t stream) {
  if (g.splits < 1) return hipErrorInvalidValue;
  const int64_t rows = batch * L;
  const dim3 grid((unsigned)((rows + kTileWaves - 1) / kTileWaves));
  if (bf16_tables) {
    pair_tile_kernel<true><<<grid, kWave * kTileWaves, 0, stream>>>(cand_idx, cand_val, prev_token, g.gate, g.splits,
                                                                     g.stride, A, B, (int)L, V, rows, out_pair);
  } else {
    pair_tile_kernel<false><<<grid, kWave * kTileWaves, 0, stream>>>(cand_idx, cand_val, prev_token, g.gate, g.splits,
                                                                      g.stride, A, B, (int)L, V, rows, out_pair);
  }
  return hipGetLastError();
}

hipError_t launch_walk(const float* pair, const int32_t* cand_idx, int64_t batch, int64_t L,
                       const WalkArgs& walk, int32_t* out_path, float* out_scores,
                       hipStream_t stream) {
  walk_kernel<<<dim3((unsigned)batch), dim3((unsigned)(kWave * L)), 0, stream>>>(
      pair, cand_idx, (int)L, walk.mode, walk.temperature, walk.seed, out_path, out_scores);
  return hipGetLastError();
}

}  // namespace dfs
