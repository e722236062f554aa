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
// the products are exact to ~2^-17 before fp32 accumulation.  The tiles stay in
// LDS and wave 0 walks them.
#include "dfs_device.h"
#include "dfs_internal.h"

namespace dfs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxL = 16;

// ---------------------------------------------------------------- Philox4x32-10
// Counter-based generator of Salmon, Moraes, Dror and Shaw (SC'11): ten rounds
// of two 32x32->64 multiplies and xors, key advanced by two Weyl constants.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// Standard Gumbel noise for (sequence b, position t, slot j), fp64:
// u = ((x >> 9) + 1/2) 2^-23 in (0, 1), g = -log(-log u).
__device__ __forceinline__ double gumbel_noise(uint64_t seed, uint32_t b, uint32_t t, uint32_t j) {
  const uint32_t x = philox_word0(j, t, b, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
  const double u = ((double)(x >> 9) + 0.5) * 0x1p-23;
  return -log(-log(u));
}

// The walk of one sequence over score tiles in LDS.  It is a chain of L dependent
// 16-way argmaxes, so one lane runs it: each step reads the predecessor's row of
// 16 scores from LDS and keeps the first maximum (lowest slot on ties).
__device__ __forceinline__ void walk_tiles(const float (*sS)[kK][kK], const double (*sN)[kK],
                                           const int32_t (*sC)[kK], int64_t b, int L, int mode,
                                           double temperature, int32_t* __restrict__ out_path,
                                           float* __restrict__ out_scores, int lane) {
  if (lane != 0) return;
  int i = 0;  // predecessor slot; every row of position 0 is the verified token's row
  for (int t = 0; t < L; ++t) {
    const float4* rp = reinterpret_cast<const float4*>(sS[t][i]);
    float row[kK];
#pragma unroll
    for (int c = 0; c < kK / 4; ++c) {
      const float4 v = rp[c];
      row[4 * c] = v.x;
      row[4 * c + 1] = v.y;
      row[4 * c + 2] = v.z;
      row[4 * c + 3] = v.w;
    }
    int j = 0;
    if (mode == 0) {
      float best = row[0];
#pragma unroll
      for (int c = 1; c < kK; ++c)
        if (row[c] > best) {
          best = row[c];
          j = c;
        }
    } else {
      double best = (double)row[0] / temperature + sN[t][0];
#pragma unroll
      for (int c = 1; c < kK; ++c) {
        const double v = (double)row[c] / temperature + sN[t][c];
        if (v > best) {
          best = v;
          j = c;
        }
      }
    }
    out_path[b * L + t] = sC[t][j];
    out_scores[b * L + t] = row[j];
    i = j;
  }
}

// Gate values g[row, e0 .. e0 + N) of the finished gate [rows, 256].
template <int N>
__device__ __forceinline__ void load_gate(const float* __restrict__ gate, int64_t row, int e0,
                                          float* g) {
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(gate + row * kE + e0 + 4 * c);
    g[4 * c] = v.x;
    g[4 * c + 1] = v.y;
    g[4 * c + 2] = v.z;
    g[4 * c + 3] = v.w;
  }
}

template <bool kBf16Tables, bool kWritePair, bool kWalk>
__global__ __launch_bounds__(kWave * kMaxL) void pair_walk_kernel(
    const int32_t* __restrict__ cand_idx, const float* __restrict__ cand_val,
    const int32_t* __restrict__ prev_token, const float* __restrict__ gate,
    const void* __restrict__ A_, const void* __restrict__ B_, int L, int64_t V,
    float* __restrict__ out_pair,
    int mode, double temperature, uint64_t seed, int32_t* __restrict__ out_path,
    float* __restrict__ out_scores) {
  __shared__ float sS[kMaxL][kK][kK];
  __shared__ double sN[kMaxL][kK];
  __shared__ int32_t sC[kMaxL][kK];
  const int lane = threadIdx.x & (kWave - 1);
  const int t = threadIdx.x / kWave;  // block position of this wave
  const int64_t b = blockIdx.x;
  const int r = lane & 15;  // predecessor slot (A operand row) and candidate slot (B column)
  const int q = lane >> 4;  // embedding quarter [64q, 64q + 64)
  const int64_t row = b * L + t;

  // Ids outside [0, V) break the caller's contract; clamp them so that no gather
  // leaves the tables.
  int64_t pred = t == 0 ? prev_token[b] : cand_idx[(row - 1) * kK + r];
  int64_t cand = cand_idx[row * kK + r];
  pred = pred < 0 ? 0 : (pred >= V ? V - 1 : pred);
  cand = cand < 0 ? 0 : (cand >= V ? V - 1 : cand);
  const float u = cand_val[row * kK + r];
  if (kWalk && lane < kK) sC[t][lane] = (int32_t)cand_idx[row * kK + lane];

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kBf16Tables) {
    // fragment c of this lane: elements [64 (c / 2) + 16 q + 8 (c % 2), + 8)
    const bf16x8* Ap = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(A_) +
                                                       pred * kE + 16 * q);
    const bf16x8* Bp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(B_) +
                                                       cand * kE + 16 * q);
    bf16x8 av[8], bv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      av[c] = Ap[8 * (c >> 1) + (c & 1)];
      bv[c] = Bp[8 * (c >> 1) + (c & 1)];
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float g[8];
      load_gate<8>(gate, row, 64 * (c >> 1) + 16 * q + 8 * (c & 1), g);
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ag = (float)av[c][e] * g[e];
        hi[e] = (__bf16)ag;
        lo[e] = (__bf16)(ag - (float)hi[e]);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv[c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv[c], acc, 0, 0, 0);
    }
  } else {
    // fp32 (one k slot per lane and step): step 4 c + s gives lane group q the value
    // e = 16 c + 4 q + s, so a lane reads e = 16 c + 4 q + 0..3 as one float4 and
    // feeds it to four consecutive steps (same mapping for A, gate and B).
    const float4* Ap = reinterpret_cast<const float4*>(static_cast<const float*>(A_) + pred * kE +
                                                       4 * q);
    const float4* Bp = reinterpret_cast<const float4*>(static_cast<const float*>(B_) + cand * kE +
                                                       4 * q);
#pragma unroll 4
    for (int c = 0; c < 16; ++c) {
      const float4 a = Ap[4 * c], bb = Bp[4 * c];
      float gv[4];
      load_gate<4>(gate, row, 16 * c + 4 * q, gv);
      const float4 g = make_float4(gv[0], gv[1], gv[2], gv[3]);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x * g.x, bb.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y * g.y, bb.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z * g.z, bb.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w * g.w, bb.w, acc, 0, 0, 0);
    }
  }
  // lane holds D[4q + i][r]: predecessor slot 4q + i, candidate slot r
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = acc[i] + u;
    if constexpr (kWalk) sS[t][4 * q + i][r] = s;
    if constexpr (kWritePair) out_pair[(row * kK + 4 * q + i) * kK + r] = s;
  }
  if constexpr (kWalk) {
    if (mode == 1 && lane < kK) sN[t][lane] = gumbel_noise(seed, (uint32_t)b, (uint32_t)t, lane);
    __syncthreads();
    if (t == 0) walk_tiles(sS, sN, sC, b, L, mode, temperature, out_path, out_scores, lane);
  }
}

// Walk over a pair tensor in memory: one wave per sequence.
__global__ __launch_bounds__(kWave) void walk_kernel(const float* __restrict__ pair,
                                                     const int32_t* __restrict__ cand_idx, int L,
                                                     int mode, double temperature, uint64_t seed,
                                                     int32_t* __restrict__ out_path,
                                                     float* __restrict__ out_scores) {
  __shared__ float sS[kMaxL][kK][kK];
  __shared__ double sN[kMaxL][kK];
  __shared__ int32_t sC[kMaxL][kK];
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;
  const float* src = pair + b * L * kK * kK;
  for (int e = lane; e < L * kK * kK; e += kWave) sS[e / (kK * kK)][(e / kK) % kK][e % kK] = src[e];
  for (int e = lane; e < L * kK; e += kWave) sC[e / kK][e % kK] = cand_idx[b * L * kK + e];
  if (mode == 1)
    for (int e = lane; e < L * kK; e += kWave)
      sN[e / kK][e % kK] = gumbel_noise(seed, (uint32_t)b, (uint32_t)(e / kK), (uint32_t)(e % kK));
  __syncthreads();
  walk_tiles(sS, sN, sC, b, L, mode, temperature, out_path, out_scores, lane);
}

template <bool kBf16, bool kWritePair, bool kWalk>
void launch_pw(int64_t batch, int64_t L, int64_t V, const int32_t* cand_idx, const float* cand_val,
               const int32_t* prev_token, const float* gate, const void* A, const void* B,
               float* out_pair, const WalkArgs* w, int32_t* out_path, float* out_scores,
               hipStream_t stream) {
  pair_walk_kernel<kBf16, kWritePair, kWalk><<<dim3((unsigned)batch), dim3((unsigned)(kWave * L)),
                                                0, stream>>>(
      cand_idx, cand_val, prev_token, gate, A, B, (int)L, V, out_pair, w ? w->mode : 0,
      w ? w->temperature : 1.0, w ? w->seed : 0ull, out_path, out_scores);
}

}  // namespace

hipError_t launch_pair_walk(const int32_t* cand_idx, const float* cand_val,
                            const int32_t* prev_token, const float* gate, const void* A,
                            const void* B, bool bf16_tables, int64_t batch, int64_t L,
                            int64_t V, float* out_pair, const WalkArgs* walk, int32_t* out_path,
                            float* out_scores, hipStream_t stream) {
  const bool wp = out_pair != nullptr;
  const bool wk = walk != nullptr;
#define DFS_PW(BF, WP, WK)                                                                      \
  launch_pw<BF, WP, WK>(batch, L, V, cand_idx, cand_val, prev_token, gate, A, B, out_pair, walk,   \
                        out_path, out_scores, stream)
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

hipError_t launch_walk(const float* pair, const int32_t* cand_idx, int64_t batch, int64_t L,
                       const WalkArgs& walk, int32_t* out_path, float* out_scores,
                       hipStream_t stream) {
  walk_kernel<<<dim3((unsigned)batch), kWave, 0, stream>>>(pair, cand_idx, (int)L, walk.mode,
                                                          walk.temperature, walk.seed, out_path,
                                                          out_scores);
  return hipGetLastError();
}

}  // namespace dfs
