// Speculative-sampling verification of drafted blocks against a target distribution.
//
// The drafted block is checked by the target model; sampled drafts are accepted by
// rejection sampling, which keeps the target's distribution exact (blog post
// "DFlash 2: Keep Drafting Parallel": the selector's sampling draws from the same
// scores, section "A Lightweight Path Selector").  The rule is the standard one for
// speculative sampling (Leviathan, Kalman and Matias, ICML 2023; Chen et al., 2023):
// draft token x_t with draft probability q_t(x_t) is kept with probability
// min(1, p_t(x_t) / q_t(x_t)); at the first rejection one token is drawn from
// norm(max(0, p_t - q_t)); with every token kept, one more is drawn from p_L.
// p_t = softmax(z_t / T) over the vocabulary, z the target logits of row t.
//
// Design (gfx950): two kernels.  lse_kernel streams the target logits once (the
// only vocabulary-wide pass) and leaves, for every run of 4096 tokens of every row
// (a segment), the running (max, sum of 2^(x - max)) of x = z log2(e) / T, each
// segment streamed by one wave with 16-byte non-temporal loads and reduced with
// DPP.  verify_kernel takes one block per workgroup: it merges a row's segments
// into its log2-sum-exp, runs the accept tests (fp64 ratio against a 23-bit Philox
// uniform), and draws the output token by inverse CDF with a 46-bit Philox
// uniform: the segments' masses (their pairs against the row's log-sum-exp, less
// the 16 candidates' min(p, q) where the residual applies) locate the segment,
// and only that segment is read again to find the token, each thread summing a
// contiguous share of it in token order.
#include "dfs_device.h"
#include "dfs_internal.h"
#include "philox.h"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
#ifndef DFS_LSE_UNROLL
#define DFS_LSE_UNROLL 2
#endif
#ifndef DFS_LSE_SEGS_PER_WAVE
#define DFS_LSE_SEGS_PER_WAVE 8  // segments a wave streams back to back (1, 2, 4, 16, 32 measured slower)
#endif
constexpr int kUnroll = DFS_LSE_UNROLL;  // 16-byte vectors per lane per step (two steps in flight)
constexpr int kSeg = 4096;           // tokens per segment of a target row
constexpr int kMaxSeg = 1024;        // segments per row the draw holds in LDS (V <= 2^22)
constexpr int kMaxL = 16;            // longest block
constexpr float kLog2e = 1.4426950408889634f;

// Running maximum and sum of 2^(x - max) (the sum in fp64, so that the mass of a
// segment is good to ~1e-7 of the row's).  An empty pair is (-inf, 0).
struct MS {
  float m;
  double s;
};

// 2^x by the hardware's v_exp_f32 (about 1 ulp; results below 2^-126, which no
// sum here can feel next to its own maximum's term 1, may come back flushed).
// The library exp2f wraps the same instruction in a denormal rescue that costs
// five more instructions per element, which would make the pass ALU-bound.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{m, 0.0};
  return MS{m, a.s * (double)fast_exp2(a.m - m) + b.s * (double)fast_exp2(b.m - m)};
}

template <bool kBf16>
__device__ __forceinline__ float logit_at(const void* p, int64_t i) {
  if constexpr (kBf16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// The values of a 16-byte vector (8 bf16 or 4 fp32), widened to fp32.
template <bool kBf16>
__device__ __forceinline__ void unpack_vec(uint4 d, float* x) {
  if constexpr (kBf16) {
    x[0] = bf16_lo(d.x); x[1] = bf16_hi(d.x);
    x[2] = bf16_lo(d.y); x[3] = bf16_hi(d.y);
    x[4] = bf16_lo(d.z); x[5] = bf16_hi(d.z);
    x[6] = bf16_lo(d.w); x[7] = bf16_hi(d.w);
  } else {
    x[0] = __uint_as_float(d.x); x[1] = __uint_as_float(d.y);
    x[2] = __uint_as_float(d.z); x[3] = __uint_as_float(d.w);
  }
}

// Add N vectors of raw logits z to a running pair of x = z * scale (scale > 0, so
// the largest z gives the largest x): one maximum and at most one rescale for the
// lot, then one fma and one v_exp_f32 per value, summed in fp32 and added to the
// fp64 sum once.
template <bool kBf16, int N>
__device__ __forceinline__ void ms_add_vecs(MS& a, const uint4* d, float scale) {
  constexpr int PV = kBf16 ? 8 : 4;
  float x[N][PV];
#pragma unroll
  for (int u = 0; u < N; ++u) unpack_vec<kBf16>(d[u], x[u]);
  float zm = -INFINITY;
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int e = 0; e < PV; ++e) zm = fmaxf(zm, x[u][e]);
  const float vm = zm * scale;
  // A new maximum is rare once a row is under way: the rescale (an exponential and
  // an fp64 product) sits behind a branch that a wave skips when none of its lanes
  // needs it, instead of running, masked, on every step (the empty volatile asm keeps
  // the compiler from turning the branch into selects).
  if (vm > a.m) {
    __asm__ volatile("");
    a.s = a.m == -INFINITY ? 0.0 : a.s * (double)fast_exp2(a.m - vm);
    a.m = vm;
  }
  if (a.m == -INFINITY) return;
  const float nm = -a.m;
  float vs = fast_exp2(fmaf(x[0][0], scale, nm));  // (the sum starts at its first term: no 0 + x)
#pragma unroll
  for (int u = 0; u < N; ++u)
#pragma unroll
    for (int e = (u == 0 ? 1 : 0); e < PV; ++e) vs += fast_exp2(fmaf(x[u][e], scale, nm));
  a.s += (double)vs;
}

__device__ __forceinline__ void ms_add(MS& a, float z, float scale) {
  const float x = z * scale;
  const float m = fmaxf(a.m, x);
  if (m == -INFINITY) return;
  a = MS{m, (m == a.m ? a.s : a.s * (double)fast_exp2(a.m - m)) + (double)fast_exp2(x - m)};
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
constexpr int kCacheNonTemporal = 2;

// Segments of a target row, in token order: the row's 16-byte aligned middle
// [vb, ve) is cut into runs of kSeg tokens from vb; segment 0 also takes the
// unaligned head [0, vb) and the last segment the tail [ve, V).  Both kernels
// derive the same cut from the row's address.
struct RowCut {
  int64_t vb, ve, nvec, nseg;
};

template <bool kBf16>
__device__ __forceinline__ RowCut row_cut(const void* rowp, int64_t V) {
  constexpr int esz = kBf16 ? 2 : 4;
  constexpr int PV = 16 / esz;
  RowCut c;
  const uintptr_t a = (uintptr_t)rowp;
  c.vb = (int64_t)(((16u - (a & 15u)) & 15u) / esz);
  if (c.vb > V) c.vb = V;
  c.nvec = (V - c.vb) / PV;
  c.ve = c.vb + c.nvec * PV;
  c.nseg = (c.nvec * PV + kSeg - 1) / kSeg;
  if (c.nseg < 1) c.nseg = 1;
  return c;
}

__device__ __forceinline__ void seg_range(const RowCut& c, int64_t V, int64_t s, int64_t& lo,
                                          int64_t& hi) {
  lo = s == 0 ? 0 : c.vb + s * kSeg;
  hi = s == c.nseg - 1 ? V : c.vb + (s + 1) * kSeg;
}

// Reduce a wave's running pair (lane 0 ends with the merge, in a fixed order).
__device__ __forceinline__ MS wave_merge(MS acc, int lane) {
#pragma unroll
  for (int k = 1; k < kWave; k <<= 1) {
    const uint64_t sb = (uint64_t)__double_as_longlong(acc.s);
    const uint32_t lo = xor_lanes((uint32_t)sb, k, lane), hi = xor_lanes((uint32_t)(sb >> 32), k, lane);
    const MS o{__uint_as_float(xor_lanes(__float_as_uint(acc.m), k, lane)),
               __longlong_as_double((long long)(((uint64_t)hi << 32) | lo))};
    acc = ms_merge(acc, o);
  }
  return acc;
}

// (max, sum) of x = z * scale for every segment of the rows.  Workgroup (row, part)
// takes a contiguous run of the row's segments and each of its waves a contiguous
// part of that; a wave streams its segments' vectors without a break (the next
// step's 16-byte non-temporal loads in flight while the current ones are added),
// and closes a segment every kSegVec vectors with one DPP reduction.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_kernel(const void* __restrict__ logits, int64_t V,
                                                       int parts, int64_t nseg_max, float scale,
                                                       double2* __restrict__ seg_out) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int PV = kBf16 ? 8 : 4;
  constexpr int kSegVec = kSeg / PV;            // vectors per segment
  constexpr int kStep = kWave * kUnroll;        // vectors per wave step
  static_assert(kSegVec % kStep == 0, "a step never straddles two segments");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t row = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const T* rowp = static_cast<const T*>(logits) + row * V;
  const RowCut c = row_cut<kBf16>(rowp, V);
  const int64_t per_wg = (c.nseg + parts - 1) / parts;
  const int64_t sa = (int64_t)part * per_wg;
  const int64_t sb = sa + per_wg < c.nseg ? sa + per_wg : c.nseg;
  const int64_t per_wave = sb > sa ? (sb - sa + kWaves - 1) / kWaves : 0;
  const int64_t wa = sa + wave * per_wave;
  const int64_t wb = wa + per_wave < sb ? wa + per_wave : sb;
  if (wa >= wb) return;

  auto scalars = [&](MS& acc, int64_t sg) {
    if (sg == 0)
      for (int64_t i = lane; i < c.vb; i += kWave) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
    if (sg == c.nseg - 1)
      for (int64_t i = c.ve + lane; i < V; i += kWave) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
  };
  auto emit = [&](MS acc, int64_t sg) {
    acc = wave_merge(acc, lane);
    if (lane == 0) seg_out[row * nseg_max + sg] = make_double2((double)acc.m, acc.s);
  };
  if (c.nvec == 0) {  // no aligned middle: the one segment is all scalars
    MS acc{-INFINITY, 0.0};
    scalars(acc, 0);
    emit(acc, 0);
    return;
  }
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(rowp + c.vb), (short)0, (int)(c.nvec * 16), kRawBufferWord3);
  auto load = [&](uint4* dst, int64_t base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t vid = (uint32_t)(base + u * kWave + lane);
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vid * 16u, 0, kCacheNonTemporal);
      dst[u] = make_uint4(w.x, w.y, w.z, w.w);  // past the row: zeros, skipped below
    }
  };
  const int64_t v0 = wa * kSegVec;
  const int64_t v1 = wb * kSegVec < c.nvec ? wb * kSegVec : c.nvec;
  MS acc{-INFINITY, 0.0};
  scalars(acc, wa);
  auto add_step = [&](const uint4* src, int64_t base) {
    if (base + kStep <= v1) {  // wave-uniform: every vector of the step is in the row
      ms_add_vecs<kBf16, kUnroll>(acc, src, scale);
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kWave + lane < v1) ms_add_vecs<kBf16, 1>(acc, src + u, scale);
    }
    const int64_t next = base + kStep;
    if (next % kSegVec == 0 || next >= v1) {  // the step closed its segment
      const int64_t sg = base / kSegVec;
      emit(acc, sg);
      acc = MS{-INFINITY, 0.0};
      if (next < v1) scalars(acc, sg + 1);
    }
  };
  uint4 bufA[kUnroll], bufB[kUnroll];
  load(bufA, v0);
  int64_t base = v0;
  for (; base + kStep < v1; base += 2 * kStep) {  // the next step is always loaded ahead
    load(bufB, base + kStep);
    add_step(bufA, base);
    load(bufA, base + 2 * kStep);
    if (base + kStep < v1) add_step(bufB, base + kStep);
  }
  if (base < v1) add_step(bufA, base);
}

// Target probability of token v in row `rowp`: 2^(x - log2-sum-exp) in fp64, x the
// fp32-scaled logit as the log-sum-exp pass saw it (the residual of a candidate
// subtracts min(p, q) from it).
template <bool kBf16>
__device__ __forceinline__ double token_weight(const void* rowp, int64_t v, float scale, double lse2) {
  return exp2((double)(logit_at<kBf16>(rowp, v) * scale) - lse2);
}

// Inclusive prefix sum over the workgroup, in a fixed order (wave scans with
// shuffles, then the wave totals in wave order); every thread passes one value.
__device__ __forceinline__ double block_prefix(double v, double* s_wave, int tid) {
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == kWave - 1) s_wave[wave] = v;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += s_wave[w];
  __syncthreads();
  return base + v;
}

constexpr int kMaxPer = 17;  // tokens per thread in the rescanned segment (kSeg / 256 + 1)

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const void* __restrict__ logits, int64_t V, int L, int64_t nseg_max, float scale,
    const double2* __restrict__ segs, const int32_t* __restrict__ path,
    const int32_t* __restrict__ cand, const float* __restrict__ q, uint64_t seed,
    int32_t* __restrict__ out_accepted, int32_t* __restrict__ out_token) {
  static_assert(kSeg / kThreads + 1 <= kMaxPer, "rescan share");
  __shared__ double s_lse2[kMaxL + 1];
  __shared__ int32_t s_cand[kK];
  __shared__ double s_corr[kK];
  __shared__ double s_mass[kMaxSeg];
  __shared__ double s_wave[kWaves];
  __shared__ int s_k, s_seg, s_pick, s_last;
  __shared__ double s_rest;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t b = blockIdx.x;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  auto row_ptr = [&](int64_t row) {
    return kBf16 ? (const void*)(static_cast<const uint16_t*>(logits) + row * V)
                 : (const void*)(static_cast<const float*>(logits) + row * V);
  };

  // log2-sum-exp of rows (b, 0..L): wave w merges rows w, w + 4, ...; a lane loads
  // segments lane, lane + 64, ... of each of its rows before any merge
  {
    constexpr int kRowsPerWave = (kMaxL + 1 + kWaves - 1) / kWaves;
    constexpr int kSegPerLane = 2;  // segment pairs a lane holds per row before merging
    double2 held[kRowsPerWave][kSegPerLane];
    int64_t nseg_of[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int t = wave + i * kWaves;
      const int64_t row = b * (L + 1) + (t <= L ? t : L);
      nseg_of[i] = row_cut<kBf16>(row_ptr(row), V).nseg;
#pragma unroll
      for (int u = 0; u < kSegPerLane; ++u) {
        const int64_t sg = lane + u * kWave;
        held[i][u] = make_double2(-INFINITY, 0.0);
        if (t <= L && sg < nseg_of[i]) held[i][u] = segs[row * nseg_max + sg];
      }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int t = wave + i * kWaves;
      const int64_t row = b * (L + 1) + (t <= L ? t : L);
      MS r{-INFINITY, 0.0};
#pragma unroll
      for (int u = 0; u < kSegPerLane; ++u) r = ms_merge(r, MS{(float)held[i][u].x, held[i][u].y});
      for (int64_t sg = lane + kSegPerLane * kWave; sg < nseg_of[i]; sg += kWave) {  // long rows
        const double2 p = segs[row * nseg_max + sg];
        r = ms_merge(r, MS{(float)p.x, p.y});
      }
      r = wave_merge(r, lane);
      if (lane == 0 && t <= L) s_lse2[t] = r.s > 0.0 ? (double)r.m + log2(r.s) : -INFINITY;
    }
  }
  __syncthreads();

  // accept tests of all positions at once (lane t of wave 0); the block keeps the
  // draft tokens before the first rejection
  if (tid < kWave) {
    bool keep = false;  // lanes >= L stand for "past the block": rejected
    if (tid < L) {
      const int t = tid;
      const int64_t row = b * (L + 1) + t;
      int32_t x = path[b * L + t];
      int32_t cj[kK];
      float qj[kK];
#pragma unroll
      for (int j = 0; j < kK; ++j) {  // every load issued before any compare
        cj[j] = cand[(b * L + t) * kK + j];
        qj[j] = q[(b * L + t) * kK + j];
      }
      float qx = 0.0f;
#pragma unroll
      for (int j = 0; j < kK; ++j) qx = cj[j] == x ? qj[j] : qx;
      x = x < 0 ? 0 : (x >= V ? (int32_t)(V - 1) : x);
      const float xs = logit_at<kBf16>(logits, row * V + x) * scale;
      const double p = exp2((double)xs - s_lse2[t]);
      uint32_t w[4];
      philox4x32_10(0u, (uint32_t)t, (uint32_t)b, 1u, k0, k1, w);
      keep = uniform23(w[0]) < p / (double)qx;
    }
    const uint64_t rejected = __ballot(!keep);  // bit L is always set (L <= 16 < 64)
    if (tid == 0) {
      const int k = (int)__builtin_ctzll(rejected);
      s_k = k < L ? k : L;
    }
  }
  __syncthreads();
  const int k = s_k;
  const int64_t row = b * (L + 1) + k;
  const void* rowp = row_ptr(row);
  const double lse2 = s_lse2[k];
  const RowCut c = row_cut<kBf16>(rowp, V);
  if (tid < kK) {
    int32_t cd = -1;
    double corr = 0.0;
    if (k < L) {
      cd = cand[(b * L + k) * kK + tid];
      const int32_t cc = cd < 0 ? 0 : (cd >= V ? (int32_t)(V - 1) : cd);
      const double p = token_weight<kBf16>(rowp, cc, scale, lse2);
      const double qc = (double)q[(b * L + k) * kK + tid];
      corr = p < qc ? p : qc;  // min(p, q): what the residual takes off token cd
    }
    s_cand[tid] = cd;
    s_corr[tid] = corr;
  }
  // the mass of every segment, from its (max, sum) pair
  for (int64_t sg = tid; sg < c.nseg; sg += kThreads) {
    const double2 p = segs[row * nseg_max + sg];
    s_mass[sg] = p.y * exp2(p.x - lse2);
  }
  if (tid == 0) {
    s_last = -1;
    s_seg = 0;  // (no segment with mass at all: the rescan below picks the segment's first token)
  }
  __syncthreads();
  if (tid == 0) {  // the residual's corrections, where they fall (in candidate order)
    for (int j = 0; j < kK; ++j) {
      const int64_t cd = s_cand[j];
      if (cd < 0 || cd >= V) continue;
      const int64_t sg = cd < c.vb + kSeg ? 0 : ((cd - c.vb) / kSeg < c.nseg ? (cd - c.vb) / kSeg : c.nseg - 1);
      s_mass[sg] -= s_corr[j];
    }
  }
  __syncthreads();
  // Which segment: thread i holds a group of g consecutive segments; a prefix sum
  // over the groups gives the group the draw falls in, its thread walks it.
  {
    const int64_t g = (c.nseg + kThreads - 1) / kThreads;
    const int64_t s0 = tid * g;
    double gm = 0.0;
    for (int64_t sg = s0; sg < s0 + g && sg < c.nseg; ++sg) gm += s_mass[sg] > 0.0 ? s_mass[sg] : 0.0;
    const double incl = block_prefix(gm, s_wave, tid);
    if (tid == kThreads - 1) s_rest = incl;  // the total mass
    __syncthreads();
    uint32_t w[4];
    philox4x32_10(0u, (uint32_t)k, (uint32_t)b, 2u, k0, k1, w);
    const double u = ((double)(w[0] >> 9) * 0x1p23 + (double)(w[1] >> 9) + 0.5) * 0x1p-46;
    const double target = u * s_rest;
    const double excl = incl - gm;
    if (gm > 0.0) atomicMax(&s_last, tid);
    __syncthreads();
    bool mine = gm > 0.0 && excl < target && target <= incl;
    if (!mine && tid == s_last && target > incl) mine = true;  // rounding past the end
    if (mine) {
      double cum = excl;
      int64_t pick = -1, lastpos = -1;
      for (int64_t sg = s0; sg < s0 + g && sg < c.nseg; ++sg) {
        const double m = s_mass[sg] > 0.0 ? s_mass[sg] : 0.0;
        if (m <= 0.0) continue;
        lastpos = sg;
        if (cum + m >= target) {
          pick = sg;
          break;
        }
        cum += m;
      }
      s_seg = (int)(pick >= 0 ? pick : lastpos);
      // past the end by rounding: a rest beyond any sum takes the segment's last token
      s_rest = pick >= 0 ? target - cum : 1e300;
    }
  }
  __syncthreads();
  // The segment, exactly: thread i weighs its contiguous share of it (candidates'
  // corrections held in registers), a prefix sum over the shares gives the share
  // the draw falls in, and its thread picks the token.
  int64_t lo, hi;
  seg_range(c, V, s_seg, lo, hi);
  const int64_t per = (hi - lo + kThreads - 1) / kThreads;
  int32_t cj[kK];
  double dj[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    cj[j] = s_cand[j];
    dj[j] = s_corr[j];
  }
  const int64_t a0 = lo + tid * per < hi ? lo + tid * per : hi;
  const int64_t e0 = a0 + per < hi ? a0 + per : hi;
  double wv[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int64_t v = a0 + i;
    double x = 0.0;
    if (v < e0) {
      x = token_weight<kBf16>(rowp, v, scale, lse2);
#pragma unroll
      for (int j = 0; j < kK; ++j) x = cj[j] == v ? x - dj[j] : x;
      x = x > 0.0 ? x : 0.0;
    }
    wv[i] = x;
  }
  double share = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) share += wv[i];
  if (tid == 0) {
    s_pick = -1;
    s_last = -1;
  }
  const double incl = block_prefix(share, s_wave, tid);  // (holds barriers)
  const double excl = incl - share;
  const double rest = s_rest;
  if (share > 0.0) atomicMax(&s_last, tid);
  __syncthreads();
  bool mine = share > 0.0 && excl < rest && rest <= incl;
  if (!mine && tid == s_last && rest > incl) mine = true;  // rounding past the end
  if (mine) {
    double cum = excl;
    int64_t pick = -1, lastpos = a0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (pick >= 0 || wv[i] <= 0.0) continue;
      lastpos = a0 + i;
      cum += wv[i];
      if (cum >= rest) pick = a0 + i;
    }
    s_pick = (int)(pick >= 0 ? pick : lastpos);
  }
  __syncthreads();
  if (tid == 0) {
    out_accepted[b] = k;
    out_token[b] = s_pick >= 0 ? s_pick : (int32_t)lo;
  }
}

}  // namespace

VerifyPlan plan_verify(int64_t batch, int64_t L, int64_t V, int esize) {
  VerifyPlan p{};
  p.batch = batch;
  p.L = L;
  p.V = V;
  p.esize = esize;
  const int64_t rows = batch * (L + 1);
  // segments per row (at most one more than the aligned middle needs)
  p.nseg = cdiv(V, kSeg) + 1;
  // workgroups per row: about eight segments per wave (32 KB of bf16 streamed back to
  // back); two per wave, many short workgroups, was 5% slower at 256 x 17 x 151936
  const int64_t parts = cdiv(p.nseg, DFS_LSE_SEGS_PER_WAVE * kWaves);
  p.parts = (int)parts;
  p.ws_bytes = align_up((size_t)rows * p.nseg * sizeof(double2), 256);
  return p;
}

int64_t verify_max_vocab() { return (int64_t)(kMaxSeg - 1) * kSeg; }

hipError_t launch_verify(const VerifyPlan& p, const void* logits, bool bf16, const int32_t* path,
                         const int32_t* cand, const float* q, double temperature, uint64_t seed,
                         void* ws, int32_t* out_accepted, int32_t* out_token, hipStream_t stream) {
  double2* segs = static_cast<double2*>(ws);
  const float scale = (float)((double)kLog2e / temperature);
  const int64_t rows = p.batch * (p.L + 1);
  const dim3 grid((unsigned)(rows * p.parts));
  if (bf16) {
    lse_kernel<true><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.nseg, scale, segs);
    verify_kernel<true><<<dim3((unsigned)p.batch), kThreads, 0, stream>>>(
        logits, p.V, (int)p.L, p.nseg, scale, segs, path, cand, q, seed, out_accepted, out_token);
  } else {
    lse_kernel<false><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.nseg, scale, segs);
    verify_kernel<false><<<dim3((unsigned)p.batch), kThreads, 0, stream>>>(
        logits, p.V, (int)p.L, p.nseg, scale, segs, path, cand, q, seed, out_accepted, out_token);
  }
  return hipGetLastError();
}

}  // namespace dfs
