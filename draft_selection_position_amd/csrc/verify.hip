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
constexpr int kUnroll = 4;           // 16-byte vectors per thread per iteration
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

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{m, 0.0};
  return MS{m, a.s * (double)exp2f(a.m - m) + b.s * (double)exp2f(b.m - m)};
}

template <bool kBf16>
__device__ __forceinline__ float logit_at(const void* p, int64_t i) {
  if constexpr (kBf16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// Add the values of one 16-byte vector (8 bf16 or 4 fp32) to a running pair.
template <bool kBf16>
__device__ __forceinline__ void ms_add_vec(MS& a, uint4 d, float scale) {
  constexpr int PV = kBf16 ? 8 : 4;
  float x[PV];
  if constexpr (kBf16) {
    x[0] = bf16_lo(d.x); x[1] = bf16_hi(d.x);
    x[2] = bf16_lo(d.y); x[3] = bf16_hi(d.y);
    x[4] = bf16_lo(d.z); x[5] = bf16_hi(d.z);
    x[6] = bf16_lo(d.w); x[7] = bf16_hi(d.w);
  } else {
    x[0] = __uint_as_float(d.x); x[1] = __uint_as_float(d.y);
    x[2] = __uint_as_float(d.z); x[3] = __uint_as_float(d.w);
  }
  float vm = -INFINITY;
#pragma unroll
  for (int e = 0; e < PV; ++e) {
    x[e] *= scale;
    vm = fmaxf(vm, x[e]);
  }
  const float m = fmaxf(a.m, vm);
  if (m == -INFINITY) return;
  float vs = 0.0f;  // the vector's own few terms in fp32, then into the fp64 sum
#pragma unroll
  for (int e = 0; e < PV; ++e) vs += exp2f(x[e] - m);
  a = MS{m, (m == a.m ? a.s : a.s * (double)exp2f(a.m - m)) + (double)vs};
}

__device__ __forceinline__ void ms_add(MS& a, float z, float scale) {
  const float x = z * scale;
  const float m = fmaxf(a.m, x);
  if (m == -INFINITY) return;
  a = MS{m, (m == a.m ? a.s : a.s * (double)exp2f(a.m - m)) + (double)exp2f(x - m)};
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

// (max, sum) of x = z * scale for every segment of the rows: workgroup (row, part)
// takes segments part, part + parts, ... of its row, one wave per segment at a
// time, 16-byte non-temporal loads of the aligned middle.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_kernel(const void* __restrict__ logits, int64_t V,
                                                       int parts, int64_t nseg_max, float scale,
                                                       double2* __restrict__ seg_out) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int PV = kBf16 ? 8 : 4;
  constexpr int kSegVec = kSeg / PV;  // vectors per segment
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t row = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const T* rowp = static_cast<const T*>(logits) + row * V;
  const RowCut c = row_cut<kBf16>(rowp, V);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(rowp + c.vb), (short)0, (int)(c.nvec * 16), kRawBufferWord3);
  for (int64_t sg = (int64_t)part * kWaves + wave; sg < c.nseg; sg += (int64_t)parts * kWaves) {
    MS acc{-INFINITY, 0.0};
    if (sg == 0)
      for (int64_t i = lane; i < c.vb; i += kWave) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
    if (sg == c.nseg - 1)
      for (int64_t i = c.ve + lane; i < V; i += kWave) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
    const int64_t v0 = sg * kSegVec;
    const int64_t v1 = v0 + kSegVec < c.nvec ? v0 + kSegVec : c.nvec;
    for (int64_t base = v0; base < v1; base += (int64_t)kWave * kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t vid = (uint32_t)(base + u * kWave + lane);
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vid * 16u, 0, kCacheNonTemporal);
        v[u] = make_uint4(w.x, w.y, w.z, w.w);  // past the row: zeros, skipped below
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kWave + lane < v1) ms_add_vec<kBf16>(acc, v[u], scale);
    }
#pragma unroll
    for (int k = 1; k < kWave; k <<= 1) {
      const uint64_t sb = (uint64_t)__double_as_longlong(acc.s);
      const uint32_t lo = xor_lanes((uint32_t)sb, k, lane), hi = xor_lanes((uint32_t)(sb >> 32), k, lane);
      const MS o{__uint_as_float(xor_lanes(__float_as_uint(acc.m), k, lane)),
                 __longlong_as_double((long long)(((uint64_t)hi << 32) | lo))};
      acc = ms_merge(acc, o);
    }
    if (lane == 0) seg_out[row * nseg_max + sg] = make_double2((double)acc.m, acc.s);
  }
}

// Target probability of token v in row `rowp`: 2^(x - log2-sum-exp) in fp64, x the
// fp32-scaled logit as the log-sum-exp pass saw it (the residual of a candidate
// subtracts min(p, q) from it).
template <bool kBf16>
__device__ __forceinline__ double token_weight(const void* rowp, int64_t v, float scale, double lse2) {
  return exp2((double)(logit_at<kBf16>(rowp, v) * scale) - lse2);
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const void* __restrict__ logits, int64_t V, int L, int64_t nseg_max, float scale,
    const double2* __restrict__ segs, const int32_t* __restrict__ path,
    const int32_t* __restrict__ cand, const float* __restrict__ q, uint64_t seed,
    int32_t* __restrict__ out_accepted, int32_t* __restrict__ out_token) {
  __shared__ double s_lse2[kMaxL + 1];
  __shared__ int32_t s_cand[kK];
  __shared__ double s_corr[kK];
  __shared__ double s_mass[kMaxSeg];
  __shared__ double s_share[kThreads];
  __shared__ int s_k, s_seg;
  __shared__ double s_rest;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);

  // log2-sum-exp of rows (b, 0..L): the row's segments merged in order
  if (tid <= L) {
    const int64_t row = b * (L + 1) + tid;
    const void* rowp = kBf16 ? (const void*)(static_cast<const uint16_t*>(logits) + row * V)
                             : (const void*)(static_cast<const float*>(logits) + row * V);
    const RowCut c = row_cut<kBf16>(rowp, V);
    MS r{-INFINITY, 0.0};
    for (int64_t i = 0; i < c.nseg; ++i) {
      const double2 p = segs[row * nseg_max + i];
      r = ms_merge(r, MS{(float)p.x, p.y});
    }
    s_lse2[tid] = r.s > 0.0 ? (double)r.m + log2(r.s) : -INFINITY;
  }
  __syncthreads();

  // accept tests, in order, up to the first rejection
  if (tid == 0) {
    int k = L;
    for (int t = 0; t < L; ++t) {
      const int64_t row = b * (L + 1) + t;
      int32_t x = path[b * L + t];
      float qx = 0.0f;
      for (int j = 0; j < kK; ++j)
        if (cand[(b * L + t) * kK + j] == x) qx = q[(b * L + t) * kK + j];
      x = x < 0 ? 0 : (x >= V ? (int32_t)(V - 1) : x);
      const float xs = logit_at<kBf16>(logits, row * V + x) * scale;
      const double p = exp2((double)xs - s_lse2[t]);
      uint32_t w[4];
      philox4x32_10(0u, (uint32_t)t, (uint32_t)b, 1u, k0, k1, w);
      if (!(uniform23(w[0]) < p / (double)qx)) {
        k = t;
        break;
      }
    }
    s_k = k;
  }
  __syncthreads();
  const int k = s_k;
  const int64_t row = b * (L + 1) + k;
  const void* rowp = kBf16 ? (const void*)(static_cast<const uint16_t*>(logits) + row * V)
                           : (const void*)(static_cast<const float*>(logits) + row * V);
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
  __syncthreads();
  if (tid == 0) {
    for (int j = 0; j < kK; ++j) {  // the residual's corrections, where they fall
      const int64_t cd = s_cand[j];
      if (cd < 0 || cd >= V) continue;
      const int64_t sg = cd < c.vb + kSeg ? 0 : (cd - c.vb) / kSeg < c.nseg ? (cd - c.vb) / kSeg
                                                                                : c.nseg - 1;
      s_mass[sg] -= s_corr[j];
    }
    double total = 0.0;
    for (int64_t sg = 0; sg < c.nseg; ++sg) total += s_mass[sg] > 0.0 ? s_mass[sg] : 0.0;
    uint32_t w[4];
    philox4x32_10(0u, (uint32_t)k, (uint32_t)b, 2u, k0, k1, w);
    const double u = ((double)(w[0] >> 9) * 0x1p23 + (double)(w[1] >> 9) + 0.5) * 0x1p-46;
    const double target = u * total;
    double cum = 0.0;
    int64_t pick = -1, last = 0;
    for (int64_t sg = 0; sg < c.nseg; ++sg) {
      const double m = s_mass[sg] > 0.0 ? s_mass[sg] : 0.0;
      if (m <= 0.0) continue;
      last = sg;
      if (cum + m >= target) {
        pick = sg;
        break;
      }
      cum += m;
    }
    if (pick < 0) {  // rounding past the end: the last segment with mass, from its end
      pick = last;
      cum = 1e300;
    }
    s_seg = (int)pick;
    s_rest = target - cum;
  }
  __syncthreads();
  // the segment, exactly: thread i sums its contiguous share of it in order
  int64_t lo, hi;
  seg_range(c, V, s_seg, lo, hi);
  const int64_t per = (hi - lo + kThreads - 1) / kThreads;
  auto weight = [&](int64_t v) {
    double wv = token_weight<kBf16>(rowp, v, scale, lse2);
#pragma unroll
    for (int j = 0; j < kK; ++j)
      if (s_cand[j] == v) wv -= s_corr[j];
    return wv > 0.0 ? wv : 0.0;
  };
  {
    const int64_t a = lo + tid * per < hi ? lo + tid * per : hi;
    const int64_t e = a + per < hi ? a + per : hi;
    double sum = 0.0;
    for (int64_t v = a; v < e; ++v) sum += weight(v);
    s_share[tid] = sum;
  }
  __syncthreads();
  if (tid == 0) {
    const double rest = s_rest;
    double cum = 0.0;
    int64_t pick = -1;
    int last_share = -1;
    for (int i = 0; i < kThreads && pick < 0; ++i) {
      if (s_share[i] <= 0.0) continue;
      last_share = i;
      if (cum + s_share[i] < rest) {
        cum += s_share[i];
        continue;
      }
      const int64_t a = lo + i * per < hi ? lo + i * per : hi;
      const int64_t e = a + per < hi ? a + per : hi;
      for (int64_t v = a; v < e; ++v) {
        const double wv = weight(v);
        if (wv <= 0.0) continue;
        cum += wv;
        if (cum >= rest) {
          pick = v;
          break;
        }
      }
    }
    if (pick < 0) {  // rounding past the end: the last token with weight
      pick = lo;
      if (last_share >= 0) {
        const int64_t a = lo + last_share * per < hi ? lo + last_share * per : hi;
        const int64_t e = a + per < hi ? a + per : hi;
        for (int64_t v = e - 1; v >= a; --v)
          if (weight(v) > 0.0) {
            pick = v;
            break;
          }
      }
    }
    out_accepted[b] = k;
    out_token[b] = (int32_t)pick;
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
  // workgroups per row: enough rows x parts to fill the chip, four segments apiece at least
  int64_t parts = 1;
  if (rows < kTargetBlocks) {
    parts = cdiv(kTargetBlocks, rows);
    const int64_t maxp = cdiv(p.nseg, kWaves);
    if (parts > maxp) parts = maxp;
  }
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
