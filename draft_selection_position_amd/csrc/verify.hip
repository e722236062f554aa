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
// only vocabulary-wide pass): each workgroup keeps a running (max, sum of 2^(x -
// max)) of x = z log2(e) / T per thread, merged across the wave with DPP and across
// waves through LDS, for a row or a chunk of one.  verify_kernel takes one block per
// workgroup: it merges the chunks into log2-sum-exp per row, runs the accept tests
// (fp64 ratio against a 23-bit Philox uniform), and draws the output token by
// inverse CDF with a 46-bit Philox uniform: every thread sums its contiguous share
// of the row's weights (as 64 sub-ranges), thread 0 finds the share and the
// sub-range the target mass falls in, and the exact token is found inside that
// sub-range.  The 16 candidates' corrections min(p, q) are subtracted where they
// fall, so the residual never needs a per-element candidate test outside the last
// sub-range.
#include "dfs_device.h"
#include "dfs_internal.h"
#include "philox.h"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;           // 16-byte vectors per thread per iteration
constexpr int kMinChunk = 4096;      // elements; below this a split does not pay
constexpr int kSub = 64;             // sub-ranges per thread share (inverse CDF)
constexpr int kMaxL = 16;            // longest block
constexpr float kLog2e = 1.4426950408889634f;

// Running maximum and sum of 2^(x - max).  An empty pair is (-inf, 0).
struct MS {
  float m, s;
};

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return MS{m, 0.0f};
  return MS{m, a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m)};
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
  float s = a.s * exp2f(a.m - m);
#pragma unroll
  for (int e = 0; e < PV; ++e) s += exp2f(x[e] - m);
  a = MS{m, s};
}

__device__ __forceinline__ void ms_add(MS& a, float z, float scale) {
  const float x = z * scale;
  const float m = fmaxf(a.m, x);
  if (m == -INFINITY) return;
  a = MS{m, a.s * exp2f(a.m - m) + exp2f(x - m)};
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
constexpr int kCacheNonTemporal = 2;

// (max, sum) of x = z * scale over chunk `part` of row `row`, one pair per workgroup.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_kernel(const void* __restrict__ logits, int64_t V,
                                                       int parts, int64_t chunk, float scale,
                                                       float2* __restrict__ partial) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int PV = kBf16 ? 8 : 4;
  __shared__ MS s_w[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t row = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const T* rowp = static_cast<const T*>(logits) + row * V;
  const int64_t beg = (int64_t)part * chunk;
  const int64_t end = beg + chunk < V ? beg + chunk : V;

  // [vb, ve): the 16-byte aligned middle of the chunk; the rest goes element by element
  const uintptr_t a_beg = (uintptr_t)(rowp + beg);
  int64_t vb = beg + (int64_t)(((16u - (a_beg & 15u)) & 15u) / sizeof(T));
  if (vb > end) vb = end;
  const int64_t nvec = (end - vb) / PV;
  const int64_t ve = vb + nvec * PV;

  MS acc{-INFINITY, 0.0f};
  for (int64_t i = beg + tid; i < vb; i += kThreads) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
  for (int64_t i = ve + tid; i < end; i += kThreads) ms_add(acc, logit_at<kBf16>(rowp, i), scale);
  if (nvec > 0) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(rowp + vb), (short)0, (int)(nvec * 16), kRawBufferWord3);
    const int64_t step = (int64_t)kThreads * kUnroll;
    for (int64_t base = 0; base < nvec; base += step) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t vid = (uint32_t)(base + u * kThreads + tid);
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, vid * 16u, 0, kCacheNonTemporal);
        v[u] = make_uint4(w.x, w.y, w.z, w.w);  // past the end: zeros, skipped below
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kThreads + tid < nvec) ms_add_vec<kBf16>(acc, v[u], scale);
    }
  }
  // across the wave (lane 0's result), then across the waves in order
#pragma unroll
  for (int k = 1; k < kWave; k <<= 1) {
    const MS o{__uint_as_float(xor_lanes(__float_as_uint(acc.m), k, lane)),
               __uint_as_float(xor_lanes(__float_as_uint(acc.s), k, lane))};
    acc = ms_merge(acc, o);
  }
  if (lane == 0) s_w[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    MS r = s_w[0];
    for (int w = 1; w < kWaves; ++w) r = ms_merge(r, s_w[w]);
    partial[blockIdx.x] = make_float2(r.m, r.s);
  }
}

// Target probability of token v in row `rowp`: 2^(x - log2-sum-exp), fp32 exp2 of
// the fp32-scaled logit (the residual of a candidate subtracts min(p, q) from it).
template <bool kBf16>
__device__ __forceinline__ double token_weight(const void* rowp, int64_t v, float scale, double lse2) {
  return (double)exp2f((float)(logit_at<kBf16>(rowp, v) * scale - (float)lse2));
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const void* __restrict__ logits, int64_t V, int L, int parts, float scale,
    const float2* __restrict__ partial, const int32_t* __restrict__ path,
    const int32_t* __restrict__ cand, const float* __restrict__ q, uint64_t seed,
    int32_t* __restrict__ out_accepted, int32_t* __restrict__ out_token) {
  __shared__ double s_lse2[kMaxL + 1];
  __shared__ int32_t s_cand[kK];
  __shared__ double s_corr[kK];
  __shared__ double s_share[kThreads];
  __shared__ double s_sub[kSub];
  __shared__ int s_k, s_share_idx, s_sub_idx;
  __shared__ double s_rest;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);

  // log2-sum-exp of rows (b, 0..L), chunks merged in order
  if (tid <= L) {
    const float2* p = partial + ((b * (L + 1)) + tid) * parts;
    MS r{-INFINITY, 0.0f};
    for (int i = 0; i < parts; ++i) r = ms_merge(r, MS{p[i].x, p[i].y});
    s_lse2[tid] = r.s > 0.0f ? (double)r.m + log2((double)r.s) : -INFINITY;
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
  if (tid < kK) {
    int32_t c = -1;
    double corr = 0.0;
    if (k < L) {
      c = cand[(b * L + k) * kK + tid];
      const int32_t cc = c < 0 ? 0 : (c >= V ? (int32_t)(V - 1) : c);
      const double p = token_weight<kBf16>(rowp, cc, scale, lse2);
      const double qc = (double)q[(b * L + k) * kK + tid];
      corr = p < qc ? p : qc;  // min(p, q): what the residual takes off token c
    }
    s_cand[tid] = c;
    s_corr[tid] = corr;
  }
  __syncthreads();

  // Thread i's share [i R, (i + 1) R) as kSub sub-ranges of R2 tokens, summed in
  // order; the same sums are rebuilt below for the share the draw falls in.
  const int64_t R = (V + kThreads - 1) / kThreads;
  const int64_t R2 = (R + kSub - 1) / kSub;
  auto sub_sum = [&](int64_t lo, int64_t hi) {
    double s = 0.0;
    for (int64_t v = lo; v < hi; ++v) s += token_weight<kBf16>(rowp, v, scale, lse2);
    for (int j = 0; j < kK; ++j) {
      const int64_t c = s_cand[j];
      if (c >= lo && c < hi) s -= s_corr[j];
    }
    return s;
  };
  {
    const int64_t lo = tid * R;
    double share = 0.0;
    for (int u = 0; u < kSub; ++u) {
      int64_t a = lo + u * R2, e = a + R2;
      const int64_t hi_share = lo + R < V ? lo + R : V;
      if (a > hi_share) a = hi_share;
      if (e > hi_share) e = hi_share;
      share += sub_sum(a, e);
    }
    s_share[tid] = share;
  }
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
    for (int i = 0; i < kThreads; ++i) total += s_share[i];
    uint32_t w[4];
    philox4x32_10(0u, (uint32_t)k, (uint32_t)b, 2u, k0, k1, w);
    const double u = ((double)(w[0] >> 9) * 0x1p23 + (double)(w[1] >> 9) + 0.5) * 0x1p-46;
    double target = u * total, cum = 0.0;
    int idx = -1;
    for (int i = 0; i < kThreads; ++i) {
      if (s_share[i] > 0.0 && cum + s_share[i] >= target) {
        idx = i;
        break;
      }
      cum += s_share[i];
    }
    if (idx < 0) {  // rounding past the end: the last share with weight
      for (int i = kThreads - 1; i >= 0; --i)
        if (s_share[i] > 0.0) {
          idx = i;
          break;
        }
      target = cum;
      cum -= idx >= 0 ? s_share[idx] : 0.0;
    }
    s_share_idx = idx < 0 ? 0 : idx;
    s_rest = target - cum;
  }
  __syncthreads();
  const int64_t lo = s_share_idx * R;
  const int64_t hi_share = lo + R < V ? lo + R : V;
  if (tid < kSub) {
    int64_t a = lo + tid * R2, e = a + R2;
    if (a > hi_share) a = hi_share;
    if (e > hi_share) e = hi_share;
    s_sub[tid] = sub_sum(a, e);
  }
  __syncthreads();
  if (tid == 0) {
    double rest = s_rest, cum = 0.0;
    int idx = -1;
    for (int u = 0; u < kSub; ++u) {
      if (s_sub[u] > 0.0 && cum + s_sub[u] >= rest) {
        idx = u;
        break;
      }
      cum += s_sub[u];
    }
    if (idx < 0) {
      for (int u = kSub - 1; u >= 0; --u)
        if (s_sub[u] > 0.0) {
          idx = u;
          break;
        }
      if (idx < 0) idx = 0;
      rest = 1e300;  // take the last token with weight in it
      cum = 0.0;
    }
    int64_t a = lo + idx * R2, e = a + R2;
    if (a > hi_share) a = hi_share;
    if (e > hi_share) e = hi_share;
    rest -= cum;
    int64_t pick = -1, last = -1;
    double run = 0.0;
    for (int64_t v = a; v < e; ++v) {
      double wv = token_weight<kBf16>(rowp, v, scale, lse2);
      for (int j = 0; j < kK; ++j)
        if (s_cand[j] == v) wv -= s_corr[j];
      if (wv > 0.0) {
        last = v;
        run += wv;
        if (run >= rest) {
          pick = v;
          break;
        }
      }
    }
    if (pick < 0) pick = last >= 0 ? last : a;
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
  const int64_t pv = 16 / esize;
  int64_t parts = 1;
  if (rows < kTargetBlocks) {
    parts = cdiv(kTargetBlocks, rows);
    int64_t maxp = V / kMinChunk;
    if (maxp < 1) maxp = 1;
    if (parts > maxp) parts = maxp;
    if (parts > 64) parts = 64;
  }
  // a chunk's byte range must fit the 32-bit range of its buffer resource
  const int64_t min_parts = cdiv(V * esize, ((int64_t)1 << 31) - 256);
  if (parts < min_parts) parts = min_parts;
  const int64_t chunk = (int64_t)align_up((size_t)cdiv(V, parts), (size_t)pv);
  p.parts = (int)cdiv(V, chunk);
  p.chunk = chunk;
  p.ws_bytes = align_up((size_t)rows * p.parts * sizeof(float2), 256);
  return p;
}

hipError_t launch_verify(const VerifyPlan& p, const void* logits, bool bf16, const int32_t* path,
                         const int32_t* cand, const float* q, double temperature, uint64_t seed,
                         void* ws, int32_t* out_accepted, int32_t* out_token, hipStream_t stream) {
  float2* partial = static_cast<float2*>(ws);
  const float scale = (float)((double)kLog2e / temperature);
  const int64_t rows = p.batch * (p.L + 1);
  const dim3 grid((unsigned)(rows * p.parts));
  if (bf16) {
    lse_kernel<true><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.chunk, scale, partial);
    verify_kernel<true><<<dim3((unsigned)p.batch), kThreads, 0, stream>>>(
        logits, p.V, (int)p.L, p.parts, scale, partial, path, cand, q, seed, out_accepted, out_token);
  } else {
    lse_kernel<false><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.chunk, scale, partial);
    verify_kernel<false><<<dim3((unsigned)p.batch), kThreads, 0, stream>>>(
        logits, p.V, (int)p.L, p.parts, scale, partial, path, cand, q, seed, out_accepted, out_token);
  }
  return hipGetLastError();
}

}  // namespace dfs
