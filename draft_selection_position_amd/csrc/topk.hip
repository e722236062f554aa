// Vocabulary-wide top-16 per row in one streaming pass over the logits.
//
// DFlash 2 keeps the 16 best candidates of each block position instead of only
// the top one (blog post "DFlash 2: Keep Drafting Parallel", section "The Right
// Tokens Are Already There").  The order is value descending, then token id
// ascending; -0 equals +0.
//
// Design (gfx950): the pass is HBM-bound, so each workgroup (4 waves) streams a
// row chunk with 16-byte coalesced non-temporal loads, the next iteration's
// vectors in flight while the current ones are scanned.  An element is only looked at
// further when it reaches the wave's admission threshold (which starts at a bound taken
// over the wave's first iteration); admitted elements are appended to a per-wave
// LDS buffer as exact 64-bit (value, index) keys, placed by one ballot when no lane holds
// more than one of a vector's admitted elements, else by a prefix count of every lane's
// admissions (chunks held whole in registers: one prefix count for all of a lane's elements),
// and the buffer is merged into the wave's sorted top-16 (held in lanes 0..15) by a
// 64-lane bitonic sort.  The 16th best key of any wave is a valid threshold for the
// whole chunk and is shared through LDS (in launches of two rounds, the bound over all
// four waves' lists).  The four wave lists are merged at the end; rows split over
// several workgroups are merged by a second kernel or by the kernel that reads them.
// Every comparison is on exact integer keys, so the result does not depend on the order
// in which elements are seen.
#include <type_traits>

#include "dfs_device.h"
#include "dfs_internal.h"
#include "gate_pack.h"
#include "gate_tile.h"
#include "topk_merge.h"

namespace dfs {
namespace {

// Tuning knobs (compile-time); the defaults are the measured best on MI355X at
// 4096 rows x 151936 bf16: three 16-byte vectors per thread per iteration (plus
// the next two in flight), registers capped for 8 waves per SIMD (exactly two
// rounds of workgroups, no ragged tail) and non-temporal loads, which keep the
// streamed logits from displacing anything in the caches.
#ifndef DFS_TOPK_UNROLL
#define DFS_TOPK_UNROLL 3
#endif
#ifndef DFS_TOPK_WAVES_PER_EU
#define DFS_TOPK_WAVES_PER_EU 8
#endif
#ifndef DFS_TOPK_NONTEMPORAL
#define DFS_TOPK_NONTEMPORAL 1
#endif
// Rows are split into chunks (merged afterwards) only while there are fewer than this
// many workgroups: few long-streaming workgroups beat many short ones (at 512 rows one
// workgroup per row took 38 us against 48 us split four ways; 16 rows run 16 ways).
#ifndef DFS_TOPK_TARGET_BLOCKS
#define DFS_TOPK_TARGET_BLOCKS 256
#endif
// Where packing jobs riding along go in the grid: 1 = first, 0 = last (in the tail).
#ifndef DFS_TOPK_PACK_FIRST
#define DFS_TOPK_PACK_FIRST 0
#endif

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = DFS_TOPK_UNROLL;  // 16-byte vectors per thread per iteration
// A wave merges its buffered keys into its list once more than kMergeAt are waiting: one
// 64-lane sort then takes the list and all of them, and the threshold it raises follows
// the stream closely (64 waiting keys took two sorts per merge and let more keys in:
// 40 measured 3.3 us faster at 512 rows x 151936, 2 us at 1024 x 262144, 1.5 us at 4096).
#ifndef DFS_TOPK_MERGE_AT
#define DFS_TOPK_MERGE_AT 40
#endif
constexpr int kMergeAt = DFS_TOPK_MERGE_AT;
constexpr int kCap = kMergeAt + 8 * kWave;  // room for one whole vector per lane on top
constexpr int kMinChunk = 4096;   // elements; below this a split does not pay
constexpr int kMinSmallChunk = 1024;  // the same for the few-row plan
// The merge sorts as inlined code (false) or as calls of one out-of-line copy (true), in
// the pass over whole rows or chunks and in the launch that carries the gate's tiles:
// merges are rare next to the scan, and one copy keeps the scan loop's code compact
// (0.2-0.9 us faster at 512-4096 rows).
#ifndef DFS_TOPK_CHUNK_COMPACT
#define DFS_TOPK_CHUNK_COMPACT true
#endif
#ifndef DFS_TOPK_GATE_COMPACT
#define DFS_TOPK_GATE_COMPACT true
#endif
// Each wave's threshold starts from a bound taken over its whole first iteration.  When
// all the pass's workgroups fit one round on the chip (256 CUs x 8 workgroups at 8 waves
// per SIMD), a barrier then lets every wave start from the best bound of its workgroup:
// every workgroup starts at once and the early threshold saves admissions (1024 rows x
// 262144: -1.8 us, 512 rows x 151936: -0.8 us); with two rounds (4096 rows) the barrier
// costs more than it saves (+1.8 us).
constexpr int64_t kWideSeedMaxBlocks = 2048;
// Launches of more than one round also raise the shared threshold to the bound over all
// four waves' lists at every merge (wave_merge): fewer admissions where the VALU is busy.
#ifndef DFS_TOPK_UNION
#define DFS_TOPK_UNION 1
#endif
// Admissions of one vector step: a bit mask per lane and one ballot for the usual case of
// at most one passing element per lane (1), or one ballot per element slot (0).
#ifndef DFS_TOPK_APPEND_BATCHED
#define DFS_TOPK_APPEND_BATCHED 1
#endif
// Few rows: workgroups the split aims for.
#ifndef DFS_TOPK_SMALL_TARGET_BLOCKS
#define DFS_TOPK_SMALL_TARGET_BLOCKS 64
#endif

template <bool kBf16>
struct Elems;
template <>
struct Elems<true> {
  static constexpr int per_vec = 8;
  using T = uint16_t;
};
template <>
struct Elems<false> {
  static constexpr int per_vec = 4;
  using T = float;
};

struct WaveTop {
  uint64_t list;  // lanes 0..15: best keys so far, descending (0 = empty slot)
  float thr;      // admission threshold, identical in every lane
  int cnt;        // keys waiting in the buffer, identical in every lane
};

// Out-of-line copy of the 64-lane sort for the compact build of the pass: merges are
// rare next to the scan, so one copy called from every merge keeps the scan's code
// small.
__device__ __attribute__((noinline)) uint64_t wave_sort_desc_call(uint64_t x, int lane) {
  return wave_sort_desc(x, lane);
}
template <bool kCompact>
__device__ __forceinline__ uint64_t sort_desc(uint64_t x, int lane) {
  if constexpr (kCompact) {
    return wave_sort_desc_call(x, lane);
  } else {
    return wave_sort_desc(x, lane);
  }
}

// The workgroup's shared words: s_thr[0] is the chunk's admission threshold key (0: none
// yet), s_thr[1 + 16 w + j] the value key of slot j of wave w's list as of its last merge.
// A slot's value never falls (each merge keeps the top 16 of a larger set), so from any
// mix of old and new words wave w holds at least j + 1 elements at or above word j; the
// waves see disjoint elements, so the 16th largest of the 64 words has 16 distinct
// elements of the chunk at or above it, whatever the other waves are doing meanwhile.
constexpr int kThrWords = 1 + kWaves * kK;

// That 16th largest word (lane l reads word 1 + l): one out-of-line copy, as merges are
// rare and the search is long.
__device__ __attribute__((noinline)) uint32_t union_bound(uint32_t* s_thr, int lane) {
  return wave_16th_largest(
      __hip_atomic_load(&s_thr[1 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// Merge the buffered keys into the wave's list and raise the threshold (kCompact: the
// out-of-line sort; kUnion: also publish the list's values and raise the threshold to the
// bound over all four waves' lists, which pays where the pass is short of issue slots,
// with eight waves per SIMD, and not where a wave's merges are on its own critical path).
template <bool kCompact, bool kUnion>
__device__ __forceinline__ void wave_merge(WaveTop& w, const uint64_t* buf, uint32_t* s_thr,
                                           int lane) {
  __builtin_amdgcn_wave_barrier();
  int cnt = w.cnt;
  while (cnt > 0) {
    const int n = cnt < 48 ? cnt : 48;
    uint64_t x = 0;
    if (lane < 16) {
      x = w.list;
    } else if (lane - 16 < n) {
      x = buf[cnt - n + (lane - 16)];
    }
    x = sort_desc<kCompact>(x, lane);
    w.list = lane < 16 ? x : 0;
    cnt -= n;
  }
  w.cnt = 0;
  __builtin_amdgcn_wave_barrier();
  const uint64_t k16 = lane_u64(w.list, 15);
  uint32_t bound = (uint32_t)(k16 >> 32);
  if constexpr (kUnion) {
    if (lane < kK) s_thr[1 + (threadIdx.x / kWave) * kK + lane] = (uint32_t)(w.list >> 32);
    const uint32_t u = (uint32_t)uniform((int)union_bound(s_thr, lane));
    bound = u > bound ? u : bound;
  }
  if (bound != 0) {
    uint32_t m = bound;
    uint32_t old = 0;
    if (lane == 0) old = atomicMax(s_thr, m);
    old = (uint32_t)__builtin_amdgcn_readlane((int)old, 0);
    m = m > old ? m : old;
    w.thr = uniformf(unmono32(m));
  }
}


// Append this lane's element to the wave buffer when `adm`.
__device__ __forceinline__ void append(WaveTop& w, bool adm, float v, uint32_t idx,
                                       uint64_t* buf) {
  const uint64_t mask = __ballot(adm);
  if (mask == 0) return;
  const int pos = w.cnt + lanes_below(mask);
  if (adm) buf[pos] = make_key(v, idx);
  w.cnt = uniform(w.cnt + __popcll(mask));
}

// 16-byte loads of the chunk's aligned middle go through a buffer resource (base
// and size in scalar registers, 32-bit byte offset per lane): fewer per-lane
// registers than 64-bit pointers, and the hardware range check returns zeros
// instead of touching memory past the end (those vectors are flagged invalid).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9-family raw (untyped) buffer
constexpr int kCacheNonTemporal = 2;         // "nt": stream through, do not keep
__device__ __forceinline__ uint4 load_vec(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, byte_off, 0,
                                                        DFS_TOPK_NONTEMPORAL ? kCacheNonTemporal : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool kBf16>
__device__ __forceinline__ float load_scalar(const typename Elems<kBf16>::T* p, int64_t i) {
  if constexpr (kBf16) {
    return bf16_to_f32(p[i]);
  } else {
    return p[i];
  }
}

// The largest of one 16-byte vector's elements (NaN, which fmaxf ignores, when invalid).
template <bool kBf16>
__device__ __forceinline__ float vec_max(uint4 d, bool valid) {
  if (!valid) return __int_as_float(0x7fffffff);
  if constexpr (kBf16) {
    return fmaxf(fmaxf(fmaxf(bf16_lo(d.x), bf16_hi(d.x)), fmaxf(bf16_lo(d.y), bf16_hi(d.y))),
                 fmaxf(fmaxf(bf16_lo(d.z), bf16_hi(d.z)), fmaxf(bf16_lo(d.w), bf16_hi(d.w))));
  } else {
    return fmaxf(fmaxf(__uint_as_float(d.x), __uint_as_float(d.y)), fmaxf(__uint_as_float(d.z), __uint_as_float(d.w)));
  }
}

// Admission test and append for one 16-byte vector (8 bf16 or 4 fp32 values),
// then a merge if the buffer has filled past kMergeAt.  A vector past the end of
// the chunk (`valid` false) is replaced by NaNs, which never pass.
template <bool kBf16, bool kCompact, bool kUnion>
__device__ __forceinline__ void scan_vec(uint4 d, bool valid, uint32_t idx0, WaveTop& w,
                                         uint64_t* buf, uint32_t* s_thr, int lane) {
  constexpr int PV = Elems<kBf16>::per_vec;
  if (!valid) d = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
  float v[PV];
  if constexpr (kBf16) {
    v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
    v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
    v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
    v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
  } else {
    v[0] = __uint_as_float(d.x); v[1] = __uint_as_float(d.y);
    v[2] = __uint_as_float(d.z); v[3] = __uint_as_float(d.w);
  }
  // fmaxf ignores NaN, so padding lanes (all-NaN) never pass.
  float m = v[0];
#pragma unroll
  for (int e = 1; e < PV; ++e) m = fmaxf(m, v[e]);
  if (__ballot(m >= w.thr) == 0) return;
#if DFS_TOPK_APPEND_BATCHED
  // Each lane's passing elements as a bit mask.  Typically every lane that passes holds
  // one passing element, which is then its maximum m: one ballot places all of them.
  // Otherwise a lane's count is summed over the lanes below it with one ballot per count
  // bit, and each lane appends its elements in order.
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < PV; ++e) bits |= (v[e] >= w.thr ? 1u : 0u) << e;
  if (__ballot(bits & (bits - 1u)) == 0) {
    const uint64_t mask = __ballot(bits != 0u);
    if (bits != 0u) buf[w.cnt + lanes_below(mask)] = make_key(m, idx0 + (uint32_t)__builtin_ctz(bits));
    w.cnt = uniform(w.cnt + __popcll(mask));
  } else {
    const int c = __popc(bits);
    int pos = w.cnt, tot = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= PV; ++b) {
      const uint64_t mb = __ballot((c >> b) & 1);
      pos += lanes_below(mb) << b;
      tot += __popcll(mb) << b;
    }
#pragma unroll
    for (int e = 0; e < PV; ++e)
      if ((bits >> e) & 1u) buf[pos++] = make_key(v[e], idx0 + e);
    w.cnt = uniform(w.cnt + tot);
  }
#else
#pragma unroll
  for (int e = 0; e < PV; ++e) append(w, v[e] >= w.thr, v[e], idx0 + e, buf);
#endif
  if (w.cnt > kMergeAt) wave_merge<kCompact, kUnion>(w, buf, s_thr, lane);
}

struct TopkLds {
  uint64_t buf[kWaves][kCap];  // per-wave key buffers
  uint64_t list[kWaves * kK];
  uint32_t thr[kThrWords];     // the chunk's threshold and the waves' published list values
};
static_assert(sizeof(TopkLds::buf) >= kPackLdsBytes, "a packing job reuses the key buffers");
static_assert(sizeof(TopkLds::buf) >= gtile::kF32LdsBytes, "a gate job reuses the key buffers");

// One (row, part) of the pass: workgroup `bid` of the rows.  kCompact: the sorts are
// out-of-line calls (few rows: each wave runs the code about once).  kU: 16-byte vectors
// per thread per iteration (two iterations in flight).
template <bool kBf16, bool kCompact, bool kWide, bool kUnion, int kU = kUnroll>
__device__ __forceinline__ void topk_body(const void* __restrict__ logits, int64_t V, int parts, int64_t chunk,
                                          uint64_t* __restrict__ partial, int32_t* __restrict__ out_idx,
                                          float* __restrict__ out_val, int64_t bid, TopkLds& lds) {
  using T = typename Elems<kBf16>::T;
  constexpr int PV = Elems<kBf16>::per_vec;
  auto& s_buf = lds.buf;
  auto& s_list = lds.list;
  uint32_t* s_thr = lds.thr;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t row = bid / parts;
  const int part = (int)(bid % parts);
  const T* rowp = static_cast<const T*>(logits) + row * V;
  const int64_t beg = (int64_t)part * chunk;
  const int64_t end = beg + chunk < V ? beg + chunk : V;

  if (tid < kThrWords) s_thr[tid] = 0u;
  __syncthreads();

  uint64_t* buf = s_buf[wave];
  WaveTop w;
  w.list = 0;
  w.thr = -INFINITY;
  w.cnt = 0;

  // [vb, ve) is the 16-byte aligned middle of the chunk; the rest is scalar.
  const uintptr_t a_beg = (uintptr_t)(rowp + beg);
  int64_t vb = beg + (int64_t)(((16u - (a_beg & 15u)) & 15u) / sizeof(T));
  if (vb > end) vb = end;
  const int64_t nvec = (end - vb) / PV;
  const int64_t ve = vb + nvec * PV;

  if (wave == 0) {
    const int nhead = (int)(vb - beg);
    const int ntail = (int)(end - ve);
    int64_t i = -1;
    if (lane < nhead) {
      i = beg + lane;
    } else if (lane < nhead + ntail) {
      i = ve + (lane - nhead);
    }
    float v = 0.0f;
    if (i >= 0) v = load_scalar<kBf16>(rowp, i);
    append(w, i >= 0 && v >= w.thr, v, (uint32_t)i, buf);  // at most 14 keys
  }

  // Main loop.  Every iteration issues the next iteration's loads before scanning
  // the current vectors; the loads are unconditional (vectors past the end come
  // back as zeros and are flagged invalid) and the two register buffers alternate
  // (no copies), so the compiler waits for exactly the vectors it is about to scan
  // and leaves the next ones in flight.
  const int64_t step = (int64_t)kThreads * kU;
  const int64_t niter = (nvec + step - 1) / step;
  if (niter > 0) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(rowp + vb), (short)0, (int)(nvec * 16), kRawBufferWord3);
    uint4 bufA[kU], bufB[kU];
    auto load_iter = [&](uint4* dst, int64_t it) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t vid = (uint32_t)(it * step) + (uint32_t)(u * kThreads + tid);
        dst[u] = load_vec(rsrc, vid * 16u);  // past the end: zeros, flagged invalid below
      }
    };
    // kCheck false: every vector of the iteration lies inside the chunk (no range test)
    auto scan_iter = [&](const uint4* src, int64_t it, auto kCheck) {
      {  // other waves may have raised the chunk's threshold
        const uint32_t m = uniform(
            (int)__hip_atomic_load(s_thr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (m != 0u) {
          const float t = unmono32(m);
          if (t > w.thr) w.thr = uniformf(t);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t vid = it * step + (int64_t)u * kThreads + tid;
        scan_vec<kBf16, kCompact, kUnion>(src[u], !decltype(kCheck)::value || vid < nvec, (uint32_t)(vb + vid * PV),
                                          w, buf, s_thr, lane);
      }
    };
    constexpr std::false_type kInside{};
    constexpr std::true_type kEdge{};
    const int64_t nfull = nvec / step;  // iterations with every vector inside the chunk
    load_iter(bufA, 0);
    {
      // The 16th-largest lane maximum over the wave's first iteration bounds the chunk's
      // top 16 (every lane maximum is a distinct element): the wave's threshold starts
      // there, and the largest such bound of the four waves is shared through LDS (with
      // a barrier when every wave should start from it, see kWideSeedMaxBlocks).
      float m = __int_as_float(0x7fffffff);
#pragma unroll
      for (int u = 0; u < kU; ++u) m = fmaxf(m, vec_max<kBf16>(bufA[u], (int64_t)u * kThreads + tid < nvec));
      const uint32_t k16 = wave_16th_largest(m == m ? mono32(m) : 0u);
      if (k16 != 0u) {
        const float t = unmono32(k16);
        if (t > w.thr) w.thr = uniformf(t);
        if (lane == 0) atomicMax(s_thr, k16);
      }
      if constexpr (kWide) __syncthreads();
    }
    int64_t it = 0;
    // bufA holds iteration `it` at the top of each loop; no exit in the middle of an
    // iteration pair, so the compiler's load waits stay exact
    for (; it + 2 <= nfull; it += 2) {
      load_iter(bufB, it + 1);
      scan_iter(bufA, it, kInside);
      load_iter(bufA, it + 2);
      scan_iter(bufB, it + 1, kInside);
    }
    for (; it + 2 <= niter; it += 2) {  // at most once: the last iteration may be ragged
      load_iter(bufB, it + 1);
      scan_iter(bufA, it, kEdge);
      load_iter(bufA, it + 2);
      scan_iter(bufB, it + 1, kEdge);
    }
    if (it < niter) scan_iter(bufA, it, kEdge);  // odd count: bufA holds the last iteration
  }

  if (w.cnt > 0) wave_merge<kCompact, false>(w, buf, s_thr, lane);
  if (lane < kK) s_list[wave * kK + lane] = w.list;
  __syncthreads();
  if (wave == 0) {
    const uint64_t x = wave_merge_runs16(s_list[lane], lane);  // the four waves' sorted lists
    if (lane < kK) {
      if (parts == 1) {
        out_idx[row * kK + lane] = (int32_t)key_index(x);
        out_val[row * kK + lane] = key_value(x);
      } else {
        partial[(row * parts + part) * kK + lane] = x;
      }
    }
  }
}

// Few rows: a chunk of at most kSmallVecs vectors per thread is loaded whole before any
// compare.  Every lane's maximum over its vectors is a distinct element, so the 16th
// largest lane maximum of any wave bounds the chunk's top 16; the largest such bound over
// the four waves (shared through LDS) is the admission threshold from the start.  A
// bitwise search over ballots finds it, typically one sort merges the admitted keys, and
// a merge of four sorted runs joins the wave lists: the critical path of a workgroup that
// runs this code once.
#ifndef DFS_TOPK_SMALL_VECS
#define DFS_TOPK_SMALL_VECS 6
#endif
#ifndef DFS_TOPK_SMALL_BATCHED
#define DFS_TOPK_SMALL_BATCHED 1
#endif
// The batched append walks each lane's set bits only (1) or every element slot (0):
// 16 x 151936 16.4 -> 15.7 us per dfs_select.
#ifndef DFS_TOPK_SMALL_BITLOOP
#define DFS_TOPK_SMALL_BITLOOP 1
#endif
constexpr int kSmallVecs = DFS_TOPK_SMALL_VECS;

template <bool kBf16>
__device__ __forceinline__ void topk_small_body(const void* __restrict__ logits, int64_t V, int parts, int64_t chunk,
                                                uint64_t* __restrict__ partial, int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_val, int64_t bid, TopkLds& lds) {
  using T = typename Elems<kBf16>::T;
  constexpr int PV = Elems<kBf16>::per_vec;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t row = bid / parts;
  const int part = (int)(bid % parts);
  const T* rowp = static_cast<const T*>(logits) + row * V;
  const int64_t beg = (int64_t)part * chunk;
  const int64_t end = beg + chunk < V ? beg + chunk : V;
  const uintptr_t a_beg = (uintptr_t)(rowp + beg);
  int64_t vb = beg + (int64_t)(((16u - (a_beg & 15u)) & 15u) / sizeof(T));
  if (vb > end) vb = end;
  const int64_t nvec = (end - vb) / PV;
  const int64_t ve = vb + nvec * PV;
  if (tid == 0) lds.thr[0] = 0u;

  uint4 d[kSmallVecs];
  if (nvec > 0) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(rowp + vb), (short)0, (int)(nvec * 16), kRawBufferWord3);
#pragma unroll
    for (int u = 0; u < kSmallVecs; ++u) d[u] = load_vec(rsrc, (uint32_t)(u * kThreads + tid) * 16u);
  }
  // the head and tail elements outside the aligned middle (at most 14), one per lane of wave 0
  const int nhead = (int)(vb - beg);
  const int ntail = (int)(end - ve);
  int64_t hi = -1;
  if (wave == 0) {
    if (lane < nhead) {
      hi = beg + lane;
    } else if (lane < nhead + ntail) {
      hi = ve + (lane - nhead);
    }
  }
  const float hv = hi >= 0 ? load_scalar<kBf16>(rowp, hi) : 0.0f;

  // lane maxima (vectors past the chunk read as NaN, which fmaxf ignores)
  float m = hi >= 0 ? hv : __int_as_float(0x7fffffff);
#pragma unroll
  for (int u = 0; u < kSmallVecs; ++u) {
    if ((int64_t)(u * kThreads + tid) >= nvec) d[u] = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
    if constexpr (kBf16) {
      m = fmaxf(m, fmaxf(fmaxf(fmaxf(bf16_lo(d[u].x), bf16_hi(d[u].x)), fmaxf(bf16_lo(d[u].y), bf16_hi(d[u].y))),
                         fmaxf(fmaxf(bf16_lo(d[u].z), bf16_hi(d[u].z)), fmaxf(bf16_lo(d[u].w), bf16_hi(d[u].w)))));
    } else {
      m = fmaxf(m, fmaxf(fmaxf(__uint_as_float(d[u].x), __uint_as_float(d[u].y)),
                         fmaxf(__uint_as_float(d[u].z), __uint_as_float(d[u].w))));
    }
  }
  __syncthreads();  // threshold cleared
  {
    const uint32_t k16 = wave_16th_largest(m == m ? mono32(m) : 0u);
    if (k16 != 0u && lane == 0) atomicMax(lds.thr, k16);
  }
  __syncthreads();
  uint64_t* buf = lds.buf[wave];
  WaveTop w;
  w.list = 0;
  w.cnt = 0;
  const uint32_t t0 = lds.thr[0];
  w.thr = t0 != 0u ? unmono32(t0) : -INFINITY;
  append(w, hi >= 0 && hv >= w.thr, hv, (uint32_t)hi, buf);  // at most 14 keys
  // Every element of the lane's vectors at or above the threshold goes to the buffer in one
  // pass: a lane's count is summed over the lanes below it with one ballot per count bit,
  // which places its keys (vectors past the chunk hold NaNs and never pass).  Inputs that
  // pass more keys than the buffer holds take the vector-by-vector scan instead.
  bool scanned = false;
#if DFS_TOPK_SMALL_BATCHED
  {
    auto elem = [&](int u, int e) -> float {
      if constexpr (kBf16) {
        const uint32_t word = (e >> 1) == 0 ? d[u].x : (e >> 1) == 1 ? d[u].y : (e >> 1) == 2 ? d[u].z : d[u].w;
        return (e & 1) ? bf16_hi(word) : bf16_lo(word);
      } else {
        return __uint_as_float(e == 0 ? d[u].x : e == 1 ? d[u].y : e == 2 ? d[u].z : d[u].w);
      }
    };
    uint32_t bits[kSmallVecs];
    int c = 0;
#pragma unroll
    for (int u = 0; u < kSmallVecs; ++u) {
      bits[u] = 0;
#pragma unroll
      for (int e = 0; e < PV; ++e) bits[u] |= (elem(u, e) >= w.thr ? 1u : 0u) << e;
      c += __popc(bits[u]);
    }
    int pos = w.cnt, tot = 0;
#pragma unroll
    for (int b = 0; (1 << b) <= kSmallVecs * PV; ++b) {
      const uint64_t mb = __ballot((c >> b) & 1);
      pos += lanes_below(mb) << b;
      tot += __popcll(mb) << b;
    }
    if (w.cnt + tot <= kCap) {
#pragma unroll
      for (int u = 0; u < kSmallVecs; ++u) {
        if (__ballot(bits[u] != 0u) == 0) continue;
        const uint32_t base = (uint32_t)(vb + ((int64_t)u * kThreads + tid) * PV);
#if DFS_TOPK_SMALL_BITLOOP
        // only the lane's set bits, lowest first (the wave loops as often as its busiest lane)
        for (uint32_t m = bits[u]; m != 0u; m &= m - 1u) {
          const int e = __builtin_ctz(m);
          float v;
          if constexpr (kBf16) {
            const int wi = e >> 1;
            const uint32_t word = wi == 0 ? d[u].x : wi == 1 ? d[u].y : wi == 2 ? d[u].z : d[u].w;
            v = (e & 1) ? bf16_hi(word) : bf16_lo(word);
          } else {
            v = __uint_as_float(e == 0 ? d[u].x : e == 1 ? d[u].y : e == 2 ? d[u].z : d[u].w);
          }
          buf[pos++] = make_key(v, base + (uint32_t)e);
        }
#else
#pragma unroll
        for (int e = 0; e < PV; ++e)
          if ((bits[u] >> e) & 1u) buf[pos++] = make_key(elem(u, e), base + (uint32_t)e);
#endif
      }
      w.cnt = uniform(w.cnt + tot);
      scanned = true;
    }
  }
#endif
  if (!scanned) {
#pragma unroll
    for (int u = 0; u < kSmallVecs; ++u) {
      const int64_t vid = (int64_t)u * kThreads + tid;
      scan_vec<kBf16, true, false>(d[u], vid < nvec, (uint32_t)(vb + vid * PV), w, buf, lds.thr, lane);
    }
  }
  if (w.cnt > 0) wave_merge<true, false>(w, buf, lds.thr, lane);
  if (lane < kK) lds.list[wave * kK + lane] = w.list;
  __syncthreads();
  if (wave == 0) {
    const uint64_t x = wave_merge_runs16(lds.list[lane], lane);  // the four waves' sorted lists
    if (lane < kK) {
      if (parts == 1) {
        out_idx[row * kK + lane] = (int32_t)key_index(x);
        out_val[row * kK + lane] = key_value(x);
      } else {
        partial[(row * parts + part) * kK + lane] = x;
      }
    }
  }
}

// The pass over `ntopk` = rows * parts workgroups; W_h packing slabs (the fused
// selector) ride as extra workgroups after or before the rows.
template <bool kBf16, bool kWide>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DFS_TOPK_WAVES_PER_EU))) void topk_chunk_kernel(
    const void* __restrict__ logits, int64_t V, int parts, int64_t chunk, uint64_t* __restrict__ partial,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, int64_t ntopk, PackJob pack, ZeroJob zero) {
  __shared__ TopkLds lds;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero.n; i += kThreads) zero.p[i] = 0u;
  const int64_t job = DFS_TOPK_PACK_FIRST ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - ntopk;
  const int64_t bid = DFS_TOPK_PACK_FIRST ? (int64_t)blockIdx.x - pack.nslabs : (int64_t)blockIdx.x;
  if (DFS_TOPK_PACK_FIRST ? job < pack.nslabs : job >= 0) {
    pack_w_slab(pack.W, pack.d, pack.Wp, job, threadIdx.x, reinterpret_cast<uint16_t(*)[kPackPitch]>(&lds.buf[0][0]));
    return;
  }
  topk_body<kBf16, DFS_TOPK_CHUNK_COMPACT, kWide, !kWide && DFS_TOPK_UNION>(logits, V, parts, chunk, partial, out_idx,
                                                                          out_val, bid, lds);
}

// The pass with the gate's jobs as the first workgroups of the launch, for up to 512
// rows: the gate tiles hold more registers than the pass's 8-waves-per-SIMD budget,
// which it does not need at those sizes (one or two of its workgroups per CU), so the
// tiles run in the CU slots it leaves free.
template <bool kBf16, bool kGateBf16>
__global__ __launch_bounds__(kThreads) void topk_gate_kernel(const void* __restrict__ logits, int64_t V, int parts,
                                                             int64_t chunk, uint64_t* __restrict__ partial,
                                                             int32_t* __restrict__ out_idx,
                                                             float* __restrict__ out_val, GateJobs g,
                                                             ZeroJob zero) {
  __shared__ TopkLds lds;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero.n; i += kThreads) zero.p[i] = 0u;
  const int64_t njobs = (int64_t)g.mtiles * g.splits;
  if ((int64_t)blockIdx.x < njobs) {
    run_gate_job(g, kGateBf16, blockIdx.x, threadIdx.x, &lds.buf[0][0]);
    return;
  }
  const int64_t bid = (int64_t)blockIdx.x - njobs;
  if (chunk <= (int64_t)kSmallVecs * kThreads * Elems<kBf16>::per_vec) {
    topk_small_body<kBf16>(logits, V, parts, chunk, partial, out_idx, out_val, bid, lds);
  } else {
    topk_body<kBf16, DFS_TOPK_GATE_COMPACT, true, false>(logits, V, parts, chunk, partial, out_idx, out_val, bid, lds);
  }
}

// Merge `parts` partial top-16 lists per row (one workgroup per row).
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(const uint64_t* __restrict__ partial,
                                                              int parts,
                                                              int32_t* __restrict__ out_idx,
                                                              float* __restrict__ out_val) {
  static_assert(kWaves == kMergeWaves, "one row per workgroup");
  __shared__ uint64_t s_list[kWaves * kK];
  const int64_t row = blockIdx.x;
  merge_row_lists(partial + row * parts * kK, parts, true, threadIdx.x / kWave, threadIdx.x & (kWave - 1),
                  s_list, out_idx + row * kK, out_val + row * kK);
}

}  // namespace

TopkPlan plan_topk(int64_t rows, int64_t V, int esize) {
  TopkPlan p{};
  p.rows = rows;
  p.V = V;
  p.esize = esize;
  const int64_t pv = 16 / esize;
  int64_t parts = 1;
  if (rows < DFS_TOPK_TARGET_BLOCKS) {
    parts = cdiv(DFS_TOPK_TARGET_BLOCKS, rows);
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
  p.ws_bytes = p.parts > 1 ? align_up((size_t)rows * p.parts * kK * sizeof(uint64_t), 256) : 0;
  return p;
}

TopkPlan plan_topk_small(int64_t rows, int64_t V, int esize) {
  TopkPlan p{};
  p.rows = rows;
  p.V = V;
  p.esize = esize;
  const int64_t pv = 16 / esize;
  const int64_t cap = (int64_t)kSmallVecs * kThreads * pv;  // elements a chunk may hold in registers
  int64_t parts = cdiv(DFS_TOPK_SMALL_TARGET_BLOCKS, rows);
  const int64_t fit = cdiv(V, cap);
  if (parts < fit) parts = fit;
  int64_t maxp = V / kMinSmallChunk;
  if (maxp < 1) maxp = 1;
  if (parts > maxp) parts = maxp;
  if (parts > kMaxMergeParts) parts = kMaxMergeParts;
  const int64_t chunk = (int64_t)align_up((size_t)cdiv(V, parts), (size_t)pv);
  p.parts = (int)cdiv(V, chunk);
  p.chunk = chunk;
  p.ws_bytes = p.parts > 1 ? align_up((size_t)rows * p.parts * kK * sizeof(uint64_t), 256) : 0;
  return p;
}

hipError_t launch_topk(const TopkPlan& p, const void* logits, bool bf16, int32_t* out_idx,
                       float* out_val, void* ws, hipStream_t stream, const PackJob* pack, bool merge, ZeroJob zero) {
  static_assert(kThreads == kPackThreads, "packing jobs run on top-16 workgroups");
  uint64_t* partial = p.parts > 1 ? static_cast<uint64_t*>(ws) : nullptr;
  const int64_t ntopk = p.rows * p.parts;
  const PackJob job = pack ? *pack : PackJob{nullptr, 0, nullptr, 0};
  const dim3 grid((unsigned)(ntopk + job.nslabs));
  const bool wide = ntopk <= kWideSeedMaxBlocks;
#define DFS_TK(LB, WS) \
  topk_chunk_kernel<LB, WS><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.chunk, partial, out_idx, out_val, ntopk, job, zero)
  if (bf16) {
    if (wide) DFS_TK(true, true); else DFS_TK(true, false);
  } else {
    if (wide) DFS_TK(false, true); else DFS_TK(false, false);
  }
#undef DFS_TK
  if (p.parts > 1 && merge) {
    topk_merge_kernel<<<dim3((unsigned)p.rows), kThreads, 0, stream>>>(partial, p.parts, out_idx,
                                                                        out_val);
  }
  return hipGetLastError();
}

hipError_t launch_topk_gate(const TopkPlan& p, const void* logits, bool bf16, int32_t* out_idx, float* out_val,
                            void* ws, const GateJobs& g, bool gate_bf16, ZeroJob zero, hipStream_t stream) {
  uint64_t* partial = p.parts > 1 ? static_cast<uint64_t*>(ws) : nullptr;
  const dim3 grid((unsigned)(p.rows * p.parts + (int64_t)g.mtiles * g.splits));
#define DFS_TG(LB, GB) \
  topk_gate_kernel<LB, GB><<<grid, kThreads, 0, stream>>>(logits, p.V, p.parts, p.chunk, partial, out_idx, out_val, g, zero)
  if (bf16) {
    if (gate_bf16) DFS_TG(true, true); else DFS_TG(true, false);
  } else {
    if (gate_bf16) DFS_TG(false, true); else DFS_TG(false, false);
  }
#undef DFS_TG
  return hipGetLastError();
}

hipError_t launch_topk_merge(const uint64_t* partial, int64_t rows, int parts, int32_t* out_idx,
                             float* out_val, hipStream_t stream) {
  topk_merge_kernel<<<dim3((unsigned)rows), kThreads, 0, stream>>>(partial, parts, out_idx, out_val);
  return hipGetLastError();
}

}  // namespace dfs
