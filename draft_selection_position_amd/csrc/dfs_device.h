// Device-side helpers shared by the selector's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfs {

constexpr int kK = 16;     // candidates per position
constexpr int kE = 256;    // embedding / gate width
constexpr int kWave = 64;  // CDNA wavefront

// ---------------------------------------------------------------- bf16 <-> f32
// bf16 is the upper half of an fp32 bit pattern; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ---------------------------------------------------------------- selection keys
// Order-preserving map from a non-NaN float to uint32, with -0 folded into +0.
__device__ __forceinline__ uint32_t mono32(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unmono32(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}
// 64-bit key: value in the high word, bit-inverted index in the low word, so a
// larger key means a larger value, then a lower index.  Key 0 is never produced
// for a non-NaN value and marks an empty slot.
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return ((uint64_t)mono32(v) << 32) | (uint32_t)(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }
__device__ __forceinline__ float key_value(uint64_t k) { return unmono32((uint32_t)(k >> 32)); }

// The context gate's nonlinearity; every kernel that applies it uses this one
// definition, so the fused and unfused paths give identical bits.
__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- wave utilities
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// x of lane (this lane ^ j) for j = 1, 2, 4, ..., 32, without going through LDS:
// DPP quad permutes for 1 and 2, DPP row shifts / rotates for 4 and 8 (a row is 16
// lanes; row_shl:n reads lane + n, row_shr:n lane - n, row_ror:8 lane ^ 8), and
// gfx950's permlane swaps for 16 and 32 (called with both operands x, the first
// result holds rows 0, 0, 2, 2 / halves 0, 0 and the second rows 1, 1, 3, 3 /
// halves 1, 1).  j must be a compile-time constant after inlining.
__device__ __forceinline__ uint32_t xor_lanes(uint32_t x, int j, int lane) {
  switch (j) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x104, 0xF, 0xF, false);
      const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x114, 0xF, 0xF, false);
      return (lane & 4) ? dn : up;
    }
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      return (lane & 16) ? p[0] : p[1];
    }
    default: {
      const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      return (lane & 32) ? p[0] : p[1];
    }
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int j, int lane) {
  const uint32_t lo = xor_lanes((uint32_t)x, j, lane);
  const uint32_t hi = xor_lanes((uint32_t)(x >> 32), j, lane);
  return ((uint64_t)hi << 32) | lo;
}
// x of lane `src` (a wave-uniform lane number), in every lane.
__device__ __forceinline__ uint64_t lane_u64(uint64_t x, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one 64-bit key per lane across the wave, descending: lane 0
// ends with the largest key.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = shfl_xor_u64(x, j, lane);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;
      // the lane keeps the larger key where lower == desc, else the smaller: one
      // compare and one select (equal keys are the same either way)
      x = ((x > y) == (lower == desc)) ? x : y;
    }
  }
  return x;
}

// The wave sorted descending when it holds four descending runs of 16 keys (lanes
// 16 r .. 16 r + 15): the odd runs are reversed (DPP row mirror), which leaves the
// alternating runs that the first four phases of the bitonic sort would have made, and
// only its last two phases run (11 exchange steps instead of 21).
__device__ __forceinline__ uint64_t wave_merge_runs16(uint64_t x, int lane) {
  const uint32_t mlo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, 0x140, 0xF, 0xF, false);
  const uint32_t mhi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), 0x140, 0xF, 0xF, false);
  if (lane & 16) x = ((uint64_t)mhi << 32) | mlo;
#pragma unroll
  for (int k = 32; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = shfl_xor_u64(x, j, lane);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;
      // the lane keeps the larger key where lower == desc, else the smaller: one
      // compare and one select (equal keys are the same either way)
      x = ((x > y) == (lower == desc)) ? x : y;
    }
  }
  return x;
}

// The 16th largest of one 32-bit key per lane (0 when fewer than 16 lanes hold a key
// above 0), found bit by bit from the top: a prefix stays when at least 16 lanes are
// at or above it.  Wave-uniform.
__device__ __forceinline__ uint32_t wave_16th_largest(uint32_t key) {
  uint32_t prefix = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    if (__popcll(__ballot(key >= cand)) >= 16) prefix = cand;
  }
  return prefix;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniformf(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

}  // namespace dfs
