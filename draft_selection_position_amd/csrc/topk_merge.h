// Merge of one row's partial top-16 lists (64-bit keys, 0 = empty; key order is value
// descending, then the lower token id) by four waves: each wave folds its share of the
// lists into its own top-16 with 64-lane merges of four sorted runs (its list plus
// three more per merge), then one wave merges the four lists.  Used by the merge pass
// of the top-16 kernel and by merge jobs that ride along in another launch.
#pragma once

#include "dfs_device.h"

namespace dfs {

constexpr int kMergeWaves = 4;  // waves per row: 4 x 16 keys = one wave of the final sort

// src: the row's lists [parts, 16]; s_list: kMergeWaves * 16 keys of LDS for this row;
// wave: 0..3 within the row's group.  Every thread of the workgroup must call it the
// same number of times (it holds one workgroup barrier); `live` false leaves the row
// untouched (a padding group).
__device__ __forceinline__ void merge_row_lists(const uint64_t* __restrict__ src, int parts, bool live,
                                                int wave, int lane, uint64_t* s_list,
                                                int32_t* __restrict__ out_idx, float* __restrict__ out_val) {
  uint64_t list = 0;
  if (live) {
    for (int p0 = wave * 3; p0 < parts; p0 += kMergeWaves * 3) {
      uint64_t x = 0;
      if (lane < kK) {
        x = list;
      } else {
        const int p = p0 + (lane - kK) / kK;
        if (p < parts) x = src[(int64_t)p * kK + (lane & (kK - 1))];
      }
      x = wave_merge_runs16(x, lane);  // the list and up to three partial lists, each sorted
      list = lane < kK ? x : 0;
    }
  }
  if (lane < kK) s_list[wave * kK + lane] = list;
  __syncthreads();
  if (live && wave == 0) {
    const uint64_t x = wave_merge_runs16(s_list[lane], lane);
    if (lane < kK) {
      out_idx[lane] = (int32_t)key_index(x);
      out_val[lane] = key_value(x);
    }
  }
}

// ---------------------------------------------------------------- one wave, one row
// Most lists one wave merges (the top-16 pass splits a row into at most this many).
constexpr int kMaxMergeParts = 64;
// Keys buffered per selection: with the running list they make 64.
constexpr int kMergeBatch = kWave - kK;
// LDS keys a merging wave needs: the buffer, the running list, the 16 output slots.
constexpr int kMergeScratch = kWave + kK;

// One wave merges one row's `parts` (1..64) sorted lists of 16 keys (src [parts, 16])
// into their top 16: lanes 0..15 of the result hold it, descending; the other lanes 0.
// merge_load issues every load (list p's key j goes to lane 16 (p % 4) + j of group
// p / 4); merge_keys then needs only the registers, so a caller can put other loads in
// flight in between.  Pruning: if some list's 16th key is T, that list alone holds 16
// keys >= T, so no key below T can be in the result; T only rises as the running list
// fills.  The survivors are appended to `scratch` (kMergeScratch keys of LDS for this
// wave) and sorted with the running list whenever the buffer would overflow, and once
// at the end.  Every lane of the wave must call both.
constexpr int kMergeGroups = kMaxMergeParts / 4;  // 4 lists per 64 lanes
struct MergeRegs {
  uint64_t x[kMergeGroups];
};

__device__ __forceinline__ void merge_load(const uint64_t* __restrict__ src, int parts, int lane, MergeRegs& m) {
  const int groups = (parts + 3) >> 2;
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) {
    m.x[g] = 0;
    const int p = 4 * g + (lane >> 4);
    if (g < groups && p < parts) m.x[g] = src[(int64_t)p * kK + (lane & (kK - 1))];
  }
}

__device__ __forceinline__ uint64_t merge_keys(MergeRegs& m, int parts, int lane, uint64_t* scratch) {
  const int groups = (parts + 3) >> 2;
  // T = the largest 16th key of any list (lanes 15, 31, 47, 63 of each group hold them)
  uint64_t t = 0;
#pragma unroll
  for (int g = 0; g < kMergeGroups; ++g) t = ((lane & (kK - 1)) == kK - 1 && m.x[g] > t) ? m.x[g] : t;
#pragma unroll
  for (int j = 1; j < kWave; j <<= 1) {
    const uint64_t o = shfl_xor_u64(t, j, lane);
    t = o > t ? o : t;
  }
  uint64_t list = 0;
  int n = 0;  // keys in the buffer (wave-uniform)
  // One pass per group plus a final one that only flushes.  The group in hand is always
  // m.x[0] (the registers shift down by one per pass), and the 64-lane sort has a single
  // call site: a wave runs this code once per call, so its size, not its loop count, is
  // what costs (every instruction fetched cold).
#pragma unroll 1
  for (int g = 0; g <= groups; ++g) {
    const bool last = g == groups;
    uint64_t v = last ? 0 : m.x[0];
#pragma unroll
    for (int i = 0; i + 1 < kMergeGroups; ++i) m.x[i] = m.x[i + 1];
#pragma unroll 1
    for (;;) {
      const bool keep = v != 0 && v >= t;
      const uint64_t mask = __ballot(keep);
      if ((n == kMergeBatch && mask != 0) || (last && n > 0)) {
        // the running list (lanes 0..15) and the buffered keys (lanes 16..): one sort
        __builtin_amdgcn_wave_barrier();
        uint64_t y = 0;
        if (lane < kK) {
          y = list;
        } else if (lane - kK < n) {
          y = scratch[lane - kK];
        }
        y = wave_sort_desc(y, lane);
        list = lane < kK ? y : 0;
        n = 0;
        const uint64_t k16 = lane_u64(list, kK - 1);
        t = k16 > t ? k16 : t;
        __builtin_amdgcn_wave_barrier();
        continue;
      }
      if (mask == 0) break;
      const int room = kMergeBatch - n;
      const int below = lanes_below(mask);
      if (keep && below < room) {
        scratch[n + below] = v;
        v = 0;  // taken
      }
      const int c = __popcll(mask);
      n += c < room ? c : room;
    }
  }
  return list;
}

// ---------------------------------------------------------------- four waves, one row
// Four waves (w4 = 0..3) of a workgroup share one row's `parts` (1..64) sorted lists:
// in round 0 wave w4 takes lists 4 w4 .. 4 w4 + 3 as its four 16-lane runs, in round
// k >= 1 its running list (lanes 0..15) and lists 16 + 12 (k - 1) + 3 w4 .. + 2; each
// round is one merge of four sorted runs.  merge4_load issues every load up front;
// merge4_wave leaves the wave's top 16 in lanes 0..15 (the others 0), and a merge of
// the four waves' lists gives the row's.  Up to 16 lists this is one merge per wave.
constexpr int kMerge4Rounds = 1 + (kMaxMergeParts - 16 + 11) / 12;
struct Merge4Regs {
  uint64_t x[kMerge4Rounds];
};

__device__ __forceinline__ void merge4_load(const uint64_t* __restrict__ src, int parts, int w4, int lane,
                                            Merge4Regs& m) {
  const int j = lane & (kK - 1);
  const int p0 = 4 * w4 + (lane >> 4);
  m.x[0] = p0 < parts ? src[(int64_t)p0 * kK + j] : 0;
#pragma unroll
  for (int k = 1; k < kMerge4Rounds; ++k) {
    const int p = 16 + 12 * (k - 1) + 3 * w4 + (lane >> 4) - 1;
    m.x[k] = (lane >= kK && p < parts) ? src[(int64_t)p * kK + j] : 0;
  }
}

__device__ __forceinline__ uint64_t merge4_wave(const Merge4Regs& m, int parts, int w4, int lane) {
  uint64_t x = wave_merge_runs16(m.x[0], lane);
  uint64_t list = lane < kK ? x : 0;
#pragma unroll
  for (int k = 1; k < kMerge4Rounds; ++k) {
    if (16 + 12 * (k - 1) + 3 * w4 < parts) {  // wave-uniform: this wave has lists in round k
      x = wave_merge_runs16(lane < kK ? list : m.x[k], lane);
      list = lane < kK ? x : 0;
    }
  }
  return list;
}

}  // namespace dfs
