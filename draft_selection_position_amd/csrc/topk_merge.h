// Merge of one row's partial top-16 lists (64-bit keys, 0 = empty; key order is value
// descending, then the lower token id) by four waves: each wave folds its share of the
// lists into its own top-16 with 64-lane sorts (its list plus three more per sort),
// then one wave sorts the four lists.  Used by the merge pass of the top-16 kernel
// and by merge jobs that ride along in another launch.
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
      x = wave_sort_desc(x, lane);
      list = lane < kK ? x : 0;
    }
  }
  if (lane < kK) s_list[wave * kK + lane] = list;
  __syncthreads();
  if (live && wave == 0) {
    const uint64_t x = wave_sort_desc(s_list[lane], lane);
    if (lane < kK) {
      out_idx[lane] = (int32_t)key_index(x);
      out_val[lane] = key_value(x);
    }
  }
}

}  // namespace dfs
