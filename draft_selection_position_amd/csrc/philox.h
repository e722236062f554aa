// Philox4x32-10 for the selector's random streams (gfx950 device code).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfs {

// ---------------------------------------------------------------- Philox4x32-10
// Counter-based generator of Salmon, Moraes, Dror and Shaw (SC'11): ten rounds
// of two 32x32->64 multiplies and xors, key advanced by two Weyl constants.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t out[4]) {
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
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// u in (0, 1) from the top 23 bits of a word, plus one half: exact in fp32 and fp64.
__device__ __forceinline__ double uniform23(uint32_t x) { return ((double)(x >> 9) + 0.5) * 0x1p-23; }

}  // namespace dfs
