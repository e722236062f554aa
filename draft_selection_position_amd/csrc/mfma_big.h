// A tile of C = A B^T on gfx950's matrix cores (bf16 operands, both K-contiguous,
// fp32 sums), for products large enough to be bound by the matrix cores.
//
// Four waves in a 2 x 2 grid, each TM x TN V_MFMA_F32_16X16X32_BF16 tiles (128 x 128
// for 8 x 8: the sums fill the 256 accumulation registers, and every fragment read
// from LDS feeds eight MFMAs; 64 x 64 for 4 x 4).  Operands go from memory straight into LDS (buffer_load_dwordx4 with
// the LDS bit: no register staging), 32 k per step into a ring of four stages, three
// steps in flight while one is computed.  A wave's load instruction fills 1 KB of
// LDS, lane i at byte 16 i: 16 rows x 64 bytes.  Within a row the four 16-byte
// chunks are stored XOR-swizzled, chunk c at slot c ^ ((row >> 1) & 3), so the 16
// rows that a fragment read touches spread over all banks.  Rows past the end of an
// operand read as zeros (buffer range check).
#pragma once

#include "dfs_device.h"

namespace dfs {
namespace big {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kThreads = 256;
constexpr int kK = 32;                         // k per step
constexpr int kRowBytes = kK * 2;              // 64 bytes of a row per step
constexpr int kStages = 4;

// Waves in a 2 x 2 grid, each TM x TN tiles of 16 x 16: the workgroup tile is
// BM = 32 TM rows of A by BN = 32 TN rows of B.
template <int TM_, int TN_>
struct Cfg {
  static constexpr int TM = TM_, TN = TN_;
  static constexpr int BM = 32 * TM, BN = 32 * TN;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLoadsPerWave = (BM + BN) / 16 / 4;  // 1 KB load instructions per wave per step
  static constexpr int kLdsBytes = kStages * kStageBytes;
  struct Acc {
    f32x4 v[TM][TN];  // C[16 TM wm + 16 mt + 4 q + i][16 TN wn + 16 nt + r] = v[mt][nt][i]
  };
  static __device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc.v[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// A raw buffer descriptor (gfx9 layout: 48-bit base, stride 0, byte range, raw
// format) over `nrows` rows of length K starting at `p`, as four scalar words.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t rows_rsrc(const uint16_t* p, int64_t nrows, int64_t K) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int32_t)(nrows * K * 2));
  r.w = kRawBufferWord3;
  return r;
}

// 16 bytes per lane from the buffer straight into LDS at lds_base + 16 lane.  Issued
// as assembly so that the compiler's wait insertion, which cannot tell the stages of
// the ring apart, does not wait for every load in flight before each LDS read; the
// loop below waits for exactly the stage it reads (vmcnt) instead.
__device__ __forceinline__ void dma16(rsrc_t rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt with vmcnt = n (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (whose release half
// waits for every load in flight): the LDS reads of the previous step are complete
// (lgkmcnt), the caller has waited for the loads it needs (vmcnt).
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The loads of one step into one stage: wave w issues instructions w, w + 4, ...;
// instruction j < BM/16 covers A rows 16 j .. 16 j + 15, the rest B rows.
template <class C>
__device__ __forceinline__ void load_step(char* stage, rsrc_t ra, rsrc_t rb, int64_t K, int ks, int wave,
                                          int lane) {
  constexpr int BM = C::BM;
  const int rr = lane >> 2;             // row within the instruction's 16
  const int slot = lane & 3;            // LDS chunk slot
  const int chunk = slot ^ ((rr >> 1) & 3);  // global chunk stored there
  const uint32_t kbyte = (uint32_t)ks * kRowBytes + 16u * chunk;
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const int j = wave + 4 * i;
    const bool isA = j < BM / 16;
    const int row = 16 * (isA ? j : j - BM / 16) + rr;
    const uint32_t voff = (uint32_t)((int64_t)row * K * 2) + kbyte;
    const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)(stage + j * 1024));
    dma16(isA ? ra : rb, voff, __builtin_amdgcn_readfirstlane(dst));
  }
}

template <class C>
struct Frags {
  bf16x8 a[C::TM], b[C::TN];
};

// This wave's operand fragments of one step, from its stage.
template <class C>
__device__ __forceinline__ void read_frags(const char* stage, int wm, int wn, int r, int q, Frags<C>& f) {
  const int sw = (q ^ ((r >> 1) & 3)) * 16;
  const char* a = stage + (16 * C::TM * wm + r) * kRowBytes + sw;
  const char* b = stage + C::BM * kRowBytes + (16 * C::TN * wn + r) * kRowBytes + sw;
#pragma unroll
  for (int t = 0; t < C::TM; ++t) f.a[t] = *reinterpret_cast<const bf16x8*>(a + 16 * t * kRowBytes);
#pragma unroll
  for (int t = 0; t < C::TN; ++t) f.b[t] = *reinterpret_cast<const bf16x8*>(b + 16 * t * kRowBytes);
}

template <class C>
__device__ __forceinline__ void mfma_frags(const Frags<C>& f, typename C::Acc& acc) {
#pragma unroll
  for (int mt = 0; mt < C::TM; ++mt)
#pragma unroll
    for (int nt = 0; nt < C::TN; ++nt)
      acc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mt], f.b[nt], acc.v[mt][nt], 0, 0, 0);
}

// acc += A[0:BM, 32 ks0 : 32 ks1] B[0:BN, same]^T.  lds: C::kLdsBytes of shared
// memory, the four stages in a row.  Every thread of the workgroup must call it; it
// ends with a barrier, after which the LDS may be reused.
//
// Step s of the loop: wait until step s + 1 has landed (this wave's loads; the
// barrier covers the other waves' and frees the stage of step s - 1), issue the
// loads of step s + 3 into that stage, read step s + 1's fragments into the spare
// register set and run step s's MFMAs from the other: the LDS reads of the next
// step overlap the matrix work of this one.
template <class C>
__device__ __forceinline__ void mma(rsrc_t ra, rsrc_t rb, int64_t K, int ks0, int ks1, char* lds,
                                    typename C::Acc& acc) {
  constexpr int kStageBytes = C::kStageBytes;
  constexpr int L = C::kLoadsPerWave;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: resources and M0 stay scalar
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n = ks1 - ks0;
  char* st[kStages] = {lds, lds + kStageBytes, lds + 2 * kStageBytes, lds + 3 * kStageBytes};
  // prologue: steps 0, 1, 2 in flight (a missing step loads the last one again)
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) load_step<C>(st[j], ra, rb, K, ks0 + (j < n ? j : n - 1), wave, lane);
  if constexpr (C::TM * C::TN > 16) {
    // 128 x 128 per wave: the accumulators fill the AGPRs, so there is no room for a
    // second fragment set; step s waits for its own stage and reads it
    for (int s = 0; s < n; s += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int cur = s + j;
        if (cur < n) {
          wait_vmcnt<2 * L>();  // this wave's loads of step cur (cur + 1's and cur + 2's remain)
          bar();
          const int nxt = cur + kStages - 1;
          load_step<C>(st[(j + kStages - 1) % kStages], ra, rb, K, ks0 + (nxt < n ? nxt : n - 1), wave, lane);
          Frags<C> f;
          read_frags<C>(st[j], wm, wn, r, q, f);
          mfma_frags<C>(f, acc);
        }
      }
    }
  } else {
    Frags<C> f[2];
    wait_vmcnt<2 * L>();
    bar();
    read_frags<C>(st[0], wm, wn, r, q, f[0]);
    for (int s = 0; s < n; s += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int cur = s + j;
        if (cur < n) {
          wait_vmcnt<L>();  // this wave's loads of step cur + 1 (only cur + 2's remain)
          bar();
          const int nxt = cur + kStages - 1;
          load_step<C>(st[(j + kStages - 1) % kStages], ra, rb, K, ks0 + (nxt < n ? nxt : n - 1), wave, lane);
          if (cur + 1 < n) read_frags<C>(st[(j + 1) % kStages], wm, wn, r, q, f[(j + 1) & 1]);
          mfma_frags<C>(f[j & 1], acc);
        }
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
}

}  // namespace big
}  // namespace dfs
