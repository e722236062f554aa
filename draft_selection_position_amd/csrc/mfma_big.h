// A tile of C = A B^T on gfx950's matrix cores (bf16 operands, both K-contiguous,
// fp32 sums), for products large enough to be bound by the matrix cores.
//
// Four waves in a 2 x 2 grid, each TM x TN V_MFMA_F32_16X16X32_BF16 tiles (128 x 128
// for 8 x 8: the sums fill the 256 accumulation registers, and every fragment read
// from LDS feeds eight MFMAs; 64 x 64 for 4 x 4).  Operands go from memory straight
// into LDS (buffer_load_dwordx4 with the LDS bit: no register staging), 32 k per step
// into a ring of S stages (four by default), S - 1 steps in flight while one is
// computed.  An operand is any layout whose 64-byte row pieces of one k step sit at
// row * row_bytes + step * step_bytes (row-major [rows, K]: 2 K and 64).  A wave's load instruction fills 1 KB of
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
constexpr int kK = 32;                         // k per MFMA
#ifndef DFS_BIG_PIPE_MAX
#define DFS_BIG_PIPE_MAX 16  // largest TM * TN that reads the next step's fragments ahead
#endif

// Waves in a 2 x 2 grid, each TM x TN tiles of 16 x 16: the workgroup tile is
// BM = 32 TM rows of A by BN = 32 TN rows of B; a ring of S stages of KK k each
// (32: a load instruction fills 16 rows x 64 bytes; 64: 8 rows x 128 bytes, whole
// cache lines).
template <int TM_, int TN_, int S_ = 4, int KK_ = 32>
struct Cfg {
  static constexpr int TM = TM_, TN = TN_;
  static constexpr int kStages = S_;
  static constexpr int KK = KK_;
  static_assert(KK_ == 32 || KK_ == 64, "k per step");
  static constexpr int KH = KK_ / kK;                   // MFMAs per tile pair per step
  static constexpr int kRowBytes = 2 * KK_;             // bytes of a row per step
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks of a row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes; // rows one load instruction fills
  // read-ahead of the next step's fragments: needs a second fragment set and a step in
  // flight beyond the one read ahead
  static constexpr bool kPipelined = TM * TN <= DFS_BIG_PIPE_MAX && S_ >= 3;
  static_assert(S_ >= 2, "a step in flight");
  // the pipelined loop's two fragment sets alternate with the step parity across ring laps
  static_assert(!kPipelined || S_ % 2 == 0, "even ring for the pipelined loop");
  static constexpr int BM = 32 * TM, BN = 32 * TN;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLoadsPerWave = (BM + BN) / kRowsPerLoad / 4;  // 1 KB load instructions per wave per step
  static_assert((S_ - 2) * kLoadsPerWave < 64, "vmcnt range");
  static constexpr int kLdsBytes = S_ * kStageBytes;
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
// format) over `bytes` bytes starting at `p`, as four scalar words.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t span_rsrc(const void* p, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r.w = kRawBufferWord3;
  return r;
}

// An operand: its range (reads past it return zeros) and where row `row`'s bytes of
// k step `ks` start: row * row_bytes + ks * step_bytes.  A 64-k step's 128 bytes are two
// 64-byte halves, the second `half_bytes` after the first (64 when the row is contiguous).
struct Operand {
  rsrc_t rsrc;
  uint32_t row_bytes, step_bytes, half_bytes;
};
__device__ __forceinline__ Operand make_operand(const void* p, int64_t bytes, uint32_t row_bytes,
                                                uint32_t step_bytes, uint32_t half_bytes = 64) {
  return Operand{span_rsrc(p, bytes), row_bytes, step_bytes, half_bytes};
}
// Row-major [nrows, K] bf16 starting at p, steps of kk.
__device__ __forceinline__ Operand rows_operand(const uint16_t* p, int64_t nrows, int64_t K, int kk = kK) {
  return make_operand(p, nrows * K * 2, (uint32_t)(K * 2), (uint32_t)(2 * kk));
}

// LDS slot of 16-byte chunk c of stage row `row`: XOR-swizzled so that the 16 rows a
// fragment read touches (one chunk each) fall on distinct banks.
template <class C>
__device__ __forceinline__ int chunk_slot(int c, int row) {
  return C::kChunks == 4 ? c ^ ((row >> 1) & 3) : c ^ (row & 7);
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
// instruction j < BM / R (R rows per instruction) covers A rows R j .. R j + R - 1,
// the rest B rows.
template <class C>
__device__ __forceinline__ void load_step(char* stage, const Operand& a, const Operand& b, int ks, int wave,
                                          int lane) {
  constexpr int BM = C::BM, R = C::kRowsPerLoad;
  const int rr = lane / C::kChunks;             // row within the instruction's R
  const int slot = lane % C::kChunks;           // LDS chunk slot
  const int chunk = chunk_slot<C>(slot, rr);    // global chunk stored there (the swizzle is an involution)
  const uint32_t ka = (uint32_t)ks * a.step_bytes + 16u * (chunk & 3) + (uint32_t)(chunk >> 2) * a.half_bytes;
  const uint32_t kb = (uint32_t)ks * b.step_bytes + 16u * (chunk & 3) + (uint32_t)(chunk >> 2) * b.half_bytes;
#pragma unroll
  for (int i = 0; i < C::kLoadsPerWave; ++i) {
    const int j = wave + 4 * i;
    const bool isA = j < BM / R;
    const int row = R * (isA ? j : j - BM / R) + rr;
    const uint32_t voff = isA ? (uint32_t)row * a.row_bytes + ka : (uint32_t)row * b.row_bytes + kb;
    const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>((lds_ptr_t)(stage + j * 1024));
    dma16(isA ? a.rsrc : b.rsrc, voff, __builtin_amdgcn_readfirstlane(dst));
  }
}

template <class C>
struct Frags {
  bf16x8 a[C::KH][C::TM], b[C::KH][C::TN];
};

// This wave's operand fragments of one step, from its stage: for the step's h-th 32 k,
// lane (r, q) takes chunk 4 h + q of its rows (16 rows apart keep the same swizzle).
template <class C>
__device__ __forceinline__ void read_frags(const char* stage, int wm, int wn, int r, int q, Frags<C>& f) {
  constexpr int RB = C::kRowBytes;
#pragma unroll
  for (int h = 0; h < C::KH; ++h) {
    const int sw = chunk_slot<C>(4 * h + q, r) * 16;
    const char* a = stage + (16 * C::TM * wm + r) * RB + sw;
    const char* b = stage + C::BM * RB + (16 * C::TN * wn + r) * RB + sw;
#pragma unroll
    for (int t = 0; t < C::TM; ++t) f.a[h][t] = *reinterpret_cast<const bf16x8*>(a + 16 * t * RB);
#pragma unroll
    for (int t = 0; t < C::TN; ++t) f.b[h][t] = *reinterpret_cast<const bf16x8*>(b + 16 * t * RB);
  }
}

// One 32-k half of a step (the loop without read-ahead).
template <class C>
struct Half {
  bf16x8 a[C::TM], b[C::TN];
};
template <class C>
__device__ __forceinline__ void read_half(const char* stage, int h, int wm, int wn, int r, int q, Half<C>& f) {
  constexpr int RB = C::kRowBytes;
  const int sw = chunk_slot<C>(4 * h + q, r) * 16;
  const char* a = stage + (16 * C::TM * wm + r) * RB + sw;
  const char* b = stage + C::BM * RB + (16 * C::TN * wn + r) * RB + sw;
#pragma unroll
  for (int t = 0; t < C::TM; ++t) f.a[t] = *reinterpret_cast<const bf16x8*>(a + 16 * t * RB);
#pragma unroll
  for (int t = 0; t < C::TN; ++t) f.b[t] = *reinterpret_cast<const bf16x8*>(b + 16 * t * RB);
}
template <class C>
__device__ __forceinline__ void mfma_half(const Half<C>& f, typename C::Acc& acc) {
#pragma unroll
  for (int mt = 0; mt < C::TM; ++mt)
#pragma unroll
    for (int nt = 0; nt < C::TN; ++nt)
      acc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mt], f.b[nt], acc.v[mt][nt], 0, 0, 0);
}

template <class C>
__device__ __forceinline__ void mfma_frags(const Frags<C>& f, typename C::Acc& acc) {
#pragma unroll
  for (int h = 0; h < C::KH; ++h)
#pragma unroll
    for (int mt = 0; mt < C::TM; ++mt)
#pragma unroll
      for (int nt = 0; nt < C::TN; ++nt)
        acc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[h][mt], f.b[h][nt], acc.v[mt][nt], 0, 0, 0);
}

// acc += A[0:BM, KK ks0 : KK ks1] B[0:BN, same]^T.  lds: C::kLdsBytes of shared
// memory, the S stages in a row.  Every thread of the workgroup must call it; it
// ends with a barrier, after which the LDS may be reused.
//
// Step s of the loop: wait until step s + 1 has landed (this wave's loads; the
// barrier covers the other waves' and frees the stage of step s - 1), issue the
// loads of step s + S - 1 into that stage, read step s + 1's fragments into the
// spare register set and run step s's MFMAs from the other: the LDS reads of the
// next step overlap the matrix work of this one.
template <class C>
__device__ __forceinline__ void mma(const Operand& a, const Operand& b, int ks0, int ks1, char* lds,
                                    typename C::Acc& acc) {
  constexpr int kStageBytes = C::kStageBytes;
  constexpr int kStages = C::kStages;
  constexpr int L = C::kLoadsPerWave;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: resources and M0 stay scalar
  const int r = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n = ks1 - ks0;
  char* st[kStages];
#pragma unroll
  for (int j = 0; j < kStages; ++j) st[j] = lds + j * kStageBytes;
  // prologue: steps 0 .. S - 2 in flight (a missing step loads the last one again)
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) load_step<C>(st[j], a, b, ks0 + (j < n ? j : n - 1), wave, lane);
  if constexpr (!C::kPipelined) {
    // 128 x 128 per wave: the accumulators fill the AGPRs, so there is no room for a
    // second fragment set; step s waits for its own stage and reads it
    for (int s = 0; s < n; s += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int cur = s + j;
        if (cur < n) {
          wait_vmcnt<(kStages - 2) * L>();  // this wave's loads of step cur (those of the S - 2 after it remain)
          bar();
          const int nxt = cur + kStages - 1;
          load_step<C>(st[(j + kStages - 1) % kStages], a, b, ks0 + (nxt < n ? nxt : n - 1), wave, lane);
#pragma unroll
          for (int h = 0; h < C::KH; ++h) {  // a 32-k half at a time: one fragment set
            Half<C> f;
            read_half<C>(st[j], h, wm, wn, r, q, f);
            mfma_half<C>(f, acc);
          }
        }
      }
    }
  } else {
    Frags<C> f[2];
    wait_vmcnt<(kStages - 2) * L>();
    bar();
    read_frags<C>(st[0], wm, wn, r, q, f[0]);
    for (int s = 0; s < n; s += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int cur = s + j;
        if (cur < n) {
          wait_vmcnt<(kStages - 3) * L>();  // this wave's loads of step cur + 1 (those of the S - 3 after it remain)
          bar();
          const int nxt = cur + kStages - 1;
          load_step<C>(st[(j + kStages - 1) % kStages], a, b, ks0 + (nxt < n ? nxt : n - 1), wave, lane);
          // unconditional (after the last step it reads a stage nobody uses): a branch here
          // would make the compiler wait for these reads before the MFMAs below
          read_frags<C>(st[(j + 1) % kStages], wm, wn, r, q, f[(j + 1) & 1]);
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
