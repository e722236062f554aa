// dfs_select_packed without a workspace argument, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its scratch is a file-scope device array of fixed size that each GPU the
// library runs on holds until the process ends; the array's device address is looked up
// once per device (hipGetSymbolAddress) and only that address is handed to kernels.
// Every call on one GPU shares that GPU's array, so calls that overlap on one GPU (two
// streams, two host threads) race: the caller must order them.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/dfs.h"
#include "dfs_internal.h"

namespace dfs {
int select_with_workspace(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                          const void* B, const void* W_h, bool wh_packed, int k, const dfs_shape_t* shape,
                          int mode, double temperature, uint64_t seed, void* ws, size_t ws_bytes,
                          int32_t* out_path, float* out_scores, hipStream_t stream);
size_t select_workspace_need(const dfs_shape_t* shape);
int select_static_checks(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                         const void* B, const void* W_h, int k, const dfs_shape_t* shape, int mode,
                         double temperature, int32_t* out_path, float* out_scores);
}  // namespace dfs

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[DFS_STATIC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (its device address), looked up on first use on
// that device; nullptr (and *st set) on failure.
void* device_scratch(int* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *st = DFS_E_HIP;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    // with `dev` current: each device holds its own copy of the array at its own address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *st = DFS_E_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int dfs_select_packed_static(const void* logits, const void* hidden, const int32_t* prev_token,
                                        const void* A, const void* B, const void* W_packed, int k,
                                        const dfs_shape_t* shape, dfs_walk_t mode, double temperature,
                                        uint64_t seed, int32_t* out_path, float* out_scores,
                                        hipStream_t stream) {
  int st = dfs::select_static_checks(logits, hidden, prev_token, A, B, W_packed, k, shape, (int)mode, temperature,
                                     out_path, out_scores);
  if (st != DFS_OK) return st;
  if (dfs::select_workspace_need(shape) > DFS_STATIC_SCRATCH_BYTES) return DFS_E_TOO_LARGE;
  void* ws = device_scratch(&st);
  if (ws == nullptr) return st;
  return dfs::select_with_workspace(logits, hidden, prev_token, A, B, W_packed, true, k, shape, mode, temperature,
                                    seed, ws, DFS_STATIC_SCRATCH_BYTES, out_path, out_scores, stream);
}
