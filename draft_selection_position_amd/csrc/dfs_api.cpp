// C ABI of the selector: argument checks, workspace layout and launch order.
// Every check happens on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/dfs.h"
#include "dfs_internal.h"

using namespace dfs;

namespace {

constexpr int64_t kMaxV = 2147483647;  // token ids are int32
constexpr int64_t kMaxD = DFS_MAX_D;    // the gate's 32-bit buffer offsets
// bf16 convolution: row tiles x column tiles stay within 2^22 workgroups
constexpr int64_t kMaxConvElems = (int64_t)1 << 36;
// LM head: rows and vocabulary within range, and its 128 x 128 tiles within 2^23
// workgroups (the launch grids stay within 2^31 work-items)
inline bool lmhead_shape_ok(int64_t rows, int64_t V, int64_t d) {
  if (rows < 1 || rows > DFS_MAX_ROWS || V < DFS_K || V > kMaxV || d < 64 || d > kMaxD) return false;
  return ((rows + 127) / 128) * ((V + 127) / 128) <= ((int64_t)1 << 23);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}
int esize(dfs_dtype_t t) { return t == DFS_BF16 ? 2 : 4; }
bool valid_dtype(int t) { return t == DFS_F32 || t == DFS_BF16; }

// gfx950 check, cached per device.  0 = unknown, 1 = ok, 2 = other arch.
std::atomic<int> g_arch_state[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return DFS_E_HIP;
  }
  if (dev < 64) {
    const int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return DFS_OK;
    if (st == 2) return DFS_E_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return DFS_E_HIP;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? DFS_OK : DFS_E_ARCH;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DFS_OK : DFS_E_HIP; }

int check_topk_args(const void* logits, int dt, int64_t rows, int64_t V, int k,
                    const int32_t* out_idx, const float* out_val) {
  if (!logits || !out_idx || !out_val) return DFS_E_NULL;
  if (!valid_dtype(dt)) return DFS_E_UNSUPPORTED;
  if (k != DFS_K) return DFS_E_UNSUPPORTED;
  if (rows < 1 || rows > DFS_MAX_ROWS || V < DFS_K || V > kMaxV) return DFS_E_SHAPE;
  if (!aligned(logits, esize((dfs_dtype_t)dt)) || !aligned(out_idx, 4) || !aligned(out_val, 4))
    return DFS_E_ALIGN;
  return DFS_OK;
}

int check_gate_args(const void* hidden, const void* W_h, int dt, int64_t rows, int64_t d,
                    int64_t E, const float* out) {
  if (!hidden || !W_h || !out) return DFS_E_NULL;
  if (!valid_dtype(dt)) return DFS_E_UNSUPPORTED;
  if (E != DFS_E) return DFS_E_UNSUPPORTED;
  if (rows < 1 || rows > DFS_MAX_ROWS || d < 1 || d > kMaxD) return DFS_E_SHAPE;
  if (d % 8 != 0) return DFS_E_UNSUPPORTED;
  if (!aligned(hidden, 16) || !aligned(W_h, 16) || !aligned(out, 4)) return DFS_E_ALIGN;
  return DFS_OK;
}

int check_walk_mode(int mode, double temperature) {
  if (mode != DFS_WALK_GREEDY && mode != DFS_WALK_GUMBEL && mode != DFS_WALK_VITERBI)
    return DFS_E_UNSUPPORTED;
  if (mode == DFS_WALK_GUMBEL && !(std::isfinite(temperature) && temperature > 0.0))
    return DFS_E_ARG;
  return DFS_OK;
}

// Workspace layout of dfs_select.
struct SelectLayout {
  TopkPlan topk;
  GatePlan gate;
  bool few;    // few rows: per-position pair workgroups (tiles, counters)
  bool tiled;  // mid-size batches: the pair tensor by position, then the walk by sequence
  size_t cand_idx_off, cand_val_off, gate_off, topk_ws_off, gate_ws_off, tiles_off, counters_off, pair_off, total;
};

// Batches up to this many sequences (beyond the few-row path, rows not split by the
// top-16 pass) score their pairs a wave per position and walk them in a second launch: a
// workgroup per sequence would leave most CUs without gathers (32 x 16 x 151936: 47.2 ->
// 44.4 us per call; 64 x 16 x 262144: 110.9 -> 107.2 us).  At 256 sequences, a workgroup
// per CU, the extra launch and the pair tensor's round trip cost more (219.7 -> 223.7 us);
// 128 lies between the sizes measured.
#ifndef DFS_TILED_MAX_BATCH
#define DFS_TILED_MAX_BATCH 128
#endif
constexpr int64_t kTiledMaxBatch = DFS_TILED_MAX_BATCH;

SelectLayout select_layout(const dfs_shape_t& s) {
  SelectLayout l{};
  const int64_t rows = s.batch * s.L;
  l.few = rows <= kPosMaxRows;
  l.topk = l.few ? plan_topk_small(rows, s.V, esize(s.logits_dtype)) : plan_topk(rows, s.V, esize(s.logits_dtype));
  l.gate = plan_gate(rows, s.d, s.act_dtype == DFS_BF16);
  size_t off = 0;
  l.cand_idx_off = off;
  off += align_up((size_t)rows * DFS_K * sizeof(int32_t), 256);
  l.cand_val_off = off;
  off += align_up((size_t)rows * DFS_K * sizeof(float), 256);
  l.gate_off = off;
  off += align_up((size_t)rows * DFS_E * sizeof(float), 256);
  l.topk_ws_off = off;
  off += l.topk.ws_bytes;
  l.gate_ws_off = off;
  off += l.gate.ws_bytes;
  l.tiles_off = off;
  l.counters_off = off;
  if (l.few) {
    off += align_up((size_t)rows * sizeof(PosTile), 256);
    l.counters_off = off;
    off += align_up((size_t)s.batch * sizeof(uint32_t), 256);
  }
  l.tiled = !l.few && l.topk.parts <= 1 && s.batch <= kTiledMaxBatch;
  l.pair_off = off;
  if (l.tiled) off += align_up((size_t)rows * DFS_K * DFS_K * sizeof(float), 256);
  l.total = off;
  return l;
}

int check_shape(const dfs_shape_t* s) {
  if (!s) return DFS_E_NULL;
  if (!valid_dtype(s->logits_dtype) || !valid_dtype(s->act_dtype) || !valid_dtype(s->table_dtype))
    return DFS_E_UNSUPPORTED;
  if (s->batch < 1 || s->L < 1 || s->L > DFS_MAX_L || s->V < DFS_K || s->V > kMaxV || s->d < 1 ||
      s->d > kMaxD)
    return DFS_E_SHAPE;
  if (s->d % 8 != 0) return DFS_E_UNSUPPORTED;
  if (s->batch > DFS_MAX_ROWS / s->L) return DFS_E_SHAPE;
  return DFS_OK;
}

}  // namespace

// The host-side checks of a dfs_select call, in order, before any device call.
static int select_host_checks(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                              const void* B, const void* W_h, int k, const dfs_shape_t* shape, dfs_walk_t mode,
                              double temperature, int32_t* out_path, float* out_scores) {
  if (!logits || !hidden || !prev_token || !A || !B || !W_h || !out_path || !out_scores)
    return DFS_E_NULL;
  int st = check_shape(shape);
  if (st != DFS_OK) return st;
  if (k != DFS_K) return DFS_E_UNSUPPORTED;
  if ((st = check_walk_mode(mode, temperature)) != DFS_OK) return st;
  const dfs_shape_t s = *shape;
  if (!aligned(logits, esize(s.logits_dtype)) || !aligned(hidden, 16) || !aligned(W_h, 16) ||
      !aligned(A, 16) || !aligned(B, 16) || !aligned(prev_token, 4) || !aligned(out_path, 4) ||
      !aligned(out_scores, 4))
    return DFS_E_ALIGN;
  return DFS_OK;
}

static int select_impl(const void* logits, const void* hidden, const int32_t* prev_token,
                       const void* A, const void* B, const void* W_h, bool wh_packed, int k,
                       const dfs_shape_t* shape, dfs_walk_t mode, double temperature,
                       uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
                       float* out_scores, float* out_q, int32_t* out_cand, hipStream_t stream) {
  int st = select_host_checks(logits, hidden, prev_token, A, B, W_h, k, shape, mode, temperature, out_path,
                              out_scores);
  if (st != DFS_OK) return st;
  const dfs_shape_t s = *shape;
  const SelectLayout l = select_layout(s);
  if (!ws || ws_bytes < l.total) return DFS_E_WORKSPACE;
  if (!aligned(ws, 256)) return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();

  char* w = static_cast<char*>(ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(w + l.cand_idx_off);
  float* cand_val = reinterpret_cast<float*>(w + l.cand_val_off);
  float* gate = reinterpret_cast<float*>(w + l.gate_off);
  char* gws = w + l.gate_ws_off;
  char* tws = w + l.topk_ws_off;
  const bool bf16_logits = s.logits_dtype == DFS_BF16;
  const bool bf16_act = s.act_dtype == DFS_BF16;
  // Two or three launches on one stream.  (1) The top-16 pass; rows split into parts
  // leave their partial lists for the pair kernel to merge.  Up to kGateTileRows rows,
  // with a gate that needs no repacking (fp32, or W_h packed by the caller), the gate's
  // tiles ride in the same launch; otherwise the W_h packing slabs (when needed) ride
  // in its tail and (2) the gate GEMM follows.  (3) Pair scores and the walk, which also merges the
  // split rows' lists and adds up the gate's K-split partial sums: one workgroup per
  // sequence, or with few rows one per position (the last of a sequence walks it; its
  // counters are zeroed by launch (1)).
  uint32_t* counters = reinterpret_cast<uint32_t*>(w + l.counters_off);
  const ZeroJob zj = l.few ? ZeroJob{counters, (int)s.batch} : ZeroJob{};
  hipError_t e;
  if (l.gate.kind == GatePlan::kJobs && s.batch * s.L <= kGateTileRows && (wh_packed || !bf16_act)) {
    const GateJobs gj = gate_jobs(l.gate, hidden, W_h, gate, gws);
    e = launch_topk_gate(l.topk, logits, bf16_logits, cand_idx, cand_val, tws, gj, bf16_act, zj, stream);
    if (e != hipSuccess) return DFS_E_HIP;
  } else {
    const PackJob job = bf16_act && !wh_packed ? gate_pack_job(l.gate, W_h, gws) : PackJob{nullptr, 0, nullptr, 0};
    e = launch_topk(l.topk, logits, bf16_logits, cand_idx, cand_val, tws, stream, &job, false, zj);
    if (e != hipSuccess) return DFS_E_HIP;
    const void* Wg = bf16_act && !wh_packed ? gate_packed_in_ws(l.gate, gws) : W_h;
    if ((e = launch_gate_gemm(l.gate, hidden, Wg, gate, gws, stream)) != hipSuccess) return DFS_E_HIP;
  }
  const CandSrc cs = l.topk.parts > 1 ? CandSrc{nullptr, nullptr, reinterpret_cast<const uint64_t*>(tws), l.topk.parts}
                                      : cand_lists(cand_idx, cand_val);
  const GateSrc gs = l.gate.splits > 1 ? GateSrc{gate_partials(l.gate, gws), l.gate.splits, s.batch * s.L * DFS_E}
                                       : GateSrc{gate, 1, 0};
  const WalkArgs wa{(int)mode, temperature, seed, out_q, out_cand};
  if (l.few) {
    e = launch_pair_pos(cs, prev_token, gs, A, B, s.table_dtype == DFS_BF16, s.batch, s.L, s.V, wa, out_path,
                        out_scores, reinterpret_cast<PosTile*>(w + l.tiles_off), counters, stream);
  } else if (l.tiled && out_q == nullptr) {
    float* pair = reinterpret_cast<float*>(w + l.pair_off);
    e = launch_pair_tiles(cand_idx, cand_val, prev_token, gs, A, B, s.table_dtype == DFS_BF16, s.batch, s.L, s.V,
                          pair, stream);
    if (e != hipSuccess) return DFS_E_HIP;
    e = launch_walk(pair, cand_idx, s.batch, s.L, wa, out_path, out_scores, stream);
  } else {
    e = launch_pair_walk(cs, prev_token, gs, A, B, s.table_dtype == DFS_BF16, s.batch, s.L, s.V, nullptr, &wa,
                         out_path, out_scores, stream);
  }
  return hip_status(e);
}

namespace dfs {
// dfs_select / dfs_select_packed with a given workspace, and the bytes it needs (0 if the
// shape is rejected), for the entry points that bring their own scratch.
int select_with_workspace(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                          const void* B, const void* W_h, bool wh_packed, int k, const dfs_shape_t* shape,
                          int mode, double temperature, uint64_t seed, void* ws, size_t ws_bytes,
                          int32_t* out_path, float* out_scores, hipStream_t stream);
size_t select_workspace_need(const dfs_shape_t* shape);
int select_static_checks(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                         const void* B, const void* W_h, int k, const dfs_shape_t* shape, int mode,
                         double temperature, int32_t* out_path, float* out_scores);
}  // namespace dfs

static int select_entry(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                        const void* B, const void* W_h, bool wh_packed, int k, const dfs_shape_t* shape,
                        dfs_walk_t mode, double temperature, uint64_t seed, void* ws, size_t ws_bytes,
                        int32_t* out_path, float* out_scores, float* out_q, int32_t* out_cand, hipStream_t stream) {
  if (out_q || out_cand) {
    if (!out_q || !out_cand) return DFS_E_NULL;
    if (!aligned(out_q, 4) || !aligned(out_cand, 4)) return DFS_E_ALIGN;
    if (!(std::isfinite(temperature) && temperature > 0.0)) return DFS_E_ARG;
  }
  return select_impl(logits, hidden, prev_token, A, B, W_h, wh_packed, k, shape, mode, temperature, seed, ws,
                     ws_bytes, out_path, out_scores, out_q, out_cand, stream);
}

extern "C" {

int dfs_abi_version(void) { return DFS_ABI_VERSION; }

const char* dfs_status_str(int status) {
  switch (status) {
    case DFS_OK: return "DFS_OK: success";
    case DFS_E_NULL: return "DFS_E_NULL: a required pointer is NULL";
    case DFS_E_SHAPE: return "DFS_E_SHAPE: a size is out of range";
    case DFS_E_UNSUPPORTED:
      return "DFS_E_UNSUPPORTED: k must be 16, E 256, d a multiple of 8 (convolution: 256), dtype and walk mode known";
    case DFS_E_WORKSPACE: return "DFS_E_WORKSPACE: workspace missing or too small";
    case DFS_E_ALIGN: return "DFS_E_ALIGN: a pointer is not aligned as required";
    case DFS_E_HIP: return "DFS_E_HIP: no usable HIP device, or a HIP launch failed";
    case DFS_E_ARCH: return "DFS_E_ARCH: the current device is not gfx950";
    case DFS_E_ARG:
      return "DFS_E_ARG: invalid argument (temperature must be finite and > 0; outputs must not overlap inputs)";
    case DFS_E_TOO_LARGE:
      return "DFS_E_TOO_LARGE: the call needs more scratch than the library's static buffer holds "
             "(dfs_select_packed_static; use dfs_select_packed with a workspace)";
    default: return "unknown dfs status";
  }
}

size_t dfs_topk_workspace_bytes(int64_t rows, int64_t V, dfs_dtype_t dt) {
  if (rows < 1 || rows > DFS_MAX_ROWS || V < DFS_K || V > kMaxV || !valid_dtype(dt)) return 0;
  return plan_topk(rows, V, esize(dt)).ws_bytes;
}

int dfs_topk(const void* logits, dfs_dtype_t dt, int64_t rows, int64_t V, int k, int32_t* out_idx,
             float* out_val, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_topk_args(logits, dt, rows, V, k, out_idx, out_val);
  if (st != DFS_OK) return st;
  const TopkPlan p = plan_topk(rows, V, esize(dt));
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes)) return DFS_E_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_topk(p, logits, dt == DFS_BF16, out_idx, out_val, ws, stream));
}

size_t dfs_gate_workspace_bytes(int64_t rows, int64_t d, dfs_dtype_t dt) {
  if (rows < 1 || rows > DFS_MAX_ROWS || d < 1 || d > kMaxD || d % 8 != 0 || !valid_dtype(dt)) return 0;
  return plan_gate(rows, d, dt == DFS_BF16).ws_bytes;
}

static int gate_entry(const void* hidden, const void* W_h, bool prepacked, dfs_dtype_t dt, int64_t rows,
                      int64_t d, int64_t E, float* out_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_gate_args(hidden, W_h, dt, rows, d, E, out_gate);
  if (st != DFS_OK) return st;
  const GatePlan p = plan_gate(rows, d, dt == DFS_BF16);
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes)) return DFS_E_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_gate(p, hidden, W_h, prepacked, out_gate, ws, stream));
}

int dfs_gate(const void* hidden, const void* W_h, dfs_dtype_t dt, int64_t rows, int64_t d,
             int64_t E, float* out_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  return gate_entry(hidden, W_h, false, dt, rows, d, E, out_gate, ws, ws_bytes, stream);
}

int dfs_gate_packed(const void* hidden, const void* W_packed, dfs_dtype_t dt, int64_t rows, int64_t d,
                    int64_t E, float* out_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  return gate_entry(hidden, W_packed, true, dt, rows, d, E, out_gate, ws, ws_bytes, stream);
}

size_t dfs_gate_pack_bytes(int64_t d, dfs_dtype_t dt) {
  if (d < 1 || d > kMaxD || d % 8 != 0 || !valid_dtype(dt)) return 0;
  return dt == DFS_BF16 ? gate_packed_bytes(d) : (size_t)d * DFS_E * sizeof(float);
}

int dfs_gate_pack(const void* W_h, dfs_dtype_t dt, int64_t d, void* out_packed, size_t out_bytes,
                  hipStream_t stream) {
  if (!W_h || !out_packed) return DFS_E_NULL;
  if (!valid_dtype(dt)) return DFS_E_UNSUPPORTED;
  if (d < 1 || d > kMaxD) return DFS_E_SHAPE;
  if (d % 8 != 0) return DFS_E_UNSUPPORTED;
  if (!aligned(W_h, 16) || !aligned(out_packed, 16)) return DFS_E_ALIGN;
  const size_t need = dfs_gate_pack_bytes(d, dt);
  if (out_bytes < need) return DFS_E_WORKSPACE;
  const size_t in_bytes = (size_t)d * DFS_E * (size_t)esize(dt);
  if (overlaps(W_h, in_bytes, out_packed, need)) return DFS_E_ARG;
  int st = check_device();
  if (st != DFS_OK) return st;
  (void)hipGetLastError();
  if (dt == DFS_F32) return hip_status(hipMemcpyAsync(out_packed, W_h, need, hipMemcpyDeviceToDevice, stream));
  return hip_status(launch_gate_pack(W_h, d, out_packed, stream));
}

int dfs_pair_scores(const int32_t* cand_idx, const float* cand_val, const int32_t* prev_token,
                    const float* gate, const void* A, const void* B, dfs_dtype_t table_dt,
                    int64_t batch, int64_t L, int64_t V, int64_t E, int k, float* out_pair,
                    hipStream_t stream) {
  if (!cand_idx || !cand_val || !prev_token || !gate || !A || !B || !out_pair) return DFS_E_NULL;
  if (!valid_dtype(table_dt) || k != DFS_K || E != DFS_E) return DFS_E_UNSUPPORTED;
  if (batch < 1 || L < 1 || L > DFS_MAX_L || batch > DFS_MAX_ROWS / L || V < DFS_K || V > kMaxV)
    return DFS_E_SHAPE;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(gate, 16) || !aligned(cand_idx, 4) ||
      !aligned(cand_val, 4) || !aligned(prev_token, 4) || !aligned(out_pair, 4))
    return DFS_E_ALIGN;
  int st = check_device();
  if (st != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_pair_walk(cand_lists(cand_idx, cand_val), prev_token, GateSrc{gate, 1, 0}, A, B,
                                     table_dt == DFS_BF16, batch, L, V, out_pair, nullptr, nullptr,
                                     nullptr, stream));
}

int dfs_walk(const float* pair, const int32_t* cand_idx, int64_t batch, int64_t L, int k,
             dfs_walk_t mode, double temperature, uint64_t seed, int32_t* out_path,
             float* out_scores, hipStream_t stream) {
  if (!pair || !cand_idx || !out_path || !out_scores) return DFS_E_NULL;
  if (k != DFS_K) return DFS_E_UNSUPPORTED;
  int st = check_walk_mode(mode, temperature);
  if (st != DFS_OK) return st;
  if (batch < 1 || L < 1 || L > DFS_MAX_L || batch > DFS_MAX_ROWS / L) return DFS_E_SHAPE;
  if (!aligned(pair, 4) || !aligned(cand_idx, 4) || !aligned(out_path, 4) ||
      !aligned(out_scores, 4))
    return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  const WalkArgs w{(int)mode, temperature, seed};
  return hip_status(launch_walk(pair, cand_idx, batch, L, w, out_path, out_scores, stream));
}

size_t dfs_select_workspace_bytes(const dfs_shape_t* shape) {
  if (check_shape(shape) != DFS_OK) return 0;
  return select_layout(*shape).total;
}

}  // extern "C"

int dfs::select_with_workspace(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                               const void* B, const void* W_h, bool wh_packed, int k, const dfs_shape_t* shape,
                               int mode, double temperature, uint64_t seed, void* ws, size_t ws_bytes,
                               int32_t* out_path, float* out_scores, hipStream_t stream) {
  return select_entry(logits, hidden, prev_token, A, B, W_h, wh_packed, k, shape, (dfs_walk_t)mode, temperature,
                      seed, ws, ws_bytes, out_path, out_scores, nullptr, nullptr, stream);
}

int dfs::select_static_checks(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                              const void* B, const void* W_h, int k, const dfs_shape_t* shape, int mode,
                              double temperature, int32_t* out_path, float* out_scores) {
  return select_host_checks(logits, hidden, prev_token, A, B, W_h, k, shape, (dfs_walk_t)mode, temperature, out_path,
                            out_scores);
}

size_t dfs::select_workspace_need(const dfs_shape_t* shape) {
  if (check_shape(shape) != DFS_OK) return 0;
  return select_layout(*shape).total;
}

extern "C" {

int dfs_select(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
               const void* B, const void* W_h, int k, const dfs_shape_t* shape, dfs_walk_t mode,
               double temperature, uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
               float* out_scores, hipStream_t stream) {
  return select_entry(logits, hidden, prev_token, A, B, W_h, false, k, shape, mode, temperature, seed, ws,
                      ws_bytes, out_path, out_scores, nullptr, nullptr, stream);
}

int dfs_select_packed(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                      const void* B, const void* W_packed, int k, const dfs_shape_t* shape, dfs_walk_t mode,
                      double temperature, uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
                      float* out_scores, hipStream_t stream) {
  return select_entry(logits, hidden, prev_token, A, B, W_packed, true, k, shape, mode, temperature, seed, ws,
                      ws_bytes, out_path, out_scores, nullptr, nullptr, stream);
}

int dfs_select_draft(const void* logits, const void* hidden, const int32_t* prev_token,
                     const void* A, const void* B, const void* W_h, int k,
                     const dfs_shape_t* shape, dfs_walk_t mode, double temperature, uint64_t seed,
                     void* ws, size_t ws_bytes, int32_t* out_path, float* out_scores,
                     float* out_q, int32_t* out_cand, hipStream_t stream) {
  if (!out_q || !out_cand) return DFS_E_NULL;
  return select_entry(logits, hidden, prev_token, A, B, W_h, false, k, shape, mode, temperature, seed, ws,
                      ws_bytes, out_path, out_scores, out_q, out_cand, stream);
}

int dfs_select_draft_packed(const void* logits, const void* hidden, const int32_t* prev_token,
                            const void* A, const void* B, const void* W_packed, int k,
                            const dfs_shape_t* shape, dfs_walk_t mode, double temperature, uint64_t seed,
                            void* ws, size_t ws_bytes, int32_t* out_path, float* out_scores,
                            float* out_q, int32_t* out_cand, hipStream_t stream) {
  if (!out_q || !out_cand) return DFS_E_NULL;
  return select_entry(logits, hidden, prev_token, A, B, W_packed, true, k, shape, mode, temperature, seed, ws,
                      ws_bytes, out_path, out_scores, out_q, out_cand, stream);
}

size_t dfs_verify_workspace_bytes(int64_t batch, int64_t L, int64_t V, dfs_dtype_t dt) {
  if (batch < 1 || L < 1 || L > DFS_MAX_L || batch > DFS_MAX_ROWS / (L + 1) || V < DFS_K ||
      V > verify_max_vocab() || !valid_dtype(dt))
    return 0;
  return plan_verify(batch, L, V, esize(dt)).ws_bytes;
}

int dfs_verify(const void* target_logits, dfs_dtype_t dt, int64_t batch, int64_t L, int64_t V,
               const int32_t* path, const int32_t* cand, const float* q, int k, double temperature,
               uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_accepted, int32_t* out_token,
               hipStream_t stream) {
  if (!target_logits || !path || !cand || !q || !out_accepted || !out_token || !ws)
    return DFS_E_NULL;
  if (!valid_dtype(dt) || k != DFS_K) return DFS_E_UNSUPPORTED;
  if (batch < 1 || L < 1 || L > DFS_MAX_L || batch > DFS_MAX_ROWS / (L + 1) || V < DFS_K ||
      V > verify_max_vocab())
    return DFS_E_SHAPE;
  if (!(std::isfinite(temperature) && temperature > 0.0)) return DFS_E_ARG;
  if (!aligned(target_logits, esize(dt)) || !aligned(path, 4) || !aligned(cand, 4) ||
      !aligned(q, 4) || !aligned(out_accepted, 4) || !aligned(out_token, 4) || !aligned(ws, 256))
    return DFS_E_ALIGN;
  const VerifyPlan p = plan_verify(batch, L, V, esize(dt));
  if (ws_bytes < p.ws_bytes) return DFS_E_WORKSPACE;
  int st = check_device();
  if (st != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_verify(p, target_logits, dt == DFS_BF16, path, cand, q, temperature,
                                  seed, ws, out_accepted, out_token, stream));
}

// Rows and width the convolution takes; 0 when they are out of range.
static int check_conv2_shape(int64_t batch, int64_t L, int64_t D, int dt) {
  if (!valid_dtype(dt)) return DFS_E_UNSUPPORTED;
  if (batch < 1 || L < 1 || L > DFS_CONV_MAX_L || D < 256 || D > kMaxD) return DFS_E_SHAPE;
  if (D % 256 != 0) return DFS_E_UNSUPPORTED;
  if (batch > DFS_MAX_ROWS / L) return DFS_E_SHAPE;
  if (batch * L * D > kMaxConvElems) return DFS_E_SHAPE;
  if (dt == DFS_F32 && batch * L * D > conv2_max_f32_elems()) return DFS_E_SHAPE;
  return DFS_OK;
}

size_t dfs_conv2_workspace_bytes(int64_t batch, int64_t L, int64_t D, dfs_dtype_t dt) {
  if (check_conv2_shape(batch, L, D, dt) != DFS_OK) return 0;
  return conv2_workspace_bytes(batch * L, D, dt == DFS_BF16);
}

int dfs_conv2(const void* x, const void* x_prev, const void* base, const void* W_c, dfs_dtype_t dt,
              int64_t batch, int64_t L, int64_t D, void* y, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  if (!x || !x_prev || !base || !W_c || !y) return DFS_E_NULL;
  int st = check_conv2_shape(batch, L, D, dt);
  if (st != DFS_OK) return st;
  if (!aligned(x, 16) || !aligned(x_prev, 16) || !aligned(base, 16) || !aligned(W_c, 16) ||
      !aligned(y, 16))
    return DFS_E_ALIGN;
  const size_t es = (size_t)esize(dt);
  const size_t ybytes = (size_t)(batch * L * D) * es;
  if (overlaps(y, ybytes, x, ybytes) || overlaps(y, ybytes, x_prev, (size_t)(batch * D) * es))
    return DFS_E_ARG;
  const size_t need = conv2_workspace_bytes(batch * L, D, dt == DFS_BF16);
  if (need > 0 && (!ws || ws_bytes < need)) return DFS_E_WORKSPACE;
  if (ws && !aligned(ws, 256)) return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_conv2(x, x_prev, base, W_c, dt == DFS_BF16, batch, L, D, y, ws, stream));
}

static int check_lmhead(const void* hidden, const void* W_lm, dfs_dtype_t dt, int64_t rows, int64_t V,
                        int64_t d) {
  if (!hidden || !W_lm) return DFS_E_NULL;
  if (dt != DFS_BF16) return DFS_E_UNSUPPORTED;
  if (!lmhead_shape_ok(rows, V, d)) return DFS_E_SHAPE;
  if (d % 64 != 0) return DFS_E_UNSUPPORTED;
  if (!aligned(hidden, 16) || !aligned(W_lm, 16)) return DFS_E_ALIGN;
  return DFS_OK;
}

size_t dfs_lmhead_topk_workspace_bytes(int64_t rows, int64_t V, int64_t d) {
  if (!lmhead_shape_ok(rows, V, d) || d % 64) return 0;
  return lmhead_workspace_bytes(rows, V, d);
}

int dfs_lmhead_topk(const void* hidden, const void* W_lm, dfs_dtype_t dt, int64_t rows, int64_t V,
                    int64_t d, int k, int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_lmhead(hidden, W_lm, dt, rows, V, d);
  if (st != DFS_OK) return st;
  if (!out_idx || !out_val || !ws) return DFS_E_NULL;
  if (k != DFS_K) return DFS_E_UNSUPPORTED;
  if (!aligned(out_idx, 4) || !aligned(out_val, 4) || !aligned(ws, 256)) return DFS_E_ALIGN;
  if (ws_bytes < lmhead_workspace_bytes(rows, V, d)) return DFS_E_WORKSPACE;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_lmhead_topk(hidden, W_lm, rows, V, d, out_idx, out_val, ws, stream));
}

int dfs_lmhead_logits(const void* hidden, const void* W_lm, dfs_dtype_t dt, int64_t rows, int64_t V,
                      int64_t d, float* out_logits, hipStream_t stream) {
  int st = check_lmhead(hidden, W_lm, dt, rows, V, d);
  if (st != DFS_OK) return st;
  if (!out_logits) return DFS_E_NULL;
  if (!aligned(out_logits, 4)) return DFS_E_ALIGN;
  if ((st = check_device()) != DFS_OK) return st;
  (void)hipGetLastError();
  return hip_status(launch_lmhead_logits(hidden, W_lm, rows, V, d, out_logits, stream));
}

}  // extern "C"
