// Host-side plans and kernel launchers of the selector (internal to libdfs).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfs {

// Workgroups a launch should offer MI355X (256 CUs) to keep every CU busy.
constexpr int64_t kTargetBlocks = 2048;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A W_h packing job (gate_pack.h) riding along with another launch (nslabs == 0: none).
struct PackJob {
  const uint16_t* W;
  int64_t d;
  uint16_t* Wp;
  int nslabs;
};

// A gate GEMM for few rows, as a list of independent 256-thread jobs (gate_tile.h):
// bf16 (pre-packed W_h) tiles of 16 rgroups rows or fp32 8-row tiles; job j = row tile
// j % mtiles of K split j / mtiles.  kchunk: k per split (a multiple of 32 for bf16).
struct GateJobs {
  const void* H = nullptr;
  const void* W = nullptr;  // packed (bf16) or as stored (fp32)
  int64_t rows = 0, d = 0, kchunk = 0;
  int mtiles = 0, splits = 0;  // mtiles * splits jobs (0: none)
  int rgroups = 1;             // bf16: 16-row groups per tile (1 or gtile::kTallGroups)
  float* partial = nullptr;    // [splits, rows, 256] when splits > 1
  float* out = nullptr;        // [rows, 256] when splits == 1
};
// Counters a later launch of the same call needs at zero, cleared by the top-16 launch.
struct ZeroJob {
  uint32_t* p = nullptr;
  int n = 0;
};

// ---------------------------------------------------------------- top-16
struct TopkPlan {
  int64_t rows, V;
  int esize;       // bytes per logit
  int parts;       // chunks per row (1 = no merge pass)
  int64_t chunk;   // elements per chunk, a multiple of the 16-byte vector width
  size_t ws_bytes; // partial lists when parts > 1
};
TopkPlan plan_topk(int64_t rows, int64_t V, int esize);
// Few rows (the fused selector's gate-carrying launch): chunks small enough to be held in
// registers whole where the vocabulary allows it.
TopkPlan plan_topk_small(int64_t rows, int64_t V, int esize);
// `pack` (may be null): W_h packing slabs run as extra workgroups of the same launch.
// merge false (rows split, parts > 1): the partial lists are left in ws for a merge job
// placed elsewhere (topk_merge_job), and out_idx / out_val are not written.
hipError_t launch_topk(const TopkPlan& p, const void* logits, bool bf16, int32_t* out_idx,
                       float* out_val, void* ws, hipStream_t stream,
                       const PackJob* pack = nullptr, bool merge = true, ZeroJob zero = ZeroJob{});

// The top-16 pass (merge false) with the gate's jobs as extra workgroups of the same
// launch (ahead of the rows), for few rows; gate_bf16 selects the gate tile kind.
hipError_t launch_topk_gate(const TopkPlan& p, const void* logits, bool bf16, int32_t* out_idx, float* out_val,
                            void* ws, const GateJobs& g, bool gate_bf16, ZeroJob zero, hipStream_t stream);

// Merge of per-row partial top-16 lists [rows, parts, 16] (64-bit keys, 0 = empty).
hipError_t launch_topk_merge(const uint64_t* partial, int64_t rows, int parts, int32_t* out_idx,
                             float* out_val, hipStream_t stream);

// ---------------------------------------------------------------- gate
// Up to this many rows the bf16 gate runs as 16-row tiles (gate_tile.h), and the fused
// selector puts those tiles (or the fp32 tiles) into its top-16 launch when W_h needs no
// repacking: the top-16 pass runs at most two workgroups per CU there and leaves room.
constexpr int64_t kGateTileRows = 512;

struct GatePlan {
  enum Kind { kJobs = 0, kTile64 = 1, kDma = 2 };
  int64_t rows, d;
  bool bf16;
  int kind;            // kJobs: independent 256-thread tiles (bf16 16 rows, fp32 8 rows);
                       // kTile64: 64-row tiles of eight waves; kDma: 128 x 128 LDS-DMA tiles
  int mtiles;          // row tiles
  int rgroups;         // kJobs, bf16: 16-row groups per tile
  int splits;          // K splits (partial sums added in split order before the sigmoid)
  int64_t kchunk;      // hidden elements per split
  size_t packed_off, packed_bytes;    // W_h packed for the matrix cores (bf16 path)
  size_t partial_off, partial_bytes;  // [splits, rows, 256] fp32
  size_t ws_bytes;
};
GatePlan plan_gate(int64_t rows, int64_t d, bool bf16);
// Bytes of W_h [d, 256] bf16 packed for the matrix cores: [ceil(d/32)][256][32], zero past d.
size_t gate_packed_bytes(int64_t d);
hipError_t launch_gate_pack(const void* W_h, int64_t d, void* Wp, hipStream_t stream);
// The whole gate: pack W_h into the workspace (bf16, unless `prepacked`: W_h is then
// the packed weight), GEMM, finish (when split).
hipError_t launch_gate(const GatePlan& p, const void* hidden, const void* W_h, bool prepacked, float* out_gate,
                       void* ws, hipStream_t stream);
// Its parts, for callers that place them themselves.  The packing job (bf16 only;
// nslabs == 0 otherwise) must complete before the GEMM; with splits > 1 the GEMM
// leaves partial sums [splits, rows, 256] at gate_partials() and out_gate is only
// written by the finish.  W: the packed weight (bf16) or W_h as stored (fp32).
PackJob gate_pack_job(const GatePlan& p, const void* W_h, void* ws);
const void* gate_packed_in_ws(const GatePlan& p, const void* ws);
hipError_t launch_gate_gemm(const GatePlan& p, const void* hidden, const void* W, float* out_gate, void* ws,
                            hipStream_t stream);
hipError_t launch_gate_finish(const GatePlan& p, float* out_gate, void* ws, hipStream_t stream);
const float* gate_partials(const GatePlan& p, const void* ws);
// kind == kJobs: the GEMM as independent workgroup jobs another launch can carry.
GateJobs gate_jobs(const GatePlan& p, const void* hidden, const void* W, float* out_gate, void* ws);

// ---------------------------------------------------------------- pair scores and walk
struct WalkArgs {
  int mode;  // 0 greedy, 1 gumbel, 2 best path
  double temperature;
  uint64_t seed;
  float* out_q = nullptr;       // optional [B, L, 16] draft distributions (fused walk only)
  int32_t* out_cand = nullptr;  // with out_q: [B, L, 16] candidate ids
};
// Where the pair kernel finds the gate: the finished gate [rows, 256] (splits 1), or
// K-split partial sums [splits, rows, 256], `stride` floats apart, which it adds up in
// split order and passes through the sigmoid (the gate's finish kernel does the same).
struct GateSrc {
  const float* gate;
  int splits;
  int64_t stride;
};
// Where it finds the candidates: final lists idx / val [rows, 16] (parts <= 1), or the
// top-16 pass's `parts` (2..64) sorted partial lists per row [rows, parts, 16] of 64-bit
// keys, which it merges itself.
struct CandSrc {
  const int32_t* idx;
  const float* val;
  const uint64_t* partial;
  int parts;
};
inline CandSrc cand_lists(const int32_t* idx, const float* val) { return CandSrc{idx, val, nullptr, 1}; }
// Pair scores for every (sequence, position); optionally written to out_pair and
// optionally followed by the walk in the same kernel (out_path/out_scores non-null).
hipError_t launch_pair_walk(const CandSrc& cand, const int32_t* prev_token, const GateSrc& gate,
                            const void* A, const void* B, bool bf16_tables, int64_t batch, int64_t L,
                            int64_t V, float* out_pair, const WalkArgs* walk, int32_t* out_path,
                            float* out_scores, hipStream_t stream);
// Few rows: one workgroup per (sequence, position), the walk by the last position of each
// sequence to finish (see pair_pos_kernel).  tiles [batch * L]; counters [batch], zero
// before the launch (the top-16 launch of the same call zeroes them) and zero after it.
struct PosTile {
  int32_t next[16];  // successor slot of each predecessor slot
  float best[16];    // its score
  int32_t cand[16];  // candidate ids
  float tile[16][16];
};
constexpr int64_t kPosMaxRows = 64;  // dfs_select takes this path up to this many rows
hipError_t launch_pair_pos(const CandSrc& cand, const int32_t* prev_token, const GateSrc& gate, const void* A,
                           const void* B, bool bf16_tables, int64_t batch, int64_t L, int64_t V,
                           const WalkArgs& walk, int32_t* out_path, float* out_scores, PosTile* tiles,
                           uint32_t* counters, hipStream_t stream);
// Mid-size batches: the [rows, 16, 16] pair tensor from final candidate lists, one wave
// per (sequence, position); launch_walk then walks it.
hipError_t launch_pair_tiles(const int32_t* cand_idx, const float* cand_val, const int32_t* prev_token,
                             const GateSrc& gate, const void* A, const void* B, bool bf16_tables, int64_t batch,
                             int64_t L, int64_t V, float* out_pair, hipStream_t stream);
hipError_t launch_walk(const float* pair, const int32_t* cand_idx, int64_t batch, int64_t L,
                       const WalkArgs& walk, int32_t* out_path, float* out_scores,
                       hipStream_t stream);

// ---------------------------------------------------------------- verification
struct VerifyPlan {
  int64_t batch, L, V;
  int esize;       // bytes per target logit
  int parts;       // workgroups per target row in the log-sum-exp pass
  int64_t nseg;    // segment slots per row
  size_t ws_bytes; // (max, sum) per segment [batch * (L + 1), nseg], fp64 pairs
};
VerifyPlan plan_verify(int64_t batch, int64_t L, int64_t V, int esize);
int64_t verify_max_vocab();  // the draw keeps a row's segment masses in LDS
hipError_t launch_verify(const VerifyPlan& p, const void* logits, bool bf16, const int32_t* path,
                         const int32_t* cand, const float* q, double temperature, uint64_t seed,
                         void* ws, int32_t* out_accepted, int32_t* out_token, hipStream_t stream);

// ---------------------------------------------------------------- two-tap convolution
// bf16: one fused kernel (no workspace).  fp32: correction [rows, D/8] in `ws`, then
// an elementwise kernel; its launches need rows * D below conv2_max_f32_elems().
size_t conv2_workspace_bytes(int64_t rows, int64_t D, bool bf16);
int64_t conv2_max_f32_elems();
hipError_t launch_conv2(const void* x, const void* x_prev, const void* base, const void* W_c,
                        bool bf16, int64_t batch, int64_t L, int64_t D, void* y, void* ws,
                        hipStream_t stream);

// ---------------------------------------------------------------- LM head -> top-16
// bf16 hidden [rows, d] and W_lm [V, d], d a multiple of 64.
size_t lmhead_workspace_bytes(int64_t rows, int64_t V, int64_t d);
hipError_t launch_lmhead_topk(const void* hidden, const void* W_lm, int64_t rows, int64_t V, int64_t d,
                              int32_t* out_idx, float* out_val, void* ws, hipStream_t stream);
hipError_t launch_lmhead_logits(const void* hidden, const void* W_lm, int64_t rows, int64_t V, int64_t d,
                                float* out, hipStream_t stream);

}  // namespace dfs
