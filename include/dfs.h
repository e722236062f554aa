/*
 * dfs.h -- C ABI of the DFlash 2 draft-path selector for AMD Instinct MI355X (gfx950).
 *
 * What is computed (blog post "DFlash 2: Keep Drafting Parallel", Inco AI, 2026):
 *   1. per block position t, keep the 16 highest-logit candidates C_t of the
 *      drafter's vocabulary logits U_t                     (section "The Right Tokens
 *      Are Already There");
 *   2. score every adjacent (predecessor a, candidate b) pair
 *         S_t(a,b) = U_t(b) + < A(a) (elementwise) H(h_t), B(b) >
 *      with 256-wide token embeddings A, B and a context gate H(h_t) computed from
 *      the drafter hidden state h_t   (section "A Lightweight Path Selector"; the
 *      equation itself survives in the twiscan.com Chinese translation);
 *   3. walk the precomputed scores once from the last verified token: greedy takes
 *      the best successor at each step, sampling draws from the same scores;
 *   4. no extra backbone or LM-head pass: only the drafter's outputs are read.
 *
 * Parameterisation chosen here where the pages are silent:
 *   H(h_t) = sigmoid(h_t W_h), W_h of shape [d, 256];  A, B are [V, 256] tables.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, except the
 *     dfs_shape_t pointer, which is host memory read during the call only.  The
 *     library allocates no memory and keeps no pointer after it returns.
 *   - Every call only enqueues kernels on `stream` (NULL = the device's null
 *     stream) on the current HIP device and returns without synchronising.
 *     Results are valid once the stream has reached that point.
 *   - All tensors are dense and row-major (C order) with the shapes given.
 *   - Return value: DFS_OK (0) or one of the positive dfs_status_t codes.
 *     Arguments are checked on the host before anything is enqueued; on an error
 *     nothing is enqueued and no output is written.  dfs_status_str() names a code.
 *   - Device-side contracts that are not checked: logits hold no NaN (-inf is
 *     allowed), every token id passed in lies in [0, V), and input and output
 *     buffers do not overlap.
 *   - Calls on different streams may run concurrently; calls that share a
 *     workspace buffer must be ordered by the caller.
 *   - Results are bitwise deterministic for identical inputs.
 */
#ifndef DFS_H_
#define DFS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFS_K 16      /* candidates kept per block position */
#define DFS_E 256     /* embedding and gate width */
#define DFS_MAX_L 16  /* longest block handled; the post's blocks span 4 to 16 tokens */
#define DFS_MAX_D (1 << 20) /* widest hidden state handled */
/* Most rows per call: logit or hidden-state rows (B*L; B*(L+1) target rows for verification).
   Larger calls return DFS_E_SHAPE before anything is launched, so that no launch grid
   exceeds 2^31 work-items. */
#define DFS_MAX_ROWS (1 << 22)
#define DFS_CONV_MAX_L 65536 /* longest run of positions dfs_conv2 takes per sequence */

/* C++ builds give the enums int as their fixed underlying type, so that every int a caller
   passes (an unknown dtype or walk mode, say) is a value of the type that the argument
   checks then reject, as in C; the size and calling convention are those of int either way. */
#ifdef __cplusplus
#define DFS_ENUM_BASE : int
#else
#define DFS_ENUM_BASE
#endif

typedef enum DFS_ENUM_BASE {
  DFS_OK = 0,
  DFS_E_NULL = 1,        /* a required pointer is NULL */
  DFS_E_SHAPE = 2,       /* a size is out of range (batch, rows < 1; V < 16; L not in [1,16];
                            d not in [1, DFS_MAX_D]; ...) */
  DFS_E_UNSUPPORTED = 3, /* k != 16, E != 256, an unknown dtype or walk mode, or d not a multiple of 8 */
  DFS_E_WORKSPACE = 4,   /* workspace NULL or smaller than the matching *_workspace_bytes() */
  DFS_E_ALIGN = 5,       /* a pointer is not aligned as documented */
  DFS_E_HIP = 6,         /* no usable HIP device, or a HIP launch error */
  DFS_E_ARCH = 7,        /* the current device is not gfx950 */
  DFS_E_ARG = 8,         /* an argument is invalid (temperature <= 0 for sampling; an output
                            that overlaps an input) */
  DFS_E_TOO_LARGE = 9    /* dfs_select_packed_static: the call needs more scratch than
                            DFS_STATIC_SCRATCH_BYTES */
} dfs_status_t;

typedef enum DFS_ENUM_BASE { DFS_F32 = 0, DFS_BF16 = 1 } dfs_dtype_t;

typedef enum DFS_ENUM_BASE {
  DFS_WALK_GREEDY = 0, /* argmax successor at each step, lowest candidate slot on ties */
  DFS_WALK_GUMBEL = 1, /* Gumbel-max draw from softmax(S / temperature) over the 16 candidates */
  DFS_WALK_VITERBI = 2 /* the path of largest summed score (dynamic programming), see dfs_walk */
} dfs_walk_t;

/* Shape of one dfs_select call. */
typedef struct {
  int64_t batch;             /* sequences, >= 1 */
  int64_t L;                 /* block positions per sequence, 1..16 */
  int64_t V;                 /* vocabulary size, 16..2^31-1 */
  int64_t d;                 /* drafter hidden width, 8..DFS_MAX_D, multiple of 8 */
  dfs_dtype_t logits_dtype;  /* logits */
  dfs_dtype_t act_dtype;     /* hidden and W_h */
  dfs_dtype_t table_dtype;   /* A and B */
} dfs_shape_t;

/* ---------------------------------------------------------------- top-16
 * Step 1.  The post observes that the right token is usually among the drafter's 16
 * best candidates even when its top pick is wrong, and keeps those 16 per block
 * position (blog post "DFlash 2: Keep Drafting Parallel", section "The Right Tokens Are
 * Already There", Table 1's recall@16).
 * For each of `rows` rows of `logits` [rows, V] (dtype dt), the k = 16 largest
 * entries ordered by value descending, then token id ascending (ties go to the
 * lower id); -0 and +0 count as equal and +0 is reported.
 *   out_idx [rows, 16] int32 token ids;  out_val [rows, 16] fp32 values (exact
 *   widening of the input values).
 * Alignment: logits to its element size; out_idx, out_val to 4 bytes; ws to 256.
 * ws: dfs_topk_workspace_bytes(rows, V, dt) bytes of scratch (may be 0, then ws may
 * be NULL).                                                                      */
size_t dfs_topk_workspace_bytes(int64_t rows, int64_t V, dfs_dtype_t dt);
int dfs_topk(const void* logits, dfs_dtype_t dt, int64_t rows, int64_t V, int k,
             int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- context gate
 * Step 2.  The score weights each candidate pair's embedding match by a context gate
 * computed from the drafter's hidden state, H(h_t) (section "A Lightweight Path
 * Selector"; the symbol survives in the twiscan.com Chinese translation's equation).
 * The pages do not say how H is built; this library takes a sigmoid of a linear map:
 * out_gate[r, e] = sigmoid( sum_c hidden[r, c] * W_h[c, e] ),  r < rows, e < E = 256.
 *   hidden [rows, d] and W_h [d, 256] of dtype dt; products and sums in fp32;
 *   out_gate [rows, 256] fp32.
 * Alignment: hidden, W_h 16 bytes; out_gate 4 bytes; ws 256 bytes.
 * ws: dfs_gate_workspace_bytes(rows, d, dt) bytes of scratch.                       */
size_t dfs_gate_workspace_bytes(int64_t rows, int64_t d, dfs_dtype_t dt);
int dfs_gate(const void* hidden, const void* W_h, dfs_dtype_t dt, int64_t rows, int64_t d,
             int64_t E, float* out_gate, void* ws, size_t ws_bytes, hipStream_t stream);

/* W_h packed once for the gate's matrix cores, for callers that keep the weight across
 * calls (it is a constant of the drafter).  bf16: the packed layout is
 * [ceil(d/32)][256][32] (slab kb, column n, then the 32 k values 32 kb .. 32 kb + 31 of
 * that column; zero past d); fp32: a plain copy of W_h.  out_packed must hold
 * dfs_gate_pack_bytes(d, dt) bytes (16-byte aligned) and must not overlap W_h; it is
 * caller-owned device memory, written on `stream`.  dfs_gate_packed,
 * dfs_select_packed and dfs_select_draft_packed take it in place of W_h and give the
 * same bits as their unpacked forms, without repacking W_h on every call. */
size_t dfs_gate_pack_bytes(int64_t d, dfs_dtype_t dt);
int dfs_gate_pack(const void* W_h, dfs_dtype_t dt, int64_t d, void* out_packed, size_t out_bytes,
                  hipStream_t stream);
int dfs_gate_packed(const void* hidden, const void* W_packed, dfs_dtype_t dt, int64_t rows, int64_t d,
                    int64_t E, float* out_gate, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- pair scores
 * Step 3.  Every adjacent (predecessor a, candidate b) pair is scored at once by
 *   S_t(a, b) = U_t(b) + < A(a) (elementwise) H(h_t), B(b) >
 * (section "A Lightweight Path Selector", equation as printed in the twiscan.com
 * Chinese and decomputer.nl Dutch translations; the bud-325 wiki summary notes the
 * 16 x 16 x K score tensor is computed once).  U_t(b) is the drafter's own logit.
 * For sequence b and position t (row r = b*L + t):
 *   t >= 1:  out_pair[b, t, i, j] = cand_val[r, j]
 *              + sum_e A[cand_idx[r-1, i], e] * gate[r, e] * B[cand_idx[r, j], e]
 *   t == 0:  the predecessor is prev_token[b] for every slot i (the row repeats).
 *   cand_idx [batch, L, 16] int32, cand_val [batch, L, 16] fp32 (a dfs_topk result),
 *   prev_token [batch] int32 (last verified token), gate [batch*L, 256] fp32
 *   (a dfs_gate result), A, B [V, 256] of dtype table_dt.
 *   out_pair [batch, L, 16, 16] fp32.  Sums in fp32 on the matrix cores; for bf16
 *   tables the gated predecessor embedding is split into two bf16 terms, so the
 *   product is exact to about 2^-17 relative before fp32 accumulation.
 * Alignment: A, B, gate 16 bytes; the int32/fp32 arrays 4 bytes.                   */
int dfs_pair_scores(const int32_t* cand_idx, const float* cand_val, const int32_t* prev_token,
                    const float* gate, const void* A, const void* B, dfs_dtype_t table_dt,
                    int64_t batch, int64_t L, int64_t V, int64_t E, int k, float* out_pair,
                    hipStream_t stream);

/* ---------------------------------------------------------------- walk
 * Step 4, the only sequential work: from the last verified token, greedy follows the
 * best successor at each step and sampling draws from the same scores (section "A
 * Lightweight Path Selector").
 * One walk per sequence over pair [batch, L, 16, 16] (a dfs_pair_scores result):
 * start at predecessor slot 0 of position 0 (the last verified token's row); at
 * step t choose slot j* in row i (the previous choice):
 *   greedy:  j* = argmax_j pair[b,t,i,j], lowest j on ties;
 *   gumbel:  j* = argmax_j pair[b,t,i,j] / temperature + g(seed, b, t, j), in fp64,
 *            g = -log(-log(u)), u = ((x >> 9) + 0.5) * 2^-23, x = word 0 of
 *            Philox4x32-10 with counter (j, t, b, 0) and key (seed low, seed high).
 *   viterbi: the slot path maximising sum_t pair[b, t, j_{t-1}, j_t] (j_{-1} = 0), found
 *            by dynamic programming in fp32: best_0[j] = pair[b,0,0,j], best_t[j] =
 *            max_i best_{t-1}[i] + pair[b,t,i,j] keeping the lowest i on ties, last
 *            slot the lowest j of largest best_{L-1}[j], read back from there.  The
 *            pages leave better selectors than the greedy one open (blog post, section
 *            "A Lightweight Path Selector"); this is the exact best path over the
 *            same scores.
 *   out_path [batch, L] int32 = cand_idx[b, t, j*];
 *   out_scores [batch, L] fp32 = pair[b, t, i, j*] (un-noised, not divided by T).
 * temperature must be finite and > 0 in gumbel mode (ignored otherwise).          */
int dfs_walk(const float* pair, const int32_t* cand_idx, int64_t batch, int64_t L, int k,
             dfs_walk_t mode, double temperature, uint64_t seed, int32_t* out_path,
             float* out_scores, hipStream_t stream);

/* ---------------------------------------------------------------- fused selector
 * The whole selector: dfs_topk over logits [batch, L, V], dfs_gate over hidden
 * [batch, L, d] with W_h [d, 256], then pair scores and the walk fused in one
 * kernel (scores stay on chip).  Same results, bit for bit, as calling the four
 * steps in turn.  Everything is enqueued on `stream` alone.
 * prev_token [batch] int32; A, B [V, 256]; out_path [batch, L] int32; out_scores
 * [batch, L] fp32.  Alignment as in the step entry points; ws 256 bytes.
 * ws: dfs_select_workspace_bytes(shape) bytes of scratch (about 24 MB at batch 256,
 * L 16, V 151936, d 5120).                                                        */
size_t dfs_select_workspace_bytes(const dfs_shape_t* shape);
int dfs_select(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
               const void* B, const void* W_h, int k, const dfs_shape_t* shape, dfs_walk_t mode,
               double temperature, uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
               float* out_scores, hipStream_t stream);
/* dfs_select with W_h already packed by dfs_gate_pack (the same bits).  With few rows
 * (batch * L <= 512) the gate then runs inside the top-16 launch; up to 64 rows a call
 * is two kernels. */
int dfs_select_packed(const void* logits, const void* hidden, const int32_t* prev_token, const void* A,
                      const void* B, const void* W_packed, int k, const dfs_shape_t* shape, dfs_walk_t mode,
                      double temperature, uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
                      float* out_scores, hipStream_t stream);

/* ---------------------------------------------------------------- draft distributions
 * dfs_select plus the draft distribution the walk drew from at every position:
 *   out_q [batch, L, 16] fp32: q[b, t, j] = softmax_j(S_t(slot[t-1], j) / temperature),
 *     slot[-1] = 0 (the last verified token's row), over the 16 candidates of position
 *     t; in gumbel mode this is exactly the distribution each step was drawn from.
 *   out_cand [batch, L, 16] int32: the candidate ids (cand_idx of the top-16 step).
 * temperature must be finite and > 0 in every mode here.  Together with out_path
 * these are what speculative-sampling verification (dfs_verify) needs.            */
int dfs_select_draft(const void* logits, const void* hidden, const int32_t* prev_token,
                     const void* A, const void* B, const void* W_h, int k,
                     const dfs_shape_t* shape, dfs_walk_t mode, double temperature,
                     uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
                     float* out_scores, float* out_q, int32_t* out_cand, hipStream_t stream);
/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): dfs_select_packed without a workspace.
 * Its scratch is a device array of DFS_STATIC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends (its device address is looked up on the first call on
 * each device, which must therefore happen outside graph capture).  It allocates nothing
 * and gives the same bits as dfs_select_packed.  Calls needing more scratch than the array
 * holds (dfs_select_workspace_bytes(shape) > DFS_STATIC_SCRATCH_BYTES) return
 * DFS_E_TOO_LARGE before anything is launched.  Every call on one GPU uses that GPU's one
 * array: calls that overlap on one GPU (two streams, two host threads) race and must be
 * ordered by the caller.  The array keeps nothing that a later call relies on. */
#define DFS_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int dfs_select_packed_static(const void* logits, const void* hidden, const int32_t* prev_token,
                             const void* A, const void* B, const void* W_packed, int k,
                             const dfs_shape_t* shape, dfs_walk_t mode, double temperature,
                             uint64_t seed, int32_t* out_path, float* out_scores, hipStream_t stream);

/* dfs_select_draft with W_h packed by dfs_gate_pack. */
int dfs_select_draft_packed(const void* logits, const void* hidden, const int32_t* prev_token,
                            const void* A, const void* B, const void* W_packed, int k,
                            const dfs_shape_t* shape, dfs_walk_t mode, double temperature,
                            uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_path,
                            float* out_scores, float* out_q, int32_t* out_cand, hipStream_t stream);

/* ---------------------------------------------------------------- verification
 * Speculative-sampling verification of drafted blocks (Leviathan, Kalman and Matias,
 * ICML 2023; Chen et al., 2023) against a target distribution p_t = softmax(z_t / T)
 * over the vocabulary, z = target_logits [batch, L + 1, V] (dtype dt; row L is the
 * target's next token after the whole block).  For block b and t = 0, 1, ...: the
 * draft token x = path[b, t] with q_x = q[b, t, j] (cand[b, t, j] == x) is accepted
 * when u < p_t(x) / q_x, u = ((w0 >> 9) + 0.5) 2^-23 from word w0 of Philox4x32-10
 * counter (0, t, b, 1), key (seed low, seed high), ratio in fp64.  At the first
 * rejection t = k (or k = L when all are accepted) one token is drawn by inverse CDF
 * over the vocabulary, in id order, from weights max(0, p_k - q_k) (q_k zero off the
 * candidates; k = L: p_L): the smallest v whose running weight reaches u2 times the
 * total, u2 = ((w0 >> 9) 2^23 + (w1 >> 9) + 0.5) 2^-46 from counter (0, k, b, 2).
 * Probabilities in fp32 against an fp32 log-sum-exp; running sums in fp64.
 *   path [batch, L] int32, cand / q [batch, L, 16] (dfs_select_draft outputs);
 *   out_accepted [batch] int32 = k; out_token [batch] int32 = the drawn token.
 * temperature finite and > 0.  Alignment: target_logits to its element size, the
 * int32 / fp32 arrays 4 bytes, ws 256 bytes.
 * ws: dfs_verify_workspace_bytes(batch, L, V, dt) bytes of scratch (never 0).     */
size_t dfs_verify_workspace_bytes(int64_t batch, int64_t L, int64_t V, dfs_dtype_t dt);
int dfs_verify(const void* target_logits, dfs_dtype_t dt, int64_t batch, int64_t L, int64_t V,
               const int32_t* path, const int32_t* cand, const float* q, int k, double temperature,
               uint64_t seed, void* ws, size_t ws_bytes, int32_t* out_accepted, int32_t* out_token,
               hipStream_t stream);

/* ---------------------------------------------------------------- two-tap convolution
 * The drafter's two-tap dynamic depthwise convolution across block positions (blog
 * post "DFlash 2: Keep Drafting Parallel", section "A Lightweight Local
 * Convolution"; its equation Conv_k(x)_t = k_{t,0} . x_t + k_{t,1} . x_{t-1}):
 *   c_t[2g + tap]   = sum_i W_c[g, tap, i] x_t[i]          (one correction per 16 channels)
 *   k_{t,tap}[ch]   = base[tap, ch] + c_t[2 (ch / 16) + tap]
 *   y_t[ch]         = k_{t,0}[ch] x_t[ch] + k_{t,1}[ch] x_{t-1}[ch],  x_{-1} = x_prev
 *   x [batch, L, D]   the sublayer input at every block position (row-major)
 *   x_prev [batch, D] the last verified token's representation at the same site
 *   base [2, D]       the learned base kernel (tap 0: current position, tap 1: predecessor)
 *   W_c [D/16, 2, D]  correction weights, K-contiguous (row 2g + tap)
 *   y [batch, L, D]   output, same dtype as the inputs; must not overlap x or x_prev
 * All of dtype dt (bf16: correction on the matrix cores with fp32 sums, y rounded to
 * nearest-even bf16; fp32: fp32 throughout).  D a multiple of 256 in [256, DFS_MAX_D],
 * 1 <= L <= DFS_CONV_MAX_L, batch * L <= DFS_MAX_ROWS, batch * L * D <= 2^36 (fp32: <= 2^32).  Every
 * pointer 16-byte aligned, ws 256-byte aligned.
 * ws: dfs_conv2_workspace_bytes(batch, L, D, dt) bytes: split partial sums of the bf16
 * correction when the shape is too small to fill the chip, else 0 (ws may then be NULL). */
size_t dfs_conv2_workspace_bytes(int64_t batch, int64_t L, int64_t D, dfs_dtype_t dt);
int dfs_conv2(const void* x, const void* x_prev, const void* base, const void* W_c, dfs_dtype_t dt,
              int64_t batch, int64_t L, int64_t D, void* y, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* ---------------------------------------------------------------- LM head -> top-16
 * The candidates straight from the drafter's hidden state: the selector reads the
 * drafter's logits and needs no extra LM-head pass (blog post "DFlash 2: Keep
 * Drafting Parallel", section "A Lightweight Path Selector"); the logits are
 * U = h W_lm^T, and the 16 largest per row are the candidates (section "The Right
 * Tokens Are Already There").  dfs_lmhead_topk computes the product on the matrix
 * cores (fp32 sums) and keeps only the running top-16 per row: U is not written
 * (for at most 32 rows, where U is small, it goes through the workspace and the
 * top-16 pass, the faster way there; the result is the same).
 *   hidden [rows, d] bf16 (row-major), W_lm [V, d] bf16 (one row per token)
 *   out_idx [rows, 16] int32, out_val [rows, 16] fp32: value descending, then the
 *     lower id, on the fp32 sums -- exactly dfs_topk run on dfs_lmhead_logits' U.
 * dt must be DFS_BF16; d a multiple of 64 in [64, DFS_MAX_D]; 16 <= V < 2^31;
 * 1 <= rows <= DFS_MAX_ROWS and ceil(rows / 128) * ceil(V / 128) <= 2^23.  hidden and W_lm
 * 16-byte aligned, outputs 4, ws 256.
 * ws: dfs_lmhead_topk_workspace_bytes(rows, V, d) bytes (never 0): per-row lists of
 * the column stripes, merged at the end (for <= 32 rows: U and the top-16 pass's
 * lists).  Finite inputs whose sums stay finite. */
size_t dfs_lmhead_topk_workspace_bytes(int64_t rows, int64_t V, int64_t d);
int dfs_lmhead_topk(const void* hidden, const void* W_lm, dfs_dtype_t dt, int64_t rows, int64_t V,
                    int64_t d, int k, int32_t* out_idx, float* out_val, void* ws, size_t ws_bytes,
                    hipStream_t stream);
/* The same product written out: out_logits [rows, V] fp32 (the unfused chain's first
 * step, and the reference the fused result is checked against). */
int dfs_lmhead_logits(const void* hidden, const void* W_lm, dfs_dtype_t dt, int64_t rows, int64_t V,
                      int64_t d, float* out_logits, hipStream_t stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* dfs_status_str(int status);

/* ABI version of this header and library (major * 100 + minor). */
#define DFS_ABI_VERSION 105
int dfs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFS_H_ */
