/*
 * msattn.h -- C ABI of the MInference-style dynamic sparse pre-filling
 * attention library for AMD Instinct MI355X (gfx950).
 *
 * What it computes (the pages this follows):
 *   - MInference abstract (taxoreview listing): long-context attention falls
 *     into three shapes, A-shape, Vertical-Slash and Block-Sparse; a pattern is
 *     fixed per head offline, sparse indices are built per prompt at inference,
 *     and attention is computed only over those indices.
 *   - "MInference 1.0: Accelerating Pre-filling for Long-Context LLMs via
 *     Dynamic Sparse Attention" (research.elamur.ai summary), section
 *     "Summary": the three stages (offline pattern search, online index
 *     estimation, sparse kernels); section "Key points": Vertical-Slash heads
 *     score the last queries against every key, Block-Sparse heads mean-pool
 *     queries and keys in 64-token blocks.
 *   - PIT abstract fragment (same listing): sparse shapes and GPU tiles do not
 *     line up, so the index must say which keys each query tile covers.
 *
 * Conventions for every call:
 *   Layout.   K and V are [H_kv][n][128]; Q and out are [H_q][m][128] with
 *             m = n - 64*q_block0 rows: the queries of sequence positions
 *             64*q_block0 .. n-1 (m = n unless a chunk of a longer prefill is
 *             computed, see ms_problem); bfloat16, row-major, 16-byte aligned
 *             base pointers.  Attention is causal (pre-filling).  Q head h reads
 *             KV head h / (H_q / H_kv).  A batch of sequences of one length is
 *             served by stacking them along the head axis (B*H_q Q heads,
 *             B*H_kv KV heads, sequence-major), within the head limit.
 *   Memory.   Every tensor pointer is a device pointer owned by the caller.
 *             The library allocates nothing and keeps no global state besides a
 *             thread-local error string and, for ms_sparse_attn_noalloc only,
 *             its static scratch array on each GPU and that array's address.
 *             Workspaces and the index arena are caller-allocated, sized by the
 *             *_bytes queries.
 *   Errors.   Arguments are validated on the host before anything is enqueued;
 *             an invalid call returns a status, writes nothing and enqueues
 *             nothing.  MS_ERR_DEVICE carries the HIP message in ms_last_error().
 *             Faults inside kernels surface at the caller's next stream sync.
 *   Streams.  Every call enqueues on the given stream and returns at once; no
 *             call synchronises the device or copies to the host.
 *   Results.  Deterministic: identical inputs give bitwise-identical outputs.
 */
#ifndef MSATTN_H
#define MSATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MS_OK = 0,
  MS_ERR_INVALID_ARG = 1, /* null/misaligned pointer, out-of-range parameter */
  MS_ERR_UNSUPPORTED = 2, /* well-formed but outside this build (head_dim != 128, n % 64 != 0, ...) */
  MS_ERR_CAPACITY = 3,    /* workspace or index arena smaller than the query returned */
  MS_ERR_DEVICE = 4       /* a HIP launch failed; see ms_last_error() */
} ms_status;

/* Per-head sparse pattern (MInference abstract: the three shapes; DENSE is the
 * full causal baseline; GRID is the video pattern the MMInference abstract
 * names: keys at the same spatial position in earlier frames). */
typedef enum { MS_A_SHAPE = 0, MS_VERTICAL_SLASH = 1, MS_BLOCK_SPARSE = 2, MS_DENSE = 3, MS_GRID = 4 } ms_pattern;

typedef enum { MS_OUT_BF16 = 0, MS_OUT_F32 = 1 } ms_out_dtype;

/* One attention layer.  Limits of this build: head_dim == 128, n % 64 == 0,
 * 64 <= n <= 8388608, 1 <= n_q_heads <= 128, n_kv_heads divides n_q_heads,
 * 0 <= q_block0 < n/64.  Below, NBq = n/64 - q_block0 is the number of query
 * blocks of the call; "query block b" is a block of the sequence
 * (q_block0 <= b < n/64) and arrays over query blocks are indexed by
 * b - q_block0. */
typedef struct {
  int64_t n;          /* sequence length: rows of Q and of K/V */
  int32_t n_q_heads;  /* H_q */
  int32_t n_kv_heads; /* H_kv */
  int32_t head_dim;   /* must be 128 */
  float scale;        /* softmax scale on q.k; 0 selects 1/sqrt(head_dim) */
  int32_t out_dtype;  /* ms_out_dtype */
  int32_t q_block0;   /* chunked prefill: the call computes query blocks
                         q_block0 .. n/64-1 only (rows 64*q_block0 .. n-1),
                         attending to all n keys; 0 for the whole sequence.
                         Every result equals the corresponding rows of the
                         whole-sequence call: estimation only reads the last
                         64 query rows and the query blocks' own pools. */
} ms_problem;

/* Pattern and budgets of one Q head (the offline search's output; MInference
 * 1.0 summary, "Summary", first stage).  Fields a pattern does not use are
 * ignored. */
typedef struct {
  int32_t pattern;      /* ms_pattern */
  int32_t last_q;       /* VS: last rows scored against all keys; must be 64 */
  int32_t n_vertical;   /* VS: key columns kept, 0..n */
  int32_t n_slash;      /* VS: diagonals kept, 0..n */
  int32_t block;        /* BS: pooling block; must be 64.  VS: query rows per
                           block of the index, 64 (or 0) or 32 (finer spans:
                           a slash keeps 32 keys per 32-row block) */
  int32_t top_k_blocks; /* BS: key blocks kept per query block, 1..n/64 */
  int32_t sink;         /* A-shape: initial keys kept, 0..n */
  int32_t window;       /* A-shape: local causal window in keys, 1..n; GRID: local offsets 0..window-1, 1..n */
  int32_t grid_stride;  /* GRID: tokens per frame P, 1..n */
  int32_t grid_frames;  /* GRID: earlier frames T kept at the same position, 0..n */
  int32_t grid_width;   /* GRID: half-width w of the kept neighbourhood, 0..n */
} ms_head_params;

/* `params` below always points to n_q_heads entries. */

const char* ms_status_string(ms_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* ms_last_error(void);
int32_t ms_version(void);

/* Host-only check of a problem and its per-head parameters. */
ms_status ms_validate(const ms_problem* prob, const ms_head_params* params);

/* Sizes (in int32 elements) of the packed selection arrays:
 *   vert  : for each VS head in head order, n_vertical ascending key indices j;
 *   slash : for each VS head in head order, n_slash ascending offsets o = i - j;
 *   blocks: for each BS head in head order, [NBq][top_k_blocks] ascending key
 *           block indices per query block, padded with -1 (early query blocks
 *           have fewer than top_k candidates).
 * Heads of other patterns take no space. */
ms_status ms_selection_sizes(const ms_problem* prob, const ms_head_params* params,
                             int64_t* n_vert, int64_t* n_slash, int64_t* n_blocks);

/* Workspace of ms_estimate_vs / ms_estimate_block (same buffer serves both). */
ms_status ms_estimate_workspace_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes);

/* Index arena of ms_build_index: worst-case size, fixed by the parameters (no
 * device round trip).  Per head it holds a CSR over the NBq query blocks:
 *   rng_ptr[NBq+1] int32, rng[2*R] int32 pairs [lo, hi) of key ranges,
 *   col_ptr[NBq+1] int32, col[C] int32 single key columns.
 * ms_index_layout() returns, for each Q head h, the byte offsets
 *   offsets[4h+0] rng_ptr, [4h+1] rng, [4h+2] col_ptr, [4h+3] col
 * from the arena base, and the capacities caps[2h+0] = R_max, caps[2h+1] = C_max
 * (both arrays caller-owned host memory).  Ranges of a query block are sorted,
 * disjoint and non-touching; columns are ascending and lie in no range.  A
 * Vertical-Slash head with block == 32 has a CSR over the 2*NBq query blocks
 * of 32 rows (rows 32b .. 32b+31 for block b - 2*q_block0). */
ms_status ms_index_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes);
ms_status ms_index_layout(const ms_problem* prob, const ms_head_params* params,
                          int64_t* offsets, int64_t* caps);

/* Workspace of the attention kernels: an fp16 copy of V and, from n = 131072
 * on, the counters the per-head kernel's paced mode keeps (4 B per XCD,
 * 8192-key segment and launch of 1024 workgroups; 2 MB at n = 2^20 with 32
 * heads).  The size covers every head set of the problem; ms_dense_attn uses
 * only the V copy. */
ms_status ms_attn_workspace_bytes(const ms_problem* prob, size_t* bytes);

/* Workspace of the one-shot ms_sparse_attn (estimation + index + attention). */
ms_status ms_workspace_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes);

/* Online Vertical-Slash estimation for every VS head (MInference 1.0 summary,
 * "Key points": the last queries scored against all keys).  For rows
 * i in [n-64, n): p_ij = softmax over j <= i of scale * q_i.k_j; vertical
 * scores v_j = sum_i p_ij; slash scores s_o = sum_i p_{i,i-o}.  The top
 * n_vertical of v and top n_slash of s are written ascending to vert/slash
 * (packed, see ms_selection_sizes); equal scores go to the lower index.
 * dbg_v / dbg_s (nullable, fp32 [H_q][n]) receive the scores of VS heads.
 * The last 64 rows of q are rows n-64 .. n-1 of the sequence, so m >= 64. 
 * q, k: device bf16.  ws: device, >= ms_estimate_workspace_bytes. */
ms_status ms_estimate_vs(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                         int32_t* vert, int32_t* slash, float* dbg_v, float* dbg_s,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Online Block-Sparse estimation for every BS head (MInference 1.0 summary,
 * "Key points": 64-token mean pooling).  S_bc = mean(q over block b) .
 * mean(k over block c) for c <= b, in fp32; the top min(top_k, b+1) key
 * blocks per query block go to `blocks` ascending, -1 padded.  dbg_scores
 * (nullable, fp32 [H_q][NBq][n/64]) receives S of BS heads, -inf above the
 * diagonal. */
ms_status ms_estimate_block(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                            int32_t* blocks, float* dbg_scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* Index conversion (MInference abstract: sparse indices from the assigned
 * pattern; PIT fragment: tile coverage).  Per Q head and 64-row query block b:
 *   VS: each slash o <= 64b+63 keeps keys [max(0, 64b-o), 64b+64-o); spans that
 *       overlap or touch merge into ranges; verticals j <= 64b+63 outside every
 *       range become columns.  With block == 32 the same per 32-row block b:
 *       [max(0, 32b-o), 32b+32-o) for o <= 32b+31, verticals j <= 32b+31.
 *   BS: selected key blocks c give [64c, 64c+64), consecutive ones merged.
 *   A-shape: [0, min(sink, 64b+64)) and [max(0, 64b-window+1), 64b+64), merged.
 *   GRID: as VS with no verticals and the fixed offsets 0 .. window-1 and
 *       tP-w .. tP+w for t = 1..T (those >= 0): the same keys of the same
 *       spatial neighbourhood in each of the T previous frames, plus the
 *       local window.
 *   DENSE: [0, 64b+64).
 * vert/slash/blocks: device arrays as written by the estimators (may be null
 * when no head needs them).  index: device arena of >= ms_index_bytes. */
ms_status ms_build_index(const ms_problem* prob, const ms_head_params* params, const int32_t* vert,
                         const int32_t* slash, const int32_t* blocks, void* index, size_t index_bytes,
                         hipStream_t stream);

/* Sparse attention over a built index (MInference 1.0 summary, "Summary",
 * third stage).  Row i of head h attends key j iff j <= i, j lies in a range
 * or column of block i/64, and, for A-shape heads, j < sink or i - j < window.
 * out_i = sum_j softmax_j(scale * q_i.k_j) v_j; a row with no key gives 0.
 * out: bf16 or fp32 per prob->out_dtype.  lse (nullable, fp32 [H_q][m]):
 * natural-log log-sum-exp of the scaled logits, -inf for empty rows.
 * ws: >= ms_attn_workspace_bytes.  Precondition: |v| < 65504 (V is staged as
 * fp16 for the P.V product). */
ms_status ms_sparse_attn_indexed(const ms_problem* prob, const ms_head_params* params, const void* q,
                                 const void* k, const void* v, const void* index, size_t index_bytes, void* out,
                                 float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* One layer end to end: estimation, index conversion and sparse attention.
 * ws: >= ms_workspace_bytes (holds selections, the index and the V copy). */
ms_status ms_sparse_attn(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                         const void* v, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as ms_sparse_attn, computed with the same kernels and bitwise the same
 * results, but with its workspace in a static scratch array inside the
 * library (MS_NOALLOC_SCRATCH_MIB MiB per GPU, reserved when the library's
 * device code is loaded on that GPU and held until the process ends).  The
 * call allocates nothing.  The caller still owns q, k, v, out and lse
 * (layouts as for ms_sparse_attn).  A layer whose ms_workspace_bytes exceeds
 * the scratch returns MS_ERR_CAPACITY before anything is enqueued.  Every call
 * on one GPU uses that GPU's one scratch array (the current device's), which
 * keeps the previous call's contents (nothing in the path needs it zeroed):
 * calls that may overlap on one GPU (different streams or host threads
 * without ordering between them) race and must be serialised by the caller. */
#define MS_NOALLOC_SCRATCH_MIB 128
ms_status ms_sparse_attn_noalloc(const ms_problem* prob, const ms_head_params* params, const void* q,
                                 const void* k, const void* v, void* out, float* lse, hipStream_t stream);
/* Size in bytes of that static scratch. */
ms_status ms_noalloc_scratch_bytes(size_t* bytes);

/* Full causal attention with the same kernel and no index (the baseline the
 * speedups are measured against).  ws: >= ms_attn_workspace_bytes. */
ms_status ms_dense_attn(const ms_problem* prob, const void* q, const void* k, const void* v, void* out,
                        float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* Index-quality instrument (MInference 1.0 summary, "Key points": the share
 * of the attention mass that the kept entries capture).  With lse_sparse from
 * ms_sparse_attn / ms_sparse_attn_indexed and lse_dense from ms_dense_attn on
 * the same q, k and scale (device fp32 [H_q][m] each), the full causal
 * attention of row i puts mass exp(lse_sparse_i - lse_dense_i) on the kept
 * keys of that row; recall[h] (device fp32 [H_q]) receives the mean of that
 * mass over the m rows of head h (an empty sparse row counts 0).  The sum is
 * taken in float64 in a fixed order (deterministic). */
ms_status ms_attention_recall(const ms_problem* prob, const float* lse_sparse, const float* lse_dense,
                              float* recall, hipStream_t stream);

/* Test hook of the paced attention mode: the number of counter reads one wait
 * of a workgroup for the others of its XCD may take (default 4096, about
 * 1 us each) before that workgroup stops pacing for the rest of its walk.
 * 0 turns the waiting off for calls enqueued afterwards (process-wide).
 * Results never depend on it; only the order in which keys are read does.
 * Negative values are rejected (MS_ERR_INVALID_ARG). */
ms_status ms_set_pace_polls(int32_t polls);

/* Test hook of the selection kernel: the k largest of x[0..n) (device fp32),
 * ties to the lower index, written ascending to idx[0..min(k, n)) (device).
 * -0.0 ranks equal to +0.0; x must hold no NaN.  1 <= n <= 2^30, 0 <= k. */
ms_status ms_topk_f32(const float* x, int64_t n, int32_t k, int32_t* idx, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MSATTN_H */
