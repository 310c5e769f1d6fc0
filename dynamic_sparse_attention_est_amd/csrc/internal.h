// Internal declarations shared by the host dispatcher and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msattn.h"

namespace msa {

constexpr int kD = 128;        // head dimension
constexpr int kBM = 64;        // query rows per query block; Block-Sparse pooling block
constexpr int kLastQ = 64;     // rows scored by the Vertical-Slash estimator
constexpr int kMaxHeads = 128; // Q heads per call

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Per-Q-head record at the start of the index arena (written by a small
// kernel from kernel arguments, read by the index builders and attention).
struct HeadDesc {
  int32_t pattern;
  int32_t p0, p1;    // VS: n_vertical, n_slash.  BS: top_k, -.  A: sink, window.  GRID: stride, window
  int32_t vs_slot;   // rank among VS heads (-1 if not VS)
  int32_t bs_slot;   // rank among BS heads (-1 if not BS)
  int32_t p2, p3;    // GRID: frames, width
  int32_t qrows;     // query rows per block of the head's CSR: 64, or 32 for a VS head that asks for it
  int64_t vert_off;  // int32 elements into the packed vert array (VS)
  int64_t slash_off; // into the packed slash array (VS)
  int64_t blk_off;   // into the packed blocks array (BS)
  int64_t rng_ptr_off, rng_off, col_ptr_off, col_off, run_off;  // bytes from arena base
};
static_assert(sizeof(HeadDesc) == 96, "HeadDesc layout");
constexpr int64_t kTableBytes = (int64_t)kMaxHeads * sizeof(HeadDesc);

// Query heads per attention workgroup: the heads of one KV head are served
// together in chunks of hpw_of(group size) heads.
inline __host__ __device__ int hpw_of(int grp) { return grp % 4 == 0 ? 4 : grp % 2 == 0 ? 2 : 1; }

// Per-chunk record (after the head table in the index arena): up to four Q
// heads of one KV head that attention serves together, and the union of
// their index (union_index.hip).
struct GroupDesc {
  int16_t head[4];   // Q heads head[0 .. nheads)
  int32_t kvh, nheads;
  int64_t urng_ptr_off, urng_off, ucol_ptr_off, ucol_off, umask_off;  // bytes from arena base
  int64_t pad;
};
static_assert(sizeof(GroupDesc) == 64, "GroupDesc layout");
constexpr int64_t kGroupTableBytes = (int64_t)kMaxHeads * sizeof(GroupDesc);
struct GroupTableArgs {
  static constexpr int kMax = 32;
  GroupDesc g[kMax];
};

// ------------------------------------------------------------------ launchers
// Every launcher enqueues on `s` and returns hipGetLastError().

// Writes `count` descriptors at table[first..first+count).
hipError_t launch_write_table(HeadDesc* table, const HeadDesc* host_descs, int first, int count, hipStream_t s);

// Vertical-Slash estimation.
struct VsGroups {
  int32_t n_groups;                 // KV heads that serve VS heads, at most four VS heads a group
  int16_t kv_head[kMaxHeads];       // per group
  int16_t q_begin[kMaxHeads + 1];   // per group: range into q_head[]
  int16_t q_head[kMaxHeads];        // VS Q heads, grouped by KV head
  int16_t q_slot[kMaxHeads];        // their VS slot
};
// Tiles of 64 keys per estimation workgroup for a sequence of n keys and
// n_groups groups (the workspace holds per-chunk partials).
int vs_chunk_tiles(int64_t n, int n_groups);
// q: the call's query rows [H_q][qm][128], the last of them row n - 1.  Every
// group holds at most four VS heads.  part_mz: [n_vs][chunks][64][2] floats,
// stats: [n_vs][64][2], diag_part: [n_vs][chunks][128], v/s_scores: [n_vs][n].
hipError_t launch_vs_estimate(const uint16_t* q, const uint16_t* k, int64_t n, int64_t qm, float scale_log2,
                              const VsGroups& groups, int n_vs, int chunk_tiles, float* part_mz, float* stats,
                              float* diag_part, float* v_scores, float* s_scores, hipStream_t s);

// Block-Sparse estimation.
hipError_t launch_bs_pool(const uint16_t* src, int64_t n, const int16_t* heads, int nheads, float* pooled,
                          hipStream_t s);
// Rows: the call's nbq query blocks from qb0; columns: the nb key blocks.
hipError_t launch_bs_scores(const float* qpool, const float* kpool, int nb, int nbq, int qb0,
                            const int16_t* kv_slot_of_bs,
                            int n_bs, float* scores, hipStream_t s);

// Exact top-k (ties to the lower index, ascending output).
struct TopkJobs {            // up to kMaxJobs problems in one launch
  static constexpr int kMaxJobs = 128;
  int32_t count;
  int64_t src_off[kMaxJobs]; // float elements from the source base
  int64_t dst_off[kMaxJobs]; // int32 elements from the destination base
  int32_t k[kMaxJobs];
};
hipError_t launch_topk_rows(const float* src, int64_t n, const TopkJobs& jobs, int32_t* dst, hipStream_t s);
// Same selection with many workgroups per problem (for long vectors); every
// job's k must lie in 1..n.  Jobs 0 .. split-1 write to dst + dst_off, the
// rest to dst2 + dst_off (two selections share one chain of launches).
// scratch: device, >= topk_scratch_bytes(n, jobs).
size_t topk_scratch_bytes(int64_t n, int problems);
hipError_t launch_topk_chunked(const float* src, int64_t n, const TopkJobs& jobs, int32_t* dst, int32_t* dst2,
                               int split, void* scratch, hipStream_t s);
// Block-Sparse selection: for every BS slot and local query block bl (query
// block b = qb0 + bl), top-min(k, b+1) of scores[slot][bl][0..b] into blocks
// row bl (-1 padded to k).  k_of_slot and dst_off_of_slot are host arrays of
// n_bs entries.
hipError_t launch_bs_select(const float* scores, int nb, int nbq, int qb0, int n_bs, const int32_t* k_of_slot,
                            const int64_t* dst_off_of_slot, int32_t* blocks, hipStream_t s);

// Attention-mass recall per head from the sparse and dense log-sum-exps.
hipError_t launch_recall(const float* lse_sparse, const float* lse_dense, int64_t n, int hq, float* recall,
                         hipStream_t s);

// Index conversion.
// Over the call's nb query blocks, the first of them query block qb0.
hipError_t launch_index_build(const HeadDesc* table, char* arena, int hq, int nb, int qb0, const int32_t* vert,
                              const int32_t* slash, const int32_t* blocks, hipStream_t s);

// Attention.
hipError_t launch_v_to_f16(const uint16_t* v, _Float16* v16, int64_t elems, hipStream_t s);
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const _Float16* v16;
  void* out;
  float* lse;
  const HeadDesc* table;   // null => implicit dense
  const char* arena;
  int64_t n;               // keys (rows of K and V)
  int64_t qm;              // rows of Q, out and lse per head: query rows qb0*64 .. n-1
  int32_t qb0;             // first query block
  int32_t hq, hkv, grp, nb;  // nb: query blocks of the call (the index's blocks)
  float scale_log2;        // softmax scale * log2(e)
  int32_t out_f32;
  // Work list: the Q heads (per-head sparse kernel) or the number of chunks
  // (grouped sparse kernel) of this launch.
  int32_t n_list;
  int16_t list[kMaxHeads];
  // Paced mode of the per-head kernel: query blocks [seg_b0, seg_b0 +
  // seg_nb) of every listed head (blocks of the heads' CSR: 64 or 32 rows),
  // each walked whole (columns, then ranges in key order) by one workgroup
  // that keeps pace with the other workgroups of its XCD: before it starts
  // keys of segment s (2^seg_shift keys) it waits, for a bounded time, until
  // all of them have passed segment s - pace - 1.  pace_cnt: seg_n counters
  // per XCD (zero before the launch).
  int32_t seg_shift, seg_b0, seg_nb, seg_n;
  uint32_t* pace_cnt;
  int32_t pace;
  int32_t pace_polls;  // counter reads a wait may take before pacing stops for the walk
};
// rows: query rows per block of the listed heads' CSR (64 or 32; a 32-row
// block is one wavefront's work item).
hipError_t launch_sparse_attn(const AttnArgs& a, int rows, hipStream_t s);
// Paced mode: one launch over the chunk's blocks of `rows` rows (64 or 32).
hipError_t launch_sparse_attn_paced(const AttnArgs& a, int rows, hipStream_t s);
// Zeroes `count` 32-bit words (a kernel, so that the call can be captured).
hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s);
// Full causal attention, query heads that share a KV head served together.
hipError_t launch_group_dense(const AttnArgs& a, hipStream_t s);
// A-shape heads listed in a.list (one head per KV head), four consecutive
// query blocks of a head per workgroup.
hipError_t launch_group_ashape(const AttnArgs& a, hipStream_t s);
// Chunks of hpw (1, 2 or 4) heads of one KV head with dense key sets (any
// pattern with a CSR), 4 / hpw consecutive query blocks per workgroup, over
// every key below the group's last row: a.list[hpw u + j] is head j of chunk
// u (-1 for none), a.n_list chunks.
hipError_t launch_group_csr(const AttnArgs& a, int hpw, hipStream_t s);
// Sparse attention over the union index (groups: device table of the
// a.n_list chunks, hpw = 2 or 4 heads per workgroup, chunks of at most hpw).
hipError_t launch_group_sparse(const AttnArgs& a, const GroupDesc* groups, int hpw, hipStream_t s);
// Union index of every chunk (after the per-head index is complete).
hipError_t launch_union_build(const HeadDesc* table, GroupDesc* groups, const GroupDesc* host_groups, char* arena,
                              int n_groups, int nb, hipStream_t s);

}  // namespace msa
