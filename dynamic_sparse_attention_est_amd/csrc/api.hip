// Host side of the C ABI declared in msattn.h: argument validation, the
// layout of workspaces and of the index arena, and the launch sequence of
// each call.  Nothing here allocates device memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"

namespace msa {
namespace {

thread_local std::string g_err;

ms_status fail(ms_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ms_status device_fail(hipError_t e, const char* what) {
  return fail(MS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Paced mode of the per-head kernel, for heads served one by one whose key
// sets are long (on average at least kLongKeys keys per query block) on
// sequences of at least kPaceMinN keys: launches of kPaceSlots workgroups
// (the resident count at four per CU, set by LDS for both the two-wave
// 64-row and the one-wave 32-row workgroups), segments of 2^kPaceShift keys,
// a workgroup at most kPaceLag + 1 segments ahead of the slowest of its XCD.
// On a 1M-key Vertical-Slash layer the workgroups of an XCD then read their
// K/V rows from L2 (92% hits against 33% for the scheme it replaced, one
// workgroup per (block, 32768-key segment) with partial results combined
// afterwards; HBM reads 31 -> 3.4 TB per call) and attention takes 12% less
// time.  Swept there: 2^10..2^15-key segments, lag 0..4; 2^13 with lag 1 was
// fastest.
constexpr int64_t kPaceMinN = 131072;
constexpr double kLongKeys = 32768.0;
constexpr int kPaceShift = 13;
constexpr int kPaceLag = 1;
constexpr int kPaceSlots = 1024;
// Counter reads one pacing wait may take (about 1 us each) before the
// workgroup stops pacing for the rest of its walk; ms_set_pace_polls sets it.
std::atomic<int32_t> g_pace_polls{4096};

// Paced mode: query blocks per launch for `heads` heads, and the pacing
// counters of all launches of a call over nb 64-row blocks split in blocks
// of `rows` rows (per launch, 8 XCDs x segments).
int64_t pace_blocks(int heads) { return std::max<int64_t>(1, kPaceSlots / std::max(heads, 1)); }
size_t pace_counter_words(int64_t n, int64_t nb, int heads, int rows) {
  const int64_t nseg = ((n - 1) >> kPaceShift) + 1;
  const int64_t nblk = nb * (kBM / rows);
  const int64_t launches = (nblk + pace_blocks(heads) - 1) / pace_blocks(heads);
  return (size_t)launches * 8 * (size_t)nseg;
}

struct Plan {
  int64_t n = 0, nb = 0;
  int64_t qb0 = 0, nbq = 0, qm = 0;  // first query block, query blocks and query rows of the call
  int hq = 0, hkv = 0, grp = 0;
  float scale_log2 = 0.f;
  int out_f32 = 0;
  std::vector<ms_head_params> p;
  int n_vs = 0, n_bs = 0;
  std::vector<int> vs_slot, bs_slot;
  std::vector<int16_t> vs_heads, bs_heads;       // Q heads by slot
  std::vector<int16_t> bs_kv_heads;              // distinct KV heads read by BS heads
  std::vector<int16_t> bs_kv_slot;               // per BS slot: index into bs_kv_heads
  std::vector<int64_t> vert_off, slash_off, blk_off;
  int64_t n_vert = 0, n_slash = 0, n_blocks = 0;
  VsGroups vsg{};     // VS heads by KV head, at most four a group
  int vs_chunk = 0;   // 64-key tiles per estimation workgroup
  int vs_nchunks = 0;
  // estimation workspace (byte offsets)
  size_t e_part = 0, e_stats = 0, e_diag = 0, e_v = 0, e_s = 0, e_qpool = 0, e_kpool = 0, e_scores = 0, e_topk = 0;
  size_t est_bytes = 0;
  // index arena
  std::vector<int64_t> cap_r, cap_c;
  std::vector<HeadDesc> desc;
  int hpw = 1;
  std::vector<GroupDesc> gdesc;  // chunks served by the grouped sparse kernel
  int n_wide = 0;                // the first n_wide chunks run with hpw heads per workgroup, the rest with 2
  std::vector<int16_t> solo;     // heads served one by one (64-row blocks)
  std::vector<int16_t> solo32;   // heads served one by one with 32-row blocks
  std::vector<int16_t> ablk;     // A-shape heads of MHA layers, four query blocks per workgroup
  std::vector<int16_t> cblk;     // heads alone with dense key sets, four query blocks per workgroup
  std::vector<int16_t> hdense4;  // chunks of heads with dense key sets (4 entries each, -1 padded), no union
  std::vector<int16_t> hdense2;  // the same, chunks of two
  size_t index_bytes = 0;
  // attention workspace: fp16 V copy, then the pacing counters (without
  // params: the most any head set needs)
  size_t v16_bytes = 0, attn_bytes = 0;
  std::vector<int16_t> solo_paced;    // heads served one by one in paced mode (64-row blocks)
  std::vector<int16_t> solo32_paced;  // the same with 32-row blocks
  size_t pace_off = 0, pace_words = 0;  // pacing counters in the attention workspace
  // one-shot workspace
  size_t o_vert = 0, o_slash = 0, o_blocks = 0, o_est = 0, o_index = 0, o_attn = 0, o_total = 0;
};

ms_status validate(const ms_problem* prob, const ms_head_params* params, bool need_params) {
  if (!prob) return fail(MS_ERR_INVALID_ARG, "prob is null");
  if (need_params && !params) return fail(MS_ERR_INVALID_ARG, "params is null");
  if (prob->head_dim != kD) return fail(MS_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", prob->head_dim);
  if (prob->n < kBM || prob->n % kBM != 0)
    return fail(MS_ERR_UNSUPPORTED, "n = %lld: must be a positive multiple of 64", (long long)prob->n);
  if (prob->n > (int64_t{1} << 23)) return fail(MS_ERR_UNSUPPORTED, "n = %lld exceeds 2^23", (long long)prob->n);
  if (prob->n_q_heads < 1 || prob->n_q_heads > kMaxHeads)
    return fail(MS_ERR_INVALID_ARG, "n_q_heads = %d: must be 1..%d", prob->n_q_heads, kMaxHeads);
  if (prob->n_kv_heads < 1 || prob->n_q_heads % prob->n_kv_heads != 0)
    return fail(MS_ERR_INVALID_ARG, "n_kv_heads = %d must divide n_q_heads = %d", prob->n_kv_heads, prob->n_q_heads);
  if (prob->out_dtype != MS_OUT_BF16 && prob->out_dtype != MS_OUT_F32)
    return fail(MS_ERR_INVALID_ARG, "out_dtype = %d", prob->out_dtype);
  if (prob->q_block0 < 0 || prob->q_block0 >= prob->n / kBM)
    return fail(MS_ERR_INVALID_ARG, "q_block0 = %d: must be 0..n/64-1", prob->q_block0);
  if (!std::isfinite(prob->scale) || prob->scale < 0.f) return fail(MS_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (!need_params) return MS_OK;
  const int64_t n = prob->n, nb = n / kBM;
  for (int h = 0; h < prob->n_q_heads; ++h) {
    const ms_head_params& q = params[h];
    switch (q.pattern) {
      case MS_VERTICAL_SLASH:
        if (q.last_q != kLastQ) return fail(MS_ERR_UNSUPPORTED, "head %d: last_q = %d, only 64 is supported", h, q.last_q);
        if (q.block != 0 && q.block != 32 && q.block != kBM)
          return fail(MS_ERR_UNSUPPORTED, "head %d: block = %d, Vertical-Slash query blocks are 64 (or 0) or 32 rows",
                      h, q.block);
        if (q.n_vertical < 0 || q.n_vertical > n) return fail(MS_ERR_INVALID_ARG, "head %d: n_vertical = %d out of 0..n", h, q.n_vertical);
        if (q.n_slash < 0 || q.n_slash > n) return fail(MS_ERR_INVALID_ARG, "head %d: n_slash = %d out of 0..n", h, q.n_slash);
        break;
      case MS_BLOCK_SPARSE:
        if (q.block != kBM) return fail(MS_ERR_UNSUPPORTED, "head %d: block = %d, only 64 is supported", h, q.block);
        if (q.top_k_blocks < 1 || q.top_k_blocks > nb)
          return fail(MS_ERR_INVALID_ARG, "head %d: top_k_blocks = %d out of 1..n/64", h, q.top_k_blocks);
        break;
      case MS_A_SHAPE:
        if (q.sink < 0 || q.sink > n) return fail(MS_ERR_INVALID_ARG, "head %d: sink = %d out of 0..n", h, q.sink);
        if (q.window < 1 || q.window > n) return fail(MS_ERR_INVALID_ARG, "head %d: window = %d out of 1..n", h, q.window);
        break;
      case MS_GRID:
        if (q.grid_stride < 1 || q.grid_stride > n)
          return fail(MS_ERR_INVALID_ARG, "head %d: grid_stride = %d out of 1..n", h, q.grid_stride);
        if (q.grid_frames < 0 || q.grid_frames > n)
          return fail(MS_ERR_INVALID_ARG, "head %d: grid_frames = %d out of 0..n", h, q.grid_frames);
        if (q.grid_width < 0 || q.grid_width > n)
          return fail(MS_ERR_INVALID_ARG, "head %d: grid_width = %d out of 0..n", h, q.grid_width);
        if (q.window < 1 || q.window > n) return fail(MS_ERR_INVALID_ARG, "head %d: window = %d out of 1..n", h, q.window);
        break;
      case MS_DENSE:
        break;
      default:
        return fail(MS_ERR_INVALID_ARG, "head %d: pattern = %d", h, q.pattern);
    }
  }
  return MS_OK;
}

// Query rows per block of a head's CSR: 32 for a Vertical-Slash head that
// asks for them, 64 otherwise.
int head_rows(const ms_head_params& q) { return q.pattern == MS_VERTICAL_SLASH && q.block == 32 ? 32 : kBM; }

// Per-head capacities of the CSR, the sums over query blocks of the bounds
// the index kernels clamp to.
std::pair<int64_t, int64_t> head_caps(const ms_head_params& q, int64_t qb0, int64_t nb) {
  int64_t r = 0, c = 0;
  if (q.pattern == MS_VERTICAL_SLASH) {
    // run starts of the sorted offsets are more than `rows` apart
    const int64_t rows = head_rows(q), per = kBM / rows;
    for (int64_t b = qb0 * per; b < nb * per; ++b) {
      const int64_t last = b * rows + rows - 1;
      r += std::min<int64_t>(q.n_slash, last / (rows + 1) + 1);
      c += std::min<int64_t>(q.n_vertical, last + 1);
    }
    return {r, c};
  }
  for (int64_t b = qb0; b < nb; ++b) {
    const int64_t last = b * kBM + kBM - 1;
    switch (q.pattern) {
      case MS_BLOCK_SPARSE:
        r += std::min<int64_t>(std::min<int64_t>(q.top_k_blocks, b + 1), b / 2 + 1);
        break;
      case MS_A_SHAPE:
        r += 2;
        break;
      case MS_GRID:  // at most one range per frame group that reaches the block, plus the local one
        r += std::min<int64_t>(q.grid_frames, (last + q.grid_width) / q.grid_stride) + 1;
        break;
      default:
        r += 1;
    }
  }
  return {r, c};
}

// Expected fraction of the causal (row, key) pairs a head keeps, from its
// parameters alone: Vertical-Slash spans of 64 keys at scattered offsets cover
// 1 - exp(-64 n_slash / n) of a row; Block-Sparse keeps min(1, k / (b + 1))
// of block b; A-shape about (sink + window) keys of a row.
double expected_density(const ms_head_params& q, int64_t n) {
  const double nd = (double)n;
  switch (q.pattern) {
    case MS_VERTICAL_SLASH:
      return std::min(1.0, 1.0 - std::exp(-(double)head_rows(q) * q.n_slash / nd) + q.n_vertical / nd);
    case MS_BLOCK_SPARSE: {
      const int64_t nb = n / kBM;
      double s = 0.0;
      for (int64_t b = 0; b < nb; ++b) s += std::min(1.0, (double)q.top_k_blocks / (double)(b + 1));
      return s / (double)nb;
    }
    case MS_A_SHAPE:
      return std::min(1.0, ((double)q.sink + (double)q.window) / (0.5 * nd));
    case MS_GRID:  // a 64-row block keeps window + 63 local keys and 2w + 64 per frame
      return std::min(1.0, ((double)q.window + 63.0 + (double)q.grid_frames * (2.0 * q.grid_width + 64.0)) /
                               (0.5 * nd));
    default:
      return 1.0;
  }
}

ms_status make_plan(const ms_problem* prob, const ms_head_params* params, Plan& P) {
  const bool have_params = params != nullptr;
  ms_status st = validate(prob, params, have_params);
  if (st != MS_OK) return st;
  P.n = prob->n;
  P.nb = P.n / kBM;
  P.qb0 = prob->q_block0;
  P.nbq = P.nb - P.qb0;
  P.qm = P.nbq * kBM;
  P.hq = prob->n_q_heads;
  P.hkv = prob->n_kv_heads;
  P.grp = P.hq / P.hkv;
  const float scale = prob->scale == 0.f ? 1.f / std::sqrt((float)kD) : prob->scale;
  P.scale_log2 = scale * 1.4426950408889634f;
  P.out_f32 = prob->out_dtype == MS_OUT_F32;
  P.v16_bytes = align_up((size_t)P.hkv * (size_t)P.n * kD * 2);
  P.attn_bytes = P.v16_bytes + (P.n >= kPaceMinN ? align_up((pace_counter_words(P.n, P.nbq, P.hq, kBM) +
                                                              pace_counter_words(P.n, P.nbq, P.hq, 32)) * 4)
                                                  : 0);
  if (!have_params) return MS_OK;
  P.p.assign(params, params + P.hq);
  P.vs_slot.assign(P.hq, -1);
  P.bs_slot.assign(P.hq, -1);
  P.vert_off.assign(P.hq, 0);
  P.slash_off.assign(P.hq, 0);
  P.blk_off.assign(P.hq, 0);
  std::vector<int> kv_slot_of(P.hkv, -1);
  for (int h = 0; h < P.hq; ++h) {
    const ms_head_params& q = P.p[h];
    if (q.pattern == MS_VERTICAL_SLASH) {
      P.vs_slot[h] = P.n_vs++;
      P.vs_heads.push_back((int16_t)h);
      P.vert_off[h] = P.n_vert;
      P.slash_off[h] = P.n_slash;
      P.n_vert += q.n_vertical;
      P.n_slash += q.n_slash;
    } else if (q.pattern == MS_BLOCK_SPARSE) {
      P.bs_slot[h] = P.n_bs++;
      P.bs_heads.push_back((int16_t)h);
      P.blk_off[h] = P.n_blocks;
      P.n_blocks += P.nbq * q.top_k_blocks;
      const int kv = h / P.grp;
      if (kv_slot_of[kv] < 0) {
        kv_slot_of[kv] = (int)P.bs_kv_heads.size();
        P.bs_kv_heads.push_back((int16_t)kv);
      }
      P.bs_kv_slot.push_back((int16_t)kv_slot_of[kv]);
    }
  }
  // Vertical-Slash estimation groups: the VS heads of one KV head, four at a
  // time (one estimation workgroup reads a K tile once for its group).
  P.vsg = VsGroups{};
  for (int kv = 0; kv < P.hkv; ++kv) {
    int cnt = 0;
    for (int h = kv * P.grp; h < (kv + 1) * P.grp; ++h) {
      if (P.vs_slot[h] < 0) continue;
      if (cnt == 4) {
        ++P.vsg.n_groups;
        cnt = 0;
      }
      const int i = P.vsg.q_begin[P.vsg.n_groups] + cnt;
      P.vsg.q_head[i] = (int16_t)h;
      P.vsg.q_slot[i] = (int16_t)P.vs_slot[h];
      P.vsg.kv_head[P.vsg.n_groups] = (int16_t)kv;
      P.vsg.q_begin[P.vsg.n_groups + 1] = (int16_t)(i + 1);
      ++cnt;
    }
    if (cnt) ++P.vsg.n_groups;
  }
  // Estimation workspace.
  if (P.n_vs) {
    P.vs_chunk = vs_chunk_tiles(P.n, P.vsg.n_groups);
    P.vs_nchunks = (int)((P.n / 64 + P.vs_chunk - 1) / P.vs_chunk);
  }
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const size_t f = sizeof(float);
  P.e_part = take((size_t)P.n_vs * P.vs_nchunks * kLastQ * 2 * f);
  P.e_stats = take((size_t)P.n_vs * kLastQ * 2 * f);
  P.e_diag = take((size_t)P.n_vs * P.vs_nchunks * 128 * f);
  P.e_v = take((size_t)P.n_vs * P.n * f);
  P.e_s = take((size_t)P.n_vs * P.n * f);
  P.e_qpool = take((size_t)P.n_bs * P.nbq * kD * f);
  P.e_kpool = take((size_t)P.bs_kv_heads.size() * P.nb * kD * f);
  P.e_scores = take((size_t)P.n_bs * P.nbq * P.nb * f);
  P.e_topk = take(topk_scratch_bytes(P.n, std::max(std::min(2 * P.n_vs, TopkJobs::kMaxJobs), 1)));
  P.est_bytes = std::max<size_t>(off, kAlign);
  // Index arena: head table, chunk table, then each head's CSR, then each
  // chunk's union CSR.
  off = align_up((size_t)(kTableBytes + kGroupTableBytes));
  P.cap_r.assign(P.hq, 0);
  P.cap_c.assign(P.hq, 0);
  P.desc.assign(P.hq, HeadDesc{});
  std::map<std::tuple<int, int, int, int, int, int>, std::pair<int64_t, int64_t>> memo;
  for (int h = 0; h < P.hq; ++h) {
    const ms_head_params& q = P.p[h];
    const int a = q.pattern == MS_VERTICAL_SLASH ? q.n_vertical : q.pattern == MS_BLOCK_SPARSE ? q.top_k_blocks : 0;
    const int b = q.pattern == MS_VERTICAL_SLASH ? q.n_slash : 0;
    const bool gr = q.pattern == MS_GRID;
    const auto key = std::make_tuple(q.pattern, a, b, gr ? q.grid_stride : head_rows(q), gr ? q.grid_frames : 0,
                                     gr ? q.grid_width : 0);
    auto it = memo.find(key);
    if (it == memo.end()) it = memo.emplace(key, head_caps(q, P.qb0, P.nb)).first;
    P.cap_r[h] = it->second.first;
    P.cap_c[h] = it->second.second;
    if (P.cap_r[h] >= (int64_t{1} << 31) || P.cap_c[h] >= (int64_t{1} << 31))
      return fail(MS_ERR_UNSUPPORTED, "head %d: index capacity exceeds int32", h);
    HeadDesc& d = P.desc[h];
    d.pattern = q.pattern;
    d.qrows = head_rows(q);
    d.vs_slot = P.vs_slot[h];
    d.bs_slot = P.bs_slot[h];
    if (q.pattern == MS_VERTICAL_SLASH) {
      d.p0 = q.n_vertical;
      d.p1 = q.n_slash;
    } else if (q.pattern == MS_BLOCK_SPARSE) {
      d.p0 = q.top_k_blocks;
    } else if (q.pattern == MS_A_SHAPE) {
      d.p0 = q.sink;
      d.p1 = q.window;
    } else if (q.pattern == MS_GRID) {
      d.p0 = q.grid_stride;
      d.p1 = q.window;
      d.p2 = q.grid_frames;
      d.p3 = q.grid_width;
    }
    d.vert_off = P.vert_off[h];
    d.slash_off = P.slash_off[h];
    d.blk_off = P.blk_off[h];
    const int64_t nblk = P.nbq * (kBM / d.qrows);  // CSR blocks of this head
    d.rng_ptr_off = (int64_t)take((size_t)(nblk + 1) * 4);
    d.rng_off = (int64_t)take((size_t)P.cap_r[h] * 8);
    d.col_ptr_off = (int64_t)take((size_t)(nblk + 1) * 4);
    d.col_off = (int64_t)take((size_t)P.cap_c[h] * 4);
    d.run_off = (int64_t)take(q.pattern == MS_VERTICAL_SLASH ? (size_t)(q.n_slash + 1) * 4 : 4);
  }
  // Heads of one KV head whose key sets overlap heavily are served together,
  // up to hpw per chunk, by the grouped kernel over the union of their index;
  // the rest one by one.  Heavy overlap: every head dense enough (expected
  // density >= 1/2), or heads whose index the parameters alone fix (A-shape,
  // Grid) with equal parameters, whose union is each one's index.
  P.hpw = hpw_of(P.grp);
  P.gdesc.clear();
  P.solo.clear();
  P.cblk.clear();
  P.hdense4.clear();
  P.hdense2.clear();
  auto emit_chunks = [&](int kv, const std::vector<int>& heads) {
    for (size_t c = 0; c < heads.size();) {
      size_t m = std::min<size_t>(P.hpw, heads.size() - c);
      // A four-head workgroup costs about the same per piece however many of
      // its heads are present, so three heads run as a chunk of two and a
      // head alone.
      if (m == 3) m = 2;
      if (m < 2) {
        P.solo.push_back((int16_t)heads[c++]);
        continue;
      }
      // Chunks whose heads all keep most causal keys walk every key with
      // per-head masks (group_csr_heads) instead of a union index.
      bool all_dense = true;
      for (size_t j = 0; j < m; ++j)
        all_dense = all_dense && P.p[heads[c + j]].pattern != MS_A_SHAPE &&
                    expected_density(P.p[heads[c + j]], P.n) >= 0.75;
      if (all_dense) {
        std::vector<int16_t>& l = m > 2 ? P.hdense4 : P.hdense2;
        for (size_t j = 0; j < (m > 2 ? 4u : 2u); ++j) l.push_back(j < m ? (int16_t)heads[c + j] : (int16_t)-1);
        c += m;
        continue;
      }
      GroupDesc g{};
      g.kvh = kv;
      g.nheads = (int)m;
      for (size_t j = 0; j < m; ++j) g.head[j] = (int16_t)heads[c + j];
      P.gdesc.push_back(g);
      c += m;
    }
  };
  auto static_key = [&](const ms_head_params& q) {
    return std::make_tuple(q.pattern, q.sink, q.window, q.grid_stride, q.grid_frames, q.grid_width);
  };
  for (int kv = 0; kv < P.hkv; ++kv) {
    std::vector<int> dense_heads, fixed_heads;
    for (int j = 0; j < P.grp; ++j) {
      const int h = kv * P.grp + j;
      const int pat = P.p[h].pattern;
      if (head_rows(P.p[h]) != kBM)
        P.solo32.push_back((int16_t)h);  // 32-row blocks: the per-head kernel only
      else if (P.hpw > 1 && expected_density(P.p[h], P.n) >= 0.5)
        dense_heads.push_back(h);
      else if (P.hpw > 1 && (pat == MS_A_SHAPE || pat == MS_GRID))
        fixed_heads.push_back(h);
      else if (P.hpw == 1 && pat == MS_A_SHAPE && P.p[h].window >= 256)
        // one head per KV head: four query blocks share one walk of the
        // sink and the union of their windows (a window of at least 256 keys
        // keeps most of that walk useful to every block)
        P.ablk.push_back((int16_t)h);
      else
        P.solo.push_back((int16_t)h);
    }
    emit_chunks(kv, dense_heads);
    // fixed-index heads with equal parameters, in head order within a set
    std::stable_sort(fixed_heads.begin(), fixed_heads.end(),
                     [&](int x, int y) { return static_key(P.p[x]) < static_key(P.p[y]); });
    for (size_t i = 0; i < fixed_heads.size();) {
      size_t e = i + 1;
      while (e < fixed_heads.size() && static_key(P.p[fixed_heads[e]]) == static_key(P.p[fixed_heads[i]])) ++e;
      emit_chunks(kv, std::vector<int>(fixed_heads.begin() + i, fixed_heads.begin() + e));
      i = e;
    }
  }
  // Heads served alone whose key sets cover most causal keys (expected
  // density >= 3/4; not A-shape, whose windows need a per-row mask) take four
  // query blocks per workgroup over every key below the group's last row, so
  // each K/V tile feeds 256 rows instead of 64.
  {
    std::vector<int16_t> keep;
    for (int16_t h : P.solo)
      (P.p[h].pattern != MS_A_SHAPE && expected_density(P.p[h], P.n) >= 0.75 ? P.cblk : keep).push_back(h);
    P.solo = keep;
  }
  // With four heads per workgroup, chunks of two go to the two-head kernel
  // instead: the four-head chunks first, then those.
  P.n_wide = (int)P.gdesc.size();
  if (P.hpw == 4) {
    std::stable_partition(P.gdesc.begin(), P.gdesc.end(), [](const GroupDesc& g) { return g.nheads > 2; });
    P.n_wide = (int)std::count_if(P.gdesc.begin(), P.gdesc.end(), [](const GroupDesc& g) { return g.nheads > 2; });
  }
  for (GroupDesc& g : P.gdesc) {
    int64_t ur = 0, uc = 0;
    for (int j = 0; j < g.nheads; ++j) {
      ur += P.cap_r[g.head[j]];
      uc += P.cap_c[g.head[j]];
    }
    if (ur >= (int64_t{1} << 31) || uc >= (int64_t{1} << 31))
      return fail(MS_ERR_UNSUPPORTED, "KV head %d: union index capacity exceeds int32", g.kvh);
    g.urng_ptr_off = (int64_t)take((size_t)(P.nbq + 1) * 4);
    g.urng_off = (int64_t)take((size_t)ur * 8);
    g.ucol_ptr_off = (int64_t)take((size_t)(P.nbq + 1) * 4);
    g.ucol_off = (int64_t)take((size_t)uc * 4);
    g.umask_off = (int64_t)take((size_t)uc);
  }
  // Solo heads with long key sets (on average at least kLongKeys keys per
  // query block) on long sequences run paced: the workgroups in flight then
  // share a stretch of K/V in L2 instead of streaming every block's keys from
  // HBM.  Short, local key sets (A-shape, small Block-Sparse budgets) stay
  // whole.
  P.solo_paced.clear();
  P.solo32_paced.clear();
  if (P.n >= kPaceMinN) {
    for (auto [solo, paced] :
         {std::make_pair(&P.solo, &P.solo_paced), std::make_pair(&P.solo32, &P.solo32_paced)}) {
      std::vector<int16_t> keep;
      for (int16_t h : *solo)
        (expected_density(P.p[h], P.n) * 0.5 * (double)P.n >= kLongKeys ? *paced : keep).push_back(h);
      *solo = keep;
    }
  }
  // Workgroups go round-robin over the 8 XCDs, so order each list to keep
  // the heads of one KV head on one XCD when the count allows.
  for (std::vector<int16_t>* l : {&P.solo, &P.solo_paced, &P.solo32, &P.solo32_paced}) {
    if (l->size() % 8 != 0 || l->empty()) continue;
    const size_t per = l->size() / 8;
    std::vector<int16_t> ordered(l->size());
    for (size_t i = 0; i < l->size(); ++i) ordered[i] = (*l)[(i % 8) * per + i / 8];
    *l = ordered;
  }
  P.attn_bytes = P.v16_bytes;
  P.pace_off = P.attn_bytes;
  P.pace_words = 0;
  if (!P.solo_paced.empty()) P.pace_words += pace_counter_words(P.n, P.nbq, (int)P.solo_paced.size(), kBM);
  if (!P.solo32_paced.empty()) P.pace_words += pace_counter_words(P.n, P.nbq, (int)P.solo32_paced.size(), 32);
  P.attn_bytes += align_up(P.pace_words * 4);
  P.index_bytes = off;
  // One-shot workspace.
  off = 0;
  P.o_vert = take((size_t)P.n_vert * 4);
  P.o_slash = take((size_t)P.n_slash * 4);
  P.o_blocks = take((size_t)P.n_blocks * 4);
  P.o_est = take(P.est_bytes);
  P.o_index = take(P.index_bytes);
  P.o_attn = take(P.attn_bytes);
  P.o_total = off;
  return MS_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

ms_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(MS_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned(p, 16)) return fail(MS_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MS_OK;
}

ms_status check_ws(const void* ws, size_t have, size_t need, const char* name) {
  if (need == 0) return MS_OK;
  if (!ws) return fail(MS_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned(ws, kAlign)) return fail(MS_ERR_INVALID_ARG, "%s is not 256-byte aligned", name);
  if (have < need) return fail(MS_ERR_CAPACITY, "%s holds %zu bytes, %zu needed", name, have, need);
  return MS_OK;
}

// Scratch of ms_sparse_attn_noalloc: a fixed array in the library's device
// code, one copy per GPU (each GPU's copy lives at its own address, held until
// the process ends).  Host code never passes `scratch` itself to a kernel (on
// the host the name is only a stand-in); it takes the device address of the
// current GPU's copy from hipGetSymbolAddress, once per device, and uses that.
constexpr size_t kScratchBytes = size_t{MS_NOALLOC_SCRATCH_MIB} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ms_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MS_ERR_DEVICE, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_fail(e, "address of the static scratch");
    if (!ptr || !aligned(ptr, kAlign)) return fail(MS_ERR_DEVICE, "static scratch address is null or misaligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MS_OK;
}

#define MS_TRY(x)                          \
  do {                                     \
    const ms_status st_ = (x);             \
    if (st_ != MS_OK) return st_;          \
  } while (0)
#define HIP_TRY(x, what)                   \
  do {                                     \
    const hipError_t e_ = (x);             \
    if (e_ != hipSuccess) return device_fail(e_, what); \
  } while (0)

// ---------------------------------------------------------------- stages
ms_status run_estimate_vs(const Plan& P, const uint16_t* q, const uint16_t* k, int32_t* vert, int32_t* slash,
                          float* dbg_v, float* dbg_s, char* ws, hipStream_t s) {
  if (P.n_vs == 0) return MS_OK;
  float* v_sc = reinterpret_cast<float*>(ws + P.e_v);
  float* s_sc = reinterpret_cast<float*>(ws + P.e_s);
  HIP_TRY(launch_vs_estimate(q, k, P.n, P.qm, P.scale_log2, P.vsg, P.n_vs, P.vs_chunk,
                             reinterpret_cast<float*>(ws + P.e_part),
                             reinterpret_cast<float*>(ws + P.e_stats), reinterpret_cast<float*>(ws + P.e_diag), v_sc,
                             s_sc, s),
          "vertical-slash estimation launch");
  // Both selections of every VS head in one chain of launches: the vertical
  // jobs (scores v_sc, written to vert) first, then the slash jobs (scores
  // s_sc, which follows v_sc in the workspace, written to slash).
  struct Job {
    int64_t src_off, dst_off;
    int32_t k;
    bool slash;
  };
  std::vector<Job> all;
  for (int i = 0; i < P.n_vs; ++i) {
    const int h = P.vs_heads[i];
    if (P.p[h].n_vertical > 0) all.push_back({(int64_t)i * P.n, P.vert_off[h], P.p[h].n_vertical, false});
  }
  const int64_t s_base = (int64_t)(P.e_s - P.e_v) / (int64_t)sizeof(float);
  for (int i = 0; i < P.n_vs; ++i) {
    const int h = P.vs_heads[i];
    if (P.p[h].n_slash > 0) all.push_back({s_base + (int64_t)i * P.n, P.slash_off[h], P.p[h].n_slash, true});
  }
  // batches of at most kMaxJobs, each with its vertical jobs first
  void* tk = ws + P.e_topk;
  for (size_t b0 = 0; b0 < all.size(); b0 += TopkJobs::kMaxJobs) {
    TopkJobs j{};
    int split = 0;
    for (size_t x = b0; x < all.size() && j.count < TopkJobs::kMaxJobs; ++x) {
      j.src_off[j.count] = all[x].src_off;
      j.dst_off[j.count] = all[x].dst_off;
      j.k[j.count++] = all[x].k;
      if (!all[x].slash) split = j.count;
    }
    HIP_TRY(launch_topk_chunked(v_sc, P.n, j, vert, slash, split, tk, s), "top-k launch");
  }
  for (int i = 0; i < P.n_vs; ++i) {
    const int h = P.vs_heads[i];
    if (dbg_v)
      HIP_TRY(hipMemcpyAsync(dbg_v + (int64_t)h * P.n, v_sc + (int64_t)i * P.n, P.n * 4, hipMemcpyDeviceToDevice, s),
              "copy of vertical scores");
    if (dbg_s)
      HIP_TRY(hipMemcpyAsync(dbg_s + (int64_t)h * P.n, s_sc + (int64_t)i * P.n, P.n * 4, hipMemcpyDeviceToDevice, s),
              "copy of slash scores");
  }
  return MS_OK;
}

ms_status run_estimate_block(const Plan& P, const uint16_t* q, const uint16_t* k, int32_t* blocks, float* dbg_scores,
                             char* ws, hipStream_t s) {
  if (P.n_bs == 0) return MS_OK;
  float* qpool = reinterpret_cast<float*>(ws + P.e_qpool);
  float* kpool = reinterpret_cast<float*>(ws + P.e_kpool);
  float* scores = reinterpret_cast<float*>(ws + P.e_scores);
  HIP_TRY(launch_bs_pool(q, P.qm, P.bs_heads.data(), P.n_bs, qpool, s), "query pooling launch");
  HIP_TRY(launch_bs_pool(k, P.n, P.bs_kv_heads.data(), (int)P.bs_kv_heads.size(), kpool, s), "key pooling launch");
  HIP_TRY(launch_bs_scores(qpool, kpool, (int)P.nb, (int)P.nbq, (int)P.qb0, P.bs_kv_slot.data(), P.n_bs, scores, s),
          "block score launch");
  std::vector<int32_t> kk(P.n_bs);
  std::vector<int64_t> off(P.n_bs);
  for (int i = 0; i < P.n_bs; ++i) {
    kk[i] = P.p[P.bs_heads[i]].top_k_blocks;
    off[i] = P.blk_off[P.bs_heads[i]];
  }
  HIP_TRY(launch_bs_select(scores, (int)P.nb, (int)P.nbq, (int)P.qb0, P.n_bs, kk.data(), off.data(), blocks, s),
          "block selection launch");
  if (dbg_scores)
    for (int i = 0; i < P.n_bs; ++i)
      HIP_TRY(hipMemcpyAsync(dbg_scores + (int64_t)P.bs_heads[i] * P.nbq * P.nb, scores + (int64_t)i * P.nbq * P.nb,
                             (size_t)P.nbq * P.nb * 4, hipMemcpyDeviceToDevice, s),
              "copy of block scores");
  return MS_OK;
}

ms_status run_build_index(const Plan& P, const int32_t* vert, const int32_t* slash, const int32_t* blocks,
                          char* index, hipStream_t s) {
  HIP_TRY(launch_write_table(reinterpret_cast<HeadDesc*>(index), P.desc.data(), 0, P.hq, s), "index table launch");
  HIP_TRY(launch_index_build(reinterpret_cast<const HeadDesc*>(index), index, P.hq, (int)P.nbq, (int)P.qb0, vert, slash,
                             blocks, s),
          "index build launch");
  if (!P.gdesc.empty())
    HIP_TRY(launch_union_build(reinterpret_cast<const HeadDesc*>(index),
                               reinterpret_cast<GroupDesc*>(index + kTableBytes), P.gdesc.data(), index,
                               (int)P.gdesc.size(), (int)P.nbq, s),
            "union index launch");
  return MS_OK;
}

ms_status run_attention(const Plan& P, const void* q, const void* k, const void* v, const char* index, void* out,
                        float* lse, char* attn_ws, hipStream_t s) {
  _Float16* v16 = reinterpret_cast<_Float16*>(attn_ws);
  HIP_TRY(launch_v_to_f16(static_cast<const uint16_t*>(v), v16, (int64_t)P.hkv * P.n * kD, s), "V conversion launch");
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v16 = v16;
  a.out = out;
  a.lse = lse;
  a.table = reinterpret_cast<const HeadDesc*>(index);
  a.arena = index;
  a.n = P.n;
  a.hq = P.hq;
  a.hkv = P.hkv;
  a.grp = P.grp;
  a.nb = (int)P.nbq;
  a.qb0 = (int)P.qb0;
  a.qm = P.qm;
  a.scale_log2 = P.scale_log2;
  a.out_f32 = P.out_f32;
  if (!P.gdesc.empty()) {
    const GroupDesc* chunks = reinterpret_cast<const GroupDesc*>(index + kTableBytes);
    if (P.n_wide > 0) {
      a.n_list = P.n_wide;
      HIP_TRY(launch_group_sparse(a, chunks, P.hpw, s), "attention launch");
    }
    if ((int)P.gdesc.size() > P.n_wide) {
      a.n_list = (int)P.gdesc.size() - P.n_wide;
      HIP_TRY(launch_group_sparse(a, chunks + P.n_wide, 2, s), "attention launch");
    }
  }
  if (!P.ablk.empty()) {
    a.n_list = (int)P.ablk.size();
    for (size_t i = 0; i < P.ablk.size(); ++i) a.list[i] = P.ablk[i];
    HIP_TRY(launch_group_ashape(a, s), "attention launch");
  }
  if (!P.cblk.empty()) {
    a.n_list = (int)P.cblk.size();
    for (size_t i = 0; i < P.cblk.size(); ++i) a.list[i] = P.cblk[i];
    HIP_TRY(launch_group_csr(a, 1, s), "attention launch");
  }
  for (auto [list, slots] : {std::make_pair(&P.hdense4, 4), std::make_pair(&P.hdense2, 2)}) {
    if (list->empty()) continue;
    a.n_list = (int)list->size() / slots;
    for (size_t i = 0; i < list->size(); ++i) a.list[i] = (*list)[i];
    HIP_TRY(launch_group_csr(a, slots, s), "attention launch");
  }
  for (auto [list, rows] : {std::make_pair(&P.solo, kBM), std::make_pair(&P.solo32, 32)}) {
    if (list->empty()) continue;
    a.n_list = (int)list->size();
    for (size_t i = 0; i < list->size(); ++i) a.list[i] = (*list)[i];
    HIP_TRY(launch_sparse_attn(a, rows, s), "attention launch");
  }
  if (P.pace_words > 0) {
    uint32_t* cnt = reinterpret_cast<uint32_t*>(attn_ws + P.pace_off);
    HIP_TRY(launch_zero_u32(cnt, (int64_t)P.pace_words, s), "pacing counter launch");
    const int64_t nseg = ((P.n - 1) >> kPaceShift) + 1;
    a.seg_shift = kPaceShift;
    a.seg_n = (int)nseg;
    a.pace = kPaceLag;
    a.pace_polls = g_pace_polls.load(std::memory_order_relaxed);
    for (auto [list, rows] : {std::make_pair(&P.solo_paced, kBM), std::make_pair(&P.solo32_paced, 32)}) {
      if (list->empty()) continue;
      a.n_list = (int)list->size();
      for (size_t i = 0; i < list->size(); ++i) a.list[i] = (*list)[i];
      // launches of the list's blocks of `rows` rows, longest first, each
      // with its own counters
      const int64_t nblk = P.nbq * (kBM / rows);
      const int64_t cb = pace_blocks(a.n_list);
      for (int64_t b0 = 0; b0 < nblk; b0 += cb) {
        a.seg_b0 = (int)std::max<int64_t>(0, nblk - b0 - cb);
        a.seg_nb = (int)(nblk - b0 - a.seg_b0);
        a.pace_cnt = cnt;
        cnt += 8 * nseg;
        HIP_TRY(launch_sparse_attn_paced(a, rows, s), "attention launch");
      }
    }
  }
  return MS_OK;
}

ms_status check_selection_ptrs(const Plan& P, const void* vert, const void* slash, const void* blocks, bool vs,
                               bool bs) {
  if (vs && P.n_vert > 0 && !vert) return fail(MS_ERR_INVALID_ARG, "vert is null but a Vertical-Slash head keeps verticals");
  if (vs && P.n_slash > 0 && !slash) return fail(MS_ERR_INVALID_ARG, "slash is null but a Vertical-Slash head keeps slashes");
  if (bs && P.n_blocks > 0 && !blocks) return fail(MS_ERR_INVALID_ARG, "blocks is null but a Block-Sparse head is present");
  for (const void* p : {vert, slash, blocks})
    if (p && !aligned(p, 4)) return fail(MS_ERR_INVALID_ARG, "selection arrays must be 4-byte aligned");
  return MS_OK;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

const char* ms_status_string(ms_status s) {
  switch (s) {
    case MS_OK: return "ok";
    case MS_ERR_INVALID_ARG: return "invalid argument";
    case MS_ERR_UNSUPPORTED: return "unsupported";
    case MS_ERR_CAPACITY: return "insufficient capacity";
    case MS_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* ms_last_error(void) { return g_err.c_str(); }

int32_t ms_version(void) { return 10000; }

ms_status ms_validate(const ms_problem* prob, const ms_head_params* params) {
  g_err.clear();
  Plan P;
  return make_plan(prob, params, P);
}

ms_status ms_selection_sizes(const ms_problem* prob, const ms_head_params* params, int64_t* n_vert, int64_t* n_slash,
                             int64_t* n_blocks) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  if (n_vert) *n_vert = P.n_vert;
  if (n_slash) *n_slash = P.n_slash;
  if (n_blocks) *n_blocks = P.n_blocks;
  return MS_OK;
}

ms_status ms_estimate_workspace_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes) {
  g_err.clear();
  if (!params || !bytes) return fail(MS_ERR_INVALID_ARG, "params and bytes must be non-null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  *bytes = P.est_bytes;
  return MS_OK;
}

ms_status ms_index_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes) {
  g_err.clear();
  if (!params || !bytes) return fail(MS_ERR_INVALID_ARG, "params and bytes must be non-null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  *bytes = P.index_bytes;
  return MS_OK;
}

ms_status ms_index_layout(const ms_problem* prob, const ms_head_params* params, int64_t* offsets, int64_t* caps) {
  g_err.clear();
  if (!params || !offsets || !caps) return fail(MS_ERR_INVALID_ARG, "params, offsets and caps must be non-null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  for (int h = 0; h < P.hq; ++h) {
    offsets[4 * h + 0] = P.desc[h].rng_ptr_off;
    offsets[4 * h + 1] = P.desc[h].rng_off;
    offsets[4 * h + 2] = P.desc[h].col_ptr_off;
    offsets[4 * h + 3] = P.desc[h].col_off;
    caps[2 * h + 0] = P.cap_r[h];
    caps[2 * h + 1] = P.cap_c[h];
  }
  return MS_OK;
}

ms_status ms_attn_workspace_bytes(const ms_problem* prob, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MS_ERR_INVALID_ARG, "bytes is null");
  Plan P;
  MS_TRY(make_plan(prob, nullptr, P));
  *bytes = P.attn_bytes;
  return MS_OK;
}

ms_status ms_workspace_bytes(const ms_problem* prob, const ms_head_params* params, size_t* bytes) {
  g_err.clear();
  if (!params || !bytes) return fail(MS_ERR_INVALID_ARG, "params and bytes must be non-null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  *bytes = P.o_total;
  return MS_OK;
}

ms_status ms_estimate_vs(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                         int32_t* vert, int32_t* slash, float* dbg_v, float* dbg_s, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  if (P.n_vs == 0) return MS_OK;
  MS_TRY(check_tensor(q, "q"));
  MS_TRY(check_tensor(k, "k"));
  MS_TRY(check_selection_ptrs(P, vert, slash, nullptr, true, false));
  if ((dbg_v && !aligned(dbg_v, 4)) || (dbg_s && !aligned(dbg_s, 4)))
    return fail(MS_ERR_INVALID_ARG, "debug score arrays must be 4-byte aligned");
  MS_TRY(check_ws(ws, ws_bytes, P.est_bytes, "ws"));
  return run_estimate_vs(P, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), vert, slash, dbg_v,
                         dbg_s, static_cast<char*>(ws), stream);
}

ms_status ms_estimate_block(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                            int32_t* blocks, float* dbg_scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  if (P.n_bs == 0) return MS_OK;
  MS_TRY(check_tensor(q, "q"));
  MS_TRY(check_tensor(k, "k"));
  MS_TRY(check_selection_ptrs(P, nullptr, nullptr, blocks, false, true));
  if (dbg_scores && !aligned(dbg_scores, 4)) return fail(MS_ERR_INVALID_ARG, "dbg_scores must be 4-byte aligned");
  MS_TRY(check_ws(ws, ws_bytes, P.est_bytes, "ws"));
  return run_estimate_block(P, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), blocks, dbg_scores,
                            static_cast<char*>(ws), stream);
}

ms_status ms_build_index(const ms_problem* prob, const ms_head_params* params, const int32_t* vert,
                         const int32_t* slash, const int32_t* blocks, void* index, size_t index_bytes,
                         hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  MS_TRY(check_selection_ptrs(P, vert, slash, blocks, true, true));
  MS_TRY(check_ws(index, index_bytes, P.index_bytes, "index"));
  return run_build_index(P, vert, slash, blocks, static_cast<char*>(index), stream);
}

ms_status ms_sparse_attn_indexed(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                                 const void* v, const void* index, size_t index_bytes, void* out, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  MS_TRY(check_tensor(q, "q"));
  MS_TRY(check_tensor(k, "k"));
  MS_TRY(check_tensor(v, "v"));
  MS_TRY(check_tensor(out, "out"));
  if (lse && !aligned(lse, 4)) return fail(MS_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  MS_TRY(check_ws(index, index_bytes, P.index_bytes, "index"));
  MS_TRY(check_ws(ws, ws_bytes, P.attn_bytes, "ws"));
  return run_attention(P, q, k, v, static_cast<const char*>(index), out, lse, static_cast<char*>(ws), stream);
}

ms_status ms_sparse_attn(const ms_problem* prob, const ms_head_params* params, const void* q, const void* k,
                         const void* v, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  MS_TRY(check_tensor(q, "q"));
  MS_TRY(check_tensor(k, "k"));
  MS_TRY(check_tensor(v, "v"));
  MS_TRY(check_tensor(out, "out"));
  if (lse && !aligned(lse, 4)) return fail(MS_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  MS_TRY(check_ws(ws, ws_bytes, P.o_total, "ws"));
  char* w = static_cast<char*>(ws);
  int32_t* vert = reinterpret_cast<int32_t*>(w + P.o_vert);
  int32_t* slash = reinterpret_cast<int32_t*>(w + P.o_slash);
  int32_t* blocks = reinterpret_cast<int32_t*>(w + P.o_blocks);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  MS_TRY(run_estimate_vs(P, qq, kk, vert, slash, nullptr, nullptr, w + P.o_est, stream));
  MS_TRY(run_estimate_block(P, qq, kk, blocks, nullptr, w + P.o_est, stream));
  MS_TRY(run_build_index(P, vert, slash, blocks, w + P.o_index, stream));
  return run_attention(P, q, k, v, w + P.o_index, out, lse, w + P.o_attn, stream);
}

ms_status ms_sparse_attn_noalloc(const ms_problem* prob, const ms_head_params* params, const void* q,
                                 const void* k, const void* v, void* out, float* lse, hipStream_t stream) {
  g_err.clear();
  if (!params) return fail(MS_ERR_INVALID_ARG, "params is null");
  Plan P;
  MS_TRY(make_plan(prob, params, P));
  if (P.o_total > kScratchBytes)
    return fail(MS_ERR_CAPACITY, "the layer needs %zu bytes of workspace; the static scratch holds %zu (%d MiB)",
                P.o_total, kScratchBytes, (int)(kScratchBytes >> 20));
  void* ws = nullptr;
  MS_TRY(scratch_of_current_device(&ws));
  return ms_sparse_attn(prob, params, q, k, v, out, lse, ws, kScratchBytes, stream);
}

ms_status ms_noalloc_scratch_bytes(size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MS_ERR_INVALID_ARG, "bytes is null");
  *bytes = kScratchBytes;
  return MS_OK;
}

ms_status ms_dense_attn(const ms_problem* prob, const void* q, const void* k, const void* v, void* out, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  Plan P;
  MS_TRY(make_plan(prob, nullptr, P));
  MS_TRY(check_tensor(q, "q"));
  MS_TRY(check_tensor(k, "k"));
  MS_TRY(check_tensor(v, "v"));
  MS_TRY(check_tensor(out, "out"));
  if (lse && !aligned(lse, 4)) return fail(MS_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  MS_TRY(check_ws(ws, ws_bytes, P.v16_bytes, "ws"));
  _Float16* v16 = reinterpret_cast<_Float16*>(ws);
  HIP_TRY(launch_v_to_f16(static_cast<const uint16_t*>(v), v16, (int64_t)P.hkv * P.n * kD, stream),
          "V conversion launch");
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v16 = v16;
  a.out = out;
  a.lse = lse;
  a.table = nullptr;
  a.arena = nullptr;
  a.n = P.n;
  a.hq = P.hq;
  a.hkv = P.hkv;
  a.grp = P.grp;
  a.nb = (int)P.nbq;
  a.qb0 = (int)P.qb0;
  a.qm = P.qm;
  a.scale_log2 = P.scale_log2;
  a.out_f32 = P.out_f32;
  HIP_TRY(launch_group_dense(a, stream), "attention launch");
  return MS_OK;
}

ms_status ms_set_pace_polls(int32_t polls) {
  g_err.clear();
  if (polls < 0) return fail(MS_ERR_INVALID_ARG, "polls = %d is negative", polls);
  g_pace_polls.store(polls, std::memory_order_relaxed);
  return MS_OK;
}

ms_status ms_topk_f32(const float* x, int64_t n, int32_t k, int32_t* idx, hipStream_t stream) {
  g_err.clear();
  if (!x || !idx) return fail(MS_ERR_INVALID_ARG, "x and idx must be non-null");
  if (n < 1 || n > (int64_t{1} << 30)) return fail(MS_ERR_INVALID_ARG, "n = %lld out of 1..2^30", (long long)n);
  if (k < 0) return fail(MS_ERR_INVALID_ARG, "k = %d is negative", k);
  if (!aligned(x, 4) || !aligned(idx, 4)) return fail(MS_ERR_INVALID_ARG, "x and idx must be 4-byte aligned");
  TopkJobs j{};
  j.count = 1;
  j.src_off[0] = 0;
  j.dst_off[0] = 0;
  j.k[0] = k;
  HIP_TRY(launch_topk_rows(x, n, j, idx, stream), "top-k launch");
  return MS_OK;
}

ms_status ms_attention_recall(const ms_problem* prob, const float* lse_sparse, const float* lse_dense,
                              float* recall, hipStream_t stream) {
  g_err.clear();
  Plan P;
  MS_TRY(make_plan(prob, nullptr, P));
  if (!lse_sparse || !lse_dense || !recall) return fail(MS_ERR_INVALID_ARG, "lse_sparse, lse_dense and recall must be non-null");
  if (!aligned(lse_sparse, 4) || !aligned(lse_dense, 4) || !aligned(recall, 4))
    return fail(MS_ERR_INVALID_ARG, "lse_sparse, lse_dense and recall must be 4-byte aligned");
  HIP_TRY(launch_recall(lse_sparse, lse_dense, P.qm, P.hq, recall, stream), "recall launch");
  return MS_OK;
}

}  // extern "C"
