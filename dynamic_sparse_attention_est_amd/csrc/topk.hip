// Exact top-k selection for gfx950: the k largest scores, equal scores going
// to the lower index, written in ascending index order.  This is the selection
// step of both online estimators (MInference 1.0 summary, "Key points": the
// top vertical / slash lines of Vertical-Slash heads, the top key blocks of
// Block-Sparse heads).
//
// One workgroup per problem.  Scores are mapped to order-preserving uint32
// keys (-0 folded onto +0).  Four 8-bit radix passes (LDS histograms) find the
// exact key T of the k-th largest and how many keys equal to T are needed;
// a final pass in index order keeps every key > T and the first `need` keys
// == T, compacting with block-wide prefix sums, so the output is ascending
// and independent of thread timing.
#include "internal.h"
#include "block_scan.h"

namespace msa {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u << 1) == 0) u = 0;  // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
struct TopkSmem {
  int hist[256];
  int warp_sum[NT / 64];
  uint32_t prefix, mask;
  int rem;
};

// Top-k of x[0..n) into out[0..min(k, n)).  All threads of the block call it.
template <int NT>
__device__ void block_topk(const float* x, int64_t n, int k, int32_t* out, TopkSmem<NT>& sm) {
  const int tid = threadIdx.x;
  if (k <= 0) return;
  if ((int64_t)k >= n) {
    for (int64_t i = tid; i < n; i += NT) out[i] = (int32_t)i;
    return;
  }
  if (tid == 0) {
    sm.prefix = 0;
    sm.mask = 0;
    sm.rem = k;
  }
  __syncthreads();
  static_assert(NT >= 256, "one thread per digit");
  const int lane = tid & 63;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sm.prefix, mask = sm.mask;
    const int rem = sm.rem;
    for (int64_t i0 = 0; i0 < n; i0 += NT) {
      const int64_t i = i0 + tid;
      const uint32_t key = i < n ? order_key(x[i]) : 0u;
      bool left = i < n && (key & mask) == prefix;
      const uint32_t d = (key >> shift) & 255;
      if (shift == 24) {
        // the first digit (sign and upper exponent bits) is mostly shared by
        // neighbouring scores: the lanes of the wave's two most common digits
        // add their counts in one atomic each
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint64_t pend = __ballot(left);
          if (pend == 0) break;
          const int ld = (int)__builtin_ctzll(pend);
          const uint32_t dl = __builtin_amdgcn_readlane(d, ld);
          const bool mine = left && d == dl;
          const uint64_t same = __ballot(mine);
          if (lane == ld) atomicAdd(&sm.hist[dl], (int)__builtin_popcountll(same));
          left = left && !mine;
        }
      }
      if (left) atomicAdd(&sm.hist[d], 1);
    }
    __syncthreads();
    // Digit of the rem-th largest key: thread t holds bin 255 - t, so its
    // exclusive prefix sum counts the keys in higher bins; the one thread
    // whose bin holds the rem-th key records it (bin 0 when no higher bin
    // does).
    const int bin = 255 - tid;
    const int cnt = tid < 256 ? sm.hist[bin] : 0;
    int tot;
    const int above = block_excl_scan<NT>(cnt, sm.warp_sum, &tot);
    if (tid < 256 && above < rem && (above + cnt >= rem || bin == 0)) {
      sm.rem = rem - above;
      sm.prefix = prefix | ((uint32_t)bin << shift);
      sm.mask = mask | (255u << shift);
    }
    __syncthreads();
  }
  const uint32_t T = sm.prefix;
  const int need = sm.rem;  // keys equal to T that are taken (>= 1)
  int base = 0, eq_base = 0;
  for (int64_t start = 0; start < n && base < k; start += NT) {
    const int64_t i = start + tid;
    const uint32_t key = i < n ? order_key(x[i]) : 0u;
    const int gt = (i < n) & (key > T);
    const int eq = (i < n) & (key == T);
    int eq_total, sel_total;
    const int eq_rank = eq_base + block_excl_scan<NT>(eq, sm.warp_sum, &eq_total);
    const int sel = gt | (eq & (eq_rank < need));
    const int pos = base + block_excl_scan<NT>(sel, sm.warp_sum, &sel_total);
    if (sel) out[pos] = (int32_t)i;
    base += sel_total;
    eq_base += eq_total;
  }
}

constexpr int kTopkThreads = 512;

// Jobs 0 .. split-1 write to dst + dst_off, the rest to dst2 + dst_off.
__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* src, int64_t n, TopkJobs jobs,
                                                          int32_t* dst, int32_t* dst2, int split) {
  __shared__ TopkSmem<kTopkThreads> sm;
  const int j = blockIdx.x;
  block_topk<kTopkThreads>(src + jobs.src_off[j], n, jobs.k[j], (j < split ? dst : dst2) + jobs.dst_off[j], sm);
}

constexpr int kSelThreads = 256;

// Block-Sparse selection: local query block bl (query block b = qb0 + bl) of
// BS slot `slot` keeps the top min(k, b+1) of scores[slot][bl][0..b]; the
// rest of its k-wide row is -1.
struct BsSelArgs {
  int32_t k[kMaxHeads];
  int64_t dst_off[kMaxHeads];
};

// Rows of up to kRankMax candidates rank every candidate directly: with
// key_j = (order key of score j, ~j) as one 64-bit value, candidate i is kept
// iff fewer than min(k, b+1) keys exceed key_i (larger score, or equal score
// and lower index); the kept ones are compacted in index order.
constexpr int kRankMax = 512;  // (b+1)^2 comparisons per row: short rows only

__global__ __launch_bounds__(kSelThreads) void bs_select(const float* scores, int nb, int nbq, int qb0,
                                                         BsSelArgs sa, int32_t* blocks) {
  __shared__ TopkSmem<kSelThreads> sm;
  __shared__ uint64_t kv[kRankMax];
  const int t = threadIdx.x;
  const int bl = blockIdx.x, slot = blockIdx.y;
  const int b = qb0 + bl;
  const int k = sa.k[slot];
  int32_t* row = blocks + sa.dst_off[slot] + (int64_t)bl * k;
  const float* x = scores + ((int64_t)slot * nbq + bl) * nb;
  const int m = b + 1;  // candidate key blocks 0..b
  const int cnt = min(k, m);
  if (cnt == m) {
    for (int i = t; i < m; i += kSelThreads) row[i] = i;
  } else if (m <= kRankMax) {
    for (int i = t; i < m; i += kSelThreads)
      kv[i] = ((uint64_t)order_key(x[i]) << 32) | (uint64_t)(~(uint32_t)i);
    __syncthreads();
    int base = 0;
    for (int r0 = 0; r0 < m; r0 += kSelThreads) {
      const int i = r0 + t;
      int sel = 0;
      if (i < m) {
        const uint64_t me = kv[i];
        int above = 0;
#pragma unroll 8
        for (int j = 0; j < m; ++j) above += kv[j] > me;
        sel = above < cnt;
      }
      int total;
      const int pos = base + block_excl_scan<kSelThreads>(sel, sm.warp_sum, &total);
      if (sel) row[pos] = i;
      base += total;
    }
  } else {
    block_topk<kSelThreads>(x, m, k, row, sm);
  }
  for (int i = cnt + t; i < k; i += kSelThreads) row[i] = -1;
}

// ---------------------------------------------------------------------------
// Many workgroups per problem (long score vectors): the same radix select with
// chunk histograms merged in a fixed order, then an ordered compaction whose
// per-chunk output offsets come from a scan over the chunks.
constexpr int kChunk = 16384;  // elements per workgroup
constexpr int kMT = 256;

struct TopkState {
  uint32_t prefix, mask;
  int rem;   // keys equal to the final prefix still to take
  int pad;
};

__global__ void topk_init(TopkJobs jobs, TopkState* st) {
  const int j = threadIdx.x;
  if (j < jobs.count) st[j] = TopkState{0u, 0u, jobs.k[j], 0};
}

// A chunk of kChunk scores is read as kChunk / (4 kMT) rounds of one 16-byte
// load per thread, all issued before any is used, so a workgroup has its
// whole chunk in flight at once; thread t takes scores 4 (kMT r + t) .. +3 of
// round r.  Score vectors start 16-byte aligned and hold a multiple of 64
// scores, so a round is either inside the chunk or past its end.
constexpr int kRounds = kChunk / (4 * kMT);

struct ChunkKeys {
  uint32_t key[kRounds][4];
  bool valid[kRounds];
};

__device__ __forceinline__ void load_chunk(const float* x, int64_t n, int c, int t, ChunkKeys& ck) {
  const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
  f32x4 v[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t i4 = (int64_t)c * (kChunk / 4) + (int64_t)kMT * r + t;  // 4-score group
    ck.valid[r] = 4 * i4 < n;
    v[r] = ck.valid[r] ? x4[i4] : f32x4{};
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) ck.key[r][e] = order_key(v[r][e]);
}

// The last pass (shift 0) also counts the chunk's keys whose upper 24 bits
// exceed the prefix (above[j][c]) and stores suffix sums (entry d: keys with
// the prefix and a low byte >= d), so that once the last digit is known a
// chunk's counts above and at the threshold are two reads, not another pass.
__global__ __launch_bounds__(kMT) void topk_hist(const float* src, int64_t n, TopkJobs jobs, const TopkState* st,
                                                 int* hist, int* above, int nchunks, int shift) {
  __shared__ int h[256];
  __shared__ int red[kMT / 64];
  const int c = blockIdx.x, j = blockIdx.y, t = threadIdx.x;
  h[t] = 0;
  const float* x = src + jobs.src_off[j];
  const uint32_t prefix = st[j].prefix, mask = st[j].mask;
  ChunkKeys ck;
  load_chunk(x, n, c, t, ck);
  __syncthreads();
  int ab = 0;
  const int lane = t & 63;
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = ck.key[r][e];
      const bool act = ck.valid[r] && (key & mask) == prefix;
      const uint32_t d = (key >> shift) & 255;
      bool left = act;
      if (shift == 24) {
        // The first digit is the sign and the exponent's upper bits, which
        // neighbouring scores mostly share: the lanes of the two digits met
        // first add their counts in one LDS atomic per digit instead of one
        // each on the same address.  (Later digits vary from lane to lane.)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint64_t pend = __ballot(left);
          if (pend == 0) break;
          const int ld = (int)__builtin_ctzll(pend);
          const uint32_t dl = __builtin_amdgcn_readlane(d, ld);
          const bool mine = left && d == dl;
          const uint64_t same = __ballot(mine);
          if (lane == ld) atomicAdd(&h[dl], (int)__builtin_popcountll(same));
          left = left && !mine;
        }
      }
      if (left) atomicAdd(&h[d], 1);
      if (shift == 0) ab += ck.valid[r] & ((key >> 8) > (prefix >> 8));
    }
  __syncthreads();
  int v = h[t];
  if (shift == 0) {
    // suffix sums over the 256 bins (thread t ends with bins t .. 255)
#pragma unroll
    for (int d = 1; d < 256; d <<= 1) {
      const int u = t + d < 256 ? h[t + d] : 0;
      __syncthreads();
      v += u;
      h[t] = v;
      __syncthreads();
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) ab += __shfl_xor(ab, d);
    if ((t & 63) == 0) red[t >> 6] = ab;
    __syncthreads();
    if (t == 0) {
      int sum = 0;
      for (int wv = 0; wv < kMT / 64; ++wv) sum += red[wv];
      above[(int64_t)j * nchunks + c] = sum;
    }
  }
  hist[((int64_t)j * nchunks + c) * 256 + t] = v;
}

__global__ __launch_bounds__(256) void topk_digit(TopkState* st, const int* hist, int nchunks, int shift) {
  __shared__ int tot[256];
  const int j = blockIdx.x, t = threadIdx.x;
  // four independent sums, loads issued sixteen chunks at a time
  int s4[4] = {0, 0, 0, 0};
  const int* hj = hist + (int64_t)j * nchunks * 256 + t;
  int c = 0;
  for (; c + 16 <= nchunks; c += 16) {
#pragma unroll
    for (int u = 0; u < 16; ++u) s4[u & 3] += hj[(int64_t)(c + u) * 256];
  }
  for (; c < nchunks; ++c) s4[0] += hj[(int64_t)c * 256];
  tot[t] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  __syncthreads();
  if (shift == 0) {
    // the last pass stores suffix sums: back to per-bin counts
    const int next = t < 255 ? tot[t + 1] : 0;
    __syncthreads();
    tot[t] -= next;
    __syncthreads();
  }
  // Digit of the rem-th largest key: thread t takes bin 255 - t, so its
  // exclusive prefix sum counts the keys in higher bins; the one thread whose
  // bin holds the rem-th key records it (bin 0 when no higher bin does).
  __shared__ int wsum[4];
  const int rem = st[j].rem;
  const int bin = 255 - t, cnt = tot[bin];
  int total;
  const int above = block_excl_scan<256>(cnt, wsum, &total);
  if (above < rem && (above + cnt >= rem || bin == 0)) {
    st[j].rem = rem - above;
    st[j].prefix |= (uint32_t)bin << shift;
    st[j].mask |= 255u << shift;
  }
}

// Per chunk: output offset of its first selected key, and the number of
// threshold-equal keys in earlier chunks.
// A chunk's keys above the threshold T and equal to it come from the last
// pass: above[c] plus the suffix sum past T's low byte, and the difference of
// the suffix sums at and past it.
__global__ __launch_bounds__(64) void topk_bases(const TopkState* st, const int* hist, const int* above, int* bases,
                                                 int nchunks) {
  const int j = blockIdx.x, lane = threadIdx.x;
  const int need = st[j].rem;
  const int d4 = (int)(st[j].prefix & 255u);
  int gtp = 0, eqp = 0;  // counts of the chunks before this window
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    // one chunk per lane; exclusive prefix sums over the window by shuffles
    const int c = c0 + lane;
    const int64_t o = ((int64_t)j * nchunks + c) * 2;
    int g = 0, e = 0;
    if (c < nchunks) {
      const int* hc = hist + ((int64_t)j * nchunks + c) * 256;
      const int past = d4 < 255 ? hc[d4 + 1] : 0;
      g = above[(int64_t)j * nchunks + c] + past;
      e = hc[d4] - past;
    }
    int gs = g, es = e;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int gu = __shfl_up(gs, d), eu = __shfl_up(es, d);
      if (lane >= d) {
        gs += gu;
        es += eu;
      }
    }
    if (c < nchunks) {
      bases[o] = gtp + gs - g + min(need, eqp + es - e);
      bases[o + 1] = eqp + es - e;
    }
    gtp += __shfl(gs, 63);
    eqp += __shfl(es, 63);
  }
}

// Ordered compaction of a chunk: per round, thread t's four scores are
// consecutive in index order, so one workgroup scan per round places them.
__global__ __launch_bounds__(kMT) void topk_write(const float* src, int64_t n, TopkJobs jobs, const TopkState* st,
                                                  const int* bases, int32_t* dst, int32_t* dst2, int split,
                                                  int nchunks) {
  __shared__ int warp_sum[kMT / 64];
  const int c = blockIdx.x, j = blockIdx.y, t = threadIdx.x;
  const float* x = src + jobs.src_off[j];
  int32_t* out = (j < split ? dst : dst2) + jobs.dst_off[j];
  const uint32_t T = st[j].prefix;
  const int need = st[j].rem;
  int base = bases[((int64_t)j * nchunks + c) * 2];
  int eq_base = bases[((int64_t)j * nchunks + c) * 2 + 1];
  ChunkKeys ck;
  load_chunk(x, n, c, t, ck);
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    int gt[4], eq[4], eqc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gt[e] = ck.valid[r] & (ck.key[r][e] > T);
      eq[e] = ck.valid[r] & (ck.key[r][e] == T);
      eqc += eq[e];
    }
    int eq_total, sel_total;
    int eq_rank = eq_base + block_excl_scan<kMT>(eqc, warp_sum, &eq_total);
    int sel[4], selc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sel[e] = gt[e] | (eq[e] & (eq_rank < need));
      eq_rank += eq[e];
      selc += sel[e];
    }
    int pos = base + block_excl_scan<kMT>(selc, warp_sum, &sel_total);
    const int64_t i0 = 4 * ((int64_t)c * (kChunk / 4) + (int64_t)kMT * r + t);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sel[e]) out[pos++] = (int32_t)(i0 + e);
    base += sel_total;
    eq_base += eq_total;
  }
}

}  // namespace

hipError_t launch_topk_rows(const float* src, int64_t n, const TopkJobs& jobs, int32_t* dst, hipStream_t s) {
  if (jobs.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows, dim3((unsigned)jobs.count), dim3(kTopkThreads), 0, s, src, n, jobs, dst, dst,
                     jobs.count);
  return hipGetLastError();
}

size_t topk_scratch_bytes(int64_t n, int problems) {
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  return 256 + (size_t)problems * sizeof(TopkState) + (size_t)problems * nchunks * (256 + 3) * sizeof(int);
}

hipError_t launch_topk_chunked(const float* src, int64_t n, const TopkJobs& jobs, int32_t* dst, int32_t* dst2,
                               int split, void* scratch, hipStream_t s) {
  if (jobs.count <= 0) return hipSuccess;
  // Short vectors: one workgroup per vector runs every pass, every vector of
  // both selections in one launch (the same selection; launch latency
  // dominates at these sizes).
  if (n <= 2 * kChunk) {
    hipLaunchKernelGGL(topk_rows, dim3((unsigned)jobs.count), dim3(kTopkThreads), 0, s, src, n, jobs, dst, dst2,
                       split);
    return hipGetLastError();
  }
  const int nchunks = (int)((n + kChunk - 1) / kChunk);
  char* w = static_cast<char*>(scratch);
  TopkState* st = reinterpret_cast<TopkState*>(w);
  int* hist = reinterpret_cast<int*>(w + 256 + (size_t)jobs.count * sizeof(TopkState));
  int* above = hist + (size_t)jobs.count * nchunks * 256;
  int* bases = above + (size_t)jobs.count * nchunks;
  const dim3 grid((unsigned)nchunks, (unsigned)jobs.count);
  hipLaunchKernelGGL(topk_init, dim3(1), dim3(TopkJobs::kMaxJobs), 0, s, jobs, st);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(topk_hist, grid, dim3(kMT), 0, s, src, n, jobs, st, hist, above, nchunks, shift);
    hipLaunchKernelGGL(topk_digit, dim3((unsigned)jobs.count), dim3(256), 0, s, st, hist, nchunks, shift);
  }
  hipLaunchKernelGGL(topk_bases, dim3((unsigned)jobs.count), dim3(64), 0, s, st, hist, above, bases, nchunks);
  hipLaunchKernelGGL(topk_write, grid, dim3(kMT), 0, s, src, n, jobs, st, bases, dst, dst2, split, nchunks);
  return hipGetLastError();
}

hipError_t launch_bs_select(const float* scores, int nb, int nbq, int qb0, int n_bs, const int32_t* k_of_slot,
                            const int64_t* dst_off_of_slot, int32_t* blocks, hipStream_t s) {
  if (n_bs <= 0) return hipSuccess;
  BsSelArgs sa;
  for (int i = 0; i < n_bs; ++i) {
    sa.k[i] = k_of_slot[i];
    sa.dst_off[i] = dst_off_of_slot[i];
  }
  hipLaunchKernelGGL(bs_select, dim3((unsigned)nbq, (unsigned)n_bs), dim3(kSelThreads), 0, s, scores, nb, nbq, qb0,
                     sa, blocks);
  return hipGetLastError();
}

}  // namespace msa
