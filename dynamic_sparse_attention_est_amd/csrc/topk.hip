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
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sm.prefix, mask = sm.mask;
    for (int64_t i = tid; i < n; i += NT) {
      const uint32_t key = order_key(x[i]);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, d = 255;
      for (; d > 0; --d) {
        if (above + sm.hist[d] >= sm.rem) break;
        above += sm.hist[d];
      }
      sm.rem -= above;
      sm.prefix = prefix | ((uint32_t)d << shift);
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

__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* src, int64_t n, TopkJobs jobs,
                                                          int32_t* dst) {
  __shared__ TopkSmem<kTopkThreads> sm;
  const int j = blockIdx.x;
  block_topk<kTopkThreads>(src + jobs.src_off[j], n, jobs.k[j], dst + jobs.dst_off[j], sm);
}

constexpr int kSelThreads = 256;

// Block-Sparse selection: query block b of BS slot `slot` keeps the top
// min(k, b+1) of scores[slot][b][0..b]; the rest of its k-wide row is -1.
struct BsSelArgs {
  int32_t k[kMaxHeads];
  int64_t dst_off[kMaxHeads];
};

__global__ __launch_bounds__(kSelThreads) void bs_select(const float* scores, int nb, BsSelArgs sa,
                                                         int32_t* blocks) {
  __shared__ TopkSmem<kSelThreads> sm;
  const int b = blockIdx.x, slot = blockIdx.y;
  const int k = sa.k[slot];
  int32_t* row = blocks + sa.dst_off[slot] + (int64_t)b * k;
  const float* x = scores + ((int64_t)slot * nb + b) * nb;
  const int cnt = min(k, b + 1);
  block_topk<kSelThreads>(x, b + 1, k, row, sm);
  for (int i = cnt + threadIdx.x; i < k; i += kSelThreads) row[i] = -1;
}

}  // namespace

hipError_t launch_topk_rows(const float* src, int64_t n, const TopkJobs& jobs, int32_t* dst, hipStream_t s) {
  if (jobs.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows, dim3((unsigned)jobs.count), dim3(kTopkThreads), 0, s, src, n, jobs, dst);
  return hipGetLastError();
}

hipError_t launch_bs_select(const float* scores, int nb, int n_bs, const int32_t* k_of_slot,
                            const int64_t* dst_off_of_slot, int32_t* blocks, hipStream_t s) {
  if (n_bs <= 0) return hipSuccess;
  BsSelArgs sa;
  for (int i = 0; i < n_bs; ++i) {
    sa.k[i] = k_of_slot[i];
    sa.dst_off[i] = dst_off_of_slot[i];
  }
  hipLaunchKernelGGL(bs_select, dim3((unsigned)nb, (unsigned)n_bs), dim3(kSelThreads), 0, s, scores, nb, sa, blocks);
  return hipGetLastError();
}

}  // namespace msa
