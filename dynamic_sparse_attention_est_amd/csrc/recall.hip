// Attention-mass recall of a sparse index (MInference 1.0 summary, "Key
// points": the share of the attention mass the kept entries capture is the
// pages' evidence that the estimated indices are good).  For row i of a head,
// the full causal attention puts mass exp(s_ij - lse_i) on key j, so the mass
// on the kept keys of the row is exp(lse_sparse_i - lse_dense_i): the ratio of
// the sparse kernel's normaliser to the dense kernel's.  One workgroup per
// head sums it over the rows in a fixed order (float64), and writes the mean.
#include "internal.h"

namespace msa {
namespace {

constexpr int kRT = 256;

__global__ __launch_bounds__(kRT) void recall_rows(const float* lse_sparse, const float* lse_dense, int64_t n,
                                                   float* recall) {
  __shared__ double part[kRT];
  const int h = blockIdx.x, t = threadIdx.x;
  const float* ls = lse_sparse + (int64_t)h * n;
  const float* ld = lse_dense + (int64_t)h * n;
  double acc = 0.0;
  for (int64_t i = t; i < n; i += kRT) {
    const float s = ls[i], d = ld[i];
    // an empty sparse row (lse -inf) keeps no mass
    if (s != -INFINITY && d != -INFINITY) acc += exp((double)s - (double)d);
  }
  part[t] = acc;
  __syncthreads();
  for (int half = kRT / 2; half > 0; half >>= 1) {
    if (t < half) part[t] += part[t + half];
    __syncthreads();
  }
  if (t == 0) recall[h] = (float)(part[0] / (double)n);
}

}  // namespace

hipError_t launch_recall(const float* lse_sparse, const float* lse_dense, int64_t n, int hq, float* recall,
                         hipStream_t s) {
  hipLaunchKernelGGL(recall_rows, dim3((unsigned)hq), dim3(kRT), 0, s, lse_sparse, lse_dense, n, recall);
  return hipGetLastError();
}

}  // namespace msa
