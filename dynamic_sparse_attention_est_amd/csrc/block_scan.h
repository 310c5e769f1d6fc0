// Workgroup-wide exclusive prefix sum for gfx950 (64-lane wavefronts):
// a shuffle scan inside each wavefront, then the wavefront totals through LDS.
#pragma once

#include <hip/hip_runtime.h>

namespace msa {

// All NT threads of the block call it with their value x; returns the sum of
// the values of lower threads and stores the block total in *total.
// warp_sum: LDS array of NT/64 ints.  Contains two block barriers.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int x, int* warp_sum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) warp_sum[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int ws = warp_sum[i];
    before += i < wv ? ws : 0;
    all += ws;
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

}  // namespace msa

namespace msa {

// Workgroup-wide inclusive and exclusive prefix maxima (exclusive of thread 0
// is `lowest`); *total receives the block maximum.  warp_buf: LDS array of
// NT/64 ints.  Contains two block barriers.
template <int NT>
__device__ __forceinline__ void block_scan_max(int x, int lowest, int* warp_buf, int* incl_out, int* excl_out,
                                               int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl = max(incl, y);
  }
  if (lane == 63) warp_buf[wv] = incl;
  __syncthreads();
  int before = lowest, all = lowest;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int ws = warp_buf[i];
    if (i < wv) before = max(before, ws);
    all = max(all, ws);
  }
  __syncthreads();
  const int prev = __shfl_up(incl, 1);
  *incl_out = max(before, incl);
  *excl_out = lane == 0 ? before : max(before, prev);
  *total = all;
}

}  // namespace msa
