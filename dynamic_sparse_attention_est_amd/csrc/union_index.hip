// Per-chunk union of the sparse index for the grouped attention kernel
// (gfx950).  A chunk is up to four query heads of one KV head that one
// workgroup serves together; that workgroup streams each key it needs through
// LDS once, so it walks the union of its heads' key sets:
//   urng: the union of the heads' ranges of query block b (sorted, disjoint,
//         non-touching half-open ranges), CSR over the blocks;
//   ucol: the union of the heads' column lists (ascending, no repeats), CSR,
//         with umask[k] = bit j set when head j of the group lists column k.
// Every head still attends only to its own keys: the attention kernel masks
// per head (from the head's own ranges for range pieces, from umask for
// column pieces).  One thread merges the lists of one (group, block): count
// pass, per-group scan, fill pass; counts never exceed the sums of the heads'
// per-block counts, which bound the arrays.
#include "block_scan.h"
#include "internal.h"

namespace msa {
namespace {

struct UnionArgs {
  const HeadDesc* table;
  const GroupDesc* groups;
  char* arena;
  int32_t n_groups;
  int32_t nb;
};

// Merge state over the (at most four) heads' lists of one block.
struct Lists {
  const int2* rng[4];
  int r[4], r_end[4];
  const int32_t* col[4];
  int c[4], c_end[4];
  int nh;
};

__device__ __forceinline__ void open_lists(const UnionArgs& a, const GroupDesc& gd, int b, Lists& L) {
  L.nh = gd.nheads;
  for (int j = 0; j < 4; ++j) {
    L.r[j] = L.r_end[j] = L.c[j] = L.c_end[j] = 0;
    L.rng[j] = nullptr;
    L.col[j] = nullptr;
    if (j >= L.nh) continue;
    const HeadDesc& d = a.table[gd.head[j]];
    const int32_t* rp = reinterpret_cast<const int32_t*>(a.arena + d.rng_ptr_off);
    const int32_t* cp = reinterpret_cast<const int32_t*>(a.arena + d.col_ptr_off);
    L.rng[j] = reinterpret_cast<const int2*>(a.arena + d.rng_off);
    L.col[j] = reinterpret_cast<const int32_t*>(a.arena + d.col_off);
    L.r[j] = rp[b];
    L.r_end[j] = rp[b + 1];
    L.c[j] = cp[b];
    L.c_end[j] = cp[b + 1];
  }
}

template <bool kFill>
__global__ __launch_bounds__(256) void union_pass(UnionArgs a) {
  const int64_t items = (int64_t)a.n_groups * a.nb;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int u = (int)(it / a.nb), b = (int)(it - (int64_t)u * a.nb);
    const GroupDesc gd = a.groups[u];
    int32_t* urp = reinterpret_cast<int32_t*>(a.arena + gd.urng_ptr_off);
    int32_t* ucp = reinterpret_cast<int32_t*>(a.arena + gd.ucol_ptr_off);
    int2* urng = reinterpret_cast<int2*>(a.arena + gd.urng_off);
    int32_t* ucol = reinterpret_cast<int32_t*>(a.arena + gd.ucol_off);
    uint8_t* umask = reinterpret_cast<uint8_t*>(a.arena + gd.umask_off);
    Lists L;
    open_lists(a, gd, b, L);
    int rbase = 0, rlim = 0, cbase = 0, clim = 0;
    if (kFill) {
      rbase = urp[b];
      rlim = urp[b + 1] - rbase;
      cbase = ucp[b];
      clim = ucp[b + 1] - cbase;
    }

    // Ranges: repeatedly take the lowest start among the heads' cursors.
    int nr = 0;
    int lo = 0, hi = -1;  // current union range (none while hi < 0)
    for (;;) {
      int best = -1, blo = 0, bhi = 0;
      for (int j = 0; j < L.nh; ++j) {
        if (L.r[j] < L.r_end[j]) {
          const int2 x = L.rng[j][L.r[j]];
          if (best < 0 || x.x < blo) {
            best = j;
            blo = x.x;
            bhi = x.y;
          }
        }
      }
      if (best < 0) break;
      ++L.r[best];
      if (bhi <= blo) continue;  // empty range
      if (hi >= 0 && blo <= hi) {
        hi = max(hi, bhi);
      } else {
        if (hi >= 0) {
          if (kFill && nr < rlim) urng[rbase + nr] = make_int2(lo, hi);
          ++nr;
        }
        lo = blo;
        hi = bhi;
      }
    }
    if (hi >= 0) {
      if (kFill && nr < rlim) urng[rbase + nr] = make_int2(lo, hi);
      ++nr;
    }

    // Columns: merge, one entry per distinct key, with the mask of its heads.
    int nc = 0;
    for (;;) {
      int key = 0x7fffffff;
      for (int j = 0; j < L.nh; ++j)
        if (L.c[j] < L.c_end[j]) key = min(key, L.col[j][L.c[j]]);
      if (key == 0x7fffffff) break;
      int m = 0;
      for (int j = 0; j < L.nh; ++j) {
        if (L.c[j] < L.c_end[j] && L.col[j][L.c[j]] == key) {
          m |= 1 << j;
          ++L.c[j];
        }
      }
      if (kFill && nc < clim) {
        ucol[cbase + nc] = key;
        umask[cbase + nc] = (uint8_t)m;
      }
      ++nc;
    }

    if (!kFill) {
      urp[b + 1] = nr;
      ucp[b + 1] = nc;
      if (b == 0) {
        urp[0] = 0;
        ucp[0] = 0;
      }
    }
  }
}

// In-place inclusive scan of ptr[1..nb] for both CSR pointers of a group.
__global__ __launch_bounds__(1024) void union_scan(UnionArgs a) {
  __shared__ int warp_sum[1024 / 64];
  const GroupDesc gd = a.groups[blockIdx.x];
  for (int which = 0; which < 2; ++which) {
    int32_t* ptr = reinterpret_cast<int32_t*>(a.arena + (which ? gd.ucol_ptr_off : gd.urng_ptr_off));
    int carry = 0;
    for (int s0 = 0; s0 < a.nb; s0 += 1024) {
      const int i = s0 + threadIdx.x;
      const int x = i < a.nb ? ptr[1 + i] : 0;
      int tot;
      const int ex = block_excl_scan<1024>(x, warp_sum, &tot);
      if (i < a.nb) ptr[1 + i] = carry + ex + x;
      carry += tot;
    }
  }
}

__global__ void write_groups(GroupDesc* dst, GroupTableArgs ga, int count) {
  const int i = threadIdx.x;
  if (i < count) dst[i] = ga.g[i];
}

}  // namespace

hipError_t launch_union_build(const HeadDesc* table, GroupDesc* groups, const GroupDesc* host_groups, char* arena,
                              int n_groups, int nb, hipStream_t s) {
  for (int g0 = 0; g0 < n_groups; g0 += GroupTableArgs::kMax) {
    GroupTableArgs ga;
    const int m = n_groups - g0 < GroupTableArgs::kMax ? n_groups - g0 : GroupTableArgs::kMax;
    for (int i = 0; i < m; ++i) ga.g[i] = host_groups[g0 + i];
    hipLaunchKernelGGL(write_groups, dim3(1), dim3(GroupTableArgs::kMax), 0, s, groups + g0, ga, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  UnionArgs a{table, groups, arena, n_groups, nb};
  const int64_t items = (int64_t)n_groups * nb;
  const unsigned grid = (unsigned)((items + 255) / 256);
  hipLaunchKernelGGL(union_pass<false>, dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(union_scan, dim3((unsigned)n_groups), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(union_pass<true>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
