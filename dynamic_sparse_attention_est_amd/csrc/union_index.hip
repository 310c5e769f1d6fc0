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
// column pieces).  One workgroup merges the lists of one (chunk, block): each
// entry's place in the merged order is its index in its own list plus, by
// binary search, the number of entries of the other lists that come before it
// (equal starts or keys ordered by list); a prefix maximum of the range ends
// then marks where a new union range starts, and equal keys sit next to each
// other.  Count pass, per-chunk scan, fill pass; counts never exceed the sums
// of the heads' per-block counts, which bound the arrays.  Lists longer than
// LDS holds are merged in windows of the merged order: a window takes, from
// every list, the entries below the smallest of the lists' (cap / heads)-th
// next keys, so it never exceeds the cap and always advances; prefix maxima
// and counts carry from window to window, and a union range's end is written
// when the next one starts (or after the last window).
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

constexpr int kUT = 256;
constexpr int kCapR = 4096;  // ranges of one (chunk, block) merged in LDS
constexpr int kCapC = 8192;  // columns of one (chunk, block) merged in LDS

// Entries of the other lists that precede x: for lists before `mine`, entries
// <= x; for lists after it, entries < x (ties ordered by list).
__device__ __forceinline__ int preceding(const int* keys, const int* off, int nh, int mine, int x) {
  int r = 0;
  for (int j = 0; j < nh; ++j) {
    if (j == mine) continue;
    int lo = off[j], hi = off[j + 1];
    const bool le = j < mine;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (le ? keys[mid] <= x : keys[mid] < x) lo = mid + 1; else hi = mid;
    }
    r += lo - off[j];
  }
  return r;
}

// Whether the ascending keys[lo, hi) hold x.
__device__ __forceinline__ bool contains(const int* keys, int lo, int hi, int x) {
  const int end = hi;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo < end && keys[lo] == x;
}

template <bool kFill>
__global__ __launch_bounds__(kUT) void union_block(UnionArgs a) {
  __shared__ int s_key[kCapC];   // list entries (range starts / columns), lists one after another
  __shared__ int s_aux[kCapC];   // range ends (ranges), merged keys (columns)
  __shared__ int s_end[kCapR];   // merged range ends
  __shared__ int s_off[5];       // window: entries of list j at [s_off[j], s_off[j+1])
  __shared__ int s_pos[4], s_wend[4];
  __shared__ int s_bound;
  __shared__ int s_wbuf[kUT / 64];
  const int b = blockIdx.x, u = blockIdx.y, t = threadIdx.x;
  const GroupDesc gd = a.groups[u];
  int32_t* urp = reinterpret_cast<int32_t*>(a.arena + gd.urng_ptr_off);
  int32_t* ucp = reinterpret_cast<int32_t*>(a.arena + gd.ucol_ptr_off);
  int2* urng = reinterpret_cast<int2*>(a.arena + gd.urng_off);
  int32_t* ucol = reinterpret_cast<int32_t*>(a.arena + gd.ucol_off);
  uint8_t* umask = reinterpret_cast<uint8_t*>(a.arena + gd.umask_off);
  Lists L;
  open_lists(a, gd, b, L);
  const int nh = L.nh;
  int rbase = 0, rlim = 0, cbase = 0, clim = 0;
  if (kFill) {
    rbase = urp[b];
    rlim = urp[b + 1] - rbase;
    cbase = ucp[b];
    clim = ucp[b + 1] - cbase;
  }

  // Next window of the merged order: list j contributes its entries from
  // s_pos[j] whose key is below s_bound, the smallest of the lists'
  // (cap/nh)-th next keys (0x7fffffff: every list has fewer left, the last
  // window).  key(j, i) is entry i's key in list j.  Returns the window size.
  auto next_window = [&](int cap, const int* end, auto key) -> int {
    if (t == 0) {
      const int q = cap / nh;
      int x = 0x7fffffff;
      for (int j = 0; j < nh; ++j)
        if (s_pos[j] + q < end[j]) x = min(x, key(j, s_pos[j] + q));
      s_bound = x;
    }
    __syncthreads();
    if (t < nh) {
      int lo = s_pos[t], hi = end[t];
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (key(t, mid) < s_bound) lo = mid + 1; else hi = mid;
      }
      s_wend[t] = lo;
    }
    __syncthreads();
    if (t == 0) {
      s_off[0] = 0;
      for (int j = 0; j < nh; ++j) s_off[j + 1] = s_off[j] + (s_wend[j] - s_pos[j]);
    }
    __syncthreads();
    return s_off[nh];
  };

  // ---- ranges
  if (t < nh) s_pos[t] = L.r[t];
  __syncthreads();
  int carry_max = -1, carry_n = 0;
  for (;;) {
    const int R = next_window(kCapR, L.r_end, [&](int j, int i) { return L.rng[j][i].x; });
    for (int e = t; e < R; e += kUT) {
      int j = 0;
      while (e >= s_off[j + 1]) ++j;
      const int2 x = L.rng[j][s_pos[j] + e - s_off[j]];
      s_key[e] = x.x;
      s_aux[e] = x.y;
    }
    __syncthreads();
    for (int e = t; e < R; e += kUT) {
      int j = 0;
      while (e >= s_off[j + 1]) ++j;
      const int x = s_key[e];
      const int rank = (e - s_off[j]) + preceding(s_key, s_off, nh, j, x);
      s_end[rank] = s_aux[e];
      s_aux[kCapR + rank] = x;  // merged starts in the upper half of s_aux
    }
    __syncthreads();
    for (int c0 = 0; c0 < R; c0 += kUT) {
      const int e = c0 + t;
      const bool valid = e < R;
      const int lo = valid ? s_aux[kCapR + e] : 0x7fffffff;
      const int hi = valid ? s_end[e] : -1;
      const bool empty = valid && hi <= lo;
      int incl, excl, tot;
      block_scan_max<kUT>(valid && !empty ? hi : -1, -1, s_wbuf, &incl, &excl, &tot);
      excl = max(excl, carry_max);
      // a range starts a union range when it begins after every end before it,
      // which is then where the previous union range ends
      const bool is_new = valid && !empty && (lo > excl || excl < 0);
      int ntot;
      const int gid = carry_n + block_excl_scan<kUT>(is_new ? 1 : 0, s_wbuf, &ntot);
      if (kFill && is_new) {
        if (gid < rlim) urng[rbase + gid].x = lo;
        if (gid >= 1 && gid - 1 < rlim) urng[rbase + gid - 1].y = excl;
      }
      carry_max = max(carry_max, tot);
      carry_n += ntot;
    }
    const bool last = s_bound == 0x7fffffff;
    __syncthreads();
    if (t < nh) s_pos[t] = s_wend[t];
    __syncthreads();
    if (last) break;
  }
  if (kFill && t == 0 && carry_n >= 1 && carry_n - 1 < rlim) urng[rbase + carry_n - 1].y = carry_max;
  const int nr = carry_n;
  __syncthreads();

  // ---- columns
  if (t < nh) s_pos[t] = L.c[t];
  __syncthreads();
  int ccarry_n = 0, carry_last = -1;
  for (;;) {
    const int C = next_window(kCapC, L.c_end, [&](int j, int i) { return L.col[j][i]; });
    for (int e = t; e < C; e += kUT) {
      int j = 0;
      while (e >= s_off[j + 1]) ++j;
      s_key[e] = L.col[j][s_pos[j] + e - s_off[j]];
    }
    __syncthreads();
    for (int e = t; e < C; e += kUT) {
      int j = 0;
      while (e >= s_off[j + 1]) ++j;
      const int x = s_key[e];
      s_aux[(e - s_off[j]) + preceding(s_key, s_off, nh, j, x)] = x;
    }
    __syncthreads();
    for (int c0 = 0; c0 < C; c0 += kUT) {
      const int e = c0 + t;
      const bool valid = e < C;
      const int x = valid ? s_aux[e] : 0;
      const bool first = valid && (e == 0 ? x != carry_last : s_aux[e - 1] != x);
      int ntot;
      const int pos = ccarry_n + block_excl_scan<kUT>(first ? 1 : 0, s_wbuf, &ntot);
      if (kFill && first && pos < clim) {
        int m = 0;
        for (int j = 0; j < nh; ++j)
          if (contains(s_key, s_off[j], s_off[j + 1], x)) m |= 1 << j;
        ucol[cbase + pos] = x;
        umask[cbase + pos] = (uint8_t)m;
      }
      ccarry_n += ntot;
    }
    if (C > 0) carry_last = s_aux[C - 1];
    const bool last = s_bound == 0x7fffffff;
    __syncthreads();
    if (t < nh) s_pos[t] = s_wend[t];
    __syncthreads();
    if (last) break;
  }
  const int nc = ccarry_n;

  if (!kFill && t == 0) {
    urp[b + 1] = nr;
    ucp[b + 1] = nc;
    if (b == 0) {
      urp[0] = 0;
      ucp[0] = 0;
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
  const dim3 grid((unsigned)nb, (unsigned)n_groups);
  hipLaunchKernelGGL(union_block<false>, grid, dim3(kUT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(union_scan, dim3((unsigned)n_groups), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(union_block<true>, grid, dim3(kUT), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
