// Index conversion for gfx950: selected verticals / slashes / key blocks ->
// per-query-block key ranges plus gathered column lists (the MInference
// abstract: sparse indices built from each head's pattern; the PIT fragment:
// sparse shapes do not line up with GPU tiles, so each 64-row query tile gets
// the exact key spans it covers).
//
// Per head the index is a CSR over the call's query blocks (NBq = n/64 -
// q_block0 of them; local block bl is query block b = q_block0 + bl):
//   rng_ptr[NBq+1], rng[] = (lo, hi) half-open key ranges, sorted, disjoint,
//   non-touching; col_ptr[NBq+1], col[] = ascending single keys in no range.
// Query block b (rows 64b .. 64b+63, last = 64b+63):
//   Vertical-Slash: slash o <= last keeps [max(0, 64b-o), 64b+64-o).  Sorted
//     offsets whose gaps are <= 64 form runs; a run's spans merge into one
//     range and different runs never touch, so per head the runs are found
//     once (vs_template) and each block reads its ranges off them.  Vertical j
//     <= last is a column unless some offset lies in [max(0, 64b-j), 64b+63-j].
//   Block-Sparse: selected block c keeps [64c, 64c+64); consecutive c merge.
//   A-shape: [0, min(sink, 64b+64)) and [max(0, 64b-window+1), 64b+64), merged
//     when they touch (the per-row window is applied by the attention kernel).
//   Dense: [0, 64b+64).
// A Vertical-Slash head may ask for 32-row query blocks: its CSR then lists
// the 2 NBq blocks of 32 rows, each built by the same rules with 32 in place
// of 64 (a slash keeps [max(0, 32b-o), 32b+32-o), runs break at gaps > 32),
// and the workgroup of a 64-row block writes both of its halves.
// Three launches over (query block, head): count -> per-head scan -> fill.
// Counts are clamped to per-block capacities that the host also uses to size
// the arena, so malformed selections can never write past it, and every value
// written is clamped into [0, end of the block).
#include "block_scan.h"
#include "internal.h"

namespace msa {
namespace {

constexpr int kT = 256;

struct TableArgs {
  HeadDesc d[32];
};

__global__ void write_table(HeadDesc* table, TableArgs ta, int count) {
  const int i = threadIdx.x;
  if (i < count) table[i] = ta.d[i];
}

__device__ __forceinline__ int upper_bound(const int32_t* a, int n, int x) {  // # of a[i] <= x
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int lower_bound(const int32_t* a, int n, int x) {  // # of a[i] < x
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Per-block capacities (same formulas as the host's arena sizing); b counts
// blocks of the head's own height (d.qrows rows for Vertical-Slash heads).
__device__ __forceinline__ int cap_ranges(const HeadDesc& d, int b) {
  const int last = b * kBM + kBM - 1;
  switch (d.pattern) {
    case MS_VERTICAL_SLASH: return min(d.p1, (b * d.qrows + d.qrows - 1) / (d.qrows + 1) + 1);
    case MS_BLOCK_SPARSE: return min(min(d.p0, b + 1), b / 2 + 1);
    case MS_A_SHAPE: return 2;
    case MS_GRID: return min(d.p2, (last + d.p3) / d.p0) + 1;
    default: return 1;
  }
}
__device__ __forceinline__ int cap_cols(const HeadDesc& d, int b) {
  return d.pattern == MS_VERTICAL_SLASH ? min(d.p0, b * d.qrows + d.qrows) : 0;
}

struct IdxArgs {
  const HeadDesc* table;
  char* arena;
  const int32_t* vert;
  const int32_t* slash;
  const int32_t* blocks;  // Block-Sparse selections, [NBq][k] per head
  int32_t nb;             // query blocks of the call (NBq)
  int32_t qb0;            // first query block
};

// Runs of the sorted slash offsets (consecutive offsets at most the block
// height apart share a run): run[0] = number of runs, run[1 + r] = index of
// run r's first offset.
__global__ __launch_bounds__(kT) void vs_template(IdxArgs a) {
  __shared__ int warp_sum[kT / 64];
  const HeadDesc d = a.table[blockIdx.x];
  if (d.pattern != MS_VERTICAL_SLASH) return;
  const int32_t* S = a.slash + d.slash_off;
  int32_t* run = reinterpret_cast<int32_t*>(a.arena + d.run_off);
  const int ks = d.p1;
  int base = 0;
  for (int s0 = 0; s0 < ks; s0 += kT) {
    const int i = s0 + threadIdx.x;
    const int start = i < ks && (i == 0 || S[i] - S[i - 1] > d.qrows);
    int tot;
    const int pos = base + block_excl_scan<kT>(start, warp_sum, &tot);
    if (start) run[1 + pos] = i;
    base += tot;
  }
  if (threadIdx.x == 0) run[0] = base;
}

// Ranges / columns of one (head, block), counted (kFill = false) or written.
template <bool kFill>
__global__ __launch_bounds__(kT) void index_pass(IdxArgs a) {
  __shared__ int warp_sum[kT / 64];
  const int bl = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int b = a.qb0 + bl;  // query block; bl indexes the CSR
  const HeadDesc d = a.table[h];
  const int row0 = b * kBM, last = row0 + kBM - 1, end = row0 + kBM;
  int32_t* rng_ptr = reinterpret_cast<int32_t*>(a.arena + d.rng_ptr_off);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(a.arena + d.col_ptr_off);
  int2* rng = reinterpret_cast<int2*>(a.arena + d.rng_off);
  int32_t* col = reinterpret_cast<int32_t*>(a.arena + d.col_off);
  int nr = 0, nc = 0;
  int rbase = 0, cbase = 0, rlim = 0, clim = 0;
  auto csr_block = [&](int cb) {  // this workgroup's CSR block cb: its slots
    if (kFill) {
      rbase = rng_ptr[cb];
      rlim = rng_ptr[cb + 1] - rbase;
      cbase = col_ptr[cb];
      clim = col_ptr[cb + 1] - cbase;
    }
  };

  if (d.pattern == MS_VERTICAL_SLASH) {
    const int32_t* S = a.slash + d.slash_off;
    const int32_t* V = a.vert + d.vert_off;
    const int32_t* run = reinterpret_cast<const int32_t*>(a.arena + d.run_off);
    const int ks = d.p1, kv = d.p0, nruns = run[0];
    const int rows = d.qrows, per = kBM / rows;
    // the 64-row block's one or two CSR blocks of `rows` rows
    for (int half = 0; half < per; ++half) {
      const int cb = bl * per + half;           // CSR block
      const int gb = b * per + half;            // query block of `rows` rows in the sequence
      const int hrow0 = gb * rows, hlast = hrow0 + rows - 1, hend = hrow0 + rows;
      csr_block(cb);
      const int ub = upper_bound(S, ks, hlast);  // offsets that reach this block
      int hr = ub == 0 ? 0 : upper_bound(run + 1, nruns, ub - 1);
      hr = min(hr, cap_ranges(d, gb));
      if (kFill) {
        for (int p = tid; p < min(hr, rlim); p += kT) {
          const int r = hr - 1 - p;  // runs of larger offsets give lower keys
          const int first = run[1 + r];
          const int stop = min(r + 1 < nruns ? run[2 + r] : ks, ub);
          const int lo = min(max(0, hrow0 - S[stop - 1]), hend);
          const int hi = min(max(lo, hrow0 + rows - S[first]), hend);
          rng[rbase + p] = make_int2(lo, hi);
        }
      }
      const int ubv = upper_bound(V, kv, hlast);
      int cnt = 0;
      for (int s0 = 0; s0 < ubv; s0 += kT) {
        const int i = s0 + tid;
        int keep = 0;
        int j = 0;
        if (i < ubv) {
          j = V[i];
          const int lbo = lower_bound(S, ks, max(0, hrow0 - j));
          keep = j >= 0 && !(lbo < ks && S[lbo] <= hlast - j);
        }
        int tot;
        const int pos = cnt + block_excl_scan<kT>(keep, warp_sum, &tot);
        if (kFill && keep && pos < clim) col[cbase + pos] = j;
        cnt += tot;
      }
      const int hc = min(cnt, cap_cols(d, gb));
      if (!kFill && tid == 0) {
        rng_ptr[cb + 1] = hr;
        col_ptr[cb + 1] = hc;
        if (cb == 0) {
          rng_ptr[0] = 0;
          col_ptr[0] = 0;
        }
      }
    }
    return;
  }
  csr_block(bl);
  const int rcap = cap_ranges(d, b);
  if (d.pattern == MS_BLOCK_SPARSE) {
    const int k = d.p0;
    const int32_t* B = a.blocks + d.blk_off + (int64_t)bl * k;
    const int cnt = min(k, b + 1);  // leading entries hold the selection
    // Run r starts at the r-th start and ends at the r-th stop; a run may
    // start in one pass of kT entries and stop in a later one, so starts and
    // stops are ranked with counters of their own.
    int runs = 0, stops = 0;
    for (int s0 = 0; s0 < cnt; s0 += kT) {
      const int i = s0 + tid;
      int start = 0, stop = 0, c = 0;
      if (i < cnt) {
        c = B[i];
        start = i == 0 || B[i - 1] + 1 != c;
        stop = i == cnt - 1 || B[i + 1] != c + 1;
      }
      int t1, t2;
      const int ps = runs + block_excl_scan<kT>(start, warp_sum, &t1);
      const int pe = stops + block_excl_scan<kT>(stop, warp_sum, &t2);
      if (kFill) {
        if (start && ps < rlim) rng[rbase + ps].x = min(max(0, c * kBM), end);
        if (stop && pe < rlim) rng[rbase + pe].y = min(max(0, c * kBM + kBM), end);
      }
      runs += t1;
      stops += t2;
    }
    nr = min(runs, rcap);
  } else if (d.pattern == MS_A_SHAPE) {
    const int sink = d.p0, window = d.p1;
    const int wlo = max(0, row0 - window + 1);
    const int shi = min(sink, end);
    if (sink > 0 && wlo > shi) {
      nr = 2;
      if (kFill && tid == 0 && rlim >= 2) {
        rng[rbase] = make_int2(0, shi);
        rng[rbase + 1] = make_int2(wlo, end);
      }
    } else {
      nr = 1;
      if (kFill && tid == 0 && rlim >= 1) rng[rbase] = make_int2(sink > 0 ? 0 : wlo, end);
    }
  } else if (d.pattern == MS_GRID) {
    // Offsets (o = i - j) kept: the local interval 0 .. window-1 and frame
    // group t = tP-w .. tP+w for t = 1..T, cut to <= last (groups with tP-w >
    // last do not reach the block: t <= tmax).  Offsets at most 64 apart give
    // key spans that touch, so intervals that close form one run, and a run
    // [ra, rb] of offsets keeps keys [max(0, row0 - rb), row0 + 64 - ra).
    //   P - 2w <= 64: consecutive groups touch; groups 1..tmax are one run,
    //     merged with the local one when it starts within 64 of it.
    //   P - 2w > 64: groups never touch each other; group t joins the local
    //     run iff tP - w <= window + 63 (t <= t1), the others are runs alone.
    // Ranges ascending in key order = runs in descending offset order.
    const int P = d.p0, W = d.p1, T = d.p2, wd = d.p3;
    const int tmax = min(T, (last + wd) / P);
    const int lob = min(W - 1, last);  // local interval [0, lob]
    if (P - 2 * wd <= kBM) {
      const bool grp = tmax >= 1;
      const int goa = max(0, P - wd), gob = min(last, tmax * P + wd);
      const bool merged = grp && goa - lob <= kBM;
      nr = grp && !merged ? 2 : 1;
      if (kFill && tid == 0) {
        if (!grp || merged) {
          if (rlim >= 1) rng[rbase] = make_int2(max(0, row0 - (grp ? max(lob, gob) : lob)), end);
        } else if (rlim >= 2) {
          rng[rbase] = make_int2(max(0, row0 - gob), end - goa);
          rng[rbase + 1] = make_int2(max(0, row0 - lob), end);
        }
      }
    } else {
      const int t1 = min(tmax, (W + 63 + wd) / P);
      const int alone = tmax - t1;  // groups t1+1 .. tmax, one run each
      nr = alone + 1;
      if (kFill) {
        for (int u = tid; u < alone && u < rlim; u += kT) {
          const int t = tmax - u;
          rng[rbase + u] = make_int2(max(0, row0 - min(last, t * P + wd)), end - (t * P - wd));
        }
        if (tid == 0 && alone < rlim) {
          const int rb = t1 >= 1 ? max(lob, min(last, t1 * P + wd)) : lob;
          rng[rbase + alone] = make_int2(max(0, row0 - rb), end);
        }
      }
    }
    nr = min(nr, rcap);
  } else {  // dense
    nr = 1;
    if (kFill && tid == 0 && rlim >= 1) rng[rbase] = make_int2(0, end);
  }

  if (!kFill && tid == 0) {
    rng_ptr[bl + 1] = nr;
    col_ptr[bl + 1] = nc;
    if (bl == 0) {
      rng_ptr[0] = 0;
      col_ptr[0] = 0;
    }
  }
}

// In-place inclusive scan of ptr[1..nblk] (ptr[0] = 0) for both CSR pointers
// (nblk = the call's query blocks of the head's own height).
__global__ __launch_bounds__(1024) void index_scan(IdxArgs a) {
  __shared__ int warp_sum[1024 / 64];
  const HeadDesc d = a.table[blockIdx.x];
  const int nblk = d.pattern == MS_VERTICAL_SLASH ? a.nb * (kBM / d.qrows) : a.nb;
  for (int which = 0; which < 2; ++which) {
    int32_t* ptr = reinterpret_cast<int32_t*>(a.arena + (which ? d.col_ptr_off : d.rng_ptr_off));
    int carry = 0;
    for (int s0 = 0; s0 < nblk; s0 += 1024) {
      const int i = s0 + threadIdx.x;
      const int x = i < nblk ? ptr[1 + i] : 0;
      int tot;
      const int ex = block_excl_scan<1024>(x, warp_sum, &tot);
      if (i < nblk) ptr[1 + i] = carry + ex + x;
      carry += tot;
    }
  }
}

}  // namespace

hipError_t launch_write_table(HeadDesc* table, const HeadDesc* host_descs, int first, int count, hipStream_t s) {
  for (int c0 = 0; c0 < count; c0 += 32) {
    TableArgs ta;
    const int m = count - c0 < 32 ? count - c0 : 32;
    for (int i = 0; i < m; ++i) ta.d[i] = host_descs[c0 + i];
    hipLaunchKernelGGL(write_table, dim3(1), dim3(32), 0, s, table + first + c0, ta, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_index_build(const HeadDesc* table, char* arena, int hq, int nb, int qb0, const int32_t* vert,
                              const int32_t* slash, const int32_t* blocks, hipStream_t s) {
  IdxArgs a{table, arena, vert, slash, blocks, nb, qb0};
  hipLaunchKernelGGL(vs_template, dim3((unsigned)hq), dim3(kT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(index_pass<false>, dim3((unsigned)nb, (unsigned)hq), dim3(kT), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(index_scan, dim3((unsigned)hq), dim3(1024), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(index_pass<true>, dim3((unsigned)nb, (unsigned)hq), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
