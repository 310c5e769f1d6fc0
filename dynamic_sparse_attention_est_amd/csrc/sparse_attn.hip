// Sparse FlashAttention-style forward kernel for gfx950 (MInference 1.0
// summary, "Summary", third stage: attention computed only over the estimated
// indices; FlashAttention-2's online softmax is the published algorithm the
// pages' kernels build on).
//
// Work item: one 64-row query block of one Q head = one workgroup of two
// wavefronts, each owning 32 rows (a head indexed by 32-row query blocks: one
// 32-row block = one workgroup of one wavefront, which loads its tiles
// alone).  The block's keys are its ranges, cut into pieces of up to 32
// consecutive keys (a range's last piece, when short, continuing with the
// next range's first keys), then its column list in pieces of up to 32
// gathered keys.  Both waves share one LDS copy of a piece's K and V rows,
// written by buffer loads that go straight to LDS (no staging registers)
// from per-row keys, so every piece kind takes one load form.  Software
// pipeline, per iteration i (four pieces in flight, in slots fixed at compile
// time):
//   - loads issued: K rows of piece i+2, V rows of piece i+1;
//   - S^T of piece i+1 (32 keys x 32 rows) = K . Q^T   v_mfma_f32_32x32x16_bf16
//     interleaved with the exponentials of piece i, whose S^T the previous
//     iteration produced;
//   - O^T (128 x 32 rows) += V^T . P^T of piece i       v_mfma_f32_32x32x16_f16
//   - one barrier.
// The online softmax works in the log2 domain; the running max may lag the
// true max by up to 8 (P <= 256), so the O rescale only runs when a row's max
// grows by more than that.  Buffer-load range checks (one KV head's rows) turn
// reads past the sequence into zeros, so piece tails need no clamping.
//
// Paced variant (sparse_attn_paced, sparse_attn_paced32), for long sequences:
// each workgroup walks its block's whole index (columns first, which every
// block of the head shares, then the ranges in key order).  A launch holds as
// many workgroups as are resident at once, and the workgroups of one XCD
// (which share its L2) keep pace: one that is about to start keys of segment
// s waits until all of them have passed segment s - pace - 1 (one counter per
// XCD and segment; bounded waits, so a workgroup never waits for good on one
// that is not resident).  The pacing orders work only; results do not depend
// on it.
//
// LDS tiles are row-major (one 256-byte row per key) with the 16-byte chunks
// of row r XOR-swizzled: chunk c sits at chunk slot c ^ swz(r).  One
// load-to-LDS instruction fills four whole rows (1 KiB of memory per four
// keys, contiguous for a range piece), and both the K fragment reads and the
// transposed V reads (ds_read_b64_tr_b16) are free of bank conflicts; the
// per-lane read offsets are precomputed, so LDS addresses cost no VALU work
// in the loop.  P and V enter the second product as fp16 (V from an exact
// fp16 copy).
#include "internal.h"

namespace msa {
namespace {

constexpr int kKP = 32;                       // keys per piece
constexpr int kRowBytes = kD * 2;             // one K or V row
constexpr int kTileBytes = kKP * kRowBytes;   // one K or V tile (8 KiB)
constexpr float kLag = 8.f;                   // allowed lag of the running max (log2 units)

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const int global_int;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Transposed LDS read (gfx950): within each group of 16 lanes, lane i gets
// element i%4 of the 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ f16x4 lds_read_tr(const char* p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// max / sum of a value and its partner in the other half of the wavefront
// (lanes l and l^32 hold the same query row).
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32); }

struct Piece {
  int start;   // first key (range piece) or first column slot (column piece)
  int count;   // 1..32 (0: past the end of the walk)
  int is_col;  // keys listed per tile row (a column piece or a two-range piece)
  int mask;    // masking the piece needs (set by the kernel when the piece is taken)
};

// A range piece whose range ends before 32 keys takes the next range's first
// keys as well: rows 0 .. split - 1 hold keys start .., rows split .. count -
// 1 hold keys start2 ..  (split = 0: one range, or a column piece).  Without
// this, every range's last piece is on average half empty (ranges of a 1M
// Vertical-Slash layer average about 250 keys, so 6% of the matrix work).
struct Split {
  int start2, split;
};

// Start key of a piece past the end: its tile offsets (start * 256 + ...)
// are >= 2^31, beyond any KV head's bytes (n <= 2^23).
constexpr int kPastEnd = 1 << 23;

// Walks a query block's ranges in pieces of <= 32 consecutive keys, then its
// column list in pieces of <= 32 listed keys.  The position is uniform.  Range
// descriptors come 64 at a time, one per lane (lane l holds range wbase + l),
// and are read with readlane: a wait for memory happens once per 64 ranges,
// not at every range (a wait there would also wait for the K/V tiles in
// flight).
template <bool kPace>
struct PieceIter {
  const int2* rng;
  int r, r_end;
  int lo, hi;
  int c, c_end;
  int wbase;     // first range of the window
  int wlo, whi;  // this lane's range of the window
  // kPace: the segment of the last range piece (pieces are not cut at
  // segment edges; a piece belongs to the segment of its first key), the
  // first key past it, the segment count of the launch, this XCD's counters
  // and group size, whether this wave reports arrivals, and whether pacing
  // is still on (a wait that runs out switches it off for the rest of the
  // walk, so a workgroup never waits on one that is not resident); polls
  // bounds the counter reads of one wait.
  int seg, seg_end, nseg, shift, pace, members, polls;
  uint32_t* cnt;
  bool reporter, paced;
  __device__ __forceinline__ void load_window(int first) {
    typedef __attribute__((address_space(1))) const u32x2 g_u32x2;
    wbase = first;
    const int k = first + (int)(threadIdx.x & 63);
    wlo = whi = 0;
    if (k < r_end) {
      const u32x2 v = *reinterpret_cast<g_u32x2*>(reinterpret_cast<uint64_t>(rng + k));
      wlo = (int)v[0];
      whi = (int)v[1];
    }
    // The window is settled here (the compiler waits for the load before this
    // use) and from then on counts as defined by this statement, so later
    // reads of it wait for nothing.
    asm volatile("" : "+v"(wlo), "+v"(whi));
  }
  __device__ __forceinline__ void start() {
    if (r < r_end) load_window(r);
  }
  // Segments seg .. s_new - 1 are done (their pieces enumerated).
  __device__ __forceinline__ void arrive(int s_new) {
    if (reporter && (threadIdx.x & 63) == 0)
      for (int s = seg; s < s_new; ++s) __hip_atomic_fetch_add(cnt + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Moves to segment s_new: reports the segments passed, then waits until
  // every workgroup of the group has passed segment s_new - pace - 1.
  __device__ __forceinline__ void enter(int s_new) {
    arrive(s_new);
    seg = s_new;
    seg_end = (s_new + 1) << shift;
    const int need = s_new - pace - 1;
    if (!paced || need < 0) return;
    for (int t = 0;; ++t) {
      uint32_t v = 0;
      if ((threadIdx.x & 63) == 0) v = __hip_atomic_load(cnt + need, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v = __builtin_amdgcn_readfirstlane(v);
      if (v >= (uint32_t)members) return;
      if (t >= polls) {
        paced = false;
        return;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  // join: a range piece that ends its range short of 32 keys may continue
  // with the next range (paced: only within the same key segment).
  __device__ __forceinline__ bool next(Piece& p, Split& sp, bool join) {
    sp.split = 0;
    sp.start2 = 0;
    if (kPace && c < c_end) {  // columns first: every block of a head reads them
      p.start = c;
      p.count = min(kKP, c_end - c);
      p.is_col = 1;
      c += p.count;
      return true;
    }
    while (lo >= hi && r < r_end) {
      if (r - wbase >= 64) load_window(r);
      lo = __builtin_amdgcn_readlane(wlo, r - wbase);
      hi = __builtin_amdgcn_readlane(whi, r - wbase);
      ++r;
    }
    if (lo < hi) {
      if (kPace && lo >= seg_end) enter(lo >> shift);
      p.start = lo;
      p.count = min(kKP, hi - lo);
      p.is_col = 0;
      lo += p.count;
      if (join && p.count < kKP && r < r_end) {
        if (r - wbase >= 64) load_window(r);
        const int nlo = __builtin_amdgcn_readlane(wlo, r - wbase);
        const int nhi = __builtin_amdgcn_readlane(whi, r - wbase);
        if (!kPace || nlo < seg_end) {
          const int take = min(kKP - p.count, nhi - nlo);
          sp.split = p.count;
          sp.start2 = nlo;
          p.count += take;
          p.is_col = 1;
          lo = nlo + take;
          hi = nhi;
          ++r;
        }
      }
      return true;
    }
    if (kPace) {
      if (seg < nseg) arrive(nseg);
      seg = nseg;
      return false;
    }
    if (c < c_end) {
      p.start = c;
      p.count = min(kKP, c_end - c);
      p.is_col = 1;
      c += p.count;
      return true;
    }
    return false;
  }
};

// Chunk slot of 16-byte chunk c of tile row r is c ^ swz(r).  For 16
// consecutive rows swz takes 16 distinct values, and for 4 consecutive rows
// starting at a multiple of 4 it takes 4 values that differ in bits 2-3.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Loads to LDS: load j (0..3) of wave w fills tile rows 16w + 4j + lane/16;
// lane writes chunk slot lane%16 and so fetches chunk (lane%16) ^ swz(row),
// at byte key_of_row * 256 + 16 ((lane%16) ^ swz(row)).

// Column pieces: the key of a tile row (rows past the piece repeat its last
// key; the mask drops them).  Global (not flat) loads, which only vmcnt
// tracks, so LDS waits do not stall on them.
__device__ __forceinline__ int col_key(const Piece& p, global_int* col, int row) {
  return col[p.start + min(row, p.count - 1)];
}

// kL loads per wave and tile: kL = 4 when two waves share a tile (rows 16w ..
// 16w + 15 from wave w), 8 when one wave fills all 32 rows.
template <int kL>
struct ColKeys {
  int k[kL];  // keys of rows (32 / (8 / kL)) w + 4j + lane/16
};

// Every piece's tile rows come as per-row keys (a range piece's are
// consecutive), so one address form serves all pieces and the loads need no
// branch on the piece kind.  The whole byte offset stays in the vector
// offset, which the buffer range check covers (a piece past the end of the
// walk reads zeros).
template <int kL>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, char* tile, int w, const uint32_t* cofs,
                                          const ColKeys<kL>& ck) {
  // One wave filling whole tiles (kL = 8): the wave's offset is made opaque
  // here, so the LDS destinations (M0) are formed at each load instead of
  // being precomputed and held across the loop, where they made the
  // compiler spill scalar registers (2.5% on a 1M layer of 32-row blocks;
  // the two-wave kernel runs best with them precomputed).
  int wofs = 256 * 4 * kL * w;
  if constexpr (kL == 8) asm volatile("" : "+s"(wofs));
  char* const base = tile + wofs;
#pragma unroll
  for (int j = 0; j < kL; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + 1024 * j), 16,
                                             (uint32_t)ck.k[j] * (uint32_t)kRowBytes + cofs[j], 0, 0, 0);
}

// Work items are the listed heads' query blocks of kRows rows (the blocks of
// their CSR; per = 64 / kRows of them per 64-row block).  Longest blocks
// first (causal work grows with the block); within a block index, workgroup x
// takes head list[x % n_list].  Workgroups are dealt round-robin over the 8
// XCDs, so the host orders the list to keep the Q heads of one KV head on one
// XCD, whose L2 then serves their common K/V rows.  b: the item's CSR block.
template <int kRows>
__device__ __forceinline__ void map_work(int x, const AttnArgs& a, int& h, int& b) {
  const int bi = x / a.n_list, hi = x - bi * a.n_list;
  b = a.nb * (kBM / kRows) - 1 - bi;
  h = a.list[hi];
}

// Paced mode: workgroup x takes the item bl-th from the top of the chunk's
// blocks [seg_b0, seg_b0 + seg_nb) and head list[hi]; its pacing group is its
// XCD (x % 8, as workgroups are dealt round-robin over the XCDs).
__device__ __forceinline__ void map_work_paced(int x, const AttnArgs& a, int& h, int& b) {
  const int bl = x / a.n_list, hi = x - bl * a.n_list;
  b = a.seg_b0 + a.seg_nb - 1 - bl;
  h = a.list[hi];
}

template <int kRows, bool kPace>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  constexpr int kWaves = kRows / 32;  // one wavefront per 32 query rows
  constexpr int kL = 4 * (2 / kWaves);  // load-to-LDS instructions per wave and tile
  constexpr int kPer = kBM / kRows;     // work items per 64-row block
  __shared__ __attribute__((aligned(1024))) char kb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[kTileBytes];
  __shared__ int key_lds[4][kKP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int h, b;
  if (kPace)
    map_work_paced(blockIdx.x, a, h, b);
  else
    map_work<kRows>(blockIdx.x, a, h, b);
  const int kvh = h / a.grp;
  const int64_t n = a.n;
  // b indexes the call's query blocks of kRows rows (and the CSR); row0 is
  // the block's first query row in the sequence, qrow0 its row in Q and out.
  const int row0 = (a.qb0 * kPer + b) * kRows;
  const int64_t qrow0 = (int64_t)b * kRows;

  // Q fragments: B operand of S^T = K Q^T; lane holds row l32 of this wave's
  // 32 rows and d = 16t + 8g .. +8.
  const uint16_t* qh = a.q + ((int64_t)h * a.qm + qrow0 + 32 * w) * kD;
  bf16x8 qf[8];
  auto load_q = [&]() {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + l32 * kD + 16 * t + 8 * g));
  };

  PieceIter<kPace> it{};
  if (kPace) {
    const int total = a.n_list * a.seg_nb, grp = blockIdx.x & 7;
    it.members = total / 8 + (grp < total % 8 ? 1 : 0);
    it.nseg = (((a.qb0 * kPer + a.seg_b0 + a.seg_nb) * kRows - 1) >> a.seg_shift) + 1;
    it.cnt = a.pace_cnt + grp * a.seg_n;
    it.shift = a.seg_shift;
    it.pace = a.pace;
    it.seg = 0;
    it.seg_end = 1 << a.seg_shift;
    it.reporter = w == 0;
    it.paced = true;
    it.polls = a.pace_polls;
  }
  global_int* col = nullptr;
  bool ashape = false;
  int sink = 0, window = 0;
  if (a.table) {
    const HeadDesc& d = a.table[h];
    const int* rng_ptr = reinterpret_cast<const int*>(a.arena + d.rng_ptr_off);
    const int* col_ptr = reinterpret_cast<const int*>(a.arena + d.col_ptr_off);
    it.rng = reinterpret_cast<const int2*>(a.arena + d.rng_off);
    it.r = rng_ptr[b];
    it.r_end = rng_ptr[b + 1];
    it.c = col_ptr[b];
    it.c_end = col_ptr[b + 1];
    col = reinterpret_cast<global_int*>(reinterpret_cast<uint64_t>(a.arena + d.col_off));
    if (d.pattern == MS_A_SHAPE) {
      ashape = true;
      sink = d.p0;
      window = d.p1;
    }
  } else {
    it.lo = 0;
    it.hi = row0 + kRows;
  }

  // Byte size of one KV head (<= 2^31 for n <= 2^23), taken as unsigned by the
  // range check.
  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);

  load_q();

  // Per-lane constants.  Loads: this lane's row rw_j = 4 kL w + 4j + lane/16
  // and chunk (lane%16) ^ swz(rw_j); cofs = that chunk's byte offset (the
  // row's key * 256 is added per piece).
  const int rq = lane >> 4;
  uint32_t cofs[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) cofs[j] = 16u * (uint32_t)((lane & 15) ^ swz(4 * kL * w + 4 * j + rq));
  // K fragment t: row l32, chunk 2t + g.
  int kofs[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) kofs[t] = l32 * kRowBytes + 16 * ((2 * t + g) ^ swz(l32));
  // V^T fragment (kh2, dt, hi): row 16kh2 + 8hi + 4g + (lane%16)/4, chunk
  // 4dt + 2((lane/16)%2) + (lane%4)/2, byte half lane%2; swz ignores the
  // 16kh2 part, which becomes an immediate.
  int vofs[2][4];
  {
    const int s16 = lane & 15;
    const int vc = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int ra = 8 * hi + 4 * g + (s16 >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vofs[hi][dt] = ra * kRowBytes + 16 * ((4 * dt + vc) ^ swz(ra)) + 8 * (s16 & 1);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int row = row0 + 32 * w + l32;  // this lane's query row
  const float sl2 = a.scale_log2;
  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};

  // Pieces in flight: piece i + k sits in slot (i + k) & 3, k = 0..3, with
  // its column keys (this lane's rows of the piece's tiles).  The loop body
  // is unrolled four times, so slots, tile buffers and key slots are
  // compile-time choices and nothing is copied from slot to slot.  A piece
  // with count 0 lies past the end of the walk: its tile loads fall outside
  // the KV head (the range check returns zeros without reading memory) and
  // it is never computed.  mask: 0 none, 1 the piece's tail only (a range
  // piece of fewer than 32 keys), 2 per element (the diagonal block, an
  // A-shape window edge, or a column piece).
  Piece pc0{}, pc1{}, pc2{}, pc3{};
  ColKeys<kL> ck0{}, ck1{}, ck2{}, ck3{};
  // slot K's piece and column keys (K a compile-time constant)
  auto pc = [&](auto k) __attribute__((always_inline)) -> Piece& {
    constexpr int K = decltype(k)::value & 3;
    if constexpr (K == 0) return pc0;
    else if constexpr (K == 1) return pc1;
    else if constexpr (K == 2) return pc2;
    else return pc3;
  };
  auto ck = [&](auto k) __attribute__((always_inline)) -> ColKeys<kL>& {
    constexpr int K = decltype(k)::value & 3;
    if constexpr (K == 0) return ck0;
    else if constexpr (K == 1) return ck1;
    else if constexpr (K == 2) return ck2;
    else return ck3;
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  // Two-range pieces only where no A-shape window test needs the piece's
  // first key.
  const bool join = !ashape;
  auto fetch = [&](Piece& p, ColKeys<kL>& c) __attribute__((always_inline)) {
    Piece q;
    Split sp;
    // The usual case, without the iterator's other checks: a full piece
    // inside the current range (paced: starting in the current key segment),
    // no A-shape window.
    if (join && it.lo + kKP <= it.hi && (!kPace || it.lo < it.seg_end)) {
      q.start = it.lo;
      q.count = kKP;
      q.is_col = 0;
      sp.split = 0;
      it.lo += kKP;
    } else if (!it.next(q, sp, join)) {
      q.start = kPastEnd;
      q.count = 0;
      q.is_col = 0;
      sp.split = 0;
    }
    const int kmax = sp.split ? sp.start2 + q.count - sp.split - 1 : q.start + q.count - 1;
    const bool far = ashape && kmax >= sink && row0 + kRows - 1 - max(q.start, sink) >= window;
    // (every field is written on every path, so the compiler keeps the
    // slots in registers)
    q.mask = q.count == 0 ? 0 : (q.is_col && !sp.split) || kmax > row0 || far ? 2 : q.count < kKP ? 1 : 0;
    p = q;
    // the keys of this lane's tile rows
    if (!q.is_col) {
#pragma unroll
      for (int j = 0; j < kL; ++j) c.k[j] = q.start + 4 * kL * w + 4 * j + rq;
    } else if (sp.split) {
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        const int rw = 4 * kL * w + 4 * j + rq;
        c.k[j] = rw < sp.split ? q.start + rw : sp.start2 + rw - sp.split;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kL; ++j) c.k[j] = col_key(q, col, 4 * kL * w + 4 * j + rq);
    }
  };
  // Mask keys of a column piece: lanes with lane%16 == 0 hold rows 4 kL w + 4j.
  auto store_keys = [&](int* dst, const ColKeys<kL>& c) __attribute__((always_inline)) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < kL; ++j) dst[4 * kL * w + 4 * j + rq] = c.k[j];
    }
  };
  it.start();
  fetch(pc0, ck0);
  fetch(pc1, ck1);
  fetch(pc2, ck2);
  __builtin_amdgcn_s_waitcnt(0);
  load_tile(kr, kb0, w, cofs, ck0);
  load_tile(vr, vb0, w, cofs, ck0);
  if (pc0.is_col) store_keys(key_lds[0], ck0);
  load_tile(kr, kb1, w, cofs, ck1);
  if (pc1.is_col) store_keys(key_lds[1], ck1);
  // Settle every outstanding load (Q fragments, first tiles) here, so the
  // wait for them is not placed inside the loop.
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(qf[t]));  // defined here, not by a load
  __syncthreads();
  f32x16 s_cur = f32x16{};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb0 + kofs[t]));
    s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[t], s_cur, 0, 0, 0);
  }
  __syncthreads();  // kb0 is refilled in the first iteration

  // One pipeline iteration for piece i with PAR = i & 3.
  auto step = [&](auto par) __attribute__((always_inline)) -> bool {
    constexpr int PAR = decltype(par)::value;
    using S1 = std::integral_constant<int, (PAR + 1) & 3>;
    using S2 = std::integral_constant<int, (PAR + 2) & 3>;
    using S3 = std::integral_constant<int, (PAR + 3) & 3>;
    const Piece& cur = pc(par);
    char* const kfill = (PAR & 1) ? kb1 : kb0;        // K of piece i+2 (piece i's buffer)
    const char* const kread = (PAR & 1) ? kb0 : kb1;  // K of piece i+1
    char* const vfill = (PAR & 1) ? vb0 : vb1;        // V of piece i+1
    const char* const vread = (PAR & 1) ? vb1 : vb0;  // V of piece i

    load_tile(kr, kfill, w, cofs, ck(S2{}));
    if (pc(S2{}).is_col) store_keys(key_lds[S2::value], ck(S2{}));
    load_tile(vr, vfill, w, cofs, ck(S1{}));
    fetch(pc(S3{}), ck(S3{}));

    // Softmax of piece i, masked as its mask kind says (the mask itself per
    // element without branches).
    f32x16& s = s_cur;  // masked in place; s_cur takes the next piece's S^T at the end
    if (cur.mask == 1) {
      // Only the piece's tail (slots >= count) is masked: element r is slot
      // 8 (r / 4) + r % 4 + 4 g, so it stays iff 8 (r / 4) + r % 4 < count - 4 g.
      const int thr = cur.count - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) < thr ? s[r] : -INFINITY;
    } else if (cur.mask == 2) {
      // Slot of element r: 8 (r / 4) + 4 g + r % 4.  The base is made opaque
      // here so the sixteen slots are formed inside the masked path instead of
      // being held in registers across the loop.
      const int* keys = key_lds[PAR];
      int g4 = 4 * g;
      asm volatile("" : "+v"(g4));
      int key[16];
      if (cur.is_col) {
#pragma unroll
        for (int r = 0; r < 16; ++r) key[r] = keys[8 * (r >> 2) + g4 + (r & 3)];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) key[r] = cur.start + 8 * (r >> 2) + g4 + (r & 3);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int slot = 8 * (r >> 2) + g4 + (r & 3);
        const bool ok = (slot < cur.count) & (key[r] <= row) &
                        !(ashape & (key[r] >= sink) & (row - key[r] >= window));
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    // This lane's half of the row decides whether any row's max ran ahead;
    // only a rescale needs the whole row's max (both halves).
    mx *= sl2;
    if (__any(mx > m_run + kLag)) {
      const float mn = fmaxf(m_run, max_halves(mx));
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;

    // S^T of the next piece (its K tile arrived during the previous
    // iteration) = 8 MFMAs; P = exp2(s - m) of this piece; O^T += V^T P^T of
    // this piece = 8 MFMAs.  Issued in groups of one or two MFMAs with the
    // exponentials, LDS reads and row sums that fit beside them, so the wave
    // issues VALU work while the matrix core runs.  V^T fragment (kh2, dt) is
    // the A operand of the second product: lane holds d = 32dt + l32 and keys
    // 16kh2 + 8(e/4) + 4g + e%4; its B operand is P^T from the S registers.
    auto kfrag = [&](int t) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kread + kofs[t]));
    };
    auto vfrag = [&](int kh2, int dt) {
      const f16x4 lo = lds_read_tr(vread + vofs[0][dt] + 4096 * kh2);
      const f16x4 hi = lds_read_tr(vread + vofs[1][dt] + 4096 * kh2);
      return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    f32x16 s_nxt = f32x16{};
    f16x8 pb[2];
    bf16x8 kf[8];
    f16x8 va[8];
    float sum = 0.f;
    kf[0] = kfrag(0);
    kf[1] = kfrag(1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 2 < 8) kf[t + 2] = kfrag(t + 2);
      va[t] = vfrag(t >> 2, t & 3);
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t], s_nxt, 0, 0, 0);
      const int r = 2 * t;
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -msub));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -msub));
      pb[r >> 3][r & 7] = (_Float16)e0;
      pb[r >> 3][(r & 7) + 1] = (_Float16)e1;
      const f16x2 e = {(_Float16)e0, (_Float16)e1};
      sum = __builtin_amdgcn_fdot2(e, ones, sum, false);  // row sum of the fp16 P the MFMA consumes
      if (t >= 4) o[t - 4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[t - 4], pb[0], o[t - 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[4 + dt], pb[1], o[dt], 0, 0, 0);
    l_run += sum;
    __syncthreads();
    s_cur = s_nxt;
    return pc(S1{}).count != 0;
  };
  if (pc0.count != 0) {
    while (step(C0{}) && step(C1{}) && step(C2{}) && step(C3{})) {
    }
  }

  const float lt = sum_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // Epilogue: out = O / l, lse = m ln2 + ln l.
  const int64_t orow = (int64_t)h * a.qm + qrow0 + 32 * w + l32;  // this lane's row of out and lse
  const int64_t obase = orow * kD;
  float* out_f32 = reinterpret_cast<float*>(a.out);
  float* lse = a.lse;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const float x0 = o[dt][4 * q4 + 0] * inv, x1 = o[dt][4 * q4 + 1] * inv;
      const float x2 = o[dt][4 * q4 + 2] * inv, x3 = o[dt][4 * q4 + 3] * inv;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(out_f32 + obase + d0) = f32x4{x0, x1, x2, x3};
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) = y;
      }
    }
  }
  if (lse && g == 0)
    lse[orow] = lt > 0.f ? m_run * 0.69314718055994530942f + logf(lt) : -INFINITY;
}

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_fwd(AttnArgs a) {
  attn_body<64, false>(a);
}

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_paced(AttnArgs a) {
  attn_body<64, true>(a);
}

// 32-row query blocks: one wavefront per work item, filling its tiles alone.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_fwd32(AttnArgs a) {
  attn_body<32, false>(a);
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_paced32(AttnArgs a) {
  attn_body<32, true>(a);
}

__global__ __launch_bounds__(256) void v_to_f16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                 int64_t chunks) {
  // One chunk = 8 values: bf16 in, fp16 out (exact for 2^-14 <= |v| < 65504).
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= chunks) return;
  const u32x4 x = src[i];
  f16x8 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = (_Float16)__builtin_bit_cast(float, x[e] << 16);
    y[2 * e + 1] = (_Float16)__builtin_bit_cast(float, x[e] & 0xffff0000u);
  }
  dst[i] = __builtin_bit_cast(u32x4, y);
}

}  // namespace

hipError_t launch_v_to_f16(const uint16_t* v, _Float16* v16, int64_t elems, hipStream_t s) {
  const int64_t chunks = elems / 8;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(v_to_f16, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const u32x4*>(v),
                     reinterpret_cast<u32x4*>(v16), chunks);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs& a, int rows, hipStream_t s) {
  if (rows != kBM && rows != 32) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)a.n_list * a.nb * (kBM / rows);
  if (rows == kBM)
    hipLaunchKernelGGL(sparse_attn_fwd, dim3((unsigned)blocks), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(sparse_attn_fwd32, dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_paced(const AttnArgs& a, int rows, hipStream_t s) {
  if (rows != kBM && rows != 32) return hipErrorInvalidValue;
  const int per = kBM / rows;
  const int nseg = (((a.qb0 * per + a.seg_b0 + a.seg_nb) * rows - 1) >> a.seg_shift) + 1;
  if (nseg > a.seg_n || !a.table) return hipErrorInvalidValue;
  if (rows == kBM)
    hipLaunchKernelGGL(sparse_attn_paced, dim3((unsigned)(a.seg_nb * a.n_list)), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(sparse_attn_paced32, dim3((unsigned)(a.seg_nb * a.n_list)), dim3(64), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_u32(uint32_t* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p, count);
  return hipGetLastError();
}


}  // namespace msa
