// Sparse FlashAttention-style forward kernel for gfx950 (MInference 1.0
// summary, "Summary", third stage: attention computed only over the estimated
// indices; FlashAttention-2's online softmax is the published algorithm the
// pages' kernels build on).
//
// Work item: one 64-row query block of one Q head = one workgroup of two
// wavefronts, each owning 32 rows.  The block's keys are its ranges, cut into
// pieces of up to 32 consecutive keys, then its column list in pieces of up to
// 32 gathered keys.  Both waves share one LDS copy of a piece's K and V rows,
// written by buffer loads that go straight to LDS (no staging registers).
// Software pipeline, per iteration i:
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
// Key-segment variant (sparse_attn_seg + seg_combine), for long sequences:
// a workgroup takes the keys of one query block that fall in one segment of
// 2^seg_shift keys (its share of the block's ranges, cut at the segment
// edges, and of its columns, found by a wave-wide search of the CSR) and
// writes O / l and the log-sum-exp of that share; the combine kernel merges a
// block's segment records in segment order.  Workgroups are numbered segment
// first, so the ones in flight read the same segment of K/V and L2 serves the
// rows that several of them read; per (query block, key) the work is
// unchanged.
//
// LDS tiles are row-major (one 256-byte row per key) with the 16-byte chunks
// of row r XOR-swizzled: chunk c sits at chunk slot c ^ swz(r).  One
// load-to-LDS instruction fills four whole rows (1 KiB of contiguous memory
// per four keys), and both the K fragment reads and the transposed V reads
// (ds_read_b64_tr_b16) are free of bank conflicts; the per-lane read offsets
// are precomputed, so LDS addresses cost no VALU work in the loop.  P and V
// enter the second product as fp16 (V from an exact fp16 copy).
#include "internal.h"

namespace msa {
namespace {

constexpr int kKP = 32;                       // keys per piece
constexpr int kRowBytes = kD * 2;             // one K or V row
constexpr int kTileBytes = kKP * kRowBytes;   // one K or V tile (8 KiB)
constexpr float kLag = 8.f;                   // allowed lag of the running max (log2 units)
constexpr int kThreads = 128;

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
  int count;   // 1..32
  int is_col;
};

// Walks a query block's ranges in pieces of <= 32 consecutive keys, then its
// column list in pieces of <= 32 listed keys.  The position is uniform.  Range
// descriptors come 64 at a time, one per lane (lane l holds range wbase + l),
// and are read with readlane: a wait for memory happens once per 64 ranges,
// not at every range (a wait there would also wait for the K/V tiles in
// flight).
template <bool kClip>
struct PieceIter {
  const int2* rng;
  int r, r_end;
  int lo, hi;
  int c, c_end;
  int clo, chi;  // kClip: ranges are cut to the key segment [clo, chi)
  int wbase;     // first range of the window
  int wlo, whi;  // this lane's range of the window
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
  __device__ __forceinline__ bool next(Piece& p) {
    while (lo >= hi && r < r_end) {
      if (r - wbase >= 64) load_window(r);
      lo = __builtin_amdgcn_readlane(wlo, r - wbase);
      hi = __builtin_amdgcn_readlane(whi, r - wbase);
      if (kClip) {
        lo = max(lo, clo);
        hi = min(hi, chi);
      }
      ++r;
    }
    if (lo < hi) {
      p.start = lo;
      p.count = min(kKP, hi - lo);
      p.is_col = 0;
      lo += p.count;
      return true;
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
// lane writes chunk slot lane%16 and so fetches chunk (lane%16) ^ swz(row).
// lofs[j] is that chunk's byte offset within a four-row group of keys plus
// the row's offset, so the address is key_of_row0 * 256 + lofs[j] for a range
// piece.

// Column pieces: the key of a tile row (rows past the piece repeat its last
// key; the mask drops them).  Global (not flat) loads, which only vmcnt
// tracks, so LDS waits do not stall on them.
__device__ __forceinline__ int col_key(const Piece& p, global_int* col, int row) {
  return col[p.start + min(row, p.count - 1)];
}

struct ColKeys {
  int k[4];  // keys of rows 16w + 4j + lane/16
};

__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, char* tile, int w, const uint32_t* lofs,
                                          const uint32_t* cofs, const Piece& p, const ColKeys& ck) {
  char* const base = tile + 4096 * w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t off = p.is_col ? (uint32_t)ck.k[j] * (uint32_t)kRowBytes + cofs[j]
                                  : (uint32_t)p.start * (uint32_t)kRowBytes + lofs[j];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + 1024 * j), 16, off, 0, 0, 0);
  }
}

// Longest query blocks first (causal work grows with b); within a block
// index, workgroup x takes head list[x % n_list].  Workgroups are dealt
// round-robin over the 8 XCDs, so the host orders the list to keep the Q
// heads of one KV head on one XCD, whose L2 then serves their common K/V rows.
__device__ __forceinline__ void map_work(int x, const AttnArgs& a, int& h, int& b) {
  const int bi = x / a.n_list, hi = x - bi * a.n_list;
  b = a.nb - 1 - bi;
  h = a.list[hi];
}

// Key-segment mode: workgroup x takes segment x / (seg_nb * n_list) of block
// seg_b0 + seg_nb - 1 - bl and head list[hi], (bl, hi) from the rest, so the
// workgroups in flight share one segment of every KV head's K/V rows; slot is
// its partial record.
__device__ __forceinline__ void map_work_seg(int x, const AttnArgs& a, int& h, int& b, int& sg, int& slot) {
  const int per = a.seg_nb * a.n_list;
  sg = __builtin_amdgcn_readfirstlane(x / per);
  const int y = x - sg * per;
  const int bl = __builtin_amdgcn_readfirstlane(y / a.n_list);
  const int hi = y - bl * a.n_list;
  b = a.seg_b0 + a.seg_nb - 1 - bl;
  h = a.list[hi];
  slot = (bl * a.n_list + hi) * a.seg_n + sg;
}

// Four lower bounds at once: for search j, the first i in [lo_j, hi_j) with
// key_j(i) >= x_j (hi_j if none), every key nondecreasing in i.  All lanes of
// the wave probe together, 64 probes per search and round, and the four
// searches' probes of a round are issued together so they share one memory
// latency.  Keys: j = 0 range ends, 1 range starts, 2 and 3 columns.
struct Bound {
  int lo, hi, x;
};
__device__ __forceinline__ void wave_lower_bounds(Bound (&s)[4], const int2* rng, global_int* col, int lane) {
  bool done[4] = {false, false, false, false};
  for (;;) {
    int probe[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int size = s[j].hi - s[j].lo;
      const int step = size > 64 ? (size + 63) >> 6 : 1;
      const int i = s[j].lo + lane * step;
      probe[j] = 0x7fffffff;
      if (!done[j] && i < s[j].hi) probe[j] = j == 0 ? rng[i].y : j == 1 ? rng[i].x : col[i];
    }
    bool all = true;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (done[j]) continue;
      const int size = s[j].hi - s[j].lo;
      if (size <= 64) {
        s[j].lo += __popcll(__ballot(probe[j] < s[j].x));
        s[j].hi = s[j].lo;
        done[j] = true;
        continue;
      }
      const int step = (size + 63) >> 6;
      const uint64_t ge = __ballot(probe[j] >= s[j].x);
      if (ge & 1) {
        s[j].hi = s[j].lo;
        done[j] = true;
        continue;
      }
      const int t = ge ? __builtin_ctzll(ge) : 64;  // key(lo + (t-1) step) < x
      if (t < 64) s[j].hi = min(s[j].hi, s[j].lo + t * step);
      s[j].lo = s[j].lo + (t - 1) * step + 1;
      all = false;
    }
    if (all) return;
  }
}

template <bool kSeg>
__device__ __forceinline__ void attn_body(const AttnArgs& a) {
  __shared__ __attribute__((aligned(1024))) char kb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[kTileBytes];
  __shared__ int key_lds[4][kKP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int h, b, sg = 0;
  if (kSeg) {
    int slot;
    map_work_seg(blockIdx.x, a, h, b, sg, slot);
  } else
    map_work(blockIdx.x, a, h, b);
  const int kvh = h / a.grp;
  const int64_t n = a.n;
  // b indexes the call's query blocks (and the CSR); row0 is the block's
  // first query row in the sequence, qrow0 its row in Q and out.
  const int row0 = (a.qb0 + b) * kBM;
  const int64_t qrow0 = (int64_t)b * kBM;
  const int seg_lo = sg << a.seg_shift;
  if (kSeg && seg_lo > row0 + kBM - 1) return;  // past the block's last key: no record
  const int seg_hi = seg_lo + (1 << a.seg_shift);

  // Q fragments: B operand of S^T = K Q^T; lane holds row l32 of this wave's
  // 32 rows and d = 16t + 8g .. +8.  The segment variant issues them before
  // its index search, so the two latencies overlap.
  const uint16_t* qh = a.q + ((int64_t)h * a.qm + qrow0 + 32 * w) * kD;
  bf16x8 qf[8];
  auto load_q = [&]() {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + l32 * kD + 16 * t + 8 * g));
  };
  if (kSeg) load_q();

  PieceIter<kSeg> it{};
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
    if (kSeg) {
      // This segment's share of the block's index: ranges that end after
      // seg_lo and start before seg_hi (cut to the segment), and columns in
      // [seg_lo, seg_hi).
      Bound sb[4] = {{it.r, it.r_end, seg_lo + 1}, {it.r, it.r_end, seg_hi}, {it.c, it.c_end, seg_lo},
                     {it.c, it.c_end, seg_hi}};
      wave_lower_bounds(sb, it.rng, col, lane);
      it.r = __builtin_amdgcn_readfirstlane(sb[0].lo);
      it.r_end = __builtin_amdgcn_readfirstlane(sb[1].lo);
      it.c = __builtin_amdgcn_readfirstlane(sb[2].lo);
      it.c_end = __builtin_amdgcn_readfirstlane(sb[3].lo);
      it.clo = seg_lo;
      it.chi = seg_hi;
    }
  } else {
    it.lo = kSeg ? seg_lo : 0;
    it.hi = kSeg ? min(seg_hi, row0 + kBM) : row0 + kBM;
  }

  // Byte size of one KV head (<= 2^31 for n <= 2^23), taken as unsigned by the
  // range check.
  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);

  if (!kSeg) load_q();

  // Per-lane constants.  Loads: this lane's row rw_j = 16w + 4j + lane/16
  // and chunk (lane%16) ^ swz(rw_j); lofs = row offset + chunk offset,
  // cofs = chunk offset alone (column pieces add key * 256).
  const int rq = lane >> 4;
  uint32_t lofs[4], cofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rw = 16 * w + 4 * j + rq;
    cofs[j] = 16u * (uint32_t)((lane & 15) ^ swz(rw));
    lofs[j] = (uint32_t)rw * (uint32_t)kRowBytes + cofs[j];
  }
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

  // Pieces i (cur), i+1, i+2, i+3.  Column keys (this lane's four rows):
  // ck1 of piece i+1 (its V tile is loaded this iteration), ck2 of piece i+2
  // (K tile this iteration, V tile next), ck3 fetched this iteration.
  Piece cur{}, p1{}, p2{}, p3{};
  ColKeys ck0{}, ck1{}, ck2{}, ck3{};
  auto fetch_keys = [&](const Piece& p, ColKeys& ck) {
    if (p.is_col) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ck.k[j] = col_key(p, col, 16 * w + 4 * j + rq);
    }
  };
  // Mask keys of a column piece: lanes with lane%16 == 0 hold rows 16w + 4j.
  auto store_keys = [&](int* dst, const ColKeys& ck) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[16 * w + 4 * j + rq] = ck.k[j];
    }
  };
  it.start();
  const bool h0 = it.next(cur);
  bool h1 = h0 && it.next(p1);
  bool h2 = h1 && it.next(p2);
  if (h0) fetch_keys(cur, ck0);
  if (h1) fetch_keys(p1, ck1);
  if (h2) fetch_keys(p2, ck2);
  __builtin_amdgcn_s_waitcnt(0);
  if (h0) {
    load_tile(kr, kb0, w, lofs, cofs, cur, ck0);
    load_tile(vr, vb0, w, lofs, cofs, cur, ck0);
    if (cur.is_col) store_keys(key_lds[0], ck0);
  }
  if (h1) {
    load_tile(kr, kb1, w, lofs, cofs, p1, ck1);
    if (p1.is_col) store_keys(key_lds[1], ck1);
  }
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

  int i = 0;
  // One pipeline iteration; PAR = i & 1 picks the buffers at compile time, so
  // the compiler sees that the tiles being loaded are not the ones being read.
  auto step = [&](auto par) -> bool {
    constexpr int PAR = decltype(par)::value;
    char* const kfill = PAR ? kb1 : kb0;        // K of piece i+2 (piece i's buffer)
    const char* const kread = PAR ? kb0 : kb1;  // K of piece i+1
    char* const vfill = PAR ? vb0 : vb1;        // V of piece i+1
    const char* const vread = PAR ? vb1 : vb0;  // V of piece i

    if (h2) {
      load_tile(kr, kfill, w, lofs, cofs, p2, ck2);
      if (p2.is_col) store_keys(key_lds[(i + 2) & 3], ck2);
    }
    if (h1) load_tile(vr, vfill, w, lofs, cofs, p1, ck1);
    const bool h3 = h2 && it.next(p3);
    if (h3) fetch_keys(p3, ck3);

    // Softmax of piece i.  Masks (causal, piece tail, A-shape window): whether
    // any is needed is decided per piece, the mask itself per element without
    // branches.
    f32x16 s = s_cur;
    const int* keys = key_lds[i & 3];
    const int kmin = cur.is_col ? keys[0] : cur.start;
    const int kmax = cur.is_col ? keys[cur.count - 1] : cur.start + cur.count - 1;
    const bool far = ashape && kmax >= sink && row0 + kBM - 1 - max(kmin, sink) >= window;
    if (cur.count < kKP || kmax > row0 || far) {
      // Slot of element r: 8 (r / 4) + 4 g + r % 4.  In the segment variant
      // the base is made opaque here so the sixteen slots are formed inside
      // the masked path instead of being held in registers across the loop.
      int g4 = 4 * g;
      if (kSeg) asm volatile("" : "+v"(g4));
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
    mx = max_halves(mx) * sl2;
    if (__any(mx > m_run + kLag)) {
      const float mn = fmaxf(m_run, mx);
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
    if (!h1) return false;
    s_cur = s_nxt;
    cur = p1;
    p1 = p2;
    p2 = p3;
    h1 = h2;
    h2 = h3;
    ck1 = ck2;
    ck2 = ck3;
    ++i;
    return true;
  };
  if (h0) {
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  }

  const float lt = sum_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // Epilogue: out = O / l, lse = m ln2 + ln l.  The segment variant writes
  // the same two results to its partial record (fp32 rows of 128, then the
  // 64 lse values), with the base pointers shifted so the row offsets match.
  const int64_t orow = (int64_t)h * a.qm + qrow0 + 32 * w + l32;  // this lane's row of out and lse
  const int64_t obase = orow * kD;
  float* out_f32 = reinterpret_cast<float*>(a.out);
  float* lse = a.lse;
  if (kSeg) {
    int hh, bb, ss, slot;
    map_work_seg(blockIdx.x, a, hh, bb, ss, slot);
    float* rec = a.part + (int64_t)__builtin_amdgcn_readfirstlane(slot) * kSegRecFloats;
    out_f32 = rec - ((int64_t)h * a.qm + qrow0) * kD;
    lse = rec + kSegRowFloats - ((int64_t)h * a.qm + qrow0);
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dt + 8 * q4 + 4 * g;
      const float x0 = o[dt][4 * q4 + 0] * inv, x1 = o[dt][4 * q4 + 1] * inv;
      const float x2 = o[dt][4 * q4 + 2] * inv, x3 = o[dt][4 * q4 + 3] * inv;
      if (kSeg || a.out_f32) {
        *reinterpret_cast<f32x4*>(out_f32 + obase + d0) = f32x4{x0, x1, x2, x3};
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) = y;
      }
    }
  }
  if ((kSeg || lse) && g == 0)
    lse[orow] = lt > 0.f ? m_run * 0.69314718055994530942f + logf(lt) : -INFINITY;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_fwd(AttnArgs a) {
  attn_body<false>(a);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_seg(AttnArgs a) {
  attn_body<true>(a);
}

// Combination of a (head, block)'s segment records (O_s / l_s and lse_s per
// row): with M the largest lse_s of a row and c_s = e^(lse_s - M), out =
// sum_s c_s (O_s / l_s) / sum_s c_s and lse = M + ln(sum_s c_s), summed in
// segment order.  Threads 0..63 turn each row's lse_s into the weights c_s
// (LDS, [segment][row], up to 64 segments at a time); every thread then
// accumulates 16-byte pieces q = 256 j + t of the records (row q / 32), so
// each load instruction of a wave reads 1 KiB of contiguous memory.
constexpr int kCombThreads = 256;
constexpr int kCombSegs = 64;  // segments whose weights LDS holds at once
__global__ __launch_bounds__(kCombThreads) void seg_combine(AttnArgs a) {
  __shared__ float cw[kCombSegs][kBM];
  __shared__ float inv[kBM];
  const int t = threadIdx.x;
  const int bl = blockIdx.x / a.n_list, hi = blockIdx.x - bl * a.n_list;
  const int b = a.seg_b0 + a.seg_nb - 1 - bl;  // the call's query block
  const int h = a.list[hi];
  const int row0 = (a.qb0 + b) * kBM;           // its first query row in the sequence
  const int ns = ((row0 + kBM - 1) >> a.seg_shift) + 1;
  const float* rec0 = a.part + (int64_t)(bl * a.n_list + hi) * a.seg_n * kSegRecFloats;
  const int64_t orow0 = (int64_t)h * a.qm + (int64_t)b * kBM;  // first row of out and lse
  float mx = -INFINITY, den = 0.f;
  if (t < kBM)
    for (int sg = 0; sg < ns; ++sg) mx = fmaxf(mx, rec0[(int64_t)sg * kSegRecFloats + kSegRowFloats + t]);
  constexpr int kPer = kSegRowFloats / 4 / kCombThreads;  // 16-byte pieces per thread
  f32x4 acc[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) acc[j] = f32x4{};
  for (int s0 = 0; s0 < ns; s0 += kCombSegs) {
    const int s1 = min(ns, s0 + kCombSegs);
    if (t < kBM) {
      for (int sg = s0; sg < s1; ++sg) {
        const float ls = rec0[(int64_t)sg * kSegRecFloats + kSegRowFloats + t];
        const float c = ls == -INFINITY ? 0.f : expf(ls - mx);
        cw[sg - s0][t] = c;
        den += c;
      }
    }
    __syncthreads();
    for (int sg = s0; sg < s1; ++sg) {
      const f32x4* src = reinterpret_cast<const f32x4*>(rec0 + (int64_t)sg * kSegRecFloats);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int q = kCombThreads * j + t;
        acc[j] += cw[sg - s0][q >> 5] * src[q];
      }
    }
    __syncthreads();
  }
  if (t < kBM) {
    inv[t] = den > 0.f ? 1.f / den : 0.f;
    if (a.lse) a.lse[orow0 + t] = den > 0.f ? mx + logf(den) : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = kCombThreads * j + t;
    const int rr = q >> 5;
    const f32x4 x = acc[j] * inv[rr];
    const int64_t o = (orow0 + rr) * kD + 4 * (q & 31);
    if (a.out_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + o) = x;
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
      *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(a.out) + o) = y;
    }
  }
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

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.n_list * a.nb;
  hipLaunchKernelGGL(sparse_attn_fwd, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_seg(const AttnArgs& a, hipStream_t s) {
  // Segments that reach the chunk's longest block.
  const int nseg = (((a.qb0 + a.seg_b0 + a.seg_nb) * kBM - 1) >> a.seg_shift) + 1;
  if (nseg > a.seg_n) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)nseg * a.seg_nb * a.n_list;
  hipLaunchKernelGGL(sparse_attn_seg, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seg_combine, dim3((unsigned)(a.seg_nb * a.n_list)), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
