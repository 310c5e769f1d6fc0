// Grouped-query FlashAttention-style forward kernels for gfx950: one
// workgroup serves HPW query heads that share a KV head (the grouped-query
// layout of the pages' LLaMA-3-8B-shaped layers), so every K/V tile brought
// into LDS serves HPW x 64 query rows instead of 64.  Two kernels share the
// machinery: the full causal baseline (every key j <= i; MInference 1.0
// summary, "Summary": the dense kernel the sparse speedups are measured
// against) and sparse attention over the union of the heads' indices.
//
// Work item: query block b (64 rows) of HPW heads of one KV head = one
// workgroup of 2 HPW wavefronts, two per head (32 rows each).  Keys arrive in
// pieces of up to 32 through a ring of S LDS stages (K and V tiles of one
// piece per stage), filled by buffer loads that go straight to LDS, S - 1
// pieces ahead of the one being finished.  Iteration i: issue the loads of
// piece i+S-1; finish piece i (masks, online softmax in the log2 domain with a
// running max that may lag by up to 8, O^T += V^T P^T) while computing S^T =
// K Q^T of piece i+1, the two interleaved so that each wave keeps the matrix
// core busy during its softmax; wait for this wave's loads of piece i+2;
// barrier.  Every wave issues the same number of loads per iteration (a piece
// past the end reads out of range, which returns zeros), so each wait is a
// fixed vmcnt.
//
// LDS tiles are row-major (one 256-byte row per key) with the 16-byte chunks
// of row r XOR-swizzled (chunk c at slot c ^ swz(r)), so each load-to-LDS
// instruction writes four whole rows from 1 KiB of contiguous memory and the
// K fragment reads and transposed V reads (ds_read_b64_tr_b16) are free of
// bank conflicts.  P and V enter the second product as fp16 (V from an exact
// fp16 copy).
#include <utility>

#include "internal.h"

namespace msa {
namespace {

constexpr int kKP = 32;                      // keys per piece
constexpr int kRowBytes = kD * 2;            // one K or V row
constexpr int kTileBytes = kKP * kRowBytes;  // one K or V tile (8 KiB)
constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile
constexpr float kLag = 8.f;                  // allowed lag of the running max (log2 units)

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Index records are read through the constant address space: the arena does
// not change during the kernel, and uniform loads from it become scalar loads
// (tracked by lgkmcnt, so they never wait on the ring's loads to LDS).
typedef __attribute__((address_space(4))) const int32_t c_i32;
typedef __attribute__((address_space(4))) const GroupDesc c_group;
typedef __attribute__((address_space(4))) const HeadDesc c_head;
template <class T>
__device__ __forceinline__ T* as_const(const void* p) {
  return reinterpret_cast<T*>(reinterpret_cast<uint64_t>(p));
}
// A window of 64 consecutive [lo, hi) range records of one list in VGPRs
// (lane k holds record base + k; records past the list end are empty
// sentinels).  The walks of the sparse kernel read it with readlane, so a
// record costs no memory latency; the window is reloaded (a coalesced 512-byte
// load) only when a walk leaves it.
struct RangeWindow {
  const int2* list;
  int base, end;
  int lo, hi;  // this lane's record
  __device__ __forceinline__ void load(int first) {
    typedef __attribute__((address_space(1))) const u32x2 g_u32x2;
    base = first;
    const int k = first + (int)(threadIdx.x & 63);
    if (k < end) {
      const u32x2 v = *reinterpret_cast<g_u32x2*>(reinterpret_cast<uint64_t>(list + k));
      lo = (int)v[0];
      hi = (int)v[1];
    } else {
      lo = hi = 0x7fffffff;
    }
    // The window is settled here (the compiler waits for the load before this
    // use) and from then on counts as defined by this statement, so the
    // readlanes of later pieces wait for nothing, in particular not for the
    // ring's loads in flight.
    asm volatile("" : "+v"(lo), "+v"(hi));
  }
  __device__ __forceinline__ void init(const int2* l, int first, int end_) {
    list = l;
    end = end_;
    load(first);
  }
  // Record i (uniform; i >= base), or the sentinel past the end.
  __device__ __forceinline__ int2 at(int i) {
    if (i >= end) return make_int2(0x7fffffff, 0x7fffffff);
    if (i - base >= 64) load(i);
    return make_int2(__builtin_amdgcn_readlane(lo, i - base), __builtin_amdgcn_readlane(hi, i - base));
  }
};

// One LDS array per ring stage, so that the compiler can tell the stage being
// filled from the stages being read.
__shared__ __attribute__((aligned(1024))) char g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage3[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage4[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage5[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage6[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage7[kStageBytes];

// Keys of the current column piece (column phase of the sparse kernel).
__shared__ int g_col_keys[kKP];

template <int I>
__device__ __forceinline__ char* stage() {
  static_assert(I >= 0 && I < 8, "at most 8 stages");
  if constexpr (I == 0) return g_stage0;
  if constexpr (I == 1) return g_stage1;
  if constexpr (I == 2) return g_stage2;
  if constexpr (I == 3) return g_stage3;
  if constexpr (I == 4) return g_stage4;
  if constexpr (I == 5) return g_stage5;
  if constexpr (I == 6) return g_stage6;
  if constexpr (I == 7) return g_stage7;
}

// Chunk slot of 16-byte chunk c of tile row r is c ^ swz(r).  For 16
// consecutive rows swz takes 16 distinct values, and for 4 consecutive rows
// starting at a multiple of 4 it takes 4 values that differ in bits 2-3.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Transposed LDS read (gfx950): within each group of 16 lanes, lane i gets
// element i%4 of the 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ f16x4 lds_read_tr(const char* p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32); }

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (expcnt left alone), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without a memory fence: the fence of __syncthreads would
// wait for every load in flight, including the ring's prefetches.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int I, int N, class F>
__device__ __forceinline__ bool run_steps(F& f) {
  if constexpr (I == N) {
    return true;
  } else {
    if (!f(std::integral_constant<int, I>{})) return false;
    return run_steps<I + 1, N>(f);
  }
}

// Blocks longest first; within a block index, consecutive workgroups take
// consecutive (KV head, head chunk) pairs, and since workgroups are dealt
// round-robin over the 8 XCDs, one KV head's workgroups share an XCD's L2
// whenever the pair count is a multiple of 8.
__device__ __forceinline__ void map_group(int x, int pairs, int nb, int& pair, int& b) {
  const int bi = x / pairs;
  pair = x - bi * pairs;
  b = nb - 1 - bi;
}

}  // namespace

// Per-wave state of one head's 32 query rows and the work on one piece:
//   qk       S^T (32 keys x 32 rows) = K . Q^T          v_mfma_f32_32x32x16_bf16
//   mask     causal / key-set / A-shape window masks of S^T
//   prep     running max (log2 domain; may lag the true max by up to 8, so
//            O is rescaled only when a row's max grows by more than that)
//   pv       P = exp2(s - m) in fp16; O^T (128 x 32 rows) += V^T . P^T
//   fused    prep'd piece i's exponentials and P.V interleaved with the S^T
//            MFMAs of piece i+1, in groups that keep the matrix core busy
//            while the wave issues VALU work
struct HeadRows {
  bf16x8 qf[8];  // Q fragments: row l32, d = 16t + 8g .. +8 (B operand of S^T)
  int kofs[8];   // LDS offsets of K fragment t (row l32, chunk 2t + g)
  int vofs[2][4];
  f32x16 o[4];
  float m_run, l_run;
  int row, row0, g;
  float sl2;
  bool ashape;
  int sink, window;

  __device__ __forceinline__ void init(const uint16_t* qh, int lane, int row0_, int rows_off, float sl2_) {
    const int l32 = lane & 31;
    g = lane >> 5;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + l32 * kD + 16 * t + 8 * g));
#pragma unroll
    for (int t = 0; t < 8; ++t) kofs[t] = l32 * kRowBytes + 16 * ((2 * t + g) ^ swz(l32));
    // V^T fragment (kh2, dt, hi): row 16kh2 + 8hi + 4g + (lane%16)/4, chunk
    // 4dt + 2((lane/16)%2) + (lane%4)/2, byte half lane%2; swz ignores the
    // 16kh2 part, which becomes an immediate.
    const int s16 = lane & 15;
    const int vc = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int ra = 8 * hi + 4 * g + (s16 >> 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vofs[hi][dt] = kTileBytes + ra * kRowBytes + 16 * ((4 * dt + vc) ^ swz(ra)) + 8 * (s16 & 1);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
    row0 = row0_;
    row = row0_ + rows_off + l32;
    sl2 = sl2_;
    ashape = false;
    sink = window = 0;
  }

  // Marks the Q fragments as settled (their loads were waited for), so the
  // compiler places no wait for them inside the loop.
  __device__ __forceinline__ void settle_q() {
#pragma unroll
    for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(qf[t]));
  }

  __device__ __forceinline__ bf16x8 kfrag(const char* st, int t) const {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + kofs[t]));
  }
  __device__ __forceinline__ f16x8 vfrag(const char* st, int kh2, int dt) const {
    const f16x4 lo = lds_read_tr(st + vofs[0][dt] + 4096 * kh2);
    const f16x4 hi = lds_read_tr(st + vofs[1][dt] + 4096 * kh2);
    return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  __device__ __forceinline__ f32x16 qk(const char* st) const {
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < 8; ++t) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(st, t), qf[t], s, 0, 0, 0);
    return s;
  }

  // Element r of S^T is key slot 8(r/4) + 4g + r%4.  keys: the piece's key
  // list (column pieces) or null (key = kstart + slot).  bits: the piece's
  // keys that belong to this head.  Away from the diagonal and the A-shape
  // window only the key set matters: with lb = bits >> 4g, element r is kept
  // iff bit 8(r/4) + r%4 of lb is set (a bit test and a select per element).
  __device__ __forceinline__ void mask(f32x16& s, int kstart, const int* keys, int cnt, uint32_t bits) const {
    const int kmin = keys ? keys[0] : kstart;
    const int kmax = keys ? keys[cnt - 1] : kstart + cnt - 1;
    const bool far = ashape && kmax >= sink && row0 + kBM - 1 - max(kmin, sink) >= window;
    if (kmax <= row0 && !far) {
      if (bits != 0xffffffffu) {
        const uint32_t lb = bits >> (4 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = (lb >> (8 * (r >> 2) + (r & 3))) & 1u ? s[r] : -INFINITY;
      }
      return;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int slot = 8 * (r >> 2) + 4 * g + (r & 3);
      const int key = keys ? keys[slot] : kstart + slot;
      const bool ok = ((bits >> slot) & 1u) & (key <= row) & !(ashape & (key >= sink) & (row - key >= window));
      s[r] = ok ? s[r] : -INFINITY;
    }
  }

  // Running-max update for a masked S^T; returns the max to subtract.  The
  // check runs on each lane's own 16 elements (a wave-wide vote); only a
  // rescale, which is rare once the max has settled, needs the row max
  // across the two half-waves that hold a row.
  __device__ __forceinline__ float prep(const f32x16& s) {
    float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    mx *= sl2;
    if (__any(mx > m_run + kLag)) {
      const float mn = fmaxf(m_run, max_halves(mx));
      const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    return m_run == -INFINITY ? 0.f : m_run;
  }

  // Exponentials + P.V of a prep'd piece (V tile in stage vst).
  __device__ __forceinline__ void pv(const f32x16& s, float msub, const char* vst) {
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
    f16x8 pb[2];
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -msub));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -msub));
      const f16x2 e = {(_Float16)e0, (_Float16)e1};
      sum = __builtin_amdgcn_fdot2(e, ones, sum, false);  // row sum of the fp16 P the MFMA consumes
      pb[r >> 3][r & 7] = e[0];
      pb[r >> 3][(r & 7) + 1] = e[1];
    }
    l_run += sum;
#pragma unroll
    for (int kh2 = 0; kh2 < 2; ++kh2) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(vst, kh2, dt), pb[kh2], o[dt], 0, 0, 0);
    }
  }

  // pv(s, msub, vst) interleaved with qk(kst_next), which it returns.
  __device__ __forceinline__ f32x16 fused(const f32x16& s, float msub, const char* vst, const char* kst_next) {
    const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};
    f32x16 s_nxt = f32x16{};
    f16x8 pb[2];
    bf16x8 kf[8];
    f16x8 va[8];
    float sum = 0.f;
    kf[0] = kfrag(kst_next, 0);
    kf[1] = kfrag(kst_next, 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 2 < 8) kf[t + 2] = kfrag(kst_next, t + 2);
      va[t] = vfrag(vst, t >> 2, t & 3);
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t], s_nxt, 0, 0, 0);
      const int r = 2 * t;
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -msub));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -msub));
      const f16x2 e = {(_Float16)e0, (_Float16)e1};
      pb[r >> 3][r & 7] = e[0];
      pb[r >> 3][(r & 7) + 1] = e[1];
      sum = __builtin_amdgcn_fdot2(e, ones, sum, false);
      // keep this group's exponentials here (the compiler would otherwise
      // sink those only the last products need to the end of the block)
      asm volatile("" : "+v"(sum));
      if (t >= 4) o[t - 4] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[t - 4], pb[0], o[t - 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[4 + dt], pb[1], o[dt], 0, 0, 0);
    l_run += sum;
    return s_nxt;
  }

  // One iteration of the per-wave pipeline: finish piece i (S^T in s_cur,
  // K/V in stage cur; bits = this head's keys of the piece, 0 if none) and
  // compute S^T of piece i+1 (K in stage nxt).  One code path: a piece the
  // head does not need is fully masked (P = 0), and the S^T of a piece it
  // does not need is computed all the same (the stage always holds finite
  // data), so the work is skipped only when neither piece is needed.
  __device__ __forceinline__ void advance(f32x16& s_cur, int kstart, const int* keys, int cnt, uint32_t bits,
                                          const char* cur, bool need_n, const char* nxt) {
    if (bits != 0u || need_n) {
      f32x16 s = s_cur;
      mask(s, kstart, keys, cnt, bits);
      const float msub = prep(s);
      s_cur = fused(s, msub, cur, nxt);
    }
  }

  __device__ __forceinline__ void store(const AttnArgs& a, int h) const {
    const float lt = sum_halves(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = (int64_t)h * a.qm + row - (int64_t)a.qb0 * kBM;  // this lane's row of out and lse
    const int64_t obase = orow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * g;
        const float x0 = o[dt][4 * q4 + 0] * inv, x1 = o[dt][4 * q4 + 1] * inv;
        const float x2 = o[dt][4 * q4 + 2] * inv, x3 = o[dt][4 * q4 + 3] * inv;
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + obase + d0) = f32x4{x0, x1, x2, x3};
        } else {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
          *reinterpret_cast<bf16x4*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) = y;
        }
      }
    }
    if (a.lse && g == 0)
      a.lse[orow] = lt > 0.f ? m_run * 0.69314718055994530942f + logf(lt) : -INFINITY;
  }
};

// Loads of one piece into a ring stage: load-to-LDS instruction q = kD16 * wv
// + d (0..15) fills tile rows 4(q%8) + lane/16 of the K tile (q < 8) or the V
// tile (q >= 8); the lane writes chunk slot lane%16 and fetches chunk
// (lane%16) ^ swz(row).
template <int kD16>
struct Loader {
  __amdgpu_buffer_rsrc_t rs;
  int tile;             // 0 (K) or kTileBytes (V)
  int wv;
  int lrow[kD16];       // tile row of this lane in load d
  uint32_t lofs[kD16];  // row offset + chunk offset (range pieces: + start * 256)
  uint32_t cofs[kD16];  // chunk offset (column pieces: + key * 256)

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int wv_, int lane) {
    wv = wv_;
    const bool v = kD16 * wv >= 8;  // a wave's loads all go to one tile
    rs = v ? vr : kr;
    tile = v ? kTileBytes : 0;
#pragma unroll
    for (int d = 0; d < kD16; ++d) {
      const int q = kD16 * wv + d;
      lrow[d] = 4 * (q & 7) + (lane >> 4);
      cofs[d] = 16u * (uint32_t)((lane & 15) ^ swz(lrow[d]));
      lofs[d] = (uint32_t)lrow[d] * (uint32_t)kRowBytes + cofs[d];
    }
  }
  // Range piece from key `start` (start = n: out of range, reads zeros).
  __device__ __forceinline__ void range(char* st, int start) const {
#pragma unroll
    for (int d = 0; d < kD16; ++d) {
      const int q = kD16 * wv + d;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + tile + 1024 * (q & 7)), 16,
                                               (uint32_t)start * (uint32_t)kRowBytes + lofs[d], 0, 0, 0);
    }
  }
  // Column piece: key[d] is the key of tile row lrow[d].
  __device__ __forceinline__ void gather(char* st, const int* key) const {
#pragma unroll
    for (int d = 0; d < kD16; ++d) {
      const int q = kD16 * wv + d;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(st + tile + 1024 * (q & 7)), 16,
                                               (uint32_t)key[d] * (uint32_t)kRowBytes + cofs[d], 0, 0, 0);
    }
  }
};

// Full causal attention.  A workgroup of 8 waves serves four slots of 64
// query rows (two waves each) that read the same KV head: HPW heads of one
// query block times 4 / HPW consecutive query blocks (GQA 4:1: four heads of
// one block; two heads per KV head: two heads of two blocks; one head per KV
// head: four blocks of that head).  The keys of the slots' longest block are
// walked once; a slot's waves skip the pieces past their own block's last
// row, so every K/V tile in LDS feeds up to 256 query rows whatever the group
// size.
template <int HPW, int S>
__device__ __forceinline__ void group_dense_body(const AttnArgs& a) {
  constexpr int kSlots = 4;
  constexpr int kBQ = kSlots / HPW;                // consecutive query blocks per workgroup
  constexpr int kD16 = 16 / (2 * kSlots);          // load-to-LDS instructions per wave per piece
  static_assert(S >= 3 && kD16 >= 1 && kSlots % HPW == 0, "ring, wave and slot counts");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wv >> 1;
  const int chunks = a.grp / HPW;
  const int ngroups = (a.nb + kBQ - 1) / kBQ;     // groups of kBQ query blocks, the last one may be short
  int pair, bg;
  map_group(blockIdx.x, a.hkv * chunks, ngroups, pair, bg);
  const int kvh = pair % a.hkv, chunk = pair / a.hkv;
  const int h = kvh * a.grp + chunk * HPW + slot % HPW;
  // Group bg holds the call's query blocks bg*kBQ .. bg*kBQ + kBQ - 1 (those
  // below nb); slot j takes the (j / HPW)-th from the top.
  const int btop = min(a.nb - 1, bg * kBQ + kBQ - 1);
  const int bj = btop - slot / HPW;
  const bool active = bj >= bg * kBQ;
  const int b = active ? bj : btop;
  const int64_t n = a.n;
  const int row0 = (a.qb0 + b) * kBM;              // this slot's first query row
  const int end = active ? row0 + kBM : 0;         // this slot's keys: [0, end)
  const int npieces = ((a.qb0 + btop) * kBM) / kKP + 2;  // keys [0, top block's row0 + 64)

  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  HeadRows hr;
  hr.init(a.q + ((int64_t)h * a.qm + (int64_t)b * kBM + 32 * (wv & 1)) * kD, lane, row0, 32 * (wv & 1),
          a.scale_log2);
  Loader<kD16> ld;
  ld.init(kr, vr, wv, lane);

  auto prologue = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    ld.range(stage<ST>(), ST < npieces ? kKP * ST : (int)n);
    return true;
  };
  run_steps<0, S - 1>(prologue);
  // The Q fragments and pieces 0 and 1 must have landed; later pieces may not.
  wait_vm_lgkm0<(S - 3) * kD16>();
  hr.settle_q();
  barrier_only();
  f32x16 s_cur = hr.qk(stage<0>());

  int i = 0;
  auto step = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    const int p = i + S - 1;
    ld.range(stage<(ST + S - 1) % S>(), p < npieces ? kKP * p : (int)n);
    if constexpr (kBQ == 1) {
      // one query block: every piece up to the end holds keys of every slot
      hr.advance(s_cur, kKP * i, nullptr, kKP, 0xffffffffu, stage<ST>(), true, stage<(ST + 1) % S>());
    } else {
      // pieces at or past the slot's end hold none of its keys
      const uint32_t bits = kKP * i < end ? 0xffffffffu : 0u;
      hr.advance(s_cur, kKP * i, nullptr, kKP, bits, stage<ST>(), kKP * (i + 1) < end, stage<(ST + 1) % S>());
    }
    // Pieces i+1 (V) and i+2 (K, read ahead) must have landed (this wave's
    // share); S-3 later pieces may still be in flight.
    wait_vm_lgkm0<(S - 3) * kD16>();
    barrier_only();
    ++i;
    return i < npieces;
  };
  while (run_steps<0, S>(step)) {
  }
  wait_vm_lgkm0<0>();  // loads of pieces past the end
  if (active) hr.store(a, h);
}

// A-shape heads of one head per KV head (MHA): a workgroup of 8 waves serves
// four consecutive query blocks of one head, two waves each, like the dense
// kernel.  Their keys are the sink [0, sink) and the union of the four
// blocks' windows, [max(0, lowest row - window + 1), top block's end): at
// most two ranges, walked in pieces of up to 32 keys; a slot's waves skip the
// pieces that hold none of their own block's keys ([0, min(sink, end)) and
// [max(0, row0 - window + 1), end)) and mask the rest per row (causal and the
// row's own window), so each K/V tile in LDS feeds up to 256 query rows.
template <int S>
__device__ __forceinline__ void group_ashape_body(const AttnArgs& a) {
  constexpr int kSlots = 4;
  constexpr int kD16 = 16 / (2 * kSlots);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wv >> 1;
  // Groups are the sequence's query blocks 4g .. 4g+3 (the last one may be
  // short), so a chunk of a longer prefill walks exactly the keys the whole
  // sequence does for each of its blocks; slots below the call's first block
  // stay idle.
  const int nseq = a.qb0 + a.nb;  // query blocks of the sequence
  const int gfirst = a.qb0 / kSlots, glast = (nseq - 1) / kSlots;
  int hi, gi;
  map_group(blockIdx.x, a.n_list, glast - gfirst + 1, hi, gi);
  const int g = gfirst + gi;
  const int h = a.list[hi];
  const int kvh = h / a.grp;
  c_head* hd = as_const<c_head>(a.arena) + h;
  const int sink = hd->p0, window = hd->p1;
  const int top = min(nseq - 1, kSlots * g + kSlots - 1);  // the group's highest block
  const int sb = top - slot;                                // this slot's block of the sequence
  const bool active = sb >= max(kSlots * g, a.qb0);
  const int b = (active ? sb : top) - a.qb0;                // the call's block (rows of Q and out)
  const int64_t n = a.n;
  const int row0 = (a.qb0 + b) * kBM;
  const int end = row0 + kBM;
  // this slot's keys: [0, s_end) and [w_lo, end)
  const int s_end = active ? min(sink, end) : 0;
  const int w_lo = active ? max(0, row0 - window + 1) : 0;
  const int w_hi = active ? end : 0;
  // the workgroup's walk: [0, r1) then [r2lo, r2hi), fixed by the group
  const int top_end = top * kBM + kBM;
  const int lo_all = max(0, kSlots * g * kBM - window + 1);
  const int r1 = sink >= lo_all ? 0 : sink;
  const int r2lo = sink >= lo_all ? 0 : lo_all;
  const int r2hi = top_end;
  const int n1 = (r1 + kKP - 1) / kKP;
  const int npieces = n1 + (r2hi - r2lo + kKP - 1) / kKP;
  auto piece = [&](int p, int& start, int& count) {
    if (p < n1) {
      start = kKP * p;
      count = min(kKP, r1 - start);
    } else if (p < npieces) {
      start = r2lo + kKP * (p - n1);
      count = min(kKP, r2hi - start);
    } else {
      start = (int)n;  // past the end: reads zeros, holds no key
      count = 0;
    }
  };
  auto span_bits = [](int lo, int hi, int start, int count) -> uint32_t {
    const int a0 = max(lo, start) - start, a1 = min(hi, start + count) - start;
    if (a1 <= a0) return 0u;
    const uint32_t upto = a1 >= 32 ? 0xffffffffu : ((1u << a1) - 1u);
    return upto & ~((1u << a0) - 1u);
  };
  auto slot_bits = [&](int start, int count) -> uint32_t {
    return span_bits(0, s_end, start, count) | span_bits(w_lo, w_hi, start, count);
  };

  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  HeadRows hr;
  hr.init(a.q + ((int64_t)h * a.qm + (int64_t)b * kBM + 32 * (wv & 1)) * kD, lane, row0, 32 * (wv & 1),
          a.scale_log2);
  hr.ashape = true;
  hr.sink = sink;
  hr.window = window;
  Loader<kD16> ld;
  ld.init(kr, vr, wv, lane);

  int p_start[S], p_count[S];
  auto prologue = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    piece(ST, p_start[ST], p_count[ST]);
    ld.range(stage<ST>(), p_start[ST]);
    return true;
  };
  run_steps<0, S - 1>(prologue);
  wait_vm_lgkm0<(S - 3) * kD16>();
  hr.settle_q();
  barrier_only();
  f32x16 s_cur = hr.qk(stage<0>());

  int i = 0;
  auto step = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    constexpr int NS = (ST + S - 1) % S;
    piece(i + S - 1, p_start[NS], p_count[NS]);
    ld.range(stage<NS>(), p_start[NS]);
    const uint32_t bits = slot_bits(p_start[ST], p_count[ST]);
    constexpr int N1 = (ST + 1) % S;
    const bool need_n = i + 1 < npieces && slot_bits(p_start[N1], p_count[N1]) != 0u;
    hr.advance(s_cur, p_start[ST], nullptr, p_count[ST], bits, stage<ST>(), need_n, stage<N1>());
    wait_vm_lgkm0<(S - 3) * kD16>();
    barrier_only();
    ++i;
    return i < npieces;
  };
  while (run_steps<0, S>(step)) {
  }
  wait_vm_lgkm0<0>();
  if (active) hr.store(a, h);
}

// A window of 64 consecutive entries of an ascending key list in VGPRs (lane
// k holds entry base + k), read with readlane like RangeWindow.
struct KeyWindow {
  const int* list;
  int base, end;
  int key;  // this lane's entry
  __device__ __forceinline__ void load(int first) {
    typedef __attribute__((address_space(1))) const int32_t g_i32;
    base = first;
    const int k = first + (int)(threadIdx.x & 63);
    key = k < end ? *reinterpret_cast<g_i32*>(reinterpret_cast<uint64_t>(list + k)) : 0x7fffffff;
    asm volatile("" : "+v"(key));
  }
  __device__ __forceinline__ void init(const int* l, int first, int end_) {
    list = l;
    end = end_;
    load(first);
  }
  __device__ __forceinline__ int at(int i) {
    if (i >= end) return 0x7fffffff;
    if (i - base >= 64) load(i);
    return __builtin_amdgcn_readlane(key, i - base);
  }
};

// Heads whose key sets cover most of the causal keys (expected density >=
// 3/4; MInference 1.0 summary, "Summary", third stage), kSlots (head, query
// block) slots per workgroup of 2 kSlots waves, walking every key below the
// slots' last row in pieces of 32 aligned keys (no union index).  Each
// slot's waves compute a piece only if it holds some of the slot's keys,
// with a per-key mask from the slot's own ranges and columns (each walked
// alongside, from windows of 64 records), so each K/V tile in LDS feeds up to
// 64 kSlots query rows.  The slots are HPW heads of one KV head (a.list[HPW u
// + j], -1 for none; HPW = 1: one head served alone) times kSlots / HPW
// consecutive query blocks, in groups aligned to the sequence's blocks (the
// last one may be short), like group_ashape_body.  A slot's pieces are those
// below its own block's end, in key order, whatever its group: a chunk of a
// sequence computes what the whole sequence computes.
template <int S, int kSlots, int HPW>
__device__ __forceinline__ void group_csr_body(const AttnArgs& a) {
  constexpr int kD16 = 16 / (2 * kSlots);
  constexpr int kBQ = kSlots / HPW;  // consecutive query blocks per workgroup
  static_assert(kSlots % HPW == 0, "slot count");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wv >> 1;
  // Slots below the call's first block, or of a missing head, stay idle.
  const int nseq = a.qb0 + a.nb;
  const int gfirst = a.qb0 / kBQ, glast = (nseq - 1) / kBQ;
  int u, gi;
  map_group(blockIdx.x, a.n_list, glast - gfirst + 1, u, gi);
  const int g = gfirst + gi;
  const int top = min(nseq - 1, kBQ * g + kBQ - 1);
  const int sb = top - slot / HPW;
  const bool in_call = sb >= max(kBQ * g, a.qb0);
  const int hs = a.list[HPW * u + slot % HPW];
  const bool active = hs >= 0 && in_call;
  const int h = hs >= 0 ? hs : a.list[HPW * u];
  const int b = (in_call ? sb : top) - a.qb0;  // the call's block (CSR, rows of Q and out)
  const int top_end = top * kBM + kBM;
  const int kvh = h / a.grp;
  c_head* hd = as_const<c_head>(a.arena) + h;
  const int64_t n = a.n;
  const int row0 = (a.qb0 + b) * kBM;
  const int npieces = (top_end + kKP - 1) / kKP;
  auto piece = [&](int p, int& start, int& count) {
    if (p < npieces) {
      start = kKP * p;
      count = min(kKP, top_end - start);
    } else {
      start = (int)n;  // past the end: reads zeros, holds no key
      count = 0;
    }
  };
  // This slot's ranges and columns, walked in key order alongside the pieces.
  c_i32* rp = as_const<c_i32>(a.arena + hd->rng_ptr_off);
  c_i32* cp = as_const<c_i32>(a.arena + hd->col_ptr_off);
  int ri = active ? rp[b] : 0;
  const int r_end = active ? rp[b + 1] : 0;
  int ci = active ? cp[b] : 0;
  const int c_end = active ? cp[b + 1] : 0;
  RangeWindow rwin;
  rwin.init(reinterpret_cast<const int2*>(a.arena + hd->rng_off), ri, r_end);
  KeyWindow cwin;
  cwin.init(reinterpret_cast<const int*>(a.arena + hd->col_off), ci, c_end);
  int rlo = 0x7fffffff, rhi = 0x7fffffff;
  auto range_advance = [&]() {
    const int2 x = rwin.at(ri);
    rlo = x.x;
    rhi = x.y;
    if (ri < r_end) ++ri;
  };
  range_advance();
  int ckey = cwin.at(ci);
  // Keys of piece [start, start + count) that are this slot's (pieces come in
  // increasing order, every piece once).
  auto slot_bits = [&](int start, int count) -> uint32_t {
    if (count == 0) return 0u;
    const int e = start + count;
    uint32_t bits = 0u;
    while (rhi <= start) range_advance();
    // the usual case for these heads: one range covers the piece (columns
    // lie in no range, so none is in it)
    if (rlo <= start && rhi >= e) return count >= 32 ? 0xffffffffu : (1u << count) - 1u;
    while (rlo < e) {
      const int lo = max(rlo, start) - start, w = min(rhi, e) - start - lo;
      bits |= (w >= 32 ? 0xffffffffu : ((1u << w) - 1u)) << lo;
      if (rhi > e) break;
      range_advance();
    }
    while (ckey < e) {
      bits |= 1u << (ckey - start);
      ckey = cwin.at(++ci);
    }
    return bits;
  };

  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  HeadRows hr;
  hr.init(a.q + ((int64_t)h * a.qm + (int64_t)b * kBM + 32 * (wv & 1)) * kD, lane, row0, 32 * (wv & 1),
          a.scale_log2);
  Loader<kD16> ld;
  ld.init(kr, vr, wv, lane);

  int p_start[S], p_count[S];
  auto prologue = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    piece(ST, p_start[ST], p_count[ST]);
    ld.range(stage<ST>(), p_start[ST]);
    return true;
  };
  run_steps<0, S - 1>(prologue);
  uint32_t bits = slot_bits(p_start[0], p_count[0]);  // piece i's keys of this slot
  wait_vm_lgkm0<(S - 3) * kD16>();
  hr.settle_q();
  barrier_only();
  f32x16 s_cur = hr.qk(stage<0>());

  int i = 0;
  auto step = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    constexpr int NS = (ST + S - 1) % S;
    constexpr int N1 = (ST + 1) % S;
    piece(i + S - 1, p_start[NS], p_count[NS]);
    ld.range(stage<NS>(), p_start[NS]);
    const uint32_t bits_n = slot_bits(p_start[N1], p_count[N1]);
    hr.advance(s_cur, p_start[ST], nullptr, p_count[ST], bits, stage<ST>(), bits_n != 0u, stage<N1>());
    bits = bits_n;
    wait_vm_lgkm0<(S - 3) * kD16>();
    barrier_only();
    ++i;
    return i < npieces;
  };
  while (run_steps<0, S>(step)) {
  }
  wait_vm_lgkm0<0>();
  if (active) hr.store(a, h);
}

// Sparse attention over the union index of a chunk of HPW heads (MInference
// 1.0 summary, "Summary", third stage; union_index.hip builds the lists).
// Phase 1 streams the union ranges through the ring in pieces of up to 32
// consecutive keys; each head's waves work on a piece only if it holds some
// of the head's keys, with a per-key mask taken from the head's own ranges
// (walked alongside with scalar loads).  Phase 2 takes the union columns in
// pieces of 32 gathered keys, one piece at a time, the head's keys marked by
// umask.  Row i of head h keeps key j iff j is in h's ranges or columns of
// block i/64, j <= i, and for A-shape heads j < sink or i - j < window; a row
// with no key gives 0 (lse -inf).
template <int HPW, int S>
__device__ __forceinline__ void group_sparse_body(const AttnArgs& a, const GroupDesc* __restrict__ groups,
                                                  const char* __restrict__ arena) {
  constexpr int kD16 = 16 / (2 * HPW);
  static_assert(S >= 3 && kD16 >= 1, "ring and wave counts");
  constexpr int kNone = 0x7fffffff;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jh = wv >> 1;  // head slot within the chunk
  // Workgroup x: chunk x % n_list, query block nb - 1 - x / n_list (longest
  // blocks first).
  const int bi = (int)blockIdx.x / a.n_list;
  const int u = (int)blockIdx.x - bi * a.n_list;
  const int b = a.nb - 1 - bi;
  c_group* gd = as_const<c_group>(groups) + u;
  const int kvh = gd->kvh;
  // A chunk with fewer than HPW heads leaves the waves of the missing slots
  // idle: they load their share of the tiles and keep the barriers, nothing
  // else.
  const bool active = jh < gd->nheads;
  const int h = gd->head[active ? jh : 0];
  c_head* hd = as_const<c_head>(arena) + h;
  const int64_t n = a.n;
  const int row0 = (a.qb0 + b) * kBM;  // b indexes the call's query blocks and the CSR

  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  HeadRows hr;
  hr.init(a.q + ((int64_t)h * a.qm + (int64_t)b * kBM + 32 * (wv & 1)) * kD, lane, row0, 32 * (wv & 1),
          a.scale_log2);
  hr.ashape = hd->pattern == MS_A_SHAPE;
  hr.sink = hd->p0;
  hr.window = hd->p1;
  Loader<kD16> ld;
  ld.init(kr, vr, wv, lane);

  // Union range walk (identical in every wave): pieces of <= 32 keys.
  c_i32* urp = as_const<c_i32>(arena + gd->urng_ptr_off);
  int ur = urp[b];
  const int ur_end = urp[b + 1];
  RangeWindow uwin;
  uwin.init(reinterpret_cast<const int2*>(arena + gd->urng_off), ur, ur_end);
  int uhi = 0, pos = 0;
  auto next_piece = [&](int& start, int& count) {
    while (pos >= uhi && ur < ur_end) {
      const int2 x = uwin.at(ur);
      pos = x.x;
      uhi = x.y;
      ++ur;
    }
    if (pos < uhi) {
      start = pos;
      count = min(kKP, uhi - pos);
      pos += count;
    } else {
      start = (int)n;
      count = 0;
    }
  };
  // This head's range walk: the keys of a piece that are the head's.
  c_i32* hrp = as_const<c_i32>(arena + hd->rng_ptr_off);
  int hri = hrp[b];
  const int hr_end = hrp[b + 1];
  RangeWindow hwin;
  hwin.init(reinterpret_cast<const int2*>(arena + hd->rng_off), hri, hr_end);
  int hlo = kNone, hhi = kNone;
  auto head_advance = [&]() {
    const int2 x = hwin.at(hri);
    hlo = x.x;
    hhi = x.y;
    if (hri < hr_end) ++hri;
  };
  head_advance();
  auto head_bits = [&](int start, int count) -> uint32_t {
    if (count == 0 || !active) return 0u;
    const int e = start + count;
    while (hhi <= start) head_advance();
    // the usual case for heads that keep most keys: one range covers the piece
    if (hlo <= start && hhi >= e) return count >= 32 ? 0xffffffffu : (1u << count) - 1u;
    uint32_t bits = 0u;
    while (hlo < e) {
      const int lo = max(hlo, start) - start, w = min(hhi, e) - start - lo;
      bits |= (w >= 32 ? 0xffffffffu : ((1u << w) - 1u)) << lo;
      if (hhi > e) break;
      head_advance();
    }
    return bits;
  };

  // Phase 1: union ranges through the ring.  Per stage: piece start, key
  // count (0 = past the end) and this head's key mask.
  int r_start[S], r_count[S];
  uint32_t r_bits[S];
  auto prologue = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    next_piece(r_start[ST], r_count[ST]);
    r_bits[ST] = head_bits(r_start[ST], r_count[ST]);
    ld.range(stage<ST>(), r_start[ST]);
    return true;
  };
  run_steps<0, S - 1>(prologue);
  wait_vm_lgkm0<(S - 3) * kD16>();
  hr.settle_q();
  barrier_only();
  f32x16 s_cur = hr.qk(stage<0>());

  auto step = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    constexpr int NS = (ST + S - 1) % S;
    if (r_count[ST] == 0) return false;  // identical in every wave
    next_piece(r_start[NS], r_count[NS]);
    r_bits[NS] = head_bits(r_start[NS], r_count[NS]);
    ld.range(stage<NS>(), r_start[NS]);
    hr.advance(s_cur, r_start[ST], nullptr, r_count[ST], r_bits[ST], stage<ST>(), r_bits[(ST + 1) % S] != 0u,
               stage<(ST + 1) % S>());
    wait_vm_lgkm0<(S - 3) * kD16>();
    barrier_only();
    return true;
  };
  while (run_steps<0, S>(step)) {
  }
  wait_vm_lgkm0<0>();
  barrier_only();

  // Phase 2: union columns, one piece at a time through stage 0.
  c_i32* ucp = as_const<c_i32>(arena + gd->ucol_ptr_off);
  const int c0 = ucp[b], c1 = ucp[b + 1];
  typedef __attribute__((address_space(1))) const int32_t g_i32;
  typedef __attribute__((address_space(1))) const uint8_t g_u8;
  g_i32* ucol = reinterpret_cast<g_i32*>(reinterpret_cast<uint64_t>(arena + gd->ucol_off));
  g_u8* umask = reinterpret_cast<g_u8*>(reinterpret_cast<uint64_t>(arena + gd->umask_off));
  for (int c = c0; c < c1; c += kKP) {
    const int cnt = min(kKP, c1 - c);
    int key[kD16];
#pragma unroll
    for (int d = 0; d < kD16; ++d) key[d] = ucol[c + min(ld.lrow[d], cnt - 1)];
    const int mk = umask[c + min(lane & 31, cnt - 1)];
    const uint32_t bits = active ? (uint32_t)__ballot(lane < cnt && ((mk >> jh) & 1)) : 0u;
    if (wv == 0 && lane < kKP) g_col_keys[lane] = ucol[c + min(lane, cnt - 1)];
    ld.gather(stage<0>(), key);
    wait_vm_lgkm0<0>();
    barrier_only();
    if (bits != 0u) {
      f32x16 s = hr.qk(stage<0>());
      hr.mask(s, 0, g_col_keys, cnt, bits);
      const float msub = hr.prep(s);
      hr.pv(s, msub, stage<0>());
    }
    barrier_only();
  }
  if (active) hr.store(a, h);
}

// Dense: eight waves and eight ring stages (128 KiB of LDS, one workgroup per
// CU) for every group size; HPW heads of one KV head per workgroup, each over
// 4 / HPW consecutive query blocks.
__global__ __launch_bounds__(512) void group_dense_h4(AttnArgs a) { group_dense_body<4, 8>(a); }
__global__ __launch_bounds__(512) void group_dense_h2(AttnArgs a) { group_dense_body<2, 8>(a); }
__global__ __launch_bounds__(512) void group_dense_h1(AttnArgs a) { group_dense_body<1, 8>(a); }

// A-shape heads of MHA layers: four query blocks of one head per workgroup.
__global__ __launch_bounds__(512) void group_ashape_blocks(AttnArgs a) { group_ashape_body<8>(a); }
__global__ __launch_bounds__(512) void group_csr_blocks(AttnArgs a) { group_csr_body<8, 4, 1>(a); }
__global__ __launch_bounds__(512) void group_csr_heads2(AttnArgs a) { group_csr_body<8, 4, 2>(a); }
__global__ __launch_bounds__(512) void group_csr_heads4(AttnArgs a) { group_csr_body<8, 4, 4>(a); }

// Sparse: heads per workgroup (HPW) and ring stages: 4 heads (one workgroup
// per CU, 8 stages = 128 KiB of LDS) or 2 (two per CU, 4 stages).

__global__ __launch_bounds__(512) void group_sparse_h4(AttnArgs a, const GroupDesc* __restrict__ groups,
                                                      const char* __restrict__ arena) {
  group_sparse_body<4, 8>(a, groups, arena);
}
__global__ __launch_bounds__(256) void group_sparse_h2(AttnArgs a, const GroupDesc* __restrict__ groups,
                                                      const char* __restrict__ arena) {
  group_sparse_body<2, 4>(a, groups, arena);
}

hipError_t launch_group_sparse(const AttnArgs& a, const GroupDesc* groups, int hpw, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.nb * a.n_list));
  // chunks of two to four heads, two or four heads per workgroup
  if (hpw == 4)
    hipLaunchKernelGGL(group_sparse_h4, grid, dim3(512), 0, s, a, groups, a.arena);
  else if (hpw == 2)
    hipLaunchKernelGGL(group_sparse_h2, grid, dim3(256), 0, s, a, groups, a.arena);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_group_ashape(const AttnArgs& a, hipStream_t s) {
  const int groups = (a.qb0 + a.nb - 1) / 4 - a.qb0 / 4 + 1;
  const dim3 grid((unsigned)((int64_t)groups * a.n_list));
  hipLaunchKernelGGL(group_ashape_blocks, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_group_csr(const AttnArgs& a, int hpw, hipStream_t s) {
  if (hpw != 1 && hpw != 2 && hpw != 4) return hipErrorInvalidValue;
  const int bq = 4 / hpw;  // consecutive query blocks per workgroup
  const int groups = (a.qb0 + a.nb - 1) / bq - a.qb0 / bq + 1;
  const dim3 grid((unsigned)((int64_t)groups * a.n_list));
  if (hpw == 4)
    hipLaunchKernelGGL(group_csr_heads4, grid, dim3(512), 0, s, a);
  else if (hpw == 2)
    hipLaunchKernelGGL(group_csr_heads2, grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(group_csr_blocks, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_group_dense(const AttnArgs& a, hipStream_t s) {
  const int hpw = hpw_of(a.grp);
  const int bq = 4 / hpw;  // consecutive query blocks per workgroup
  const dim3 grid((unsigned)((int64_t)((a.nb + bq - 1) / bq) * a.hkv * (a.grp / hpw)));
  if (hpw == 4)
    hipLaunchKernelGGL(group_dense_h4, grid, dim3(512), 0, s, a);
  else if (hpw == 2)
    hipLaunchKernelGGL(group_dense_h2, grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(group_dense_h1, grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
