// Sparse FlashAttention-style forward kernel for gfx950 (MInference 1.0
// summary, "Summary", third stage: attention computed only over the estimated
// indices; FlashAttention-2's online softmax is the published algorithm the
// pages' kernels build on).
//
// Work item: one 64-row query block of one Q head = one workgroup of two
// wavefronts, each owning 32 rows.  The block's keys are its ranges, cut into
// pieces of up to 32 consecutive keys, then its column list in pieces of up to
// 32 gathered keys.  Per piece, both waves share one LDS copy of the piece's
// K and V rows, double-buffered: the next piece's rows are loaded into
// registers right after a barrier and written to the other buffer at the end
// of the iteration, a full piece of compute later.
//   S^T (32 keys x 32 rows) = K . Q^T         v_mfma_f32_32x32x16_bf16
//   online softmax in the log2 domain; the running max may lag the true max by
//   up to 8 (P <= 256), so the O rescale only runs when a row's max grows by
//   more than that
//   O^T (128 x 32 rows) += V^T . P^T           v_mfma_f32_32x32x16_f16
// K and V rows are fetched with buffer loads whose range check (one KV head's
// rows) turns reads past the sequence into zeros, so piece tails need no
// clamping.  V is read transposed out of its row-major LDS tile with
// ds_read_b64_tr_b16.  P and V enter the second product as fp16 (V from an
// exact fp16 copy).
#include "internal.h"

namespace msa {
namespace {

constexpr int kKP = 32;            // keys per piece
constexpr int kKS = 136;           // K tile row stride, 16-bit elements (272 B)
constexpr int kVS = 160;           // V tile row stride, 16-bit elements (320 B)
constexpr int kKTile = kKP * kKS;
constexpr int kVTile = kKP * kVS;
constexpr int kRowBytes = kD * 2;  // one K or V row in HBM
constexpr float kLag = 8.f;        // allowed lag of the running max (log2 units)
constexpr int kThreads = 128;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Transposed LDS read (gfx950): within each group of 16 lanes, lane i gets
// element i%4 of the 8-byte chunks addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4.
__device__ __forceinline__ f16x4 lds_read_tr(const _Float16* p) {
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

// A load the compiler keeps on the vector memory path (its address is moved
// into VGPRs first), so it is ordered with the K/V loads by vmcnt instead of
// sharing lgkmcnt with every LDS access.
__device__ __forceinline__ int2 vector_load_int2(const int2* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  uint32_t lo = (uint32_t)a, hi = (uint32_t)(a >> 32);
  asm volatile("v_mov_b32 %0, %0" : "+v"(lo));
  asm volatile("v_mov_b32 %0, %0" : "+v"(hi));
  typedef __attribute__((address_space(1))) const u32x2 global_u32x2;
  const u32x2 v = *reinterpret_cast<global_u32x2*>(((uint64_t)hi << 32) | lo);
  return make_int2((int)v[0], (int)v[1]);
}

// Walks a query block's ranges in pieces of <= 32 consecutive keys, then its
// column list in pieces of <= 32 listed keys.  The position is uniform; the
// descriptor of the next range is fetched one range ahead.
struct PieceIter {
  const int2* rng;
  int r, r_end;
  int lo, hi;
  int c, c_end;
  int2 pre;  // descriptor of range r (valid while r < r_end)
  __device__ __forceinline__ void start() {
    if (r < r_end) pre = vector_load_int2(rng + r);
  }
  __device__ __forceinline__ bool next(Piece& p) {
    while (lo >= hi && r < r_end) {
      lo = __builtin_amdgcn_readfirstlane(pre.x);
      hi = __builtin_amdgcn_readfirstlane(pre.y);
      ++r;
      if (r < r_end) pre = vector_load_int2(rng + r);
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

// Staging registers of one piece: thread t owns 16-byte chunk t%16 of rows
// t/16 + 8i (i = 0..3) of both the K tile and the V tile.
struct Stage {
  u32x4 k[4];
  u32x4 v[4];
  int key[4];  // column pieces only
};

__device__ __forceinline__ void load_piece(const Piece& p, const int* col, __amdgpu_buffer_rsrc_t kr,
                                           __amdgpu_buffer_rsrc_t vr, int row_off, int tid, Stage& st) {
  int off[4];
  if (p.is_col) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.key[i] = col[p.start + min((tid >> 4) + 8 * i, p.count - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) off[i] = st.key[i] * kRowBytes + (row_off & (kRowBytes - 1));
  } else {
    // rows past the piece hold keys that the mask drops; rows past the
    // sequence lie outside the buffer and read as zero
#pragma unroll
    for (int i = 0; i < 4; ++i) off[i] = p.start * kRowBytes + row_off + i * 8 * kRowBytes;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, off[i], 0, 0);
    st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, off[i], 0, 0);
  }
}

__device__ __forceinline__ void store_piece(const Stage& st, bool is_col, uint16_t* kt, _Float16* vt, int* keys,
                                            int tid) {
  const int c16 = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 4) + 8 * i;
    *reinterpret_cast<u32x4*>(kt + row * kKS + 8 * c16) = st.k[i];
    *reinterpret_cast<u32x4*>(vt + row * kVS + 8 * c16) = st.v[i];
  }
  if (is_col && c16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) keys[(tid >> 4) + 8 * i] = st.key[i];
  }
}

// Longest query blocks first (causal work grows with b); Q heads that share a
// KV head are kept on one XCD (workgroups are dealt round-robin over the 8
// XCDs), so that XCD's L2 serves their common K/V rows.
__device__ __forceinline__ void map_work(int x, int hq, int nb, int& h, int& b) {
  const int bi = x / hq, hi = x - bi * hq;
  b = nb - 1 - bi;
  if ((hq & 7) == 0) {
    const int per = hq >> 3;
    h = (hi & 7) * per + (hi >> 3);
  } else {
    h = hi;
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_attn_fwd(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKTile];
  __shared__ __attribute__((aligned(16))) _Float16 v_lds[2][kVTile];
  __shared__ int key_lds[2][kKP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int h, b;
  map_work(blockIdx.x, a.hq, a.nb, h, b);
  const int kvh = h / a.grp;
  const int64_t n = a.n;
  const int row0 = b * kBM;

  PieceIter it{};
  const int* col = nullptr;
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
    col = reinterpret_cast<const int*>(a.arena + d.col_off);
    if (d.pattern == MS_A_SHAPE) {
      ashape = true;
      sink = d.p0;
      window = d.p1;
    }
  } else {
    it.lo = 0;
    it.hi = row0 + kBM;
  }

  const uint16_t* qh = a.q + ((int64_t)h * n + row0 + 32 * w) * kD;
  const int nbytes = (int)(n * kRowBytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + (int64_t)kvh * n * kD), 0, nbytes, 0x00020000);
  const int row_off = (tid >> 4) * kRowBytes + (tid & 15) * 16;  // this thread's staging rows / chunk

  // Q fragments: B operand of S^T = K Q^T; lane holds row l32 of this wave's
  // 32 rows and d = 16t + 8g .. +8.
  bf16x8 qf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + l32 * kD + 16 * t + 8 * g));

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int row = row0 + 32 * w + l32;     // this lane's query row
  const float sl2 = a.scale_log2;
  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};

  Piece cur, nxt;
  Stage stg;
  it.start();
  const bool have0 = it.next(cur);
  if (have0) {
    load_piece(cur, col, kr, vr, row_off, tid, stg);
    store_piece(stg, cur.is_col, k_lds[0], v_lds[0], key_lds[0], tid);
  }
  // Settle every outstanding load (Q fragments, first piece) here, so the
  // wait for them is not placed at the top of the loop, where it would also
  // stall on the prefetch of the next piece in every iteration.
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(qf[t]));  // defined here, not by a load
  bool have_n = have0 && it.next(nxt);
  if (have_n) load_piece(nxt, col, kr, vr, row_off, tid, stg);
  __syncthreads();
  int buf = 0;
  if (have0) {
    do {
      const uint16_t* kt = k_lds[buf];
      const _Float16* vt = v_lds[buf];

      // S^T = K Q^T.  Lane: row l32, keys 8(r/4) + 4g + r%4.
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + l32 * kKS + 16 * t + 8 * g));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[t], s, 0, 0, 0);
      }

      // Masks (causal, piece tail, A-shape window); whether any is needed is
      // decided per piece, the mask itself per element without branches.
      const int* keys = key_lds[buf];
      const int kmin = cur.is_col ? keys[0] : cur.start;
      const int kmax = cur.is_col ? keys[cur.count - 1] : cur.start + cur.count - 1;
      const bool far = ashape && kmax >= sink && row0 + kBM - 1 - max(kmin, sink) >= window;
      if (cur.count < kKP || kmax > row0 || far) {
        int key[16];
        if (cur.is_col) {
#pragma unroll
          for (int r = 0; r < 16; ++r) key[r] = keys[8 * (r >> 2) + 4 * g + (r & 3)];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) key[r] = cur.start + 8 * (r >> 2) + 4 * g + (r & 3);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int slot = 8 * (r >> 2) + 4 * g + (r & 3);
          const bool ok = (slot < cur.count) & (key[r] <= row) &
                          !(ashape & (key[r] >= sink) & (row - key[r] >= window));
          s[r] = ok ? s[r] : -INFINITY;
        }
      }

      // Online softmax with a lazily updated max (log2 units).
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
      f16x8 pb[2];
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -msub));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], sl2, -msub));
        const f16x2 e = {(_Float16)e0, (_Float16)e1};
        sum = __builtin_amdgcn_fdot2(e, ones, sum, false);  // the row sum of the fp16 P fed to the MFMA
        pb[r >> 3][r & 7] = e[0];
        pb[r >> 3][(r & 7) + 1] = e[1];
      }
      l_run += sum;

      // O^T += V^T P^T.  A operand: lane holds d = 32dt + l32 and keys
      // 16kh + 8(e/4) + 4g + e%4; B operand: P^T from the S registers.
      const int s16 = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
      for (int kh2 = 0; kh2 < 2; ++kh2) {
        const int ra = 16 * kh2 + 4 * g + (s16 >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int ch = 32 * dt + 16 * dh + 4 * (s16 & 3);
          const f16x4 lo = lds_read_tr(vt + ra * kVS + ch);
          const f16x4 hi = lds_read_tr(vt + (ra + 8) * kVS + ch);
          const f16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kh2], o[dt], 0, 0, 0);
        }
      }
      const bool more = have_n;
      if (more) store_piece(stg, nxt.is_col, k_lds[buf ^ 1], v_lds[buf ^ 1], key_lds[buf ^ 1], tid);
      __syncthreads();
      cur = nxt;
      buf ^= 1;
      have_n = more && it.next(nxt);
      if (have_n) load_piece(nxt, col, kr, vr, row_off, tid, stg);
      if (!more) break;
    } while (true);
  }

  // Epilogue: out = O / l, lse = m ln2 + ln l.
  const float lt = sum_halves(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int64_t obase = ((int64_t)h * n + row) * kD;
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
    a.lse[(int64_t)h * n + row] = lt > 0.f ? m_run * 0.69314718055994530942f + logf(lt) : -INFINITY;
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
  const int64_t blocks = (int64_t)a.hq * a.nb;
  hipLaunchKernelGGL(sparse_attn_fwd, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
