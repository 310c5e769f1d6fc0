// Online Vertical-Slash estimation for gfx950 (MInference 1.0 summary, "Key
// points": for Vertical-Slash heads the last query vectors are scored against
// every key; the MInference abstract: indices are built per prompt).
//
// For the last 64 rows i = n-64+r of each Vertical-Slash head, with logits
// z_ij = scale q_i.k_j (j <= i) and p_ij = softmax_j z_ij:
//   vertical score v_j = sum_r p_ij,   slash score s_o = sum_r p_{i,i-o}.
// Column sums need the final row normalisers, so K is streamed twice:
//   vs_rows  : per chunk of keys, each row's running max and sum of exp -> part_mz
//   vs_stats : fixed-order merge of the chunk partials               -> (M_i, Z_i)
//   vs_scores: p = 2^(x - M) / Z; column sums (complete per 64-key tile) and
//              diagonal sums (complete except at chunk edges)          -> v, s
//   vs_diag  : the 64 diagonals at each chunk edge add their two halves.
//
// Both passes have one shape.  A workgroup takes one KV head and up to four of
// its Vertical-Slash Q heads, one per wavefront, over a chunk of consecutive
// 64-key tiles.  Each wave keeps its head's 64 query rows in registers for the
// whole chunk (MFMA fragments); the K tiles stream through a ring of four LDS
// stages, filled by buffer loads that go straight to LDS three tiles ahead of
// the one being scored, and every K tile is read from memory once for all the
// heads of the workgroup.  Logits come from v_mfma_f32_32x32x16_bf16.
//
// Row statistics take the logits transposed (keys x rows, one row per lane):
// each lane keeps a running max and sum for its row over its half of the keys.
// The scores pass takes them rows x keys (one key per lane), so a column sum
// is a sum within the lane plus one exchange between the two half-waves.  A
// diagonal runs across lanes: for register r, lane D of each half-wave fetches
// (ds_bpermute) the element of its own diagonal class D = (row - key) mod 32,
// and adds it to one of four accumulators by the sign and 32-block of
// row - key; a tile's negative diagonals are completed by the next tile.
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include <algorithm>
#include <utility>

#include "internal.h"

namespace msa {
namespace {

constexpr int kET = 64;                   // keys per tile
constexpr int kRowB = kD * 2;             // one K row (bytes)
constexpr int kTileB = kET * kRowB;       // one K tile (16 KiB)
constexpr int kES = 4;                    // ring stages
constexpr int kLoads = kTileB / 1024 / 4; // load-to-LDS instructions per wave per tile

typedef __attribute__((address_space(3))) void lds_void;

__shared__ __attribute__((aligned(1024))) char e_stage0[kTileB];
__shared__ __attribute__((aligned(1024))) char e_stage1[kTileB];
__shared__ __attribute__((aligned(1024))) char e_stage2[kTileB];
__shared__ __attribute__((aligned(1024))) char e_stage3[kTileB];
__shared__ __attribute__((aligned(16))) float e_rows[4][2][kLastQ];

template <int I>
__device__ __forceinline__ char* est_stage() {
  static_assert(I >= 0 && I < kES, "stage");
  if constexpr (I == 0) return e_stage0;
  if constexpr (I == 1) return e_stage1;
  if constexpr (I == 2) return e_stage2;
  if constexpr (I == 3) return e_stage3;
}

// Chunk slot of 16-byte chunk c of tile row r is c ^ swz(r) (16 distinct
// values over 16 consecutive rows), so the K fragment reads are free of bank
// conflicts.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// s_waitcnt vmcnt(N) lgkmcnt(0), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for the ring's loads in flight); the empty asm statements keep memory
// accesses on their side.
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

struct VsArgs {
  const uint16_t* q;  // [H_q][qm][128]: the call's query rows, which end at row n - 1
  const uint16_t* k;
  int64_t n;
  int64_t qm;
  int32_t ntiles;      // n / 64
  int32_t chunk_tiles; // tiles per workgroup
  int32_t nchunks;
  float sl2;           // scale * log2(e): logits are kept in log2 units
  float* part_mz;      // [n_vs][nchunks][64][2]
  float* stats;        // [n_vs][64][2]  (M, Z)
  float* diag_part;    // [n_vs][nchunks][128]: first tile's diagonals 0..63, last tile's carry
  float* v_scores;     // [n_vs][n]
  float* s_scores;     // [n_vs][n]
  VsGroups groups;
};

// Element r of a 32x32 product tile sits in lane half g at position
// 8(r/4) + 4g + r%4 along the tile's first axis.
__device__ __forceinline__ constexpr int pos5(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <bool kScores>
__device__ __forceinline__ void est_body(const VsArgs& a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int chunk = blockIdx.x, gi = blockIdx.y;
  const int q0 = a.groups.q_begin[gi];
  const bool active = w < a.groups.q_begin[gi + 1] - q0;
  const int h = active ? a.groups.q_head[q0 + w] : a.groups.q_head[q0];
  const int slot = active ? a.groups.q_slot[q0 + w] : 0;
  const int64_t n = a.n;
  const int t0 = chunk * a.chunk_tiles;
  const int t1 = min(a.ntiles, t0 + a.chunk_tiles);
  const int last_tile = a.ntiles - 1;  // the only tile with keys after some of the 64 rows

  const int nbytes = (int)((uint32_t)n * (uint32_t)kRowB);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + (int64_t)a.groups.kv_head[gi] * n * kD), 0, nbytes, 0x00020000);
  // Load d of this wave fills tile rows 16w + 4d + lane/16; the lane writes
  // slot lane%16 and fetches chunk (lane%16) ^ swz(row).
  uint32_t lofs[kLoads];
#pragma unroll
  for (int d = 0; d < kLoads; ++d) {
    const int row = 16 * w + 4 * d + (lane >> 4);
    lofs[d] = (uint32_t)row * kRowB + 16u * (uint32_t)((lane & 15) ^ swz(row));
  }
  // Tiles past the chunk read out of range (zeros, no memory traffic).
  auto issue = [&](char* st, int tile) {
    const uint32_t base = tile < t1 ? (uint32_t)tile * kTileB : (uint32_t)nbytes;
#pragma unroll
    for (int d = 0; d < kLoads; ++d)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(st + 1024 * (kLoads * w + d)), 16, base + lofs[d], 0,
                                               0, 0);
  };
  // K fragment t of key half kt: key 32kt + l32, d = 16t + 8g .. +8.
  auto kfrag = [&](const char* st, int kt, int t) {
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(st + kt * (32 * kRowB) + l32 * kRowB + 16 * ((2 * t + g) ^ swz(l32))));
  };

  // Query fragments of rows 32rt + l32 of the last 64, d = 16t + 8g .. +8.
  bf16x8 qf[2][8];
  if (active) {
    const uint16_t* qh = a.q + ((int64_t)h * a.qm + a.qm - kLastQ) * kD;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        qf[rt][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qh + (32 * rt + l32) * kD + 16 * t + 8 * g));
  }

  // Scores pass: the head's row maxima and 1 / row sums, row = lane, kept in
  // LDS (e_rows[w][0][row], e_rows[w][1][row]) and read four rows at a time.
  float stat_m = 0.f, stat_z = 1.f;
  if constexpr (kScores) {
    if (active) {
      const float* st = a.stats + ((int64_t)slot * kLastQ + lane) * 2;
      stat_m = st[0];
      stat_z = st[1];
    }
  }

  auto prologue = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    issue(est_stage<ST>(), t0 + ST);
    return true;
  };
  run_steps<0, kES - 1>(prologue);
  // The query fragments and statistics, loaded before the ring, have landed
  // once only the ring's loads are in flight; from here on they count as
  // defined by these statements, so no later use waits for memory.
  wait_vm<(kES - 1) * kLoads>();
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(qf[rt][t]));
  if constexpr (kScores) {
    asm volatile("" : "+v"(stat_m), "+v"(stat_z));
    e_rows[w][0][lane] = stat_m;
    e_rows[w][1][lane] = 1.f / stat_z;
  }

  // Row statistics state: lane's row 32rt + l32, over its half of the keys.
  float m_run[2] = {-INFINITY, -INFINITY}, z_run[2] = {0.f, 0.f};
  // Scores state: diagonal carry into the next tile (diagonals D and D + 32).
  float carry0 = 0.f, carry1 = 0.f;
  // bpermute source of register r: lane (pos5(r, g) - D) mod 32 of this half.
  const int D = l32;

  int tau = t0;
  auto step = [&](auto st_c) -> bool {
    constexpr int ST = decltype(st_c)::value;
    if (tau >= t1) return false;
    // Tile tau has landed once at most the later ops of this wave are in
    // flight: the loads of the kES-2 tiles after it and, in the scores pass,
    // two stores per tile scored since tile tau's loads were issued (gfx9
    // counts a wave's vector loads and stores in one counter that drains in
    // issue order).
    if (!(kScores && active)) {
      wait_vm<(kES - 2) * kLoads>();
    } else {
      const int k = tau - t0;
      if (k == 0)
        wait_vm<(kES - 2) * kLoads>();
      else if (k == 1)
        wait_vm<(kES - 2) * kLoads + 2>();
      else if (k == 2)
        wait_vm<(kES - 2) * kLoads + 4>();
      else
        wait_vm<(kES - 2) * kLoads + 6>();
    }
    barrier_only();
    issue(est_stage<(ST + kES - 1) % kES>(), tau + kES - 1);
    const char* st = est_stage<ST>();
    // The sequence's last tile is the only one with keys after some of the
    // rows; the statistics pass takes a copy of its code for it.
    const bool last_tile_now = tau == last_tile;
    auto score_tile = [&](auto last_c) {
      constexpr bool last = decltype(last_c)::value;
      if constexpr (!kScores && !last) {
        // Four products per tile, (key half kt, row half rt) = (g / 2, g % 2);
        // the statistics of product g-1 (max, then the exponentials and their
        // sum in element order) are interleaved with the MFMAs of product g.
        bf16x8 kf[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) kf[t] = kfrag(st, 0, t);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[0][t], acc, 0, 0, 0);
        auto stats_of = [&](const f32x16& p, int prt, auto with_mfma) {
          float mx = p[0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, p[r]);
          const float mn = fmaxf(m_run[prt], mx * a.sl2);  // finite: no key is masked in this tile
          const float alpha = m_run[prt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[prt] - mn);
          float sum = 0.f;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            with_mfma(t);
            sum += __builtin_amdgcn_exp2f(fmaf(p[2 * t], a.sl2, -mn));
            sum += __builtin_amdgcn_exp2f(fmaf(p[2 * t + 1], a.sl2, -mn));
            __builtin_amdgcn_sched_barrier(0);
          }
          z_run[prt] = fmaf(z_run[prt], alpha, sum);
          m_run[prt] = mn;
        };
#pragma unroll
        for (int gp = 1; gp < 4; ++gp) {
          const int rt = gp & 1;
          if (gp == 2) {
#pragma unroll
            for (int t = 0; t < 8; ++t) kf[t] = kfrag(st, 1, t);
          }
          f32x16 nxt = f32x16{};
          stats_of(acc, (gp - 1) & 1, [&](int t) {
            nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[rt][t], nxt, 0, 0, 0);
          });
          acc = nxt;
        }
        stats_of(acc, 1, [&](int) {});
      } else if constexpr (!kScores) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          bf16x8 kf[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) kf[t] = kfrag(st, kt, t);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            f32x16 acc = f32x16{};
#pragma unroll
            for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[rt][t], acc, 0, 0, 0);
            // acc[r]: key 32kt + pos5(r, g) of the tile, row 32rt + l32.
            if constexpr (last) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (32 * kt + pos5(r, g) > 32 * rt + l32) acc[r] = -INFINITY;
            }
            float mx = acc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
            const float mn = fmaxf(m_run[rt], mx * a.sl2);
            if (mn != -INFINITY) {
              const float alpha = m_run[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[rt] - mn);
              float s = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(fmaf(acc[r], a.sl2, -mn));
              z_run[rt] = fmaf(z_run[rt], alpha, s);
              m_run[rt] = mn;
            }
          }
        }
      } else {
        // Diagonal accumulators by 32-block of row - key: -2, -1, 0, 1.
        float bm2 = 0.f, bm1 = 0.f, b0 = 0.f, b1 = 0.f;
        float cs[2] = {0.f, 0.f};
        // Probabilities by (rt, kt): row - key = 32(rt - kt) + pos5 - l32, so
        // the streams A = (0,0) + (1,1), B = (1,0) and C = (0,1) lie in
        // 32-blocks {0,-1}, {1,0} and {-1,-2} of row - key.
        float pa[16], pb[16], pc[16];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          bf16x8 kf[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) kf[t] = kfrag(st, kt, t);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            f32x16 acc = f32x16{};
#pragma unroll
            for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rt][t], kf[t], acc, 0, 0, 0);
            // acc[r]: row 32rt + pos5(r, g), key 32kt + l32 of the tile.
            float p[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4 mq = *reinterpret_cast<const f32x4*>(&e_rows[w][0][32 * rt + pos5(4 * q4, g)]);
              const f32x4 zq = *reinterpret_cast<const f32x4*>(&e_rows[w][1][32 * rt + pos5(4 * q4, g)]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * q4 + e;
                p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], a.sl2, -mq[e])) * zq[e];
              }
            }
            if (last_tile_now) {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (32 * kt + l32 > 32 * rt + pos5(r, g)) p[r] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              cs[kt] += p[r];
              if (rt == 0 && kt == 0) pa[r] = p[r];
              if (rt == 1 && kt == 0) pb[r] = p[r];
              if (rt == 0 && kt == 1) pc[r] = p[r];
              if (rt == 1 && kt == 1) pa[r] += p[r];
            }
            // keep the four products apart (registers)
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // Register r: lane D of each half fetches the elements of diagonal
        // class D; where D exceeds the register's row position they lie one
        // 32-block lower.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int src = (((pos5(r, g) - D) & 31) | (g << 5)) << 2;
          const float va = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, pa[r])));
          const float vb = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, pb[r])));
          const float vc = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, pc[r])));
          const bool below = D > pos5(r, g);
          b0 += below ? vb : va;
          bm1 += below ? va : vc;
          b1 += below ? 0.f : vb;
          bm2 += below ? vc : 0.f;
        }
        // Half-waves hold the same diagonals for different rows: add them.
        const float t0s = b0 + __shfl_xor(b0, 32), t1s = b1 + __shfl_xor(b1, 32);
        const float tm2 = bm2 + __shfl_xor(bm2, 32), tm1 = bm1 + __shfl_xor(bm1, 32);
        // Diagonals dl = D (half 0) and D + 32 (half 1), dl = row - key,
        // offset o = n - 64 - 64 tau + dl; the previous tile's carry completes
        // them unless this is the chunk's first tile.
        const float out = g ? t1s + carry1 : t0s + carry0;
        const int64_t o = n - kLastQ - (int64_t)kET * tau + 32 * g + D;
        if (tau == t0)
          a.diag_part[((int64_t)slot * a.nchunks + chunk) * 128 + 32 * g + D] = out;
        else
          a.s_scores[(int64_t)slot * n + o] = out;
        carry0 = tm2;
        carry1 = tm1;
        // Column sums: half g writes keys 32g + l32 of the tile.
        const float c0 = cs[0] + __shfl_xor(cs[0], 32), c1 = cs[1] + __shfl_xor(cs[1], 32);
        a.v_scores[(int64_t)slot * n + (int64_t)kET * tau + 32 * g + l32] = g ? c1 : c0;
      }
    };
    if (active) {
      if constexpr (kScores) {
        score_tile(std::false_type{});
      } else {
        if (last_tile_now)
          score_tile(std::true_type{});
        else
          score_tile(std::false_type{});
      }
    }
    ++tau;
    return true;
  };
  while (run_steps<0, kES>(step)) {
  }
  wait_vm<0>();

  if (!active) return;
  if constexpr (!kScores) {
    // Merge the two half-waves' statistics of each row; half g writes row
    // 32g + l32.
    float mo[2], zo[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float m2 = __shfl_xor(m_run[rt], 32), z2 = __shfl_xor(z_run[rt], 32);
      const float mn = fmaxf(m_run[rt], m2);
      float z = 0.f;
      if (mn != -INFINITY) {
        const float za = m_run[rt] == -INFINITY ? 0.f : z_run[rt] * exp2f(m_run[rt] - mn);
        const float zb = m2 == -INFINITY ? 0.f : z2 * exp2f(m2 - mn);
        z = g ? zb + za : za + zb;  // the same order in both halves
      }
      mo[rt] = mn;
      zo[rt] = z;
    }
    float* dst = a.part_mz + (((int64_t)slot * a.nchunks + chunk) * kLastQ + 32 * g + l32) * 2;
    dst[0] = g ? mo[1] : mo[0];
    dst[1] = g ? zo[1] : zo[0];
  } else {
    // The last tile's negative diagonals: the next chunk's first tile
    // completes them (nothing follows the sequence's last tile).
    a.diag_part[((int64_t)slot * a.nchunks + chunk) * 128 + 64 + 32 * g + D] = g ? carry1 : carry0;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void vs_rows(VsArgs a) { est_body<false>(a); }
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void vs_scores(VsArgs a) { est_body<true>(a); }

// Row statistics of the last 64 rows: merge the per-chunk partials (m_c, z_c),
// m in log2 units, into M = max m_c and Z = sum z_c 2^(m_c - M).  One
// workgroup per (row, head); thread t merges chunks t, t+256, ... online, then
// the 256 partials are merged pairwise in a fixed tree order.
__device__ __forceinline__ void merge_mz(float& m, float& z, float m2, float z2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  z = (m == -INFINITY ? 0.f : z * exp2f(m - mn)) + (m2 == -INFINITY ? 0.f : z2 * exp2f(m2 - mn));
  m = mn;
}

__global__ __launch_bounds__(256) void vs_stats(const float* part_mz, float* stats, int nchunks) {
  __shared__ float sm[256], sz[256];
  const int rr = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const float* p = part_mz + (int64_t)slot * nchunks * kLastQ * 2 + rr * 2;
  float m = -INFINITY, z = 0.f;
  for (int t = tid; t < nchunks; t += 256) merge_mz(m, z, p[(int64_t)t * kLastQ * 2], p[(int64_t)t * kLastQ * 2 + 1]);
  sm[tid] = m;
  sz[tid] = z;
  __syncthreads();
  for (int half = 128; half > 0; half >>= 1) {
    if (tid < half) {
      float m1 = sm[tid], z1 = sz[tid];
      merge_mz(m1, z1, sm[tid + half], sz[tid + half]);
      sm[tid] = m1;
      sz[tid] = z1;
    }
    __syncthreads();
  }
  if (tid == 0) {
    stats[((int64_t)slot * kLastQ + rr) * 2] = sm[0];
    stats[((int64_t)slot * kLastQ + rr) * 2 + 1] = sz[0];
  }
}

// The 64 diagonals at the start of each chunk: the chunk's first tile holds
// one part, the previous chunk's last tile the other.
__global__ __launch_bounds__(64) void vs_diag(const float* diag_part, float* s_scores, int64_t n, int chunk_tiles,
                                              int nchunks) {
  const int c = blockIdx.x, slot = blockIdx.y, dl = threadIdx.x;
  const float* dp = diag_part + (int64_t)slot * nchunks * 128;
  const float head = dp[(int64_t)c * 128 + dl];
  const float s = c > 0 ? head + dp[(int64_t)(c - 1) * 128 + 64 + dl] : head;
  s_scores[(int64_t)slot * n + n - kLastQ - (int64_t)kET * c * chunk_tiles + dl] = s;
}

}  // namespace

int vs_chunk_tiles(int64_t n, int n_groups) {
  const int64_t ntiles = n / kET;
  // About 1024 workgroups (two per CU twice over); short sequences get one
  // tile per workgroup.
  const int64_t want = (ntiles * n_groups + 1023) / 1024;
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, ntiles));
}

hipError_t launch_vs_estimate(const uint16_t* q, const uint16_t* k, int64_t n, int64_t qm, float scale_log2,
                              const VsGroups& groups, int n_vs, int chunk_tiles, float* part_mz, float* stats,
                              float* diag_part, float* v_scores, float* s_scores, hipStream_t s) {
  VsArgs a;
  a.q = q;
  a.k = k;
  a.n = n;
  a.qm = qm;
  a.ntiles = (int)(n / kET);
  a.chunk_tiles = chunk_tiles;
  a.nchunks = (a.ntiles + chunk_tiles - 1) / chunk_tiles;
  a.sl2 = scale_log2;
  a.part_mz = part_mz;
  a.stats = stats;
  a.diag_part = diag_part;
  a.v_scores = v_scores;
  a.s_scores = s_scores;
  a.groups = groups;
  const dim3 grid((unsigned)a.nchunks, (unsigned)groups.n_groups);
  hipLaunchKernelGGL(vs_rows, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vs_stats, dim3((unsigned)kLastQ, (unsigned)n_vs), dim3(256), 0, s, part_mz, stats, a.nchunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_scores, grid, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_diag, dim3((unsigned)a.nchunks, (unsigned)n_vs), dim3(64), 0, s, diag_part, s_scores, n,
                     chunk_tiles, a.nchunks);
  return hipGetLastError();
}

}  // namespace msa
