// Online Vertical-Slash estimation for gfx950 (MInference 1.0 summary, "Key
// points": for Vertical-Slash heads the last query vectors are scored against
// every key; the MInference abstract: indices are built per prompt).
//
// For the last 64 rows i = n-64+r of each Vertical-Slash head, with logits
// z_ij = scale q_i.k_j (j <= i) and p_ij = softmax_j z_ij:
//   vertical score v_j = sum_r p_ij,   slash score s_o = sum_r p_{i,i-o}.
// Column sums need the final row normalisers, so K is streamed twice:
//   pass 1: per 256-key tile, partial row max and sum of exp  -> part_mz
//   stats : fixed-order merge of the tile partials             -> (M_i, Z_i)
//   pass 2: p = exp2(x - M)/Z into LDS; column sums (complete per tile) and
//           per-tile partial diagonal sums (256 + 63 diagonals) -> v, diag_part
//   diag  : each diagonal adds its (at most two) tile partials in tile order.
// One workgroup covers one 256-key tile of one KV head for every Vertical-
// Slash Q head that reads it, so each K tile is read once per pass.  Logits
// come from v_mfma_f32_32x32x16_bf16 (S^T = K Q^T, keys x rows); every
// reduction has a fixed order, so results are bitwise reproducible.
#include "internal.h"

namespace msa {
namespace {

constexpr int kT = kVsTile;      // 256 keys per workgroup, 64 per wave
constexpr int kPS = kT + 1;      // LDS row stride of the probability tile (floats)
constexpr int kDiagStride = 320; // stored diagonals per tile (319 used)

struct VsArgs {
  const uint16_t* q;  // [H_q][qm][128]: the call's query rows, which end at row n - 1
  const uint16_t* k;
  int64_t n;
  int64_t qm;
  int32_t ntiles;
  float sl2;          // scale * log2(e): logits are kept in log2 units
  float* part_mz;     // [n_vs][ntiles][64][2]
  float* stats;       // [n_vs][64][2]  (M, Z)
  float* diag_part;   // [n_vs][ntiles][320]
  float* v_scores;    // [n_vs][n]
  float* s_scores;    // [n_vs][n]
  VsGroups groups;
};

// Logit tile of one wave: keys j0 + 64w + 32kt + 8(r/4) + 4g + r%4 (kt = 0, 1)
// against rows 32rt + lane%32 (rt = 0, 1) of the last 64 rows, in log2 units,
// -inf where the key lies after the row.
__device__ __forceinline__ void logits(const bf16x8 (&kf)[2][8], const uint16_t* qlast, int64_t n, int j0w,
                                       int lane, float sl2, f32x16 (&x)[2][2]) {
  const int l32 = lane & 31, g = lane >> 5;
  bf16x8 qf[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qf[rt][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qlast + (32 * rt + l32) * kD + 16 * t + 8 * g));
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt][t], qf[rt][t], acc, 0, 0, 0);
      const int64_t row = n - kLastQ + 32 * rt + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = j0w + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
        x[kt][rt][r] = key <= row ? acc[r] * sl2 : -INFINITY;
      }
    }
}

// K fragments (A operand) of one wave: key j0w + 32kt + lane%32 (clamped
// inside the sequence; keys past n are masked as lying after every row),
// d = 16t + 8g .. +8.
__device__ __forceinline__ void load_k(const uint16_t* kb, int64_t n, int j0w, int lane, bf16x8 (&kf)[2][8]) {
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t key = min((int64_t)(j0w + 32 * kt + l32), n - 1);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      kf[kt][t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kb + key * kD + 16 * t + 8 * g));
  }
}

__global__ __launch_bounds__(256) void vs_pass1(VsArgs a) {
  __shared__ float red[4][kLastQ][2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int tile = blockIdx.x, gi = blockIdx.y;
  const int64_t n = a.n;
  const int j0w = tile * kT + 64 * w;
  bf16x8 kf[2][8];
  load_k(a.k + (int64_t)a.groups.kv_head[gi] * n * kD, n, j0w, lane, kf);

  for (int qi = a.groups.q_begin[gi]; qi < a.groups.q_begin[gi + 1]; ++qi) {
    const int h = a.groups.q_head[qi], slot = a.groups.q_slot[qi];
    f32x16 x[2][2];
    logits(kf, a.q + ((int64_t)h * a.qm + a.qm - kLastQ) * kD, n, j0w, lane, a.sl2, x);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, x[kt][rt][r]);
      m = fmaxf(m, __shfl_xor(m, 32));
      float z = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) z += exp2f(x[kt][rt][r] - m);
      }
      z += __shfl_xor(z, 32);
      if (g == 0) {
        red[w][32 * rt + l32][0] = m;
        red[w][32 * rt + l32][1] = z;
      }
    }
    __syncthreads();
    if (tid < kLastQ) {
      float m = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) m = fmaxf(m, red[ww][tid][0]);
      float z = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
        if (red[ww][tid][0] != -INFINITY) z += red[ww][tid][1] * exp2f(red[ww][tid][0] - m);
      float* dst = a.part_mz + (((int64_t)slot * a.ntiles + tile) * kLastQ + tid) * 2;
      dst[0] = m;
      dst[1] = z;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void vs_pass2(VsArgs a) {
  __shared__ float P[kLastQ * kPS];  // probabilities of the tile, [row][key]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int tile = blockIdx.x, gi = blockIdx.y;
  const int64_t n = a.n;
  const int j0 = tile * kT, j0w = j0 + 64 * w;
  bf16x8 kf[2][8];
  load_k(a.k + (int64_t)a.groups.kv_head[gi] * n * kD, n, j0w, lane, kf);

  for (int qi = a.groups.q_begin[gi]; qi < a.groups.q_begin[gi + 1]; ++qi) {
    const int h = a.groups.q_head[qi], slot = a.groups.q_slot[qi];
    f32x16 x[2][2];
    logits(kf, a.q + ((int64_t)h * a.qm + a.qm - kLastQ) * kD, n, j0w, lane, a.sl2, x);
    const float* st = a.stats + (int64_t)slot * kLastQ * 2;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int rr = 32 * rt + l32;
      const float M = st[rr * 2], invZ = 1.f / st[rr * 2 + 1];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = 64 * w + 32 * kt + 8 * (r >> 2) + 4 * g + (r & 3);
          P[rr * kPS + kl] = exp2f(x[kt][rt][r] - M) * invZ;
        }
    }
    __syncthreads();
    // Column sums: thread t owns key j0 + t (complete within the tile).
    if (j0 + tid < n) {
      float v = 0.f;
      for (int rr = 0; rr < kLastQ; ++rr) v += P[rr * kPS + tid];
      a.v_scores[(int64_t)slot * n + j0 + tid] = v;
    }
    // Partial diagonal sums: local diagonal od = rr - kl + 255 is the global
    // offset o = n - 319 - j0 + od.
    float* dp = a.diag_part + ((int64_t)slot * a.ntiles + tile) * kDiagStride;
    for (int od = tid; od < kT + kLastQ - 1; od += 256) {
      float s = 0.f;
      const int r_lo = max(0, od - (kT - 1)), r_hi = min(kLastQ - 1, od);
      for (int rr = r_lo; rr <= r_hi; ++rr) s += P[rr * kPS + rr + kT - 1 - od];
      dp[od] = s;
    }
    __syncthreads();
  }
}

// Row statistics of the last 64 rows: merge the per-tile partials (m_t, z_t),
// m in log2 units, into M = max m_t and Z = sum z_t 2^(m_t - M).  One
// workgroup per (row, head); thread t merges tiles t, t+256, ... online, then
// the 256 partials are merged pairwise in a fixed tree order.
__device__ __forceinline__ void merge_mz(float& m, float& z, float m2, float z2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  z = (m == -INFINITY ? 0.f : z * exp2f(m - mn)) + (m2 == -INFINITY ? 0.f : z2 * exp2f(m2 - mn));
  m = mn;
}

__global__ __launch_bounds__(256) void vs_stats(const float* part_mz, float* stats, int ntiles) {
  __shared__ float sm[256], sz[256];
  const int rr = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const float* p = part_mz + (int64_t)slot * ntiles * kLastQ * 2 + rr * 2;
  float m = -INFINITY, z = 0.f;
  for (int t = tid; t < ntiles; t += 256) merge_mz(m, z, p[(int64_t)t * kLastQ * 2], p[(int64_t)t * kLastQ * 2 + 1]);
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

__global__ __launch_bounds__(256) void vs_diag(const float* diag_part, float* s_scores, int64_t n, int ntiles) {
  const int slot = blockIdx.y;
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= n) return;
  // Tile t holds offsets [n - 319 - 256t, n - 1 - 256t].
  const int64_t span = kT + kLastQ - 1;
  int64_t t_hi = (n - 1 - o) / kT;
  if (t_hi > ntiles - 1) t_hi = ntiles - 1;
  const int64_t num = n - span - o;  // t >= num / 256, rounded up
  int64_t t_lo = num <= 0 ? 0 : (num + kT - 1) / kT;
  float s = 0.f;
  for (int64_t t = t_lo; t <= t_hi; ++t) {
    const int64_t od = o - (n - span - (int64_t)kT * t);
    s += diag_part[((int64_t)slot * ntiles + t) * kDiagStride + od];
  }
  s_scores[(int64_t)slot * n + o] = s;
}

}  // namespace

hipError_t launch_vs_estimate(const uint16_t* q, const uint16_t* k, int64_t n, int64_t qm, float scale_log2,
                              const VsGroups& groups, int n_vs, float* part_mz, float* stats, float* diag_part,
                              float* v_scores, float* s_scores, hipStream_t s) {
  VsArgs a;
  a.q = q;
  a.k = k;
  a.n = n;
  a.qm = qm;
  a.ntiles = (int)((n + kT - 1) / kT);
  a.sl2 = scale_log2;
  a.part_mz = part_mz;
  a.stats = stats;
  a.diag_part = diag_part;
  a.v_scores = v_scores;
  a.s_scores = s_scores;
  a.groups = groups;
  const dim3 grid((unsigned)a.ntiles, (unsigned)groups.n_groups);
  hipLaunchKernelGGL(vs_pass1, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vs_stats, dim3((unsigned)kLastQ, (unsigned)n_vs), dim3(256), 0, s, part_mz, stats, a.ntiles);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_pass2, grid, dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_diag, dim3((unsigned)((n + 255) / 256), (unsigned)n_vs), dim3(256), 0, s, diag_part,
                     s_scores, n, a.ntiles);
  return hipGetLastError();
}

}  // namespace msa
