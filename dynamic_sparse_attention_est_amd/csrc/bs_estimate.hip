// Online Block-Sparse estimation for gfx950 (MInference 1.0 summary, "Key
// points": for Block-Sparse heads, queries and keys are mean-pooled over
// 64-token blocks and the pooled blocks are scored against each other).
//
//   bs_pool   : mean of each 64-row block of Q (per BS head) or K (per KV head
//               read by a BS head), fp32, fixed summation order.  This is the
//               HBM-bound step: every Q/K byte of those heads is read once.
//   bs_scores : S[b][c] = Qpool[b] . Kpool[c] for c <= b (-inf above the
//               diagonal), a 64x64-tiled fp32 product with a fixed d order.
//               Rows are the call's query blocks (local bl = b - q_block0);
//               columns every key block.
// Selection of the top key blocks per query block lives in topk.hip.
#include "internal.h"

namespace msa {
namespace {

struct PoolArgs {
  const uint16_t* src;   // [heads][n][128] bf16
  int64_t n;
  float* pooled;         // [nheads][n/64][128]
  int16_t head[kMaxHeads];
};

// Thread t: 8 dims (chunk t%16) of rows 4(t/16) .. +3 of the block; the 16
// row-group partials are then added in order.
__global__ __launch_bounds__(256) void bs_pool(PoolArgs a) {
  __shared__ float part[16][kD];
  const int b = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const int c16 = tid & 15, rg = tid >> 4;
  const uint16_t* base = a.src + ((int64_t)a.head[slot] * a.n + (int64_t)b * kBM + 4 * rg) * kD + 8 * c16;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(base + r * kD);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __builtin_bit_cast(float, x[e] << 16);
      acc[2 * e + 1] += __builtin_bit_cast(float, x[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * c16 + e] = acc[e];
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][tid];
    const int nb = (int)(a.n / kBM);
    a.pooled[((int64_t)slot * nb + b) * kD + tid] = s * (1.f / kBM);
  }
}

struct ScoreArgs {
  const float* qpool;    // [n_bs][nbq][128]
  const float* kpool;    // [n_kv][nb][128]
  float* scores;         // [n_bs][nbq][nb]
  int32_t nb, nbq, qb0;  // key blocks, query blocks of the call, first query block
  int16_t kv_slot[kMaxHeads];  // kpool slot of each BS slot
};

constexpr int kST = 64;      // score tile
constexpr int kTP = kST + 4; // LDS stride of a transposed tile (floats; rows stay 16-byte aligned)

// Tiles are held transposed in LDS ([d][block]), so a thread's four query
// blocks (or four key blocks) at one d are one 16-byte read: two reads per 16
// FMAs.  Each sum runs over d in order.
__global__ __launch_bounds__(256) void bs_scores(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[kD * kTP];
  __shared__ __attribute__((aligned(16))) float ks[kD * kTP];
  const int ct = blockIdx.x, bt = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const int nb = a.nb, nbq = a.nbq;
  const int tx = tid & 15, ty = tid >> 4;
  float* out = a.scores + (int64_t)slot * nbq * nb;
  const int b0 = bt * kST, c0 = ct * kST;  // first local query block, first key block
  if (c0 > a.qb0 + b0 + kST - 1) {  // strictly above the diagonal: no key block is allowed
    for (int i = tid; i < kST * kST; i += 256) {
      const int bl = b0 + i / kST, c = c0 + i % kST;
      if (bl < nbq && c < nb) out[(int64_t)bl * nb + c] = -INFINITY;
    }
    return;
  }
  const float* qp = a.qpool + (int64_t)slot * nbq * kD;
  const float* kp = a.kpool + (int64_t)a.kv_slot[slot] * nb * kD;
  for (int i = tid; i < kST * kD; i += 256) {
    const int r = i / kD, d = i % kD;
    qs[d * kTP + r] = b0 + r < nbq ? qp[(int64_t)(b0 + r) * kD + d] : 0.f;
    ks[d * kTP + r] = c0 + r < nb ? kp[(int64_t)(c0 + r) * kD + d] : 0.f;
  }
  __syncthreads();
  float acc[4][4] = {};
  for (int d = 0; d < kD; ++d) {
    const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[d * kTP + 4 * ty]);
    const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[d * kTP + 4 * tx]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(qv[i], kv[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bl = b0 + 4 * ty + i, c = c0 + 4 * tx + j;
      if (bl < nbq && c < nb) out[(int64_t)bl * nb + c] = c <= a.qb0 + bl ? acc[i][j] : -INFINITY;
    }
}

}  // namespace

hipError_t launch_bs_pool(const uint16_t* src, int64_t n, const int16_t* heads, int nheads, float* pooled,
                          hipStream_t s) {
  if (nheads <= 0) return hipSuccess;
  PoolArgs a;
  a.src = src;
  a.n = n;
  a.pooled = pooled;
  for (int i = 0; i < nheads; ++i) a.head[i] = heads[i];
  hipLaunchKernelGGL(bs_pool, dim3((unsigned)(n / kBM), (unsigned)nheads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bs_scores(const float* qpool, const float* kpool, int nb, int nbq, int qb0,
                            const int16_t* kv_slot_of_bs, int n_bs, float* scores, hipStream_t s) {
  if (n_bs <= 0) return hipSuccess;
  ScoreArgs a;
  a.qpool = qpool;
  a.kpool = kpool;
  a.scores = scores;
  a.nb = nb;
  a.nbq = nbq;
  a.qb0 = qb0;
  for (int i = 0; i < n_bs; ++i) a.kv_slot[i] = kv_slot_of_bs[i];
  const unsigned tc = (unsigned)((nb + kST - 1) / kST), tq = (unsigned)((nbq + kST - 1) / kST);
  hipLaunchKernelGGL(bs_scores, dim3(tc, tq, (unsigned)n_bs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
