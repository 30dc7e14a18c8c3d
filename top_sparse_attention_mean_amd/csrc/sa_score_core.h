// sa_score_core.h -- block scores of one (b, kv head).
//
// The score of block j is the group-mean query (scale folded in) against the
// block's mean-key sketch row: the head-averaged importance of the attention-
// mass oracle ("How Much Dense Attention is Necessary?", technical summary
// §2.1) applied per page as Quest does ("The Sparse Frontier", Contributi §2).
// The pieces of the scoring kernel: the sketch-row pass and the rebuild of one
// block's sketch from K.
//
// Lane layout of a sketch-row pass: LPR = D/4 lanes per row, lane lc holds
// query columns 4*lc .. 4*lc+3 and multiplies one 16-byte row segment; the
// row's sum lands in lane lc = LPR-1 of its group.
#pragma once

#include <type_traits>

#include "sa_device.h"

namespace sa {

template <typename T>
using QCol = typename std::conditional<sizeof(T) == 2, u32x2, u32x4>::type;

// Query loads of columns 4*lc.. of the group's heads 0..7 (clamped to G-1, so
// none sits behind a branch).
template <typename T, int D>
__device__ __forceinline__ void score_q_issue(const T* Qg, int G, int lc, QCol<T> (&qv)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const T* qp = Qg + size_t(min(u, G - 1)) * D + lc * 4;
    if constexpr (sizeof(T) == 2) qv[u] = ld8(qp);
    else qv[u] = ld16(qp);
  }
}

// The scaled group mean of those columns (heads past 8 are loaded here).
template <typename T, int D>
__device__ __forceinline__ void score_q_finish(const T* Qg, int G, int lc, float scale,
                                               const QCol<T> (&qv)[8], float (&q)[4]) {
  q[0] = q[1] = q[2] = q[3] = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if constexpr (sizeof(T) == 2) {
      q[0] += u < G ? bf16lo(qv[u][0]) : 0.f; q[1] += u < G ? bf16hi(qv[u][0]) : 0.f;
      q[2] += u < G ? bf16lo(qv[u][1]) : 0.f; q[3] += u < G ? bf16hi(qv[u][1]) : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] += u < G ? __uint_as_float(qv[u][e]) : 0.f;
    }
  }
  for (int h = 8; h < G; ++h) {
    const T* qp = Qg + size_t(h) * D + lc * 4;
    if constexpr (sizeof(T) == 2) {
      const u32x2 v = ld8(qp);
      q[0] += bf16lo(v[0]); q[1] += bf16hi(v[0]); q[2] += bf16lo(v[1]); q[3] += bf16hi(v[1]);
    } else {
      const u32x4 v = ld16(qp);
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] += __uint_as_float(v[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) q[e] = (q[e] / float(G)) * scale;
}

// One row segment's share of the dot product, summed over the row's lanes.
template <int D>
__device__ __forceinline__ float score_row(const float (&q)[4], u32x4 w) {
  const float p = q[0] * __uint_as_float(w[0]) + q[1] * __uint_as_float(w[1]) +
                  q[2] * __uint_as_float(w[2]) + q[3] * __uint_as_float(w[3]);
  return group_sum_to_last<D / 4>(p);
}

// LDS of the block rebuild.
template <int D>
struct ScoreUpdLds {
  float qbar[D];
  float red[256 / (D / 8)][D + 4];
};

// Rebuild the sketch row of one block from its nj <= block K rows (Kb: the
// block's first row, [nj, D]) -- the mean over the block's tokens -- store it
// to sk_row and return its score in thread 0.  The query loads and every K row
// load are in flight together.  All 256 threads call; ends after a barrier.
template <typename T, int D>
__device__ float score_update_block(const T* Kb, int nj, const T* Qg, int G, float scale,
                                    float* sk_row, ScoreUpdLds<D>& L) {
  constexpr int CPT = 8, TPR = D / CPT, RPP = 256 / TPR;
  constexpr bool BF = sizeof(T) == 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tr = tid / TPR, tc = tid % TPR;
  float acc[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) acc[q] = 0.f;
  const T* Kp = Kb + tc * CPT;
  constexpr int NV = BF ? 1 : 2;               // 16-byte loads per row segment
  constexpr int KB = BF ? 8 : 4;               // rows per thread in flight
  auto k_batch = [&](int r0, bool with_q, T (&qs)[8]) {
    u32x4 kv[KB][NV];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int r = min(r0 + u * RPP, nj - 1);
#pragma unroll
      for (int v = 0; v < NV; ++v) kv[u][v] = ld16(Kp + size_t(r) * D + 4 * v);
    }
    if (with_q) {
      const int qd = tid < D ? tid : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) qs[u] = Qg[size_t(min(u, G - 1)) * D + qd];
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (r0 + u * RPP < nj) {
        if constexpr (BF) {
#pragma unroll
          for (int q = 0; q < 4; ++q) { acc[2 * q] += bf16lo(kv[u][0][q]); acc[2 * q + 1] += bf16hi(kv[u][0][q]); }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) { acc[q] += __uint_as_float(kv[u][0][q]); acc[4 + q] += __uint_as_float(kv[u][1][q]); }
        }
      }
    }
  };
  T qs[8];
  k_batch(tr, true, qs);                       // with the query loads
  // blocks longer than KB * RPP rows take further batches
  for (int r0 = tr + KB * RPP; r0 < nj; r0 += KB * RPP) k_batch(r0, false, qs);
  if (tid < D) {
    float sq = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float v;
      if constexpr (BF) v = bf16_to_f32(qs[u]);
      else v = qs[u];
      sq += u < G ? v : 0.f;
    }
    for (int h = 8; h < G; ++h) {
      if constexpr (BF) sq += bf16_to_f32(Qg[size_t(h) * D + tid]);
      else sq += Qg[size_t(h) * D + tid];
    }
    L.qbar[tid] = (sq / float(G)) * scale;
  }
#pragma unroll
  for (int q = 0; q < CPT; ++q) L.red[tr][tc * CPT + q] = acc[q];
  __syncthreads();
  float part = 0.f;
  if (tid < D) {
    float sum = 0.f;
    for (int g = 0; g < RPP; ++g) sum += L.red[g][tid];
    const float v = sum / float(nj);
    sk_row[tid] = v;
    part = v * L.qbar[tid];
  }
  part = wave_sum(part);
  __syncthreads();
  if (lane == 0) L.red[0][wave] = part;
  __syncthreads();
  float p = 0.f;
  if (tid == 0) {
    for (int ww = 0; ww < D / 64; ++ww) p += L.red[0][ww];
  }
  __syncthreads();
  return p;
}

}  // namespace sa
