// k_select.hip -- block scoring and deterministic top-k block selection.
//
// Scoring averages the query heads of a KV group, as the head-averaged token
// importance of the attention-mass oracle does ("How Much Dense Attention is
// Necessary?", technical summary §2.1), and scores every block's mean sketch
// with it (per-page selection over the retained cache, Quest, as described in
// "The Sparse Frontier", Contributi §2).  Selection keeps the forced sink block
// ("Pulsar Attention", Fase 1: fixed attention-sink prefix) and the local block
// ("Faster Than Flash", Metodologia §2: sink and local tokens dominate), then
// the best remaining scores with ties to the lower block index.
//
// Kernels
//   k_score         HBM-bound scan of the float32 sketch: one 256-thread
//                   workgroup per (b, kv head, 64 sketch rows); each wave issues
//                   all of its row loads before the group's mean query (scale
//                   folded in) is formed; every row dot product is reduced
//                   across 32 (D=128) or 16 (D=64) lanes with DPP row shifts.
//                   Workgroup id % (B*Hkv) picks the (b, kv head), so with
//                   B*Hkv a multiple of 8 every (b, kv head) stays on one
//                   XCD.  Optional extra
//                   workgroups rebuild one block's sketch from K and score it.
//   k_select_rows   one 256-thread workgroup per (b, kv head): the row's
//                   scores become order-preserving keys in LDS and the exact
//                   top-k is taken by the radix core of sa_select_core.h.  (The
//                   fused decode step runs the same core inside the decode
//                   kernel instead.)
//   k_prefill_select one 256-thread workgroup per (b, kv head, query block i):
//                   scores pooled query block i against key blocks [1, i-1]
//                   and selects with the same core (no cross-workgroup
//                   dependency, so scoring and selection fuse).
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"
#include "sa_score_core.h"
#include "sa_select_core.h"

namespace sa {

// ---------------------------------------------------------------- decode scoring
struct ScoreArgs {
  const void* Q;
  float* sk;
  const void* K;
  int N, block, upd;
  int BH, Hq, Hkv, G, nb, C;
  float scale;
  float* scores;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a) {
  constexpr int LPR = D / 4, RPI = 64 / LPR;
  __shared__ ScoreUpdLds<D> L;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the newest-block workgroups come first, so their K loads are not queued
  // behind the sketch stream (they would finish last otherwise)
  const int nupd = a.upd >= 0 ? a.BH : 0;
  const bool is_upd = int(blockIdx.x) < nupd;
  const int wid = int(blockIdx.x) - nupd;
  const int bh = is_upd ? int(blockIdx.x) : wid % a.BH;
  const int c = is_upd ? 0 : wid / a.BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int nb = a.nb, G = a.G;
  const T* Qg = static_cast<const T*>(a.Q) + (size_t(b) * a.Hq + kh * G) * D;
  float* srow = a.scores + size_t(bh) * nb;

  if (!is_upd) {
    // Each lane forms the 4 group-mean query columns it multiplies itself.  Its
    // query loads go out first and the sketch rows right after, so waiting for
    // the query does not wait for the rows, and each row's dot product starts
    // when that row arrives: no LDS and no barrier on this path.
    constexpr int RPWV = kScoreRows / 4;        // rows per wave
    constexpr int NLD = RPWV / RPI;             // 16-byte row loads per lane
    const int sub = lane / LPR, lc = lane % LPR;
    const int rw = c * kScoreRows + wave * RPWV;
    QCol<T> qv[8];
    score_q_issue<T, D>(Qg, G, lc, qv);
    __builtin_amdgcn_sched_barrier(0);          // keep the query loads ahead of the rows
    u32x4 w[NLD];
    const float* base = a.sk + size_t(bh) * nb * D;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = min(rw + i * RPI + sub, nb - 1);
      w[i] = ld16(base + size_t(r) * D + lc * 4);
    }
    __builtin_amdgcn_sched_barrier(0);          // every load issued before the first wait
    float q[4];
    score_q_finish<T, D>(Qg, G, lc, a.scale, qv, q);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = rw + i * RPI + sub;
      const float p = score_row<D>(q, w[i]);
      if (r < nb && r != a.upd && lc == LPR - 1) srow[r] = p;
    }
    return;
  }
  // rebuild the sketch of block upd from K, then score it
  const int t0 = a.upd * a.block, nj = min(a.block, a.N - t0);
  const float p = score_update_block<T, D>(static_cast<const T*>(a.K) + (size_t(bh) * a.N + t0) * D,
                                           nj, Qg, G, a.scale, a.sk + (size_t(bh) * nb + a.upd) * D, L);
  if (tid == 0) srow[a.upd] = p;
}

SelectPlan select_plan(int BH, int nb) {
  (void)BH;
  SelectPlan p;
  p.RPW = kScoreRows;
  p.C = cdiv(nb, p.RPW);
  return p;
}

hipError_t launch_score(const void* Q, int dtype, int B, int Hq, int Hkv, int D, float* sk,
                        int nb, const void* K, int N, int block, int upd, float scale,
                        float* scores, hipStream_t st) {
  ScoreArgs a;
  a.Q = Q; a.sk = sk; a.K = K; a.N = N; a.block = block; a.upd = upd;
  a.BH = B * Hkv; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.nb = nb;
  a.C = select_plan(a.BH, nb).C;
  a.scale = scale; a.scores = scores;
  const dim3 g(static_cast<unsigned>(long(a.BH) * a.C + (upd >= 0 ? a.BH : 0)));
  if (dtype == SA_BF16) {
    if (D == 128) k_score<uint16_t, 128><<<g, 256, 0, st>>>(a);
    else          k_score<uint16_t, 64><<<g, 256, 0, st>>>(a);
  } else {
    if (D == 128) k_score<float, 128><<<g, 256, 0, st>>>(a);
    else          k_score<float, 64><<<g, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode rows
template <int KPT>
__global__ __launch_bounds__(256) void k_select_rows(const float* __restrict__ scores, int nb,
                                                     int k, unsigned flags,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count) {
  constexpr int NT = 256;
  __shared__ SelectLdsT<NT, KPT> S;
  const int row = blockIdx.x;
  uint32_t kr[KPT];
  load_keys_reg<NT, KPT>(scores + size_t(row) * nb, nb, kr);
  int32_t* out = idx + size_t(row) * k;
  const int n = select_decode_row<NT, KPT>(kr, nb, k, flags, out, S);
  for (int j = n + threadIdx.x; j < k; j += NT) out[j] = -1;
  if (threadIdx.x == 0) count[row] = n;
}

hipError_t launch_select_rows(const float* scores, int rows, int nb, int k, unsigned flags,
                              int32_t* idx, int32_t* count, hipStream_t st) {
  const dim3 g(static_cast<unsigned>(rows));
  switch (keys_per_thread_tier(nb)) {
    case 2: k_select_rows<2><<<g, 256, 0, st>>>(scores, nb, k, flags, idx, count); break;
    case 8: k_select_rows<8><<<g, 256, 0, st>>>(scores, nb, k, flags, idx, count); break;
    default: k_select_rows<32><<<g, 256, 0, st>>>(scores, nb, k, flags, idx, count); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- prefill rows
template <int D, int KPT>
__global__ __launch_bounds__(256) void k_prefill_select(const float* __restrict__ qbar,
                                                        const float* __restrict__ ksk,
                                                        int M, int nb, int k,
                                                        unsigned flags, float scale,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ count,
                                                        float* __restrict__ score) {
  constexpr int NT = 256;
  constexpr int LPR = D / 4, RPI = 64 / LPR;
  extern __shared__ __attribute__((aligned(16))) uint32_t keys[];   // keys[M]
  __shared__ SelectLdsT<NT, KPT> S;
  const int i = blockIdx.x % M;
  const int bh = blockIdx.x / M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool sink = flags & SA_FORCE_SINK, local = flags & SA_FORCE_LOCAL;
  int32_t* out = idx + (size_t(bh) * M + i) * k;
  float* srow = score ? score + (size_t(bh) * M + i) * nb : nullptr;

  // candidates: earlier blocks, minus the forced sink; the diagonal is forced
  const int c0 = sink ? 1 : 0;
  const int c1 = local ? i : i + 1;
  const int n = max(c1 - c0, 0);
  const bool diag_forced = local && !(sink && i == 0);
  const int nF = int(sink) + int(diag_forced);
  const int nfree = min(k - nF, n);

  // scores of the candidates
  const int sub = lane / LPR, lc = lane % LPR;
  const u32x4 qv = ld16(qbar + (size_t(bh) * M + i) * D + lc * 4);
  const float* kb = ksk + size_t(bh) * nb * D;
  for (int jb = c0 + wave * RPI; jb < c1; jb += 4 * RPI) {
    const int j = jb + sub;
    const bool ok = j < c1;
    float p = 0.f;
    if (ok) {
      u32x4 w = ld16(kb + size_t(j) * D + lc * 4);
      p = __uint_as_float(qv[0]) * __uint_as_float(w[0]) +
          __uint_as_float(qv[1]) * __uint_as_float(w[1]) +
          __uint_as_float(qv[2]) * __uint_as_float(w[2]) +
          __uint_as_float(qv[3]) * __uint_as_float(w[3]);
    }
    p = group_sum_to_last<LPR>(p);
    if (ok && lc == LPR - 1) {
      p *= scale;
      keys[j] = score_key(p);
      if (srow) srow[j] = p;
    }
  }
  if (srow) {
    for (int j = tid; j < nb; j += NT)
      if (j < c0 || j >= c1) srow[j] = -__builtin_inff();
  }
  __syncthreads();
  // kept set as a bitmap over blocks [0, i]: sink, diagonal, chosen candidates
  const int W = (i + 32) >> 5;
  sel_init(S, W);
  if (nfree > 0 && nfree < n) {
    uint32_t kr[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int j = r * NT + tid;
      kr[r] = (j >= c0 && j < c1) ? keys[j] : 0u;
    }
    sel_mark_top<NT, KPT>(kr, c0, c1, nfree, S);
  } else {
    __syncthreads();
    if (nfree > 0)
      for (int j = c0 + tid; j < c1; j += NT) sel_mark(S.bm, j);
  }
  if (tid == 0) {
    if (sink) sel_mark(S.bm, 0);
    if (diag_forced) sel_mark(S.bm, i);
  }
  const int total = sel_bitmap_to_list(S, W, out, k);
  for (int j = total + tid; j < k; j += NT) out[j] = -1;
  if (tid == 0) count[size_t(bh) * M + i] = total;
}

hipError_t launch_prefill_select(const float* qbar, const float* ksk, int BH, int M, int nb,
                                 int D, int k, unsigned flags, float scale, int32_t* idx,
                                 int32_t* count, float* score, hipStream_t st) {
  const size_t lds = size_t(max(M, 1)) * sizeof(uint32_t);
  const dim3 g(static_cast<unsigned>(long(BH) * M)), t(256);
#define SA_PSEL(DD, KK) k_prefill_select<DD, KK><<<g, t, lds, st>>>(qbar, ksk, M, nb, k, flags, scale, idx, count, score)
  const int tier = keys_per_thread_tier(M);
  if (D == 128) {
    if (tier == 2) SA_PSEL(128, 2); else if (tier == 8) SA_PSEL(128, 8); else SA_PSEL(128, 32);
  } else {
    if (tier == 2) SA_PSEL(64, 2); else if (tier == 8) SA_PSEL(64, 8); else SA_PSEL(64, 32);
  }
#undef SA_PSEL
  return hipGetLastError();
}

}  // namespace sa
