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
//   k_block_score   HBM-bound scan of the float32 sketch; one 256-thread
//                   workgroup per (b, kv head, chunk of 64 blocks); the group's
//                   mean query (scale folded in) sits in registers, every row
//                   dot product is reduced across 32 (D=128) or 16 (D=64) lanes.
//                   Workgroup id % (B*Hkv) picks the (b, kv head), so with
//                   B*Hkv a multiple of 8 every (b, kv head) stays on one XCD.
//   k_topk_decode   one 1024-thread workgroup per (b, kv head): MSB-first radix
//                   select over order-preserving 32-bit keys in LDS (4 passes of
//                   8 bits), then an ordered compaction (block-wide prefix sums)
//                   that takes equal keys lowest index first.
//   k_prefill_select one 256-thread workgroup per (b, kv head, query block i):
//                   scores pooled query block i against key blocks [1, i-1]
//                   and selects with the same radix core (no cross-workgroup
//                   dependency, so scoring and selection fuse).
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------- radix core
struct TopkLds {
  uint32_t hist[256];
  int scan[17];
  int pick[2];
};

// Select the `nfree` largest of key[0..n) (ties: lower index first) and write
// their indices + `base`, ascending, to out[0..nfree).  n > nfree > 0.
// Every thread of the workgroup must call it (it contains barriers).
template <int NT>
__device__ void topk_core(const uint32_t* key, int n, int nfree, int base,
                          int32_t* __restrict__ out, TopkLds& L) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u;
  int rem = nfree;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) L.hist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += NT) {
      const uint32_t u = key[j];
      if ((u & mask) == prefix) atomicAdd(&L.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      int c[4], s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = int(L.hist[255 - 4 * tid - q]); s += c[q]; }
      int run = wave_incl_scan(s, tid) - s;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (run < rem && rem <= run + c[q]) { L.pick[0] = 255 - 4 * tid - q; L.pick[1] = rem - run; }
        run += c[q];
      }
    }
    __syncthreads();
    prefix |= uint32_t(L.pick[0]) << shift;
    mask |= 0xffu << shift;
    rem = L.pick[1];
    __syncthreads();
  }
  // keys above `prefix` are in; `rem` of the keys equal to it, lowest index first
  const uint32_t T = prefix;
  const int per = (n + NT - 1) / NT;
  const int j0 = min(tid * per, n), j1 = min(j0 + per, n);
  int neq = 0;
  for (int j = j0; j < j1; ++j) neq += key[j] == T;
  int tot;
  int eqr = block_excl_scan<NT>(neq, L.scan, &tot);
  int nsel = 0;
  {
    int e = eqr;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = key[j];
      nsel += (u > T) || (u == T && e < rem);
      e += u == T;
    }
  }
  int pos = block_excl_scan<NT>(nsel, L.scan, &tot);
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key[j];
    if ((u > T) || (u == T && eqr < rem)) out[pos++] = base + j;
    eqr += u == T;
  }
}

// ---------------------------------------------------------------- decode
// One launch scores every block and selects.  Workgroups [0, BH*C) each score
// RPW sketch rows of one (b, kv head) and add their candidates to that row's
// 2048-bin histogram of key digits (top 11 bits of the order-preserving key);
// with upd >= 0, BH more workgroups first rebuild the sketch of block `upd`
// from K and score it.  The last workgroup to arrive for a (b, kv head) finds
// the digit bin holding the cut from the histogram, ranks exactly only the
// members of that bin (ties to the lower index), writes the ascending list and
// clears the histogram and arrival counter for the next call.
constexpr int kHistBins = 2048;
constexpr int kMaxBoundary = 1024;

__device__ __forceinline__ uint32_t key_digit(uint32_t key) { return key >> 21; }

struct SelectArgs {
  const void* Q;
  float* sk;
  const void* K;
  int N, block, upd;
  int BH, Hq, Hkv, G, nb, C, RPW;
  float scale;
  int k;
  unsigned flags;
  float* scores;
  uint32_t* hist;
  uint32_t* counter;
  int32_t* idx;
  int32_t* count;
};

template <int NT>
__device__ void select_from_hist(const SelectArgs& a, int bh, uint32_t* lh, uint32_t* keys,
                                 uint32_t* bkey, int* bidx, int* bsel, int* misc, int* scan,
                                 TopkLds& L) {
  const int tid = threadIdx.x;
  const int nb = a.nb, k = a.k;
  const bool sink = a.flags & SA_FORCE_SINK, local = a.flags & SA_FORCE_LOCAL;
  uint32_t* gh = a.hist + size_t(bh) * kHistBins;
  for (int i = tid; i < kHistBins; i += NT) {
    lh[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&gh[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const float* srow = a.scores + size_t(bh) * nb;
  for (int j = tid; j < nb; j += NT) keys[j] = score_key(srow[j]);
  int32_t* out = a.idx + size_t(bh) * k;
  if (tid == 0) {
    a.count[bh] = min(k, nb);
    __hip_atomic_store(&a.counter[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (k >= nb) {
    for (int j = tid; j < k; j += NT) out[j] = j < nb ? j : -1;
    return;
  }
  const int c0 = sink ? 1 : 0, c1 = local ? nb - 1 : nb;   // nb >= 2 here
  const int nfree = k - int(sink) - int(local);
  if (tid == 0) {
    if (sink) out[0] = 0;
    if (local) out[k - 1] = nb - 1;
  }
  if (nfree <= 0) return;
  int32_t* fout = out + (sink ? 1 : 0);

  // cut bin: thread t owns bins 2047-8t .. 2040-8t (descending digits)
  constexpr int BPT = kHistBins / NT;
  int cnt[BPT], tot = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) { cnt[q] = int(lh[kHistBins - 1 - BPT * tid - q]); tot += cnt[q]; }
  int all;
  int run = block_excl_scan<NT>(tot, scan, &all);
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    if (run < nfree && nfree <= run + cnt[q]) { misc[0] = kHistBins - 1 - BPT * tid - q; misc[1] = run; }
    run += cnt[q];
  }
  __syncthreads();
  const uint32_t cut = uint32_t(misc[0]);
  const int need = nfree - misc[1];

  // boundary members (digit == cut), in index order
  const int n = c1 - c0;
  const int per = (n + NT - 1) / NT;
  const int j0 = min(tid * per, n), j1 = min(j0 + per, n);
  int nbd = 0;
  for (int j = j0; j < j1; ++j) nbd += key_digit(keys[c0 + j]) == cut;
  int m;
  const int bpos0 = block_excl_scan<NT>(nbd, scan, &m);
  if (m > kMaxBoundary) {                     // degenerate spread: full radix select
    topk_core<NT>(keys + c0, n, nfree, c0, fout, L);
    return;
  }
  {
    int p = bpos0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = keys[c0 + j];
      if (key_digit(u) == cut) { bkey[p] = u; bidx[p] = j; ++p; }
    }
  }
  __syncthreads();
  for (int i = tid; i < m; i += NT) {
    const uint32_t u = bkey[i];
    const int ji = bidx[i];
    int rank = 0;
    for (int t = 0; t < m; ++t) {
      const uint32_t v = bkey[t];
      rank += (v > u) || (v == u && bidx[t] < ji);
    }
    bsel[i] = rank < need;
  }
  __syncthreads();
  int nsel = 0;
  {
    int p = bpos0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t d = key_digit(keys[c0 + j]);
      if (d == cut) nsel += bsel[p++];
      else nsel += d > cut;
    }
  }
  int pos = block_excl_scan<NT>(nsel, scan, &all);
  {
    int p = bpos0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t d = key_digit(keys[c0 + j]);
      bool take;
      if (d == cut) take = bsel[p++];
      else take = d > cut;
      if (take) fout[pos++] = c0 + j;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_score_select(SelectArgs a) {
  constexpr int NT = 256;
  constexpr int LPR = D / 4, RPI = 64 / LPR;
  extern __shared__ uint32_t dyn[];           // nb keys (last workgroup) / sketch staging
  __shared__ uint32_t lh[kHistBins];
  __shared__ float qbar[D];
  __shared__ uint32_t bkey[kMaxBoundary];
  __shared__ int bidx[kMaxBoundary];
  __shared__ int bsel[kMaxBoundary];
  __shared__ int misc[4];
  __shared__ int scan[NT / 64 + 1];
  __shared__ TopkLds L;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nscore = a.BH * a.C;
  const bool is_upd = int(blockIdx.x) >= nscore;
  const int bh = is_upd ? int(blockIdx.x) - nscore : int(blockIdx.x) % a.BH;
  const int c = is_upd ? 0 : int(blockIdx.x) / a.BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int nb = a.nb;
  const bool sink = a.flags & SA_FORCE_SINK, local = a.flags & SA_FORCE_LOCAL;

  if (tid < D) {
    const T* Qp = static_cast<const T*>(a.Q);
    float s = 0.f;
    for (int h = 0; h < a.G; ++h) {
      const size_t o = (size_t(b) * a.Hq + kh * a.G + h) * D + tid;
      if constexpr (sizeof(T) == 2) s += bf16_to_f32(Qp[o]);
      else s += Qp[o];
    }
    qbar[tid] = (s / float(a.G)) * a.scale;
  }
  for (int i = tid; i < kHistBins; i += NT) lh[i] = 0u;
  __syncthreads();

  float* srow = a.scores + size_t(bh) * nb;
  if (!is_upd) {
    const int sub = lane / LPR, lc = lane % LPR;
    const float q0 = qbar[lc * 4], q1 = qbar[lc * 4 + 1], q2 = qbar[lc * 4 + 2],
                q3 = qbar[lc * 4 + 3];
    const int r0 = c * a.RPW, r1 = min(r0 + a.RPW, nb);
    const float* base = a.sk + size_t(bh) * nb * D;
    for (int rb = r0 + wave * RPI; rb < r1; rb += 4 * RPI) {
      const int r = rb + sub;
      const bool ok = r < r1 && r != a.upd;
      float p = 0.f;
      if (ok) {
        const u32x4 w = ld16(base + size_t(r) * D + lc * 4);
        p = q0 * __uint_as_float(w[0]) + q1 * __uint_as_float(w[1]) +
            q2 * __uint_as_float(w[2]) + q3 * __uint_as_float(w[3]);
      }
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
      if (ok && lc == 0) {
        srow[r] = p;
        if (!((sink && r == 0) || (local && r == nb - 1)))
          atomicAdd(&lh[key_digit(score_key(p))], 1u);
      }
    }
  } else {
    // rebuild the sketch of block upd from K, then score it
    constexpr int CPT = 8, TPR = D / CPT, RPP = NT / TPR;
    float* red = reinterpret_cast<float*>(dyn);            // [RPP][D + 4]
    const int t0 = a.upd * a.block, nj = min(a.block, a.N - t0);
    const int tr = tid / TPR, tc = tid % TPR;
    float acc[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) acc[q] = 0.f;
    const T* Kp = static_cast<const T*>(a.K) + (size_t(bh) * a.N + t0) * D + tc * CPT;
    for (int r = tr; r < nj; r += RPP) {
      if constexpr (sizeof(T) == 2) {
        const u32x4 w = ld16(Kp + size_t(r) * D);
#pragma unroll
        for (int q = 0; q < 4; ++q) { acc[2 * q] += bf16lo(w[q]); acc[2 * q + 1] += bf16hi(w[q]); }
      } else {
        const u32x4 w0 = ld16(Kp + size_t(r) * D), w1 = ld16(Kp + size_t(r) * D + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { acc[q] += __uint_as_float(w0[q]); acc[4 + q] += __uint_as_float(w1[q]); }
      }
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) red[tr * (D + 4) + tc * CPT + q] = acc[q];
    __syncthreads();
    float part = 0.f;
    if (tid < D) {
      float sum = 0.f;
      for (int g = 0; g < RPP; ++g) sum += red[g * (D + 4) + tid];
      const float v = sum / float(nj);
      a.sk[(size_t(bh) * nb + a.upd) * D + tid] = v;
      part = v * qbar[tid];
    }
    part = wave_sum(part);
    __syncthreads();
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (tid == 0) {
      float p = 0.f;
      for (int w = 0; w < D / 64; ++w) p += red[w];
      srow[a.upd] = p;
      if (!((sink && a.upd == 0) || (local && a.upd == nb - 1)))
        lh[key_digit(score_key(p))] += 1u;
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + size_t(bh) * kHistBins;
  for (int i = tid; i < kHistBins; i += NT) {
    const uint32_t v = lh[i];
    if (v) atomicAdd(&gh[i], v);
  }
  // publish scores and histogram, then count arrivals for this (b, kv head)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  const uint32_t total = uint32_t(a.C + (a.upd >= 0 ? 1 : 0));
  if (tid == 0) misc[3] = atomicAdd(&a.counter[bh], 1u) == total - 1u;
  __syncthreads();
  if (!misc[3]) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  select_from_hist<NT>(a, bh, lh, dyn, bkey, bidx, bsel, misc, scan, L);
}

SelectPlan select_plan(int BH, int nb) {
  SelectPlan p;
  p.RPW = 64;
  p.C = cdiv(nb, p.RPW);
  return p;
}

hipError_t launch_score_select(const void* Q, int dtype, int B, int Hq, int Hkv, int D,
                               float* sk, int nb, const void* K, int N, int block, int upd,
                               float scale, int k, unsigned flags, float* scores,
                               uint32_t* hist, uint32_t* counter, int32_t* idx, int32_t* count,
                               hipStream_t st) {
  SelectArgs a;
  a.Q = Q; a.sk = sk; a.K = K; a.N = N; a.block = block; a.upd = upd;
  a.BH = B * Hkv; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.nb = nb;
  const SelectPlan p = select_plan(a.BH, nb);
  a.C = p.C; a.RPW = p.RPW;
  a.scale = scale; a.k = k; a.flags = flags; a.scores = scores; a.hist = hist;
  a.counter = counter; a.idx = idx; a.count = count;
  const long grid = long(a.BH) * a.C + (upd >= 0 ? a.BH : 0);
  const size_t lds = max(size_t(nb) * sizeof(uint32_t), size_t(256 / (D / 8)) * (D + 4) * sizeof(float));
  if (dtype == SA_BF16) {
    if (D == 128) k_score_select<uint16_t, 128><<<dim3(unsigned(grid)), 256, lds, st>>>(a);
    else          k_score_select<uint16_t, 64><<<dim3(unsigned(grid)), 256, lds, st>>>(a);
  } else {
    if (D == 128) k_score_select<float, 128><<<dim3(unsigned(grid)), 256, lds, st>>>(a);
    else          k_score_select<float, 64><<<dim3(unsigned(grid)), 256, lds, st>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- prefill rows
template <int D>
__global__ __launch_bounds__(256) void k_prefill_select(const float* __restrict__ qbar,
                                                        const float* __restrict__ ksk,
                                                        int M, int nb, int k,
                                                        unsigned flags, float scale,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ count,
                                                        float* __restrict__ score) {
  constexpr int NT = 256;
  constexpr int LPR = D / 4, RPI = 64 / LPR;
  extern __shared__ uint32_t keys[];
  __shared__ TopkLds L;
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
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
    if (ok && lc == 0) {
      p *= scale;
      keys[j - c0] = score_key(p);
      if (srow) srow[j] = p;
    }
  }
  if (srow) {
    for (int j = tid; j < nb; j += NT)
      if (j < c0 || j >= c1) srow[j] = -__builtin_inff();
  }
  __syncthreads();
  const int total = nF + nfree;
  if (tid == 0) {
    if (sink) out[0] = 0;
    if (diag_forced) out[total - 1] = i;
    count[size_t(bh) * M + i] = total;
  }
  for (int j = total + tid; j < k; j += NT) out[j] = -1;
  int32_t* free_out = out + (sink ? 1 : 0);
  if (nfree >= n) {
    for (int j = tid; j < n; j += NT) free_out[j] = c0 + j;
  } else if (nfree > 0) {
    topk_core<NT>(keys, n, nfree, c0, free_out, L);
  }
}

hipError_t launch_prefill_select(const float* qbar, const float* ksk, int BH, int M, int nb,
                                 int D, int k, unsigned flags, float scale, int32_t* idx,
                                 int32_t* count, float* score, hipStream_t st) {
  const size_t lds = size_t(max(M, 1)) * sizeof(uint32_t);
  dim3 g(unsigned(long(BH) * M)), t(256);
  if (D == 128) k_prefill_select<128><<<g, t, lds, st>>>(qbar, ksk, M, nb, k, flags, scale, idx, count, score);
  else          k_prefill_select<64><<<g, t, lds, st>>>(qbar, ksk, M, nb, k, flags, scale, idx, count, score);
  return hipGetLastError();
}

}  // namespace sa
