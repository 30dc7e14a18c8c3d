// sa_select_core.h -- exact top-n of one score row inside one workgroup.
//
// Used by the standalone selection kernel, by the decode kernel that selects
// its own blocks and by the prefill selector.  Keys are order-preserving
// 32-bit images of float scores (score_key); among equal keys the lower index
// wins, matching the selection rule of the block selector (forced blocks
// aside, the best scores are kept, ties to the lower block index).
//
// Layout: thread tid holds the keys of indices j = r*NT + tid (r < KPT) in
// registers, so every pass over the keys is a register sweep.
//
// Usual path (several keys per thread, k small against the thread count):
// 1. A histogram of the per-thread maxima (one LDS atomic per thread) gives a
//    lower bound T0 that at least `need` keys reach, so the exact top set lies
//    in {key >= T0}.
// 2. Those keys are compacted by a block scan into an LDS list of unique
//    64-bit composites (key << 32 | ~index) and each is ranked by counting
//    the list entries above it.
// Direct path (bound too weak, or one or two keys per thread):
// 1. Range: wave min / max of the candidate keys (DPP), u = key - min.
// 2. Radix cut: up to 11 bits of u at a time, from its top set bit down, are
//    histogrammed in LDS for the keys sharing the current prefix; a block scan
//    (DPP inside each wave) finds the digit holding the cut.  This repeats
//    until the cut bin is taken whole or holds at most kBoundCap keys.  With
//    the prefix P under the mask M, a key is above the cut when (u & M) > P
//    and a boundary member when (u & M) == P.
// 3. Boundary members are appended to LDS and ranked exactly by
//    (key desc, index asc); if more than kBoundCap keys share all 32 bits,
//    the lowest indices win by a prefix count over a member bitmap.
// Both paths set one bit per kept index in an LDS bitmap; one block scan of
// the word popcounts turns it into the ascending index list.
#pragma once

#include "sa_device.h"

namespace sa {

constexpr int kSelBins = 2048;
constexpr int kBoundCap = 512;
constexpr int kSelWords = 256;    // bitmap words: rows of up to 8192 indices
constexpr int kCandCap = 512;     // pre-filtered candidate list

template <int NT, int KPT>
struct SelectLdsT {
  __attribute__((aligned(16))) uint32_t hist[kSelBins];
  __attribute__((aligned(16))) uint32_t bm[kSelWords];
  __attribute__((aligned(16))) uint32_t bkey[kBoundCap];
  __attribute__((aligned(16))) int bidx[kBoundCap];
  // (key << 32) | ~index; zero padding at [C, C + 64), per-lane discard
  // slots at [kCandCap + 64, kCandCap + 128)
  __attribute__((aligned(16))) uint64_t cand[kCandCap + 128];
  int wsum[8][NT / 64];
  int misc[8];
};

// Sum of the wave totals of waves before `wave` and of all waves.
template <int NW>
__device__ __forceinline__ int wave_base(const int* wt, int wave, int* all) {
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = wt[w];
    base += w < wave ? t : 0;
    tot += t;
  }
  *all = tot;
  return base;
}

// Clear the histogram, the bitmap words [0, W) and the member counter.  No
// barrier: the first barrier of sel_mark_top (or the caller's) publishes it.
template <int NT, int KPT>
__device__ __forceinline__ void sel_init(SelectLdsT<NT, KPT>& S, int W) {
  static_assert(NT == 256, "the cut search assumes 8 histogram bins per thread");
  const int tid = threadIdx.x;
  u32x4* h4 = reinterpret_cast<u32x4*>(S.hist);
  h4[2 * tid] = u32x4{0u, 0u, 0u, 0u};
  h4[2 * tid + 1] = u32x4{0u, 0u, 0u, 0u};
  if (tid < W) S.bm[tid] = 0u;
  if (tid == 0) S.misc[6] = 0;
}

__device__ __forceinline__ void sel_mark(uint32_t* bm, int j) {
  atomicOr(&bm[j >> 5], 1u << (j & 31));
}

// Mark in S.bm the top `need` of the ncand candidates held in registers:
// key kr[r] of index ix[r] where cand[r] (0 < need < ncand, indices distinct
// and below 32 * kSelWords).  The histogram must be zero and published by a
// barrier before the first atomic (the barrier after the range reduction
// below serves); all NT threads call.  Ends without a barrier after the last
// marks.
template <int NT, int KPT, int L>
__device__ void sel_mark_top_kv(const uint32_t (&kr)[L], const int (&ix)[L], const bool (&cand)[L],
                                int ncand, int need, SelectLdsT<NT, KPT>& S) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int r = 0; r < L; ++r)
    if (cand[r]) { lo = min(lo, kr[r]); hi = max(hi, kr[r]); }
  lo = wave_umin(lo);
  hi = wave_umax(hi);
  if (lane == 0) { S.wsum[0][wave] = int(lo); S.wsum[1][wave] = int(hi); }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, uint32_t(S.wsum[0][w]));
    hi = max(hi, uint32_t(S.wsum[1][w]));
  }
  uint32_t u[L];
#pragma unroll
  for (int r = 0; r < L; ++r) u[r] = kr[r] - lo;
  int bits = 32 - __clz(int(hi - lo));       // 0 when every candidate key is equal
  uint32_t P = 0u, M = 0u;
  int want = need, m = ncand, level = 0;
  u32x4* h4 = reinterpret_cast<u32x4*>(S.hist);
  while (bits > 0 && want < m) {
    const int width = min(bits, 11), shift = bits - width;
    const uint32_t dmask = (1u << width) - 1u;
    if (level > 0) {
      h4[2 * tid] = u32x4{0u, 0u, 0u, 0u};
      h4[2 * tid + 1] = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < L; ++r)
      if (cand[r] && (u[r] & M) == P) atomicAdd(&S.hist[(u[r] >> shift) & dmask], 1u);
    __syncthreads();
    // thread t owns bins [kSelBins - 8(t+1), kSelBins - 8t), scanned downward
    const u32x4 ha = h4[kSelBins / 4 - 2 * tid - 2], hb = h4[kSelBins / 4 - 2 * tid - 1];
    const int tot = int(ha[0] + ha[1] + ha[2] + ha[3] + hb[0] + hb[1] + hb[2] + hb[3]);
    const int incl = wave_incl_scan(tot);
    int* wt = S.wsum[3 + level];
    if (lane == 63) wt[wave] = incl;
    __syncthreads();
    int all;
    int run = incl - tot + wave_base<NW>(wt, wave, &all);
    if (run < want && want <= run + tot) {
      const uint32_t hv[8] = {hb[3], hb[2], hb[1], hb[0], ha[3], ha[2], ha[1], ha[0]};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int c = int(hv[q]);
        if (run < want && want <= run + c) {
          S.misc[0] = kSelBins - 1 - 8 * tid - q; S.misc[1] = run; S.misc[2] = c;
        }
        run += c;
      }
    }
    __syncthreads();
    want -= S.misc[1];
    m = S.misc[2];
    P |= uint32_t(S.misc[0]) << shift;
    M |= dmask << shift;
    bits = shift;
    ++level;
    if (m <= kBoundCap) break;
  }
  // above the cut: kept; boundary members: kept whole, ranked, or by index
  const bool whole = want >= m;
  const bool ranked = !whole && m <= kBoundCap;
  uint32_t* mbm = S.hist;                    // member bitmap (identical keys only)
  if (!whole && !ranked) {
    if (tid < kSelWords) mbm[tid] = 0u;      // the histogram is no longer read
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < L; ++r) {
    const int j = ix[r];
    if (!cand[r]) continue;
    const uint32_t um = u[r] & M;
    if (um > P || (whole && um == P)) {
      sel_mark(S.bm, j);
    } else if (um == P) {
      if (ranked) {
        const int p = atomicAdd(&S.misc[6], 1);
        if (p < kBoundCap) { S.bkey[p] = u[r]; S.bidx[p] = j; }
      } else {
        sel_mark(mbm, j);
      }
    }
  }
  if (whole) return;
  __syncthreads();
  if (ranked) {
    for (int i = tid; i < m; i += NT) {
      const uint32_t x = S.bkey[i];
      const int xi = S.bidx[i];
      int rk = 0;
      for (int t = 0; t < m; t += 4) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(&S.bkey[t]);
        const u32x4 ii = *reinterpret_cast<const u32x4*>(&S.bidx[t]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rk += (t + q < m) && ((kk[q] > x) || (kk[q] == x && int(ii[q]) < xi));
      }
      if (rk < want) sel_mark(S.bm, xi);
    }
    return;
  }
  // more than kBoundCap identical keys at the cut: the `want` lowest indices
  const uint32_t wv = tid < kSelWords ? mbm[tid] : 0u;
  const int c = __popc(wv);
  const int incl = wave_incl_scan(c);
  if (lane == 63) S.wsum[6][wave] = incl;
  __syncthreads();
  int all;
  int pos = incl - c + wave_base<NW>(S.wsum[6], wave, &all);
  for (uint32_t x = wv; x != 0u && pos < want; x &= x - 1u, ++pos)
    sel_mark(S.bm, tid * 32 + __ffs(int(x)) - 1);
}


// Keys of the candidates c0 <= j < c1 among kin[r] (index j = r*NT + tid);
// the others become 0, which no score maps to, so later passes need no masks
// and their stores can be unconditional.  Returns the thread's largest key.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t sel_mask_keys(const uint32_t (&kin)[KPT], int c0, int c1,
                                                  uint32_t (&kr)[KPT], int (&ix)[KPT]) {
  uint32_t tmax = 0u;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    ix[r] = r * NT + threadIdx.x;
    kr[r] = unsigned(ix[r] - c0) < unsigned(c1 - c0) ? kin[r] : 0u;
    tmax = max(tmax, kr[r]);
  }
  return tmax;
}

// Pre-filter for the top `need` of the masked keys (sel_mask_keys; sel_init
// must have run; all NT threads call).  A histogram of the per-thread maxima
// (one LDS atomic per thread) gives a lower bound T0 that at least `need` keys
// reach, so the exact top set lies in {key >= T0}.  Those C keys are compacted
// by a block scan into S.cand[0, C) as (key << 32) | ~index -- unique, ordered
// by key and then lower index first -- followed by zero padding up to the next
// multiple of 128 and to the share layout of sel_rank_all.  Returns C after a
// barrier, or -1 when the bound does not apply (one or two keys per thread,
// need above 3NT/4, nmax below need or C above kCandCap); the histogram is
// then zero again and published, ready for sel_mark_top_kv.
template <int NT, int KPT>
__device__ int sel_prefilter(const uint32_t (&kr)[KPT], const int (&ix)[KPT], uint32_t tmax,
                             int need, SelectLdsT<NT, KPT>& S) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!(KPT > 2 && need <= 3 * NT / 4)) return -1;
  // range of the per-thread maxima, then their histogram
  uint32_t lo = wave_umin(tmax != 0u ? tmax : 0xffffffffu), hi = wave_umax(tmax);
  if (lane == 0) { S.wsum[0][wave] = int(lo); S.wsum[1][wave] = int(hi); }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, uint32_t(S.wsum[0][w]));
    hi = max(hi, uint32_t(S.wsum[1][w]));
  }
  const int bits = 32 - __clz(int(hi - lo));
  const int shift = bits > 11 ? bits - 11 : 0;
  atomicAdd(&S.hist[tmax != 0u ? (tmax - lo) >> shift : 0], tmax != 0u ? 1u : 0u);
  __syncthreads();
  u32x4* h4 = reinterpret_cast<u32x4*>(S.hist);
  const u32x4 ha = h4[kSelBins / 4 - 2 * tid - 2], hb = h4[kSelBins / 4 - 2 * tid - 1];
  const int tot = int(ha[0] + ha[1] + ha[2] + ha[3] + hb[0] + hb[1] + hb[2] + hb[3]);
  const int incl = wave_incl_scan(tot);
  if (lane == 63) S.wsum[2][wave] = incl;
  __syncthreads();
  int nmax;
  int run = incl - tot + wave_base<NW>(S.wsum[2], wave, &nmax);
  if (run < need && need <= run + tot) {
    const uint32_t hv[8] = {hb[3], hb[2], hb[1], hb[0], ha[3], ha[2], ha[1], ha[0]};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = int(hv[q]);
      if (run < need && need <= run + c) S.misc[3] = kSelBins - 1 - 8 * tid - q;
      run += c;
    }
  }
  // the histogram is read: clear it for a possible direct selection
  h4[2 * tid] = u32x4{0u, 0u, 0u, 0u};
  h4[2 * tid + 1] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  if (nmax < need) return -1;
  const uint32_t T0 = lo + (uint32_t(S.misc[3]) << shift);
  int nc = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) nc += kr[r] >= T0 ? 1 : 0;
  const int inc2 = wave_incl_scan(nc);
  if (lane == 63) S.wsum[7][wave] = inc2;
  __syncthreads();
  int C;
  int pos = inc2 - nc + wave_base<NW>(S.wsum[7], wave, &C);
  if (C > kCandCap) return -1;
  // keys below T0 go to this lane's discard slot
  const int trash = kCandCap + 64 + lane;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const bool in = kr[r] >= T0;
    S.cand[in ? pos : trash] = (uint64_t(kr[r]) << 32) | uint32_t(~ix[r]);
    pos += in ? 1 : 0;
  }
  // zero padding (candidates are nonzero, so it never outranks one): to
  // R * share for sel_rank_all and to a multiple of 128 for sel_rank_entry8;
  // both ends stay below kCandCap + 64
  const int R = C <= NT / 4 ? 4 : (C <= NT / 2 ? 2 : 1);
  const int share = (((C + R - 1) / R) + 15) & ~15;
  const int pad = max(R * share, (C + 127) & ~127) - C;
  if (tid < pad) S.cand[C + tid] = 0ull;
  __syncthreads();
  return C;
}

// Mark in S.bm the top `need` of the C pre-filtered candidates (need <= C):
// each is ranked by counting the list entries above it, R threads (adjacent
// lanes) per candidate, each over its share of the list, 16 entries (8 reads)
// per step.  Ends without a barrier after the last marks.
template <int NT, int KPT>
__device__ void sel_rank_all(int C, int need, SelectLdsT<NT, KPT>& S) {
  const int tid = threadIdx.x;
  if (need >= C) {
    for (int i = tid; i < C; i += NT) sel_mark(S.bm, int(~uint32_t(S.cand[i])));
    return;
  }
  const int R = C <= NT / 4 ? 4 : (C <= NT / 2 ? 2 : 1);
  const int share = (((C + R - 1) / R) + 15) & ~15;
  for (int i0 = 0; i0 < C; i0 += NT / R) {
    const int i = i0 + tid / R, h = tid % R;
    const uint64_t x = i < C ? S.cand[i] : ~0ull;
    const uint64_t* lp = S.cand + h * share;
    int rk = 0;
    for (int t = 0; t < share; t += 16) {
      u32x4 pr[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) pr[q] = *reinterpret_cast<const u32x4*>(lp + t + 2 * q);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        rk += ((uint64_t(pr[q][1]) << 32) | pr[q][0]) > x;
        rk += ((uint64_t(pr[q][3]) << 32) | pr[q][2]) > x;
      }
    }
    if (R >= 2) rk += __shfl_xor(rk, 1, 64);
    if (R >= 4) rk += __shfl_xor(rk, 2, 64);
    if (i < C && h == 0 && rk < need) sel_mark(S.bm, int(~uint32_t(x)));
  }
}

// Rank of the list entry x = S.cand[i] (i < C) within groups of 8 adjacent
// lanes that all pass the same x: the number of entries of S.cand[0, P) above
// it, P = C rounded up to 128 (zero padded by sel_prefilter).  Lane h =
// lane % 8 counts the h-th eighth of the list; the total lands in the
// group's lane h = 7.
template <int NT, int KPT>
__device__ __forceinline__ int sel_rank_entry8(uint64_t x, int C, const SelectLdsT<NT, KPT>& S) {
  const int h = threadIdx.x & 7;
  const int e8 = ((C + 127) & ~127) >> 3;     // entries per lane: a multiple of 16
  const uint64_t* lp = S.cand + h * e8;
  int rk = 0;
  for (int t = 0; t < e8; t += 16) {
    u32x4 pr[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) pr[q] = *reinterpret_cast<const u32x4*>(lp + t + 2 * q);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      rk += ((uint64_t(pr[q][1]) << 32) | pr[q][0]) > x;
      rk += ((uint64_t(pr[q][3]) << 32) | pr[q][2]) > x;
    }
  }
  return group_isum8_to_last(rk);
}

// Mark in S.bm the top `need` of the candidates c0 <= j < c1 among the keys
// kin[r] of indices j = r*NT + tid (0 < need < c1 - c0).  sel_init must have
// run; all NT threads call.  Ends without a barrier after the last marks.
// The pre-filtered list is ranked by counting (it is short: about 1.1-1.5
// need on continuous scores; LDS atomics serialize per lane, so this avoids a
// histogram over every key); when the bound is too weak the keys are selected
// directly.
template <int NT, int KPT>
__device__ void sel_mark_top(const uint32_t (&kin)[KPT], int c0, int c1, int need,
                             SelectLdsT<NT, KPT>& S) {
  uint32_t kr[KPT];
  int ix[KPT];
  const uint32_t tmax = sel_mask_keys<NT, KPT>(kin, c0, c1, kr, ix);
  const int C = sel_prefilter<NT, KPT>(kr, ix, tmax, need, S);
  if (C >= 0) {
    sel_rank_all<NT, KPT>(C, need, S);
    return;
  }
  bool cand[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) cand[r] = kr[r] != 0u;
  sel_mark_top_kv<NT, KPT, KPT>(kr, ix, cand, c1 - c0, need, S);
}

// Ascending list of the set bits of S.bm[0, W) into out[0, min(total, cap));
// returns the total.  Starts and ends with a barrier; all NT threads call.
template <int NT, int KPT>
__device__ int sel_bitmap_to_list(SelectLdsT<NT, KPT>& S, int W, int* out, int cap) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();
  const uint32_t wv = tid < W ? S.bm[tid] : 0u;
  const int c = __popc(wv);
  const int incl = wave_incl_scan(c);
  if (lane == 63) S.wsum[4][wave] = incl;
  __syncthreads();
  int total;
  int pos = incl - c + wave_base<NW>(S.wsum[4], wave, &total);
  for (uint32_t x = wv; x != 0u; x &= x - 1u, ++pos)
    if (unsigned(pos) < unsigned(cap)) out[pos] = tid * 32 + __ffs(int(x)) - 1;
  __syncthreads();
  return total;
}

// Keys of score row srow (length nb) into registers: kr[r] <- key of index
// r*NT + tid (missing entries get key 0, never a candidate).  Every load is
// issued (clamped in bounds, no branch) before the first is waited on.
template <int NT, int KPT>
__device__ __forceinline__ void load_keys_reg(const float* srow, int nb, uint32_t (&kr)[KPT]) {
  const int tid = threadIdx.x;
  float v[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) v[r] = srow[min(r * NT + tid, nb - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < KPT; ++r) kr[r] = r * NT + tid < nb ? score_key(v[r]) : 0u;
}

// Full decode selection of one row: forced sink (block 0) and local (block
// nb-1) per flags, then the best k - forced of the rest.  Writes min(k, nb)
// ascending block ids to out (capacity k).  Returns the count.  All NT
// threads call; nb <= 32 * kSelWords.
template <int NT, int KPT>
__device__ int select_decode_row(const uint32_t (&kr)[KPT], int nb, int k, unsigned flags,
                                 int* out, SelectLdsT<NT, KPT>& S) {
  const int tid = threadIdx.x;
  if (k >= nb) {
    for (int j = tid; j < nb; j += NT) out[j] = j;
    __syncthreads();
    return nb;
  }
  const bool sink = flags & SA_FORCE_SINK, local = flags & SA_FORCE_LOCAL;
  const int c0 = sink ? 1 : 0, c1 = local ? nb - 1 : nb;   // nb >= 2 here
  const int nfree = k - int(sink) - int(local);
  const int W = (nb + 31) >> 5;
  sel_init(S, W);
  if (nfree > 0) sel_mark_top<NT, KPT>(kr, c0, c1, nfree, S);
  else __syncthreads();
  if (tid == 0) {
    if (sink) sel_mark(S.bm, 0);
    if (local) sel_mark(S.bm, nb - 1);
  }
  return sel_bitmap_to_list(S, W, out, k);
}

// Register tiers for KPT = ceil(nb / 256) rounded up: 2, 8 or 32 keys per thread.
__host__ __device__ inline int keys_per_thread_tier(int nb) {
  return nb <= 512 ? 2 : (nb <= 2048 ? 8 : 32);
}

}  // namespace sa
