// sa_select_core.h -- exact top-n of one score row inside one workgroup.
//
// Used by the standalone selection kernel, by the decode kernel that selects
// its own blocks and by the prefill selector.  Keys are order-preserving
// 32-bit images of float scores (score_key); among equal keys the lower index
// wins, matching the selection rule of the block selector (forced blocks
// aside, the best scores are kept, ties to the lower block index).
//
// Layout: thread tid holds the keys of indices j = r*NT + tid (r < KPT) in
// registers, so every pass is a register sweep.
//
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
// 4. Every kept index sets its bit in an LDS bitmap; one block scan of the
//    word popcounts turns the bitmap into the ascending index list.
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
  uint32_t ckey[kCandCap];
  int cidx[kCandCap];
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


// Mark in S.bm the top `need` of the candidates c0 <= j < c1 among the keys
// kr[r] of indices j = r*NT + tid (0 < need < c1 - c0).  sel_init must have
// run; all NT threads call.  Ends without a barrier after the last marks.
//
// Pre-filter: a histogram of the per-thread maxima (one LDS atomic per
// thread) gives a lower bound T0 that at least `need` candidate keys reach, so
// the exact top set lies in {key >= T0}.  Those keys are compacted into an LDS
// list by a block scan and the radix select runs on the list (at most two
// entries per thread) instead of on every key; LDS atomics serialize per lane,
// so this is what keeps the histogram passes short.  When the bound is too
// weak (list over kCandCap, need above 3NT/4) the keys are selected directly.
template <int NT, int KPT>
__device__ void sel_mark_top(const uint32_t (&kr)[KPT], int c0, int c1, int need,
                             SelectLdsT<NT, KPT>& S) {
  constexpr int NW = NT / 64;
  static_assert(kCandCap == 2 * NT, "two list entries per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool cand[KPT];
  int ix[KPT];
  uint32_t tmax = 0u;                 // real keys are nonzero: 0 = no candidate
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    ix[r] = r * NT + tid;
    cand[r] = ix[r] >= c0 && ix[r] < c1;
    if (cand[r]) tmax = max(tmax, kr[r]);
  }
  if (KPT > 2 && need <= 3 * NT / 4) {
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
    if (tmax != 0u) atomicAdd(&S.hist[(tmax - lo) >> shift], 1u);
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
    // the histogram is read: clear it for the list's radix select
    h4[2 * tid] = u32x4{0u, 0u, 0u, 0u};
    h4[2 * tid + 1] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    if (nmax >= need) {
      const uint32_t T0 = lo + (uint32_t(S.misc[3]) << shift);
      int nc = 0;
#pragma unroll
      for (int r = 0; r < KPT; ++r) nc += (cand[r] && kr[r] >= T0) ? 1 : 0;
      const int inc2 = wave_incl_scan(nc);
      if (lane == 63) S.wsum[7][wave] = inc2;
      __syncthreads();
      int C;
      int pos = inc2 - nc + wave_base<NW>(S.wsum[7], wave, &C);
      if (C <= kCandCap) {
#pragma unroll
        for (int r = 0; r < KPT; ++r)
          if (cand[r] && kr[r] >= T0) { S.ckey[pos] = kr[r]; S.cidx[pos] = ix[r]; ++pos; }
        __syncthreads();
        uint32_t ck[2];
        int ci[2];
        bool cc[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int i = q * NT + tid;
          cc[q] = i < C;
          ck[q] = cc[q] ? S.ckey[i] : 0u;
          ci[q] = cc[q] ? S.cidx[i] : 0;
        }
        if (need < C) sel_mark_top_kv<NT, KPT, 2>(ck, ci, cc, C, need, S);
        else {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            if (cc[q]) sel_mark(S.bm, ci[q]);
        }
        return;
      }
    }
  }
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
// r*NT + tid (missing entries get key 0, never a candidate).
template <int NT, int KPT>
__device__ __forceinline__ void load_keys_reg(const float* srow, int nb, uint32_t (&kr)[KPT]) {
  const int tid = threadIdx.x;
  float v[KPT];
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    const int j = r * NT + tid;
    v[r] = j < nb ? srow[j] : 0.f;
  }
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
