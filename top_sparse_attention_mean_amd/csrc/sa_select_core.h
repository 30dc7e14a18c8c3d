// sa_select_core.h -- exact top-n of one score row inside one workgroup.
//
// Used by the standalone selection kernel, by the decode kernel that selects
// its own blocks and by the prefill selector.  Keys are order-preserving
// 32-bit images of float scores (score_key); among equal keys the lower index
// wins, matching the selection rule of the block selector (forced blocks
// aside, the best scores are kept, ties to the lower block index).
//
// Layout: thread tid holds the keys of indices j = r*NT + tid (r < KPT) in
// registers, so every pass below is a register sweep plus LDS atomics -- no
// dependent LDS reads.
// Radix select with early exit: level 0 histograms the top 11 bits of every
// candidate key in LDS and finds the bin holding the cut (one block-wide scan);
// keys above that bin are appended to the result, and when the cut bin holds at
// most kBoundCap keys they are ranked exactly by (key desc, index asc).
// Otherwise the next 11 (then 10) bits of the cut bin's members are
// histogrammed the same way.  The small rank and sort loops read their lists
// with unrolled 16-byte LDS loads over sentinel-padded arrays.
#pragma once

#include "sa_device.h"

namespace sa {

constexpr int kSelBins = 2048;
constexpr int kBoundCap = 512;

struct SelectLds {
  uint32_t hist[kSelBins];
  __attribute__((aligned(16))) uint32_t bkey[kBoundCap + 8];
  __attribute__((aligned(16))) int bidx[kBoundCap + 8];
  int scan[17];
  int misc[8];
};

// Top `need` of the candidates c0 <= j < c1 (need < c1 - c0) among the keys
// kr[r] of indices j = r*NT + tid.  Writes the chosen indices ascending to
// out[0..need).  tmp must hold need + 8 ints of LDS (16-byte aligned).  All NT
// threads call.
template <int NT, int KPT>
__device__ void select_core(const uint32_t (&kr)[KPT], int c0, int c1, int need, int* tmp,
                            int* out, SelectLds& S) {
  const int tid = threadIdx.x;
  if (tid == 0) { S.misc[0] = 0; S.misc[4] = 0; }
  uint32_t prefix = 0u, pmask = 0u;
  int want = need;
  for (int level = 0; level < 3; ++level) {
    const int width = level < 2 ? 11 : 10;
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int nbins = 1 << width;
    const uint32_t dmask = uint32_t(nbins - 1);
    for (int i = tid; i < nbins; i += NT) S.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int j = r * NT + tid;
      const uint32_t u = kr[r];
      if (j >= c0 && j < c1 && (u & pmask) == prefix) atomicAdd(&S.hist[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    // cut bin: thread t owns bins nbins-1-bpt*t .. (descending digits)
    const int bpt = nbins / NT;
    int tot = 0;
    for (int q = 0; q < bpt; ++q) tot += int(S.hist[nbins - 1 - bpt * tid - q]);
    int all;
    int run = block_excl_scan<NT>(tot, S.scan, &all);
    for (int q = 0; q < bpt; ++q) {
      const int b = nbins - 1 - bpt * tid - q;
      const int c = int(S.hist[b]);
      if (run < want && want <= run + c) { S.misc[1] = b; S.misc[2] = run; S.misc[3] = c; }
      run += c;
    }
    __syncthreads();
    const uint32_t d = uint32_t(S.misc[1]);
    const int above = S.misc[2], m = S.misc[3];
    // keys of this prefix whose digit beats the cut bin are in
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int j = r * NT + tid;
      const uint32_t u = kr[r];
      if (j >= c0 && j < c1 && (u & pmask) == prefix && ((u >> shift) & dmask) > d)
        tmp[atomicAdd(&S.misc[0], 1)] = j;
    }
    want -= above;
    prefix |= d << shift;
    pmask |= dmask << shift;
    if (m <= kBoundCap) {
      // rank the cut bin's members exactly by (key desc, index asc)
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int j = r * NT + tid;
        const uint32_t u = kr[r];
        if (j >= c0 && j < c1 && (u & pmask) == prefix) {
          const int p = atomicAdd(&S.misc[4], 1);
          S.bkey[p] = u;
          S.bidx[p] = j;
        }
      }
      if (tid < 8) { S.bkey[m + tid] = 0u; S.bidx[m + tid] = 0x7fffffff; }  // sentinels
      __syncthreads();
      for (int i = tid; i < m; i += NT) {
        const uint32_t u = S.bkey[i];
        const int ji = S.bidx[i];
        int rk = 0;
        for (int t = 0; t < m; t += 8) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(&S.bkey[t]);
          const u32x4 kb = *reinterpret_cast<const u32x4*>(&S.bkey[t + 4]);
          const u32x4 ia = *reinterpret_cast<const u32x4*>(&S.bidx[t]);
          const u32x4 ib = *reinterpret_cast<const u32x4*>(&S.bidx[t + 4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            rk += (ka[q] > u) || (ka[q] == u && int(ia[q]) < ji);
            rk += (kb[q] > u) || (kb[q] == u && int(ib[q]) < ji);
          }
        }
        if (rk < want) tmp[atomicAdd(&S.misc[0], 1)] = ji;
      }
      break;
    }
    if (level == 2) {
      // more than kBoundCap identical keys: take the lowest indices, in index
      // order, one NT-wide chunk (r) at a time
      int taken = 0;
      for (int r = 0; r < KPT && taken < want; ++r) {
        const int j = r * NT + tid;
        const int f = (j >= c0 && j < c1 && kr[r] == prefix) ? 1 : 0;
        int tot2;
        const int pre = block_excl_scan<NT>(f, S.scan, &tot2);
        if (f && taken + pre < want) tmp[atomicAdd(&S.misc[0], 1)] = j;
        taken += tot2;
      }
      break;
    }
    __syncthreads();
  }
  __syncthreads();
  if (tid < 8) tmp[need + tid] = 0x7fffffff;  // sentinels for the sort
  __syncthreads();
  // ascending order by index (indices are distinct)
  for (int i = tid; i < need; i += NT) {
    const int v = tmp[i];
    int rk = 0;
    for (int t = 0; t < need; t += 8) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(&tmp[t]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(&tmp[t + 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) rk += (int(a0[q]) < v) + (int(a1[q]) < v);
    }
    out[rk] = v;
  }
  __syncthreads();
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
// ascending block ids to out.  tmp holds k + 8 ints of LDS.  Returns the count.
template <int NT, int KPT>
__device__ int select_decode_row(const uint32_t (&kr)[KPT], int nb, int k, unsigned flags,
                                 int* tmp, int* out, SelectLds& S) {
  const int tid = threadIdx.x;
  if (k >= nb) {
    for (int j = tid; j < nb; j += NT) out[j] = j;
    __syncthreads();
    return nb;
  }
  const bool sink = flags & SA_FORCE_SINK, local = flags & SA_FORCE_LOCAL;
  const int c0 = sink ? 1 : 0, c1 = local ? nb - 1 : nb;   // nb >= 2 here
  const int nfree = k - int(sink) - int(local);
  if (tid == 0) {
    if (sink) out[0] = 0;
    if (local) out[k - 1] = nb - 1;
  }
  if (nfree > 0) select_core<NT, KPT>(kr, c0, c1, nfree, tmp, out + (sink ? 1 : 0), S);
  __syncthreads();
  return k;
}

// Register tiers for KPT = ceil(nb / 256) rounded up: 2, 8 or 32 keys per thread.
__host__ __device__ inline int keys_per_thread_tier(int nb) {
  return nb <= 512 ? 2 : (nb <= 2048 ? 8 : 32);
}

}  // namespace sa
