// k_step.hip -- one whole bf16 decode step of one layer in one launch: the
// newest block's sketch refresh, the block scores, the top-k selection with
// the forced sink and local blocks, the split-K attention over the selected
// blocks and the exact log-sum-exp merge.  sa_decode_step runs it when
// SA_STEP_MODE is 1, 2 or 3; by default it runs the two-kernel step (k_score,
// then the selecting k_decode_blocks_mfma), which measures faster at the long
// decode shape: the selection handed across workgroups here costs more than
// the kernel boundary it removes.
//
// The method: score each block's mean-key sketch against the group-mean query
// (the head-averaged importance of "How Much Dense Attention is Necessary?",
// technical summary §2.1, applied per page as Quest does in "The Sparse
// Frontier", Contributi §2), keep the sink block ("Pulsar Attention", Fase 1)
// and the local block ("Faster Than Flash", Metodologia §2) and the best
// scores of the rest (ties to the lower block), attend exactly over the kept
// blocks and merge the split partials ("Pulsar Attention", Fase 2).
//
// Layout on the chip.  Workgroups are dispatched to the eight XCDs round
// robin (workgroup w runs on XCD w % 8), so the workgroups w = x, x + 8, ...
// form XCD x's team, and kv head bh belongs to team bh % 8: all of a head's
// workgroups share one L2.  A team of W workgroups gives each of its Hx heads
// S = W / Hx splits.  Split s of a head:
//   1. scores the sketch rows j = s, s + S, s + 2S, ... (strided, so that a
//      slowly drifting score profile spreads its best blocks over all
//      splits); the split owning the newest block rebuilds that sketch row
//      from K first;
//   2. ranks its candidate rows (forced blocks excluded) by counting, each
//      thread the rows above its own, and publishes the m best in rank order,
//      then arrives at the head's barrier;
//   3. reads every split's candidates and selects the top k - |forced| of
//      them: the weakest split's p-th best (p = ceil((k - |forced|) / S))
//      bounds the cut from below, since at least S p candidates reach it, so
//      only the candidates at or above it are ranked, again by counting.  The
//      union holds the exact selection unless some split kept back a block
//      that beats the cut, which shows as that split's weakest published
//      candidate being selected; then every split of the head selects from
//      the whole score row instead;
//   4. attends to its equal share of the selected 16-token tiles (the tile
//      pipeline of sa_decode_core.h) and publishes its partial;
//   5. after a second barrier merges 1/S of the head group's outputs from
//      every split's partial (split 0 also writes the ascending block list).
// Hand-offs inside a team go through the team's L2: plain stores, read back
// with sc1 loads (which skip the compute unit's L1 and see the L2's latest
// data).  A workgroup that finds itself on another XCD than its team's (the
// hardware register XCC_ID) makes its stores device-coherent and flags the
// barrier; when any member did, every member republishes with device-
// coherent stores before the candidates are read and writes its partial that
// way too, so the result never depends on where the workgroups ran.  Counters
// are device-scope atomics.  Every wait is a bounded poll; a poll that runs
// out sets the workspace's error word (the grid holds one workgroup per
// compute unit, so all of them are resident at once).
#include "sa_decode_core.h"
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_score_core.h"
#include "sa_select_core.h"

namespace sa {

struct StepArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  float* sk;                 // [BH, nb, D] sketch; row upd is rebuilt
  int B, Hq, Hkv, N, nb, k, upd;
  unsigned flags;
  float scale, sl2;
  int W;                     // workgroups per XCD team
  int coh_mode;              // 0 normal, 1 device-coherent stores throughout, 2 act off-team
  int32_t* idx;              // [BH, k]
  int32_t* count;            // [BH]
  float* score;              // [BH, nb] or null
  void* O;
  int out_bf16;
  float* lse;
  StepWs w;
  char* ws;
};

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 0xfu;
}

// Thread 0: add inc to the counter, then poll (device-scope atomic reads)
// until its low 16 bits reach `total`; returns the final value.  Bounded: on
// running out the error word gets `code`.  The counter is cleared after a
// later barrier that every member has passed.
__device__ __forceinline__ uint32_t team_barrier_t0(uint32_t* ctr, uint32_t inc, int total,
                                                    uint32_t* err, uint32_t code) {
  uint32_t v = __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
  for (int it = 0; int(v & 0xffffu) < total; ++it) {
    if (it >= kStepSpinLimit) {
      __hip_atomic_fetch_or(err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_fetch_add(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return v;
}

// A barrier that leaves its counter ready for the next call: the low 16 bits
// count arrivals, the high 16 bits a generation.  The last to arrive clears
// the count and advances the generation; the others poll for the new one.
// arrive() by thread 0 returns the value before its increment; wait() by
// thread 0 of every member but the last.
__device__ __forceinline__ uint32_t gen_arrive(uint32_t* ctr, int total) {
  const uint32_t v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (int(v & 0xffffu) == total - 1)
    __hip_atomic_fetch_add(ctr, 0x10000u - uint32_t(total), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
__device__ __forceinline__ void gen_wait(uint32_t* ctr, uint32_t v, uint32_t* err, uint32_t code) {
  for (int it = 0;; ++it) {
    const uint32_t c = __hip_atomic_fetch_add(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((c >> 16) != (v >> 16)) return;
    if (it >= kStepSpinLimit) {
      __hip_atomic_fetch_or(err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Workgroup barrier for LDS traffic only: each wave waits for its own LDS
// accesses, not for its outstanding global loads and stores (which the full
// __syncthreads would also wait for).  Global stores that another workgroup
// must see are waited for explicitly before the counters that publish them.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Number of threads of the workgroup with pred set (all threads call; ends
// after a barrier).  tmp: 4 ints of LDS.
__device__ __forceinline__ int block_count(bool pred, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = __popcll(__ballot(pred));
  if (lane == 0) tmp[wave] = c;
  lds_sync();
  const int t = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  lds_sync();
  return t;
}

// Exclusive prefix sum of v over the workgroup's 256 threads (thread order)
// and the total; tmp: 4 ints of LDS.  All threads call; ends after a barrier.
__device__ __forceinline__ int block_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = incl;
  lds_sync();
  int base = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) base += w < wave ? tmp[w] : 0;
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  lds_sync();
  return base + incl - v;
}

// Rank of entry x among keys[0, n): the number of entries above it.  R
// adjacent lanes share the count, each taking every R-th group of entries;
// eight 16-byte LDS reads are in flight per step, so the entries past n up to
// the last read must be zero.  K is the key type: 32-bit score keys (four per
// read) for the fast pass, 64-bit composites (key << 32 | ~index, two per read,
// unique) for the exact one.
constexpr int kRankBatch = 8;
template <int R, typename K>
__device__ __forceinline__ int rank_in(const K* keys, int n, K x) {
  constexpr int E = 16 / sizeof(K);              // entries per 16-byte read
  const int h = threadIdx.x % R;
  int rk = 0;
  for (int u0 = E * h; u0 < n; u0 += E * R * kRankBatch) {
    u32x4 pr[kRankBatch];
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q)
      pr[q] = *reinterpret_cast<const u32x4*>(keys + u0 + E * R * q);
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q) {
      if constexpr (E == 4) {
        rk += (pr[q][0] > x) + (pr[q][1] > x) + (pr[q][2] > x) + (pr[q][3] > x);
      } else {
        rk += ((uint64_t(pr[q][1]) << 32) | pr[q][0]) > x;
        rk += ((uint64_t(pr[q][3]) << 32) | pr[q][2]) > x;
      }
    }
  }
  if (R >= 2) rk += __shfl_xor(rk, 1, 64);
  if (R >= 4) rk += __shfl_xor(rk, 2, 64);
  return rk;
}
// Entries past n that rank_in may read (zeros): 32-bit keys with R <= 4,
// composites with R = 1.
constexpr int kRankPad32 = 4 * 4 * kRankBatch;
constexpr int kRankPad64 = 2 * kRankBatch;

// Exact ranks of the nonzero entries of comp[0, n) (64-bit composites,
// unique; their 32-bit keys in key32[], 0 for an empty entry), both zero
// padded past n: f(i, rank) once per nonzero entry, rank = the number of
// entries above it.  The ranks come from the 32-bit keys; when two of them are
// equal (the ranks of the e nonzero keys then do not sum to e (e - 1) / 2)
// they are recomputed from the composites.  All threads call; tmp: 4 ints of
// LDS.
template <typename F>
__device__ __forceinline__ void rank_all(const uint64_t* comp, const uint32_t* key32, int n,
                                         int* tmp, F f) {
  const int tid = threadIdx.x;
  const int R = n <= 64 ? 4 : (n <= 128 ? 2 : 1);
  const int per = 256 / R;
  int rr[2];
  int sum = 0, nz = 0;
  rr[0] = rr[1] = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c * per >= n) break;                     // uniform: no entries in the second round
    const int i = tid / R + c * per;
    const uint32_t x = i < n ? key32[i] : 0u;
    int v = 0;
    if (R == 4) v = rank_in<4>(key32, n, x);
    else if (R == 2) v = rank_in<2>(key32, n, x);
    else v = rank_in<1>(key32, n, x);
    rr[c] = v;
    const bool mine = tid % R == 0 && x != 0u;
    sum += mine ? v : 0;
    nz += mine ? 1 : 0;
  }
  int total, e;
  block_scan(sum, tmp, &total);
  block_scan(nz, tmp, &e);
  const bool ties = long(total) != long(e) * (e - 1) / 2;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = tid / R + c * per;
    if (c * per < n && i < n && tid % R == 0 && key32[i] != 0u && !ties) f(i, rr[c]);
  }
  if (!ties) return;
  for (int i = tid; i < n; i += 256)
    if (key32[i] != 0u) f(i, rank_in<1>(comp, n, comp[i]));
}

template <int D, int G, int BLOCK>
__global__ __launch_bounds__(256, 2) void k_decode_step(StepArgs a) {
  constexpr int TPB = BLOCK / 16;      // 16-token tiles per block
  constexpr int LPR = D / 4;           // lanes per sketch row (16-byte segments)
  constexpr int RPI = 64 / LPR;        // sketch rows per wave load
  constexpr int NU = 16;               // row loads per lane in flight
  constexpr int RB = 4 * RPI * NU;     // rows per batch
  constexpr int KPT = 32;              // keys per thread of the whole-row fallback
  constexpr int QC = 8;                // candidate loads per thread (S * 8 * TPS >= every m)
  __shared__ SelectLdsT<256, KPT> sel;
  __shared__ CombineLds<D, G> cmb;
  __shared__ ScoreUpdLds<D> upl;
  __shared__ float s_sc[kStepMaxRows];
  __shared__ __attribute__((aligned(16))) uint64_t s_key[kStepMaxCand + kRankPad64];
  __shared__ __attribute__((aligned(16))) uint32_t s_k32[kStepMaxCand + kRankPad32];
  __shared__ int s_rank[kStepMaxRows];
  __shared__ unsigned char s_fmin[kStepMaxCand];
  __shared__ int s_list[kMaxKFused];
  __shared__ __attribute__((aligned(16))) f32x4 s_ma[kStepMergeEnt];
  __shared__ float s_mm[kStepMergeEnt], s_ml[kStepMergeEnt];
  __shared__ int s_tmp[8];
  __shared__ int s_misc[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int BH = a.B * a.Hkv;
  const int Hx = x < BH ? (BH - x + 7) >> 3 : 0;
  if (Hx == 0) return;
  const int S = a.W / Hx;
  const int hi = r / S, s = r - hi * S;
  if (hi >= Hx) return;
  const int bh = x + 8 * hi;
  const int b = bh / a.Hkv, kh = bh - b * a.Hkv;
  const int nb = a.nb, N = a.N, k = a.k;
  const bool off = a.coh_mode == 2 || xcc_id() != uint32_t(x);
  const bool coh1 = a.coh_mode == 1 || off;          // this workgroup's first publication

  char* ws = a.ws;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws + a.w.ctr_off) + size_t(bh) * 3 * kCounterStride;
  uint64_t* pub = reinterpret_cast<uint64_t*>(ws + a.w.pub_off) + size_t(bh) * a.W * kStepPubWords;
  float* srow = reinterpret_cast<float*>(ws + a.w.srow_off) + size_t(bh) * a.W * kStepMaxRows;
  float* pacc = reinterpret_cast<float*>(ws + a.w.acc_off) + size_t(bh) * G * a.W * D;
  float* pml = reinterpret_cast<float*>(ws + a.w.ml_off) + size_t(bh) * G * a.W * 2;

  const bool sink = a.flags & SA_FORCE_SINK, local = a.flags & SA_FORCE_LOCAL;
  const int c0 = sink ? 1 : 0, c1 = local ? nb - 1 : nb;   // candidate blocks [c0, c1)
  const int nF = (sink ? 1 : 0) + (local && nb > 1 ? 1 : 0);
  const int need = k - nF;
  const bool all = k >= nb;                 // every block kept
  const bool team_sel = !all && need > 0;   // selection among candidates

  // ------------------------------------------------ 1. scores of this split's rows
  const int R = s < nb ? (nb - 1 - s) / S + 1 : 0;
  const uint16_t* Qg = a.Q + (size_t(b) * a.Hq + kh * G) * D;
  {
    const int sub = lane / LPR, lc = lane % LPR;
    const float* skb = a.sk + size_t(bh) * nb * D;
    QCol<uint16_t> qv[8];
    score_q_issue<uint16_t, D>(Qg, G, lc, qv);
    __builtin_amdgcn_sched_barrier(0);
    for (int r0 = 0; r0 < R; r0 += RB) {
      u32x4 wv[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int i = r0 + (u * 4 + wave) * RPI + sub;
        const int j = min(s + S * min(i, R - 1), nb - 1);
        wv[u] = ld16(skb + size_t(j) * D + lc * 4);
      }
      __builtin_amdgcn_sched_barrier(0);
      float q[4];
      score_q_finish<uint16_t, D>(Qg, G, lc, a.scale, qv, q);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int i = r0 + (u * 4 + wave) * RPI + sub;
        const float p = score_row<D>(q, wv[u]);
        if (i < R && lc == LPR - 1) s_sc[i] = p;
      }
    }
  }
  // The newest block's sketch row is rebuilt from K by the split owning it.
  // When that block is forced (the local or the sink block, or every block is
  // kept) its score cannot change the selection, so the rebuild waits until
  // the end of the step, off its critical path.
  const bool upd_mine = a.upd >= 0 && a.upd % S == s;
  const bool upd_late = all || (local && a.upd == nb - 1) || (sink && a.upd == 0);
  auto refresh = [&]() {
    const int t0 = a.upd * BLOCK, nj = min(BLOCK, N - t0);
    const float p = score_update_block<uint16_t, D>(a.K + (size_t(bh) * N + t0) * D, nj, Qg, G,
                                                    a.scale, a.sk + (size_t(bh) * nb + a.upd) * D,
                                                    upl);
    if (tid == 0 && a.score) a.score[size_t(bh) * nb + a.upd] = p;
    return p;
  };
  if (upd_mine && !upd_late) {
    const float p = refresh();
    if (tid == 0) s_sc[a.upd / S] = p;
  }
  lds_sync();

  // ------------------------------------------------ 2. this split's candidates
  // Thread t owns slot t of this split (R <= 256): block j = s + S t.
  const int jt = s + S * tid;
  const bool own = tid < R;
  const float sv = own ? s_sc[tid] : 0.f;
  if (own && a.score && !(upd_late && jt == a.upd)) a.score[size_t(bh) * nb + jt] = sv;
  const bool el = own && jt >= c0 && jt < c1;
  const uint64_t xk = el ? (uint64_t(score_key(sv)) << 32) | uint32_t(~jt) : 0ull;
  const int m = min(kStepPubCap, max(16, (2 * need + S - 1) / S + 8));
  bool anyoff = true;          // without a team barrier the partials go device-coherent
  if (team_sel) {
    // eligible rows: all but block 0 (sink) and block nb - 1 (local) when they fall here
    int n_el = R;
    if (sink && s == 0 && R > 0) --n_el;
    if (local && nb > 1 && nb - 1 >= s && (nb - 1 - s) % S == 0) --n_el;
    const bool full = n_el > m;
    // the slots' keys (0 for rows that are no candidates), zeros past R
    s_key[tid] = xk;
    s_k32[tid] = uint32_t(xk >> 32);
    if (tid < kRankPad32) s_k32[256 + tid] = 0u;
    if (tid < kRankPad64) s_key[256 + tid] = 0ull;
    lds_sync();
    rank_all(s_key, s_k32, R, s_tmp, [&](int i, int rr) { s_rank[i] = rr; });
    lds_sync();
    const int rk = el ? s_rank[tid] : 0x7fffffff;
    const bool pubd = el && rk < m;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(srow + size_t(s) * kStepMaxRows, kStepMaxRows * 4);
    const __amdgpu_buffer_rsrc_t rPub = make_rsrc(pub, uint32_t(S) * kStepPubWords * 8);
    auto publish = [&](bool coh) {
      const int base = s * kStepPubWords * 8;
      const u32x2 w = u32x2{uint32_t(xk), uint32_t(xk >> 32)};
      if (own) {
        if (coh) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), rS, tid * 4, 0, kCoherent);
        else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), rS, tid * 4, 0, 0);
      }
      if (pubd) {
        if (coh) bst8c(rPub, base + (2 + rk) * 8, w); else bst8(rPub, base + (2 + rk) * 8, w);
        // the weakest published candidate of a full split
        if (full && rk == m - 1) { if (coh) bst8c(rPub, base + 8, w); else bst8(rPub, base + 8, w); }
      }
      if (tid == 0) {
        const u32x2 h0 = u32x2{uint32_t(min(n_el, m)), full ? 1u : 0u};
        if (coh) bst8c(rPub, base, h0); else bst8(rPub, base, h0);
      }
      __builtin_amdgcn_s_waitcnt(0);
      lds_sync();
    };
    publish(coh1);
    // ------------------------------------------------ 3. team barrier, selection
    if (tid == 0) {
      const uint32_t v = team_barrier_t0(ctr, off ? 0x10001u : 1u, S, err, 1u);
      s_misc[0] = int(v >> 16);
    }
    lds_sync();
    const bool someoff = s_misc[0] != 0;
    anyoff = someoff || a.coh_mode == 1;
    if (someoff && a.coh_mode != 1) {
      // someone ran off the team's XCD: republish device-coherently, wait again
      publish(true);
      if (tid == 0) team_barrier_t0(ctr + kCounterStride, 1u, S, err, 2u);
      lds_sync();
    }
    // every split's candidates: split ss = tid / TPS, positions tid % TPS + TPS q
    const int TPS = 256 / S;
    const int ss = tid / TPS, sl = tid - ss * TPS;
    const bool act = ss < S;
    const int p = (need + S - 1) / S;                 // S p >= need
    const int base = (act ? ss : 0) * kStepPubWords * 8;
    const u32x2 hdr = bld8c(rPub, base);
    u32x2 cw[QC];
#pragma unroll
    for (int q = 0; q < QC; ++q) cw[q] = bld8c(rPub, base + (2 + min(sl + TPS * q, kStepPubCap - 1)) * 8);
    const int cnt_ss = act ? int(hdr[0]) : 0;
    const bool full_ss = act && hdr[1] != 0u;
    uint64_t cx[QC];
#pragma unroll
    for (int q = 0; q < QC; ++q)
      cx[q] = act && sl + TPS * q < cnt_ss ? (uint64_t(cw[q][1]) << 32) | cw[q][0] : 0ull;
    // pass 1: the `need`-th best of the splits' p best is a lower bound of the
    // cut (at least `need` candidates reach it); 0 when a split has fewer than p
    int na = 0;
#pragma unroll
    for (int q = 0; q < QC; ++q) na += cx[q] != 0ull && sl + TPS * q < p ? 1 : 0;
    int A;
    int pos = block_scan(na, s_tmp, &A);
#pragma unroll
    for (int q = 0; q < QC; ++q)
      if (cx[q] != 0ull && sl + TPS * q < p) {
        if (pos < kStepMaxCand) { s_key[pos] = cx[q]; s_k32[pos] = uint32_t(cx[q] >> 32); }
        ++pos;
      }
    const bool short_split = block_count(act && sl == 0 && cnt_ss < p, s_tmp) != 0;
    A = min(A, kStepMaxCand);
    if (tid < kRankPad32) s_k32[A + tid] = 0u;
    if (tid < kRankPad64) s_key[A + tid] = 0ull;
    if (tid == 0) { s_misc[5] = 0; s_misc[6] = 0; }
    lds_sync();
    if (!short_split && A >= need) {
      rank_all(s_key, s_k32, A, s_tmp, [&](int i, int rr) {
        if (rr == need - 1) {
          s_misc[5] = int(uint32_t(s_key[i] >> 32));
          s_misc[6] = int(uint32_t(s_key[i]));
        }
      });
    }
    lds_sync();
    const uint64_t T0 = (uint64_t(uint32_t(s_misc[5])) << 32) | uint32_t(s_misc[6]);
    // pass 2: every candidate at or above the bound, ranked; the top `need` go
    // to list slots nF + rank
    bool in[QC];
    int nin = 0;
#pragma unroll
    for (int q = 0; q < QC; ++q) {
      in[q] = cx[q] != 0ull && cx[q] >= T0;
      nin += in[q] ? 1 : 0;
    }
    int C;
    pos = block_scan(nin, s_tmp, &C);
#pragma unroll
    for (int q = 0; q < QC; ++q) {
      if (in[q]) {
        if (pos < kStepMaxCand) {
          s_key[pos] = cx[q];
          s_k32[pos] = uint32_t(cx[q] >> 32);
          s_fmin[pos] = full_ss && sl + TPS * q == m - 1;
        }
        ++pos;
      }
    }
    const bool capped = C > kStepMaxCand;
    C = min(C, kStepMaxCand);
    if (tid < kRankPad32) s_k32[C + tid] = 0u;
    if (tid < kRankPad64) s_key[C + tid] = 0ull;
    lds_sync();
    bool bad = false;
    rank_all(s_key, s_k32, C, s_tmp, [&](int i, int rr) {
      if (rr < need) {
        s_list[nF + rr] = int(~uint32_t(s_key[i]));
        bad = bad || s_fmin[i];
      }
    });
    // a capped list, or fewer bracketed candidates than slots, cannot be trusted
    bad = bad || (tid == 0 && (capped || C < need));
    const bool fallback = block_count(bad, s_tmp) != 0;
    if (tid == 0) {
      int f = 0;
      if (sink) s_list[f++] = 0;
      if (local && nb > 1) s_list[f++] = nb - 1;
      s_misc[2] = nF + need;
    }
    if (fallback) {
      // the whole score row, from every split's slot row
      const __amdgpu_buffer_rsrc_t rR = make_rsrc(srow, uint32_t(S) * kStepMaxRows * 4);
      uint32_t kx[KPT];
#pragma unroll
      for (int q = 0; q < KPT; ++q) {
        const int j = q * 256 + tid;
        const int jc = min(j, nb - 1);
        const int o = ((jc % S) * kStepMaxRows + jc / S) * 4;
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rR, o, 0, kCoherent);
        kx[q] = j < nb ? score_key(__uint_as_float(v)) : 0u;
      }
      lds_sync();
      const int P = select_decode_row<256, KPT>(kx, nb, k, a.flags, s_list, sel);
      if (tid == 0) s_misc[2] = P;
    }
  } else {
    if (all) {
      for (int j = tid; j < nb; j += 256) s_list[j] = j;
    } else if (tid == 0) {
      int f = 0;
      if (sink) s_list[f++] = 0;
      if (local && nb > 1) s_list[f++] = nb - 1;
    }
    if (tid == 0) s_misc[2] = all ? nb : nF;
  }
  lds_sync();
  const int P = s_misc[2];

  // ------------------------------------------------ 4. attention over this split's tiles
  const int T = P * TPB;
  const int g0 = int((long(s) * T) / S), g1 = int((long(s + 1) * T) / S);
  u32x4 qb[D / 32];
  tile_q_operand<D, G>(Qg, qb);
  TileAcc<D> ta;
  tile_acc_init(ta);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(a.K + size_t(bh) * N * D, uint32_t(N) * D * 2);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.V + size_t(bh) * N * D, uint32_t(N) * D * 2);
  run_tiles<D, G>(ta, qb, KRowsBf16<D>{rK}, rV, N, a.sl2, g1 - g0, [&](int t) {
    const int u = g0 + t;
    const int tok0 = s_list[u / TPB] * BLOCK + (u % TPB) * 16;
    return tok0 < N ? tok0 : -1;
  });
  store_partial<D, G>(ta, cmb, pacc, pml, S, s, anyoff);

  // ------------------------------------------------ 5. barrier, then 1/S of the merge
  __builtin_amdgcn_s_waitcnt(0);
  lds_sync();
  uint32_t* c3 = ctr + 2 * kCounterStride;
  if (tid == 0) s_misc[4] = int(gen_arrive(c3, S));
  lds_sync();
  const uint32_t v3 = uint32_t(s_misc[4]);
  if (s == 0) {
    // the ascending block list while the other splits arrive
    const int W = (nb + 31) >> 5;
    if (tid < W) sel.bm[tid] = 0u;
    lds_sync();
    for (int j = tid; j < P; j += 256) sel_mark(sel.bm, s_list[j]);
    int32_t* orow = a.idx + size_t(bh) * k;
    const int tot = sel_bitmap_to_list(sel, W, orow, k);   // starts with a barrier
    for (int j = tot + tid; j < k; j += 256) orow[j] = -1;
    if (tid == 0) a.count[bh] = tot;
  }
  if (tid == 0 && int(v3 & 0xffffu) != S - 1) gen_wait(c3, v3, err, 4u);
  lds_sync();
  if (s == 0 && tid == 0) {
    // every split has passed the first barriers: clear them for the next call
    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ctr + kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  {
    // this split's outputs: [s OPW, (s + 1) OPW) of the group's G * D, four
    // columns per entry; entry e = split s2 + S * chunk
    const int GD = G * D;
    const int OPW = ((GD + S - 1) / S + 3) & ~3;
    const int NC = OPW / 4;
    const int o0 = s * OPW;
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(pacc, uint32_t(G) * S * D * sizeof(float));
    const __amdgpu_buffer_rsrc_t rM = make_rsrc(pml, uint32_t(G) * S * 8);
    for (int e = tid; e < S * NC; e += 256) {
      const int s2 = e % S, c = e / S, o = o0 + 4 * c;
      const int h = min(o, GD - 1) / D, d = min(o, GD - 1) % D;
      const int pi = h * S + s2;
      const u32x4 av = bld16c(rP, o < GD ? (pi * D + d) * int(sizeof(float)) : kBufOOB, 0);
      const u32x2 mv = bld8c(rM, o < GD ? pi * 8 : kBufOOB);
      s_ma[e] = __builtin_bit_cast(f32x4, av);
      s_mm[e] = o < GD ? __uint_as_float(mv[0]) : -__builtin_inff();
      s_ml[e] = __uint_as_float(mv[1]);
    }
    lds_sync();
    for (int c = tid; c < NC; c += 256) {
      const int o = o0 + 4 * c;
      if (o >= GD) continue;
      const int h = o / D, d = o % D;
      float M = -__builtin_inff();
      for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, s_mm[s2 + S * c]);
      float L = 0.f;
      f32x4 A = f32x4{0.f, 0.f, 0.f, 0.f};
      if (M != -__builtin_inff()) {
        for (int s2 = 0; s2 < S; ++s2) {
          const int e = s2 + S * c;
          const float f = exp2_fast(s_mm[e] - M);
          L += s_ml[e] * f;
          const f32x4 v = s_ma[e];
#pragma unroll
          for (int q = 0; q < 4; ++q) A[q] += v[q] * f;
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const size_t oi = size_t(b * a.Hq + kh * G + h) * D + d;
      if (a.out_bf16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.O) + oi) =
            u32x2{pack_bf16x2(A[0] * inv, A[1] * inv), pack_bf16x2(A[2] * inv, A[3] * inv)};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + oi) =
            f32x4{A[0] * inv, A[1] * inv, A[2] * inv, A[3] * inv};
      }
      if (a.lse && d == 0)
        a.lse[b * a.Hq + kh * G + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
    }
  }
  if (upd_mine && upd_late) refresh();
}

// ---------------------------------------------------------------- launcher
template <int D, int BLOCK>
static void launch_step_g(const StepArgs& a, int G, dim3 g, hipStream_t st) {
  switch (G) {
    case 1: k_decode_step<D, 1, BLOCK><<<g, 256, 0, st>>>(a); break;
    case 2: k_decode_step<D, 2, BLOCK><<<g, 256, 0, st>>>(a); break;
    case 4: k_decode_step<D, 4, BLOCK><<<g, 256, 0, st>>>(a); break;
    default: k_decode_step<D, 8, BLOCK><<<g, 256, 0, st>>>(a); break;
  }
}

hipError_t launch_decode_step(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                              int N, int D, int block, float* sk, int upd, int k, unsigned flags,
                              float scale, int32_t* idx, int32_t* count, float* score, void* O,
                              int out_dtype, float* lse, void* ws, int coh_mode, hipStream_t st) {
  StepArgs a;
  a.Q = static_cast<const uint16_t*>(Q);
  a.K = static_cast<const uint16_t*>(K);
  a.V = static_cast<const uint16_t*>(V);
  a.sk = sk;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.nb = cdiv(N, block); a.k = k; a.upd = upd;
  a.flags = flags;
  a.scale = scale; a.sl2 = scale * kLog2e;
  a.W = kStepTeam;
  a.coh_mode = coh_mode;
  a.idx = idx; a.count = count; a.score = score;
  a.O = O; a.out_bf16 = out_dtype == SA_BF16; a.lse = lse;
  a.w = step_ws(B, Hq, Hkv, D);
  a.ws = static_cast<char*>(ws);
  const dim3 g(8 * kStepTeam);
  const int G = Hq / Hkv;
  if (D == 128) {
    if (block == 64) launch_step_g<128, 64>(a, G, g, st);
    else             launch_step_g<128, 128>(a, G, g, st);
  } else {
    if (block == 64) launch_step_g<64, 64>(a, G, g, st);
    else             launch_step_g<64, 128>(a, G, g, st);
  }
  return hipGetLastError();
}

}  // namespace sa
