// k_decode.hip -- split-K sparse decode attention with a fused log-sum-exp merge.
//
// Exact softmax attention recomputed on the selected support with the
// original q, K, V ("How Much Dense Attention is Necessary?", technical
// summary §2.1); only the chosen blocks are fetched from the retained cache
// ("Faster Than Flash", Metodologia §3 refinement stage; Quest in "The Sparse
// Frontier", Contributi §2).  Each split produces an online-softmax partial
// (m, l, sum p v) and the partials are merged exactly ("Pulsar Attention",
// Fase 2: online-softmax merge of per-shard attention).  The merge runs in the
// same launch: the last split workgroup of a head group to finish (an arrival
// counter; partials written and read with agent-coherent accesses) combines
// all partials.
//
// k_decode_blocks_mfma (bf16): one 256-thread workgroup per (b, kv head,
//   split); a split takes an equal share of the head's 16-token tiles.  A
//   tile is one wave's unit of work; each wave issues the loads of up to four
//   tiles before computing any of them.  The selecting variant first runs the
//   selection pre-filter of its head from the score row, then takes its tiles
//   from its own slice of the candidate list (ranking only those candidates)
//   or, when the list does not suit slices, from the fully ranked selection.  Scores of the g
//   heads for 16 tokens are one chain of v_mfma_f32_16x16x32_bf16 with the key
//   rows as the A operand and the group's queries as the B operand -- both
//   read in their natural row-major layout (contraction over d), so keys go
//   straight from HBM into matrix-core registers.  The score tile comes out
//   with lane l holding head l%16 for tokens 4*(l/16)+r, which is exactly the
//   A-operand layout of v_mfma_f32_16x16x16_bf16 for P V.  V rows are loaded as
//   row vectors and transposed in registers with v_perm_b32 so the value
//   columns land in the B operand (column d = (D/16)*n + e of MFMA e).  P is
//   split as p ~ hi + lo (two bf16) and the lo part fills the padding
//   rows g..2g-1 of the 16-row tile, so the value product is accurate to about
//   2^-17 relative with float32 accumulation.  Workgroup id % (B*Hkv) selects
//   the (b, kv head): all splits of one kv head share an XCD and its L2.
// k_decode_blocks_valu (float32): per-thread dot products, LDS softmax over
//   1024-token chunks, (head, column)-parallel value pass; float32 throughout.
// k_decode_tokens: per (b, query head, split) over an explicit token list
//   (threshold selection), reusing the selector's scores when given.
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_select_core.h"

namespace sa {

struct DecodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  int B, Hq, Hkv, G, N, block;
  float scale, sl2;
  const int32_t* idx;
  const int32_t* count;
  int idx_stride;
  const float* score;
  int S;
  float* pacc;
  float* pml;
  uint32_t* counter;
  void* O;
  int out_bf16;
  float* lse;
  // in-kernel selection (decode step): scores [B*Hkv, nb] -> top-k per row
  const float* sel_scores;
  int nb, k;
  unsigned flags;
  int32_t* sel_idx;
  int32_t* sel_count;
  int32_t* sel_ent;   // [B*Hkv, kSelEntCap] kept block (or -1) per entry of a row
};
static_assert(kSelWords * 32 >= kMaxNbDecode, "one bitmap word per 32 blocks of a row");
static_assert(2 + kCandCap <= kSelEntCap && kSelEntCap <= 3 * 256, "entries of a row: forced blocks and candidates");

// ---------------------------------------------------------------- merge tail
// Partials cross workgroups through the workspace with agent-coherent (sc1)
// stores and loads -- the accesses the compiler emits for agent-scope atomic
// stores and loads -- so no L2 writeback or invalidate is needed.
//
// Publish this workgroup's partial and count arrivals; true for the last one.
// Every wave waits until its sc1 stores have completed (s_waitcnt), then one
// thread increments the counter; an atomic is performed at the device's
// coherent level, so when it returns total - 1 every other workgroup's stores
// had completed before its increment, and the last one's sc1 loads, issued
// after that, see them.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            uint32_t(total - 1);
  __syncthreads();
  if (!*flag) return false;
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Merge the S partials of query heads h0 .. h0+nh-1 (rows of [B*Hq]):
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum acc_s 2^(m_s - M) / L,
// lse = (M + log2 L) ln 2 (scores are kept in log2 units).
// Thread t owns head t / (D/4) and 4 consecutive columns (nh * D / 4 <= 256).
// Its first kMergeChunk partial loads and the (m, l) pair loads are issued
// first; mid() (all threads call it) runs while they are in flight.  The
// pairs are staged in LDS, one row per head of stride Sp (S up to
// kMergeRegSplits: Sp = kMergeRegSplits, so one unrolled branch-free pass of
// 16-byte LDS reads serves every split; else S rounded up to 4), padded with
// m = -inf, l = 0.  Beyond kMergeRegSplits the rest follow 8 at a time.
constexpr int kMergeChunk = 32;
constexpr int kMergeRegSplits = 32;

struct NoMid {
  __device__ void operator()() const {}
};

template <int D, typename Mid = NoMid>
__device__ void merge_tail(const DecodeArgs& a, int h0, int nh, float* w, float* lv,
                           Mid mid = Mid()) {
  constexpr int CH = kMergeChunk, SR = kMergeRegSplits;
  static_assert(SR == CH && CH % 4 == 0, "one chunk holds the register path");
  const int S = a.S, Sp = S <= SR ? SR : (S + 3) & ~3, tid = threadIdx.x;
  const bool act = tid < nh * (D / 4);
  const int h = act ? tid / (D / 4) : 0, d0 = (tid % (D / 4)) * 4;
  // the head group's partials through one buffer resource: a lane offset plus
  // a scalar offset per split
  const __amdgpu_buffer_rsrc_t rP =
      make_rsrc(a.pacc + size_t(h0) * S * D, uint32_t(nh) * S * D * sizeof(float));
  const int voff = (h * S * D + d0) * int(sizeof(float));
  u32x4 v[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) v[u] = bld16c(rP, voff, min(u, S - 1) * D * int(sizeof(float)));
  // (m, l) pairs: nh * S <= 8 * kMaxSplits = 4 per thread
  static_assert(8 * kMaxSplits <= 4 * 256, "pairs per thread");
  const int np = nh * S;
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(a.pml + 2 * size_t(h0) * S, uint32_t(np) * 8);
  u32x2 ml[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) ml[q] = bld8c(rM, min(tid + 256 * q, np - 1) * 8);
  mid();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = tid + 256 * q;
    if (i < np) {
      const int hh = i / S, ss = i - hh * S;
      w[hh * Sp + ss] = __uint_as_float(ml[q][0]);
      lv[hh * Sp + ss] = __uint_as_float(ml[q][1]);
    }
  }
  for (int i = tid; i < nh * (Sp - S); i += 256) {
    const int hh = i / (Sp - S), ss = S + i % (Sp - S);
    w[hh * Sp + ss] = -__builtin_inff();
    lv[hh * Sp + ss] = 0.f;
  }
  __syncthreads();
  if (!act) return;
  const float* wh = w + h * Sp;
  const float* lh = lv + h * Sp;
  float M = -__builtin_inff();
  float L = 0.f;
  f32x4 A = f32x4{0.f, 0.f, 0.f, 0.f};
  if (S <= SR) {
    // every partial is already loaded: M from the staged m row, then one
    // unrolled pass of (m, l) 16-byte LDS reads (the -inf padding weighs 0)
    f32x4 m4[SR / 4];
#pragma unroll
    for (int q = 0; q < SR / 4; ++q) {
      m4[q] = *reinterpret_cast<const f32x4*>(wh + 4 * q);
      M = fmaxf(M, fmaxf(fmaxf(m4[q][0], m4[q][1]), fmaxf(m4[q][2], m4[q][3])));
    }
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int q = 0; q < SR / 4; ++q) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lh + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = exp2_fast(m4[q][e] - M);
          L += l4[e] * f;
#pragma unroll
          for (int c = 0; c < 4; ++c) A[c] += __uint_as_float(v[4 * q + e][c]) * f;
        }
      }
    }
  } else {
    for (int s = 0; s < S; ++s) M = fmaxf(M, wh[s]);
    if (M != -__builtin_inff()) {
      // the first CH partials are loaded; the rest follow 8 at a time
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const float f = exp2_fast(wh[u] - M);
        L += lh[u] * f;
#pragma unroll
        for (int c = 0; c < 4; ++c) A[c] += __uint_as_float(v[u][c]) * f;
      }
      for (int s0 = CH; s0 < S; s0 += 8) {
        u32x4 w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          w8[u] = bld16c(rP, voff, min(s0 + u, S - 1) * D * int(sizeof(float)));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (s0 + u < S) {
            const float f = exp2_fast(wh[s0 + u] - M);
            L += lh[s0 + u] * f;
#pragma unroll
            for (int c = 0; c < 4; ++c) A[c] += __uint_as_float(w8[u][c]) * f;
          }
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t oi = size_t(h0 + h) * D + d0;
  if (a.out_bf16) {
    const u32x2 pk = u32x2{pack_bf16x2(A[0] * inv, A[1] * inv), pack_bf16x2(A[2] * inv, A[3] * inv)};
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.O) + oi) = pk;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + oi) = f32x4{A[0] * inv, A[1] * inv, A[2] * inv, A[3] * inv};
  }
  if (a.lse && d0 == 0) a.lse[h0 + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------- bf16 MFMA
constexpr int kTileBatch = 4;

template <int D, int G, int BLOCK, int SELKPT>
__global__ __launch_bounds__(256, 2) void k_decode_blocks_mfma(DecodeArgs a) {
  constexpr bool SEL = SELKPT > 0;
  static_assert(2 * G <= 16, "g must be at most 8");
  constexpr int NST = D / 32;      // contraction steps of the score MFMA
  constexpr int EPL = D / 16;      // value columns per lane = PV MFMAs per tile
  constexpr int TPB = BLOCK / 16;  // 16-token tiles per block
  __shared__ __attribute__((aligned(16))) float s_acc[4][2 * G][D + 4];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ __attribute__((aligned(16))) float s_w[G * kMaxSplits], s_lv[G * kMaxSplits];
  __shared__ int s_flag;

  const int BH = a.B * a.Hkv, N = a.N;
  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nn = lane & 15;

  // Work is split by 16-token tiles: split s takes tiles [g0, g0 + tps) of
  // the head's slot list (slot = tile / TPB).  The range comes from
  // idx_stride, so the index loads do not wait for count; slots at or past
  // count are skipped.
  const int tps = (a.idx_stride * TPB + a.S - 1) / a.S;
  const int g0 = s * tps;
  int ntiles = max(min(g0 + tps, a.idx_stride * TPB) - g0, 0);
  int cnt = 0;
  const int32_t* ib = nullptr;
  constexpr int KPT = SEL ? SELKPT : 1;
  SelectLdsT<256, KPT>* selp = nullptr;
  // slice mode of the selecting kernel: the head's splits own tile slices of
  // the candidate list instead of the ranked selection
  bool cmode = false;
  const int* wl = nullptr;   // this wave's kept tiles (token offsets), slice mode
  const int* es = nullptr;   // kept block or -1 of the entries this split owns
  int cm_E = 0, cm_ea = 0, cm_ne = 0, cm_u0 = 0;
  if constexpr (SEL) {
    // every split runs the selection pre-filter of its kv head from the score row
    extern __shared__ __attribute__((aligned(16))) int dyn_i[];   // max(k, 320) ints
    __shared__ SelectLdsT<256, KPT> S;
    selp = &S;
    int* list = dyn_i;
    const int nb = a.nb, k = a.k;
    const bool sink = a.flags & SA_FORCE_SINK, local = a.flags & SA_FORCE_LOCAL;
    const int F = int(sink) + int(local), need = k - F, W = (nb + 31) >> 5;
    uint32_t kr[KPT];
    load_keys_reg<256, KPT>(a.sel_scores + size_t(bh) * nb, nb, kr);
    if (k >= nb) {
      for (int j = tid; j < nb; j += 256) list[j] = j;
      __syncthreads();
      cnt = nb;
    } else {
      sel_init(S, W);
      int ix[KPT];   // keys masked in place
      int C = -1;
      if (need > 0) {
        const uint32_t tmax = sel_mask_keys<256, KPT>(kr, sink ? 1 : 0, local ? nb - 1 : nb, kr, ix);
        C = sel_prefilter<256, KPT>(kr, ix, tmax, need, S);
      }
      // entries [forced blocks, candidates] of TPB tiles each: split s owns
      // the tiles [s*cpu, s*cpu + cpu) of that sequence
      const int E = F + C, U = E * TPB, cpu = (U + a.S - 1) / a.S;
      cmode = C >= 0 && cpu <= 64;
      if (cmode) {
        // rank only the entries of the owned tiles (every wave does it, so no
        // barrier; each keeps its own copy of the kept tiles, in tile order)
        const int u0 = s * cpu, u1 = min(u0 + cpu, U);
        const int ea = u0 / TPB, ne = u1 > u0 ? (u1 - 1) / TPB - ea + 1 : 0;
        const int g = lane >> 3, h = lane & 7;
        int* tl = list + wave * 64;
        int* el = list + 256;   // written and read by wave 0 only
        int nk = 0;
        for (int j0 = 0; j0 < ne; j0 += 8) {
          const int e = ea + j0 + g;
          const bool in = j0 + g < ne, forced = e < F;
          const uint64_t x = S.cand[min(max(e - F, 0), C - 1)];
          const int rk = sel_rank_entry8<256, KPT>(x, C, S);
          const int blk = forced ? (sink && e == 0 ? 0 : nb - 1) : int(~uint32_t(x));
          const uint64_t km = __ballot(h == 7 && (forced || rk < need));
          const bool keep = (km >> (8 * g + 7)) & 1ull;
          // the split holding an entry's first tile reports it
          if (wave == 0 && h == 7 && in && e * TPB >= u0) el[j0 + g] = keep ? blk : -1;
          // lane h < TPB stands for tile h of entry e
          const int u = e * TPB + h, tok0 = blk * BLOCK + h * 16;
          const bool take = keep && in && h < TPB && u >= u0 && u < u1 && tok0 < N;
          const uint64_t tm = __ballot(take);
          if (take) tl[nk + __popcll(tm & ((1ull << lane) - 1ull))] = tok0;
          nk += __popcll(tm);
        }
        wl = tl;
        es = el;
        ntiles = nk;
        cm_E = E; cm_ea = ea; cm_ne = ne; cm_u0 = u0;
      } else {
        if (C >= 0) {
          sel_rank_all<256, KPT>(C, need, S);
        } else if (need > 0) {
          bool cand[KPT];
#pragma unroll
          for (int r = 0; r < KPT; ++r) cand[r] = kr[r] != 0u;
          sel_mark_top_kv<256, KPT, KPT>(kr, ix, cand, nb - F, need, S);
        } else {
          __syncthreads();   // publishes sel_init before the forced marks
        }
        if (tid == 0) {
          if (sink) sel_mark(S.bm, 0);
          if (local) sel_mark(S.bm, nb - 1);
        }
        cnt = sel_bitmap_to_list(S, W, list, k);
      }
    }
    if (!cmode) {
      ib = list;
      if (s == 0) {
        int32_t* orow = a.sel_idx + size_t(bh) * k;
        for (int j = tid; j < k; j += 256) orow[j] = j < cnt ? list[j] : -1;
        if (tid == 0) a.sel_count[bh] = cnt;
      }
    }
  } else {
    cnt = a.count ? min(max(a.count[bh], 0), a.idx_stride) : a.idx_stride;
    ib = a.idx + size_t(bh) * a.idx_stride;
  }

  const uint16_t* Q = static_cast<const uint16_t*>(a.Q);
  u32x4 qb[NST];
  if (nn < G) {
    const uint16_t* qp = Q + (size_t(b) * a.Hq + kh * G + nn) * D + 8 * gq;
#pragma unroll
    for (int st = 0; st < NST; ++st) qb[st] = ld16(qp + 32 * st);
  } else {
#pragma unroll
    for (int st = 0; st < NST; ++st) qb[st] = u32x4{0u, 0u, 0u, 0u};
  }

  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x4 acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-(b, kv head) buffer resources: rows past N (and invalid tiles) read as
  // zeros, so every load of a batch issues unconditionally
  const __amdgpu_buffer_rsrc_t rK =
      make_rsrc(static_cast<const uint16_t*>(a.K) + size_t(bh) * N * D, uint32_t(N) * D * 2);
  const __amdgpu_buffer_rsrc_t rV =
      make_rsrc(static_cast<const uint16_t*>(a.V) + size_t(bh) * N * D, uint32_t(N) * D * 2);
  const int nbk = (N + BLOCK - 1) / BLOCK;
  const float sl2 = a.sl2;

  for (int tb = wave; tb < ntiles; tb += 4 * kTileBatch) {
    u32x4 ka[kTileBatch][NST];
    uint32_t vw[kTileBatch][4][EPL / 2];
    int tok0s[kTileBatch];
    // issue every load of the batch first
#pragma unroll
    for (int u = 0; u < kTileBatch; ++u) {
      const int t = tb + 4 * u;
      int tok0 = -1;
      if (t < ntiles) {
        if (SEL && cmode) {
          tok0 = wl[t];
        } else if ((g0 + t) / TPB < cnt) {
          const int blk = ib[(g0 + t) / TPB];
          if (blk >= 0 && blk < nbk) {
            tok0 = blk * BLOCK + ((g0 + t) % TPB) * 16;
            if (tok0 >= N) tok0 = -1;
          }
        }
      }
      tok0s[u] = tok0;
      const int koff = tok0 >= 0 ? ((tok0 + nn) * D + 8 * gq) * 2 : kBufOOB;
      const int voff = tok0 >= 0 ? ((tok0 + 4 * gq) * D + EPL * nn) * 2 : kBufOOB;
#pragma unroll
      for (int st = 0; st < NST; ++st) ka[u][st] = bld16(rK, koff + 64 * st);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (EPL == 8) {
          const u32x4 w = bld16(rV, voff + j * D * 2);
          vw[u][j][0] = w[0]; vw[u][j][1] = w[1]; vw[u][j][2] = w[2]; vw[u][j][3] = w[3];
        } else {
          const u32x2 w = bld8(rV, voff + j * D * 2);
          vw[u][j][0] = w[0]; vw[u][j][1] = w[1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kTileBatch; ++u) {
      const int tok0 = tok0s[u];
      if (tok0 < 0) continue;  // uniform across the wave
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st) sc = mfma16x16x32(ka[u][st], qb[st], sc);
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = tok0 + 4 * gq + r < N ? sc[r] * sl2 : -__builtin_inff();
      float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
      tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
      const float m_new = fmaxf(m_run, tm);          // finite: the tile has a valid token
      const float alpha = exp2_fast(m_run - m_new);  // 0 on the first tile
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = exp2_fast(sv[r] - m_new);
      l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m_run = m_new;
      // rescale accumulator row 4*gq+r by the factor of the head it belongs to
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * gq + r;
        const int hs = row < G ? row : (row < 2 * G ? row - G : 0);
        const float al = __shfl(alpha, hs, 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e][r] *= al;
      }
      // P operand: rows 0..g-1 carry bf16(p), rows g..2g-1 carry bf16(p - bf16(p))
      const uint32_t h01 = pack_bf16x2(p[0], p[1]);
      const uint32_t h23 = pack_bf16x2(p[2], p[3]);
      const uint32_t l01 = pack_bf16x2(p[0] - bf16lo(h01), p[1] - bf16hi(h01));
      const uint32_t l23 = pack_bf16x2(p[2] - bf16lo(h23), p[3] - bf16hi(h23));
      const int src = (lane - G) & 63;
      const uint32_t l01s = __shfl(l01, src, 64);
      const uint32_t l23s = __shfl(l23, src, 64);
      u32x2 pa;
      if (nn < G) pa = u32x2{h01, h23};
      else if (nn < 2 * G) pa = u32x2{l01s, l23s};
      else pa = u32x2{0u, 0u};
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int c = e >> 1;
        u32x2 bv;
        if (e & 1) bv = u32x2{pack_hi(vw[u][0][c], vw[u][1][c]), pack_hi(vw[u][2][c], vw[u][3][c])};
        else       bv = u32x2{pack_lo(vw[u][0][c], vw[u][1][c]), pack_lo(vw[u][2][c], vw[u][3][c])};
        acc[e] = mfma16x16x16(pa, bv, acc[e]);
      }
    }
  }

  // per-wave results -> LDS (16-byte stores)
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (gq == 0 && nn < G) { s_m[wave][nn] = m_run; s_l[wave][nn] = l_tot; }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * gq + r;
    if (row < 2 * G) {
#pragma unroll
      for (int e0 = 0; e0 < EPL; e0 += 4)
        *reinterpret_cast<f32x4*>(&s_acc[wave][row][EPL * nn + e0]) =
            f32x4{acc[e0][r], acc[e0 + 1][r], acc[e0 + 2][r], acc[e0 + 3][r]};
    }
  }
  __syncthreads();

  // combine the 4 waves and the hi/lo rows: one head and 4 columns per thread
  const int h0 = b * a.Hq + kh * G;
  const __amdgpu_buffer_rsrc_t rPw =
      make_rsrc(a.pacc + size_t(h0) * a.S * D, uint32_t(G) * a.S * D * sizeof(float));
  const __amdgpu_buffer_rsrc_t rMw = make_rsrc(a.pml + 2 * size_t(h0) * a.S, uint32_t(G) * a.S * 8);
  for (int o4 = tid; o4 < G * D / 4; o4 += 256) {
    const int h = o4 / (D / 4), d0 = (o4 % (D / 4)) * 4;
    float mw[4], lw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = s_m[w][h]; lw[w] = s_l[w][h]; }
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    float Ls = 0.f;
    f32x4 A = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2_fast(mw[w] - M);
        Ls += lw[w] * f;
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&s_acc[w][h][d0]);
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&s_acc[w][h + G][d0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) A[q] += (hi[q] + lo[q]) * f;
      }
    }
    const int pi = h * a.S + s;   // partial within the head group
    bst16c(rPw, (pi * D + d0) * int(sizeof(float)), __builtin_bit_cast(u32x4, A));
    if (d0 == 0) bst8c(rMw, pi * 8, u32x2{__float_as_uint(M), __float_as_uint(Ls)});
  }
  int32_t* gent = nullptr;
  if constexpr (SEL) {
    gent = a.sel_ent + size_t(bh) * kSelEntCap;
    if (cmode && wave == 0) {
      for (int i = lane; i < cm_ne; i += 64)
        if ((cm_ea + i) * TPB >= cm_u0)
          __hip_atomic_store(gent + cm_ea + i, es[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!arrive_last(&a.counter[bh * kCounterStride], a.S, &s_flag)) return;
  if constexpr (SEL) {
    // slice mode: the ascending idx row from the entries' kept blocks, built
    // while the partials load
    int ev[3] = {-1, -1, -1};
    if (cmode) {
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (tid + 256 * q < cm_E)
          ev[q] = __hip_atomic_load(gent + tid + 256 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    auto write_idx = [&]() {
      if (!cmode) return;
      const int W = (a.nb + 31) >> 5;
      if (tid < W) selp->bm[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (ev[q] >= 0) sel_mark(selp->bm, ev[q]);
      int32_t* orow = a.sel_idx + size_t(bh) * a.k;
      const int tot = sel_bitmap_to_list(*selp, W, orow, a.k);   // starts with a barrier
      for (int j = tot + tid; j < a.k; j += 256) orow[j] = -1;
      if (tid == 0) a.sel_count[bh] = tot;
    };
    merge_tail<D>(a, h0, G, s_w, s_lv, write_idx);
  } else {
    merge_tail<D>(a, h0, G, s_w, s_lv);
  }
}

// ---------------------------------------------------------------- float32 VALU
template <int D>
__global__ __launch_bounds__(256) void k_decode_blocks_valu(DecodeArgs a) {
  constexpr int CH = kValuTokensPerWG;
  constexpr int OPT = 8 * D / 256;       // (head, column) outputs per thread for g <= 8
  __shared__ float sq[8][D];
  __shared__ float sp[8][CH];
  __shared__ int stok[CH];
  __shared__ float red[8][4];
  __shared__ __attribute__((aligned(16))) float s_w[8 * kMaxSplits], s_lv[8 * kMaxSplits];
  __shared__ int s_flag;

  const int BH = a.B * a.Hkv, G = a.G, N = a.N, block = a.block;
  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cnt = a.count ? min(max(a.count[bh], 0), a.idx_stride) : a.idx_stride;
  const int bps = (cnt + a.S - 1) / a.S;
  const int blk0 = s * bps;
  const int blk1 = min(blk0 + bps, cnt);
  const int ntok = max(blk1 - blk0, 0) * block;
  const int nbk = (N + block - 1) / block;
  const int32_t* ib = a.idx + size_t(bh) * a.idx_stride;
  const float* Kb = static_cast<const float*>(a.K) + size_t(bh) * N * D;
  const float* Vb = static_cast<const float*>(a.V) + size_t(bh) * N * D;
  const float* Q = static_cast<const float*>(a.Q);
  const int h0 = b * a.Hq + kh * G;

  for (int o = tid; o < G * D; o += 256) sq[o / D][o % D] = Q[size_t(h0 + o / D) * D + o % D];
  float m_run[8], l_run[8], acc[OPT];
#pragma unroll
  for (int h = 0; h < 8; ++h) { m_run[h] = -__builtin_inff(); l_run[h] = 0.f; }
#pragma unroll
  for (int i = 0; i < OPT; ++i) acc[i] = 0.f;
  __syncthreads();

  for (int c0 = 0; c0 < ntok; c0 += CH) {
    const int n = min(CH, ntok - c0);
    for (int tt = tid; tt < n; tt += 256) {
      const int blk = ib[blk0 + (c0 + tt) / block];
      const bool okb = blk >= 0 && blk < nbk;
      const int tok = okb ? blk * block + (c0 + tt) % block : N;
      const bool ok = tok < N;
      stok[tt] = ok ? tok : -1;
      for (int h = 0; h < G; ++h) {
        float v = 0.f;
        if (ok) {
          const float* kp = Kb + size_t(tok) * D;
          for (int d = 0; d < D; d += 4) {
            const u32x4 w = ld16(kp + d);
            v += sq[h][d] * __uint_as_float(w[0]) + sq[h][d + 1] * __uint_as_float(w[1]) +
                 sq[h][d + 2] * __uint_as_float(w[2]) + sq[h][d + 3] * __uint_as_float(w[3]);
          }
        }
        sp[h][tt] = ok ? v * a.sl2 : -__builtin_inff();
      }
    }
    __syncthreads();
    for (int h = 0; h < G; ++h) {
      float m = -__builtin_inff();
      for (int tt = tid; tt < n; tt += 256) m = fmaxf(m, sp[h][tt]);
      m = wave_max(m);
      if (lane == 0) red[h][wave] = m;
    }
    __syncthreads();
    float alpha[8], mnew[8];
    for (int h = 0; h < G; ++h) {
      const float cm = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
      mnew[h] = fmaxf(m_run[h], cm);
      alpha[h] = mnew[h] == -__builtin_inff() ? 1.f : exp2_fast(m_run[h] - mnew[h]);
    }
    __syncthreads();
    for (int h = 0; h < G; ++h) {
      float l = 0.f;
      for (int tt = tid; tt < n; tt += 256) {
        const float pv = mnew[h] == -__builtin_inff() ? 0.f : exp2_fast(sp[h][tt] - mnew[h]);
        sp[h][tt] = pv;
        l += pv;
      }
      l = wave_sum(l);
      if (lane == 0) red[h][wave] = l;
    }
    __syncthreads();
    for (int h = 0; h < G; ++h) {
      l_run[h] = l_run[h] * alpha[h] + ((red[h][0] + red[h][1]) + (red[h][2] + red[h][3]));
      m_run[h] = mnew[h];
    }
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = tid + 256 * i;
      if (o < G * D) {
        const int h = o / D, d = o % D;
        float v = acc[i] * alpha[h];
        for (int tt = 0; tt < n; ++tt) {
          const int tok = stok[tt];
          if (tok >= 0) v += sp[h][tt] * Vb[size_t(tok) * D + d];
        }
        acc[i] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int o = tid + 256 * i;
    if (o < G * D) {
      const int h = o / D, d = o % D;
      const size_t pi = size_t(h0 + h) * a.S + s;
      __hip_atomic_store(a.pacc + pi * D + d, acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(a.pml + 2 * pi, m_run[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.pml + 2 * pi + 1, l_run[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (!arrive_last(&a.counter[bh * kCounterStride], a.S, &s_flag)) return;
  merge_tail<D>(a, h0, G, s_w, s_lv);
}

// ---------------------------------------------------------------- token lists
template <typename T, int D>
__global__ __launch_bounds__(256) void k_decode_tokens(DecodeArgs a) {
  constexpr int CH = kValuTokensPerWG;
  constexpr int CPL = D / 16;                 // columns per lane in the value pass
  __shared__ float sp[CH];
  __shared__ int stok[CH];
  __shared__ float sq[D];
  __shared__ float red[4];
  __shared__ float racc[16][D + 4];
  __shared__ __attribute__((aligned(16))) float s_w[kMaxSplits], s_lv[kMaxSplits];
  __shared__ int s_flag;

  const int BHq = a.B * a.Hq, N = a.N;
  const int bhq = blockIdx.x % BHq, s = blockIdx.x / BHq;
  const int b = bhq / a.Hq, h = bhq % a.Hq, kh = h / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cnt = min(max(a.count[bhq], 0), a.idx_stride);
  const int tps = (cnt + a.S - 1) / a.S;
  const int t0 = s * tps;
  const int ntok = max(min(t0 + tps, cnt) - t0, 0);
  const T* Kb = static_cast<const T*>(a.K) + (size_t(b) * a.Hkv + kh) * N * D;
  const T* Vb = static_cast<const T*>(a.V) + (size_t(b) * a.Hkv + kh) * N * D;
  const int32_t* il = a.idx + size_t(bhq) * a.idx_stride + t0;
  const float* sl = a.score ? a.score + size_t(bhq) * a.idx_stride + t0 : nullptr;

  if (!sl) {
    const T* Q = static_cast<const T*>(a.Q);
    for (int d = tid; d < D; d += 256) {
      if constexpr (sizeof(T) == 2) sq[d] = bf16_to_f32(Q[size_t(bhq) * D + d]);
      else sq[d] = Q[size_t(bhq) * D + d];
    }
  }
  __syncthreads();
  const int rg = tid >> 4, lc = tid & 15;
  float m_run = -__builtin_inff(), l_run = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

  for (int c0 = 0; c0 < ntok; c0 += CH) {
    const int n = min(CH, ntok - c0);
    for (int i = tid; i < n; i += 256) {
      const int tok = il[c0 + i];
      const bool ok = tok >= 0 && tok < N;
      float sc = -__builtin_inff();
      if (ok) {
        if (sl) {
          sc = sl[c0 + i];
        } else {
          const T* kp = Kb + size_t(tok) * D;
          float v = 0.f;
          for (int d = 0; d < D; d += 8) {
            if constexpr (sizeof(T) == 2) {
              const u32x4 w = ld16(kp + d);
#pragma unroll
              for (int q = 0; q < 4; ++q) v += sq[d + 2 * q] * bf16lo(w[q]) + sq[d + 2 * q + 1] * bf16hi(w[q]);
            } else {
              const u32x4 w0 = ld16(kp + d), w1 = ld16(kp + d + 4);
#pragma unroll
              for (int q = 0; q < 4; ++q) v += sq[d + q] * __uint_as_float(w0[q]) + sq[d + 4 + q] * __uint_as_float(w1[q]);
            }
          }
          sc = v * a.scale;
        }
      }
      sp[i] = ok ? sc * kLog2e : -__builtin_inff();
      stok[i] = ok ? tok : -1;
    }
    __syncthreads();
    float m = -__builtin_inff();
    for (int i = tid; i < n; i += 256) m = fmaxf(m, sp[i]);
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float mnew = fmaxf(m_run, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    const float alpha = mnew == -__builtin_inff() ? 1.f : exp2_fast(m_run - mnew);
    __syncthreads();
    float l = 0.f;
    for (int i = tid; i < n; i += 256) {
      const float pv = mnew == -__builtin_inff() ? 0.f : exp2_fast(sp[i] - mnew);
      sp[i] = pv;
      l += pv;
    }
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l_run = l_run * alpha + ((red[0] + red[1]) + (red[2] + red[3]));
    m_run = mnew;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] *= alpha;
    // value pass: each 16-lane row group takes every 16th token; the V rows
    // of UV of its tokens are loaded before any is used, so a row group has
    // UV loads in flight instead of one (same summation order as one at a
    // time; a missing token adds an exact zero whatever row 0 holds)
    constexpr int UV = 8;
    for (int i0 = rg; i0 < n; i0 += 16 * UV) {
      float pv[UV];
      bool ok[UV];
      const T* vp[UV];
#pragma unroll
      for (int u = 0; u < UV; ++u) {
        const int i = i0 + 16 * u;
        const int tok = i < n ? stok[i] : -1;
        ok[u] = tok >= 0;
        pv[u] = ok[u] ? sp[i] : 0.f;
        vp[u] = Vb + size_t(ok[u] ? tok : 0) * D + lc * CPL;
      }
      if constexpr (sizeof(T) == 2) {
        if constexpr (CPL == 8) {
          u32x4 w[UV];
#pragma unroll
          for (int u = 0; u < UV; ++u) w[u] = ld16(vp[u]);
#pragma unroll
          for (int u = 0; u < UV; ++u) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[2 * q] += ok[u] ? pv[u] * bf16lo(w[u][q]) : 0.f;
              acc[2 * q + 1] += ok[u] ? pv[u] * bf16hi(w[u][q]) : 0.f;
            }
          }
        } else {
          u32x2 w[UV];
#pragma unroll
          for (int u = 0; u < UV; ++u) w[u] = ld8(vp[u]);
#pragma unroll
          for (int u = 0; u < UV; ++u) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              acc[2 * q] += ok[u] ? pv[u] * bf16lo(w[u][q]) : 0.f;
              acc[2 * q + 1] += ok[u] ? pv[u] * bf16hi(w[u][q]) : 0.f;
            }
          }
        }
      } else {
        constexpr int NV = CPL / 4;
        u32x4 w[UV][NV];
#pragma unroll
        for (int u = 0; u < UV; ++u) {
#pragma unroll
          for (int c = 0; c < NV; ++c) w[u][c] = ld16(vp[u] + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < UV; ++u) {
#pragma unroll
          for (int c = 0; c < NV; ++c) {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[4 * c + q] += ok[u] ? pv[u] * __uint_as_float(w[u][c][q]) : 0.f;
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) racc[rg][lc * CPL + c] = acc[c];
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float A = 0.f;
    for (int g = 0; g < 16; ++g) A += racc[g][d];
    const size_t pi = size_t(bhq) * a.S + s;
    __hip_atomic_store(a.pacc + pi * D + d, A, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(a.pml + 2 * pi, m_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.pml + 2 * pi + 1, l_run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!arrive_last(&a.counter[bhq * kCounterStride], a.S, &s_flag)) return;
  merge_tail<D>(a, bhq, 1, s_w, s_lv);
}

// ---------------------------------------------------------------- launchers
static DecodeArgs make_args(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                            int N, int block, float scale, const int32_t* idx,
                            const int32_t* count, int idx_stride, const float* score,
                            const DecodeWs& w, void* ws, void* O, int out_dtype, float* lse) {
  DecodeArgs a;
  a.Q = Q; a.K = K; a.V = V;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.N = N; a.block = block;
  a.scale = scale; a.sl2 = scale * kLog2e;
  a.idx = idx; a.count = count; a.idx_stride = idx_stride; a.score = score;
  a.S = w.S;
  char* base = static_cast<char*>(ws);
  a.pacc = reinterpret_cast<float*>(base + w.acc_off);
  a.pml = reinterpret_cast<float*>(base + w.ml_off);
  a.counter = reinterpret_cast<uint32_t*>(base + w.cnt_off);
  a.O = O; a.out_bf16 = out_dtype == SA_BF16; a.lse = lse;
  a.sel_scores = nullptr; a.nb = 0; a.k = 0; a.flags = 0; a.sel_idx = nullptr;
  a.sel_count = nullptr;
  a.sel_ent = reinterpret_cast<int32_t*>(base + w.ent_off);
  return a;
}

template <int D, int BLOCK, int SELKPT>
static void launch_mfma_g(const DecodeArgs& a, dim3 g, size_t lds, hipStream_t st) {
  switch (a.G) {
    case 1: k_decode_blocks_mfma<D, 1, BLOCK, SELKPT><<<g, 256, lds, st>>>(a); break;
    case 2: k_decode_blocks_mfma<D, 2, BLOCK, SELKPT><<<g, 256, lds, st>>>(a); break;
    case 4: k_decode_blocks_mfma<D, 4, BLOCK, SELKPT><<<g, 256, lds, st>>>(a); break;
    default: k_decode_blocks_mfma<D, 8, BLOCK, SELKPT><<<g, 256, lds, st>>>(a); break;
  }
}

hipError_t launch_decode_blocks(const void* Q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int N, int D, float scale, int block,
                                const int32_t* idx, const int32_t* count, int idx_stride,
                                const DecodeWs& w, void* ws, void* O, int out_dtype, float* lse,
                                hipStream_t st) {
  const DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, block, scale, idx, count, idx_stride,
                                 nullptr, w, ws, O, out_dtype, lse);
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * w.S));
  if (dtype == SA_BF16) {
    if (D == 128 && block == 64) launch_mfma_g<128, 64, 0>(a, g, 0, st);
    else if (D == 128)           launch_mfma_g<128, 128, 0>(a, g, 0, st);
    else if (block == 64)        launch_mfma_g<64, 64, 0>(a, g, 0, st);
    else                         launch_mfma_g<64, 128, 0>(a, g, 0, st);
  } else {
    if (D == 128) k_decode_blocks_valu<128><<<g, 256, 0, st>>>(a);
    else          k_decode_blocks_valu<64><<<g, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_select_blocks(const void* Q, const void* K, const void* V, int B, int Hq,
                                       int Hkv, int N, int D, float scale, int block,
                                       const float* scores, int nb, int k, unsigned flags,
                                       int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                       void* O, int out_dtype, float* lse, hipStream_t st) {
  DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, block, scale, nullptr, nullptr, k, nullptr, w,
                           ws, O, out_dtype, lse);
  a.sel_scores = scores; a.nb = nb; a.k = k; a.flags = flags; a.sel_idx = idx; a.sel_count = count;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * w.S));
  const size_t lds = size_t(k > 320 ? k : 320) * sizeof(int);
  (void)D;   // the selecting variant is compiled for D = 128
  const bool small = nb <= 4096;
  if (block == 64) {
    if (small) launch_mfma_g<128, 64, 16>(a, g, lds, st);
    else       launch_mfma_g<128, 64, 32>(a, g, lds, st);
  } else {
    if (small) launch_mfma_g<128, 128, 16>(a, g, lds, st);
    else       launch_mfma_g<128, 128, 32>(a, g, lds, st);
  }
  return hipGetLastError();
}

hipError_t launch_decode_tokens(const void* Q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int N, int D, float scale, const int32_t* idx,
                                const int32_t* count, int idx_stride, const float* score,
                                const DecodeWs& w, void* ws, void* O, int out_dtype, float* lse,
                                hipStream_t st) {
  const DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, 0, scale, idx, count, idx_stride, score,
                                 w, ws, O, out_dtype, lse);
  const dim3 g(static_cast<unsigned>(long(B) * Hq * w.S));
  if (dtype == SA_BF16) {
    if (D == 128) k_decode_tokens<uint16_t, 128><<<g, 256, 0, st>>>(a);
    else          k_decode_tokens<uint16_t, 64><<<g, 256, 0, st>>>(a);
  } else {
    if (D == 128) k_decode_tokens<float, 128><<<g, 256, 0, st>>>(a);
    else          k_decode_tokens<float, 64><<<g, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace sa
