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
//   split); a split takes an equal share of the head's 16-token tiles and runs
//   them through the tile pipeline of sa_decode_core.h (scores and P V on the
//   matrix cores, up to four tiles' loads in flight per wave).  The selecting
//   variant first runs the selection pre-filter of its head from the score
//   row, then takes its tiles from its own slice of the candidate list
//   (ranking only those candidates) or, when the list does not suit slices,
//   from the fully ranked selection.  Workgroup id % (B*Hkv) selects the
//   (b, kv head): all splits of one kv head share an XCD and its L2.
// k_decode_blocks_valu (float32): one split per 64-token block; K and V rows
//   loaded by D/4 lanes each (scores summed over the row's lanes), an LDS
//   softmax per round of 256 tokens, a (head, column)-parallel value pass;
//   float32 throughout.  Its selecting variant (rows of up to 512 blocks)
//   takes the top-k of the score row in every split; for the decode step it
//   also scores the row itself, with the scoring kernel's functions, so the
//   whole step is one launch.
// k_decode_tokens: per (b, query head, split) over an explicit token list
//   (threshold selection), reusing the selector's scores when given.
#include "sa_decode_core.h"
#include "sa_device.h"
#include "sa_internal.h"
#include "sa_score_core.h"
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
  // in-kernel scoring (float32 step, k_decode_blocks_valu): the sketch
  // [B*Hkv, nb, D] (row upd rebuilt from K first, upd = -1: none) scored
  // against the group-mean query, the scores written to sc_out [B*Hkv, nb]
  float* sk;
  int upd;
  float* sc_out;
  // keys rebuilt from thumbnails (k_decode_lowbit): codes [B*Hkv, N, D/4],
  // residuals [B*Hkv, N, D], (lo, step, rstep) rows [B*Hkv, nb, 3, D]
  const uint8_t* lb_codes;
  const int8_t* lb_resid;
  const float* lb_meta;
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

// ---------------------------------------------------------------- bf16 MFMA

template <int D, int G, int BLOCK, int SELKPT>
__global__ __launch_bounds__(256, 2) void k_decode_blocks_mfma(DecodeArgs a) {
  constexpr bool SEL = SELKPT > 0;
  static_assert(2 * G <= 16, "g must be at most 8");
  constexpr int NST = D / 32;      // contraction steps of the score MFMA
  constexpr int TPB = BLOCK / 16;  // 16-token tiles per block
  __shared__ CombineLds<D, G> s_cmb;
  __shared__ __attribute__((aligned(16))) float s_w[G * kMaxSplits], s_lv[G * kMaxSplits];
  __shared__ int s_flag;

  const int BH = a.B * a.Hkv, N = a.N;
  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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

  u32x4 qb[NST];
  tile_q_operand<D, G>(static_cast<const uint16_t*>(a.Q) + (size_t(b) * a.Hq + kh * G) * D, qb);
  TileAcc<D> ta;
  tile_acc_init(ta);

  // per-(b, kv head) buffer resources: rows past N (and invalid tiles) read as
  // zeros, so every load of a batch issues unconditionally
  const __amdgpu_buffer_rsrc_t rK =
      make_rsrc(static_cast<const uint16_t*>(a.K) + size_t(bh) * N * D, uint32_t(N) * D * 2);
  const __amdgpu_buffer_rsrc_t rV =
      make_rsrc(static_cast<const uint16_t*>(a.V) + size_t(bh) * N * D, uint32_t(N) * D * 2);
  const int nbk = (N + BLOCK - 1) / BLOCK;
  run_tiles<D, G>(ta, qb, KRowsBf16<D>{rK}, rV, N, a.sl2, ntiles, [&](int t) {
    if (SEL && cmode) return wl[t];
    if ((g0 + t) / TPB < cnt) {
      const int blk = ib[(g0 + t) / TPB];
      if (blk >= 0 && blk < nbk) {
        const int tok0 = blk * BLOCK + ((g0 + t) % TPB) * 16;
        return tok0 < N ? tok0 : -1;
      }
    }
    return -1;
  });

  // combine the 4 waves and the hi/lo rows into this split's partials
  const int h0 = b * a.Hq + kh * G;
  store_partial<D, G>(ta, s_cmb, a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S,
                      a.S, s, true);
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
    merge_tail<D>(a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S, a.S,
                  MergeDst{a.O, a.out_bf16, a.lse}, h0, G, s_w, s_lv,
                  write_idx);
  } else {
    merge_tail<D>(a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S, a.S,
                  MergeDst{a.O, a.out_bf16, a.lse}, h0, G, s_w, s_lv);
  }
}

// ---------------------------------------------------------------- thumbnail keys
// k_decode_lowbit (bf16): the block-mode split-K decode with every key row
// rebuilt from its 2-bit code and 8-bit residual inside the tile pipeline
// (KRowsLowbit), so the refinement of the kept blocks and the attention over
// them are one pass over codes, residuals and values ("Faster Than Flash",
// Metodologia §3).  Split s takes the tile slice of the block decode; the
// (lo, step, rstep) rows of the slice's blocks (at most kLowbitMetaBlocks) are
// staged in LDS first.
template <int D, int G, int BLOCK>
__global__ __launch_bounds__(256, 2) void k_decode_lowbit(DecodeArgs a) {
  static_assert(2 * G <= 16, "g must be at most 8");
  constexpr int TPB = BLOCK / 16;  // 16-token tiles per block
  __shared__ CombineLds<D, G> s_cmb;
  __shared__ __attribute__((aligned(16))) float s_w[G * kMaxSplits], s_lv[G * kMaxSplits];
  __shared__ __attribute__((aligned(16))) float s_meta[kLowbitMetaBlocks][3 * D];
  __shared__ int s_flag;

  const int BH = a.B * a.Hkv, N = a.N;
  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int tps = (a.idx_stride * TPB + a.S - 1) / a.S;
  const int g0 = s * tps;
  const int ntiles = max(min(g0 + tps, a.idx_stride * TPB) - g0, 0);
  const int cnt = a.count ? min(max(a.count[bh], 0), a.idx_stride) : a.idx_stride;
  const int32_t* ib = a.idx + size_t(bh) * a.idx_stride;
  const int nbk = (N + BLOCK - 1) / BLOCK;
  // the slice's list entries [e0, e0 + ne): their (lo, step, rstep) rows
  const int e0 = g0 / TPB;
  const int ne = ntiles > 0 ? min((g0 + ntiles - 1) / TPB - e0 + 1, kLowbitMetaBlocks) : 0;
  for (int i = tid; i < ne * (3 * D / 4); i += 256) {
    const int q = i / (3 * D / 4), c4 = i % (3 * D / 4);
    const int e = e0 + q;
    const int blk = e < cnt ? ib[e] : -1;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (blk >= 0 && blk < nbk)
      v = *reinterpret_cast<const f32x4*>(a.lb_meta + (size_t(bh) * nbk + blk) * 3 * D + 4 * c4);
    *reinterpret_cast<f32x4*>(&s_meta[q][4 * c4]) = v;
  }
  u32x4 qb[D / 32];
  tile_q_operand<D, G>(static_cast<const uint16_t*>(a.Q) + (size_t(b) * a.Hq + kh * G) * D, qb);
  TileAcc<D> ta;
  tile_acc_init(ta);
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(a.lb_codes + size_t(bh) * N * (D / 4), uint32_t(N) * (D / 4));
  const __amdgpu_buffer_rsrc_t rR = make_rsrc(a.lb_resid + size_t(bh) * N * D, uint32_t(N) * D);
  const __amdgpu_buffer_rsrc_t rV =
      make_rsrc(static_cast<const uint16_t*>(a.V) + size_t(bh) * N * D, uint32_t(N) * D * 2);
  auto meta_of = [&](int t) -> const float* { return &s_meta[(g0 + t) / TPB - e0][0]; };
  const KRowsLowbit<D, decltype(meta_of)> ks{rC, rR, meta_of};
  run_tiles<D, G>(ta, qb, ks, rV, N, a.sl2, ntiles, [&](int t) {
    const int e = (g0 + t) / TPB;
    if (e < cnt && e - e0 < kLowbitMetaBlocks) {
      const int blk = ib[e];
      if (blk >= 0 && blk < nbk) {
        const int tok0 = blk * BLOCK + ((g0 + t) % TPB) * 16;
        return tok0 < N ? tok0 : -1;
      }
    }
    return -1;
  });
  const int h0 = b * a.Hq + kh * G;
  store_partial<D, G>(ta, s_cmb, a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S,
                      a.S, s, true);
  if (!arrive_last(&a.counter[bh * kCounterStride], a.S, &s_flag)) return;
  merge_tail<D>(a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S, a.S,
                MergeDst{a.O, a.out_bf16, a.lse}, h0, G, s_w, s_lv);
}

// ---------------------------------------------------------------- float32 VALU
template <int D, int G, int SELKPT>
__global__ __launch_bounds__(256) void k_decode_blocks_valu(DecodeArgs a) {
  // SELKPT > 0: the selecting variant (rows of nb <= 256 SELKPT blocks): every
  // split takes the top-k of its kv head's score row itself (the selection of
  // k_select_rows) instead of reading a list, and split 0 writes the list out
  static_assert(SELKPT >= 0, "keys per thread of the selection");
  constexpr int CH = 256;                // tokens per round: 64 per wave
  constexpr int OPT = (G * D + 255) / 256;   // (head, column) outputs per thread
  constexpr int LPR = D / 4;             // lanes per K/V row (16-byte segments)
  constexpr int RPI = 64 / LPR;          // rows per wave load
  constexpr int NL = 64 / RPI;           // loads per lane for the wave's 64 tokens
  constexpr int NC = NL > 16 ? 16 : NL;  // K and V loads per lane in flight
  __shared__ float sp[G][CH];
  __shared__ int stok[CH];
  __shared__ __attribute__((aligned(16))) float sv[CH * D];
  __shared__ float red[G][4];
  __shared__ __attribute__((aligned(16))) float s_w[8 * kMaxSplits], s_lv[8 * kMaxSplits];
  __shared__ int s_flag;

  const int BH = a.B * a.Hkv, N = a.N, block = a.block;
  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / a.Hkv, kh = bh % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / LPR, lc = lane % LPR;
  // split s takes the list slots [blk0, blk1) of idx_stride, so the index
  // loads do not wait for count; slots at or past count are skipped
  const int bps = (a.idx_stride + a.S - 1) / a.S;
  const int blk0 = s * bps;
  const int blk1 = min(blk0 + bps, a.idx_stride);
  const int ntok = max(blk1 - blk0, 0) * block;
  int cnt;
  const int32_t* ib;
  if constexpr (SELKPT > 0) {
    // the selection's LDS state lives in the value tile, unused until the
    // first round
    __shared__ int s_list[kValuSelMaxK];
    static_assert(sizeof(SelectLdsT<256, SELKPT>) <= sizeof(sv), "selection state in sv");
    auto& S = *reinterpret_cast<SelectLdsT<256, SELKPT>*>(sv);
    uint32_t kr[SELKPT];
    if (a.sk) {
      // The whole decode step in one launch: every split scores its kv head's
      // row itself with the scoring kernel's arithmetic (the same functions,
      // so the same scores bit for bit), the newest block's sketch rebuilt
      // from K; split 0 stores that sketch row and the scores.
      constexpr int SOFF = (sizeof(SelectLdsT<256, SELKPT>) + 255) / 256 * 64;   // floats
      float* srow = sv + SOFF;                                 // nb <= 256 SELKPT
      float* dummy = srow + 256 * SELKPT;                      // D floats
      auto& U = *reinterpret_cast<ScoreUpdLds<D>*>(dummy + D);
      static_assert(SOFF + 256 * SELKPT + D + sizeof(ScoreUpdLds<D>) / 4 <= CH * D,
                    "scoring state in sv");
      const int nbr = a.nb, upd = a.upd;
      const float* Qg = static_cast<const float*>(a.Q) + (size_t(b) * a.Hq + kh * G) * D;
      {
        constexpr int SLPR = D / 4, SRPI = 64 / SLPR, SB = 8;   // rows of a load batch: SB SRPI
        const int ssub = lane / SLPR, slc = lane % SLPR;
        QCol<float> qv[8];
        score_q_issue<float, D>(Qg, G, slc, qv);
        float q[4];
        score_q_finish<float, D>(Qg, G, slc, a.scale, qv, q);
        const float* base = a.sk + size_t(bh) * nbr * D;
        for (int r0 = wave * SB * SRPI; r0 < nbr; r0 += 4 * SB * SRPI) {
          u32x4 w[SB];
#pragma unroll
          for (int u = 0; u < SB; ++u)
            w[u] = ld16(base + size_t(min(r0 + u * SRPI + ssub, nbr - 1)) * D + slc * 4);
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            const int r = r0 + u * SRPI + ssub;
            const float pr = score_row<D>(q, w[u]);
            if (r < nbr && r != upd && slc == SLPR - 1) srow[r] = pr;
          }
        }
      }
      if (upd >= 0) {
        const int t0 = upd * block, nj = min(block, N - t0);
        const float pu = score_update_block<float, D>(
            static_cast<const float*>(a.K) + (size_t(bh) * N + t0) * D, nj, Qg, G, a.scale,
            s == 0 ? a.sk + (size_t(bh) * nbr + upd) * D : dummy, U);
        if (tid == 0) srow[upd] = pu;
      }
      __syncthreads();
      if (s == 0) {
        float* so = a.sc_out + size_t(bh) * nbr;
        for (int j = tid; j < nbr; j += 256) so[j] = srow[j];
      }
      load_keys_reg<256, SELKPT>(srow, nbr, kr);
      __syncthreads();                         // srow read before the selection's state is set
    } else {
      load_keys_reg<256, SELKPT>(a.sel_scores + size_t(bh) * a.nb, a.nb, kr);
    }
    cnt = select_decode_row<256, SELKPT>(kr, a.nb, a.k, a.flags, s_list, S);
    __syncthreads();
    if (s == 0) {
      int32_t* orow = a.sel_idx + size_t(bh) * a.k;
      for (int j = tid; j < a.k; j += 256) orow[j] = j < cnt ? s_list[j] : -1;
      if (tid == 0) a.sel_count[bh] = cnt;
    }
    ib = s_list;
  } else {
    cnt = a.count ? min(max(a.count[bh], 0), a.idx_stride) : a.idx_stride;
    ib = a.idx + size_t(bh) * a.idx_stride;
  }
  const int nbk = (N + block - 1) / block;
  const float* Kb = static_cast<const float*>(a.K) + size_t(bh) * N * D;
  const float* Vb = static_cast<const float*>(a.V) + size_t(bh) * N * D;
  const float* Q = static_cast<const float*>(a.Q);
  const int h0 = b * a.Hq + kh * G;

  // query columns 4*lc .. 4*lc+3 of the group's heads
  u32x4 qc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qc[h] = ld16(Q + size_t(h0 + h) * D + 4 * lc);
  float m_run[G], l_run[G], acc[OPT];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = -__builtin_inff(); l_run[h] = 0.f; }
#pragma unroll
  for (int i = 0; i < OPT; ++i) acc[i] = 0.f;

  for (int c0 = 0; c0 < ntok; c0 += CH) {
    const int n = min(CH, ntok - c0);
    {
      // thread tt resolves token c0 + tt of the split (-1: none)
      int tok = -1;
      const int slot = blk0 + (c0 + tid) / block;
      if (tid < n) {
        const int blk = ib[slot];
        if (blk >= 0 && blk < nbk && slot < cnt) tok = blk * block + (c0 + tid) % block;
        if (tok >= N) tok = -1;
      }
      stok[tid] = tok;
    }
    __syncthreads();
    // K and V rows of the wave's 64 tokens, LPR lanes per row (coalesced): the
    // key segments give each head's score (summed over the row's lanes), the
    // value rows go to LDS (zero rows for missing tokens, whose p is 0)
#pragma unroll
    for (int i0 = 0; i0 < NL; i0 += NC) {
      u32x4 kw[NC], vw[NC];
      int tk[NC];
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        tk[i] = stok[wave * 64 + (i0 + i) * RPI + sub];
        const size_t row = size_t(tk[i] >= 0 ? tk[i] : 0) * D + 4 * lc;
        kw[i] = ld16(Kb + row);
        vw[i] = ld16(Vb + row);
      }
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int t = wave * 64 + (i0 + i) * RPI + sub;
        const bool ok = tk[i] >= 0;
        reinterpret_cast<u32x4*>(sv)[t * LPR + lc] = ok ? vw[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float p = __uint_as_float(qc[h][0]) * __uint_as_float(kw[i][0]) +
                    __uint_as_float(qc[h][1]) * __uint_as_float(kw[i][1]) +
                    __uint_as_float(qc[h][2]) * __uint_as_float(kw[i][2]) +
                    __uint_as_float(qc[h][3]) * __uint_as_float(kw[i][3]);
          p = group_sum_to_last<LPR>(p);
          if (lc == LPR - 1) sp[h][t] = ok ? p * a.sl2 : -__builtin_inff();
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m = tid < n ? sp[h][tid] : -__builtin_inff();
      m = wave_max(m);
      if (lane == 0) red[h][wave] = m;
    }
    __syncthreads();
    float alpha[G], mnew[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float cm = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
      mnew[h] = fmaxf(m_run[h], cm);
      alpha[h] = mnew[h] == -__builtin_inff() ? 1.f : exp2_fast(m_run[h] - mnew[h]);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float l = 0.f;
      if (tid < n) {
        const float pv = mnew[h] == -__builtin_inff() ? 0.f : exp2_fast(sp[h][tid] - mnew[h]);
        sp[h][tid] = pv;
        l = pv;
      }
      l = wave_sum(l);
      if (lane == 0) red[h][wave] = l;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l_run[h] = l_run[h] * alpha[h] + ((red[h][0] + red[h][1]) + (red[h][2] + red[h][3]));
      m_run[h] = mnew[h];
    }
    // values from LDS: thread (head, column) outputs over the round's tokens
#pragma unroll
    for (int i = 0; i < OPT; ++i) {
      const int o = tid + 256 * i;
      if (o < G * D) {
        const int h = o / D, d = o % D;
        // four independent partial sums, so the LDS reads of a step overlap
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        int tt = 0;
        for (; tt + 8 <= n; tt += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u & 3] += sp[h][tt + u] * sv[(tt + u) * D + d];
        }
        for (; tt < n; ++tt) v[0] += sp[h][tt] * sv[tt * D + d];
        acc[i] = acc[i] * alpha[h] + ((v[0] + v[1]) + (v[2] + v[3]));
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
  merge_tail<D>(a.pacc + size_t(h0) * a.S * D, a.pml + 2 * size_t(h0) * a.S, a.S,
                  MergeDst{a.O, a.out_bf16, a.lse}, h0, G, s_w, s_lv);
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
  merge_tail<D>(a.pacc + size_t(bhq) * a.S * D, a.pml + 2 * size_t(bhq) * a.S, a.S,
                MergeDst{a.O, a.out_bf16, a.lse}, bhq, 1, s_w, s_lv);
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
  a.sk = nullptr; a.upd = -1; a.sc_out = nullptr;
  a.lb_codes = nullptr; a.lb_resid = nullptr; a.lb_meta = nullptr;
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

template <int D, int SELKPT = 0>
static void launch_valu_g(const DecodeArgs& a, int G, dim3 g, hipStream_t st) {
  switch (G) {
    case 1: k_decode_blocks_valu<D, 1, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 2: k_decode_blocks_valu<D, 2, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 3: k_decode_blocks_valu<D, 3, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 4: k_decode_blocks_valu<D, 4, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 5: k_decode_blocks_valu<D, 5, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 6: k_decode_blocks_valu<D, 6, SELKPT><<<g, 256, 0, st>>>(a); break;
    case 7: k_decode_blocks_valu<D, 7, SELKPT><<<g, 256, 0, st>>>(a); break;
    default: k_decode_blocks_valu<D, 8, SELKPT><<<g, 256, 0, st>>>(a); break;
  }
}

hipError_t launch_decode_blocks(const void* Q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int N, int D, float scale, int block,
                                const int32_t* idx, const int32_t* count, int idx_stride,
                                const DecodeWs& w, void* ws, void* O, int out_dtype, float* lse,
                                hipStream_t st) {
  DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, block, scale, idx, count, idx_stride,
                           nullptr, w, ws, O, out_dtype, lse);
  if (dtype != SA_BF16) a.S = decode_valu_splits(idx_stride, block);   // sized for by decode_ws
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * a.S));
  if (dtype == SA_BF16) {
    if (D == 128 && block == 64) launch_mfma_g<128, 64, 0>(a, g, 0, st);
    else if (D == 128)           launch_mfma_g<128, 128, 0>(a, g, 0, st);
    else if (block == 64)        launch_mfma_g<64, 64, 0>(a, g, 0, st);
    else                         launch_mfma_g<64, 128, 0>(a, g, 0, st);
  } else {
    if (D == 128) launch_valu_g<128>(a, Hq / Hkv, g, st);
    else          launch_valu_g<64>(a, Hq / Hkv, g, st);
  }
  return hipGetLastError();
}

template <int D, int BLOCK>
static void launch_lowbit_g(const DecodeArgs& a, int G, dim3 g, hipStream_t st) {
  switch (G) {
    case 1: k_decode_lowbit<D, 1, BLOCK><<<g, 256, 0, st>>>(a); break;
    case 2: k_decode_lowbit<D, 2, BLOCK><<<g, 256, 0, st>>>(a); break;
    case 4: k_decode_lowbit<D, 4, BLOCK><<<g, 256, 0, st>>>(a); break;
    default: k_decode_lowbit<D, 8, BLOCK><<<g, 256, 0, st>>>(a); break;
  }
}

hipError_t launch_decode_lowbit(const void* Q, const uint8_t* codes, const int8_t* resid,
                                const float* meta, const void* V, int B, int Hq, int Hkv, int N,
                                int D, float scale, int block, const int32_t* idx,
                                const int32_t* count, int idx_stride, const DecodeWs& w, void* ws,
                                void* O, int out_dtype, float* lse, hipStream_t st) {
  DecodeArgs a = make_args(Q, nullptr, V, B, Hq, Hkv, N, block, scale, idx, count, idx_stride,
                           nullptr, w, ws, O, out_dtype, lse);
  a.S = decode_lowbit_splits(idx_stride, block);   // within the partials decode_ws sizes
  a.lb_codes = codes; a.lb_resid = resid; a.lb_meta = meta;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * a.S));
  const int G = Hq / Hkv;
  if (D == 128) {
    if (block == 64) launch_lowbit_g<128, 64>(a, G, g, st);
    else             launch_lowbit_g<128, 128>(a, G, g, st);
  } else {
    if (block == 64) launch_lowbit_g<64, 64>(a, G, g, st);
    else             launch_lowbit_g<64, 128>(a, G, g, st);
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

hipError_t launch_decode_select_valu(const void* Q, const void* K, const void* V, int B, int Hq,
                                     int Hkv, int N, int D, float scale, int block,
                                     const float* scores, int nb, int k, unsigned flags,
                                     int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                     void* O, int out_dtype, float* lse, hipStream_t st) {
  DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, block, scale, nullptr, nullptr, k, nullptr, w,
                           ws, O, out_dtype, lse);
  a.S = decode_valu_splits(k, block);   // sized for by decode_ws
  a.sel_scores = scores; a.nb = nb; a.k = k; a.flags = flags; a.sel_idx = idx; a.sel_count = count;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * a.S));
  if (D == 128) launch_valu_g<128, kValuSelKpt>(a, Hq / Hkv, g, st);
  else          launch_valu_g<64, kValuSelKpt>(a, Hq / Hkv, g, st);
  return hipGetLastError();
}

hipError_t launch_decode_step_valu(const void* Q, const void* K, const void* V, int B, int Hq,
                                   int Hkv, int N, int D, float scale, int block, float* sketch,
                                   int update_block, float* scores, int nb, int k, unsigned flags,
                                   int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                   void* O, int out_dtype, float* lse, hipStream_t st) {
  DecodeArgs a = make_args(Q, K, V, B, Hq, Hkv, N, block, scale, nullptr, nullptr, k, nullptr, w,
                           ws, O, out_dtype, lse);
  a.S = decode_valu_splits(k, block);   // sized for by decode_ws
  a.nb = nb; a.k = k; a.flags = flags; a.sel_idx = idx; a.sel_count = count;
  a.sk = sketch; a.upd = update_block; a.sc_out = scores;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * a.S));
  if (D == 128) launch_valu_g<128, kValuSelKpt>(a, Hq / Hkv, g, st);
  else          launch_valu_g<64, kValuSelKpt>(a, Hq / Hkv, g, st);
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
