// sa_decode_core.h -- pieces of the bf16 split-K decode shared by the decode
// kernels: the per-wave pipeline over 16-token tiles, the combination of a
// workgroup's four waves into one partial per query head, and the exact merge
// of a head group's partials.
//
// Exact softmax attention is recomputed on the selected support with the
// original q, K, V ("How Much Dense Attention is Necessary?", technical
// summary §2.1); each split yields an online-softmax partial (m, l, sum p v)
// and the partials merge exactly ("Pulsar Attention", Fase 2).
//
// Tile pipeline (one wave per 16-token tile): the scores of the g heads for
// 16 tokens are one chain of v_mfma_f32_16x16x32_bf16 with the key rows as the
// A operand and the group's queries as the B operand, both in their natural
// row-major layout (contraction over d).  The score tile comes out with lane l
// holding head l%16 for tokens 4*(l/16)+r, which is the A-operand layout of
// v_mfma_f32_16x16x16_bf16 for P V.  V rows are loaded as row vectors and
// transposed in registers with v_perm_b32 so the value columns land in the B
// operand (column d = (D/16)*n + e of MFMA e).  P is split as p ~ hi + lo (two
// bf16) and the lo part fills the padding rows g..2g-1 of the 16-row tile, so
// the value product is accurate to about 2^-17 relative with float32
// accumulation.  Each wave issues the loads of up to kTileBatch tiles before
// computing any of them, through buffer resources (rows past N read as zeros).
#pragma once

#include "sa_device.h"

namespace sa {

constexpr int kTileBatch = 4;   // tiles per wave whose loads are issued together

// Running state of one wave: lane l keeps (m, l) of head l%16 (< g) in log2
// units and accumulator rows 4*(l/16)+r (hi rows 0..g-1, lo rows g..2g-1).
template <int D>
struct TileAcc {
  float m_run, l_run;
  f32x4 acc[D / 16];
};

template <int D>
__device__ __forceinline__ void tile_acc_init(TileAcc<D>& t) {
  t.m_run = -__builtin_inff();
  t.l_run = 0.f;
#pragma unroll
  for (int e = 0; e < D / 16; ++e) t.acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// B operand of the score MFMA: lane (gq, nn) holds d-slots 8*gq + 32*st .. +7
// of query head nn of the group (zeros for nn >= g).  Qg: the group's first head.
template <int D, int G>
__device__ __forceinline__ void tile_q_operand(const uint16_t* Qg, u32x4 (&qb)[D / 32]) {
  const int lane = threadIdx.x & 63, gq = lane >> 4, nn = lane & 15;
  if (nn < G) {
    const uint16_t* qp = Qg + size_t(nn) * D + 8 * gq;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) qb[st] = ld16(qp + 32 * st);
  } else {
#pragma unroll
    for (int st = 0; st < D / 32; ++st) qb[st] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Key sources of the tile pipeline.  issue() starts the loads of lane
// (gq, nn)'s share of a tile's key rows (row tok0 + nn, channels
// 8 gq + 32 st .. + 7 for st < D / 32) into a raw register set; finish()
// turns them into the score MFMA's A operand once they are needed.
//
// KRowsBf16: bf16 key rows through a buffer resource over the head's K (rows
// past N, and tok0 < 0, read as zeros).
template <int D>
struct KRowsBf16 {
  __amdgpu_buffer_rsrc_t rK;
  struct Raw {
    u32x4 k[D / 32];
  };
  __device__ __forceinline__ void issue(int tok0, int /*t*/, Raw& r) const {
    const int lane = threadIdx.x & 63, gq = lane >> 4, nn = lane & 15;
    const int koff = tok0 >= 0 ? ((tok0 + nn) * D + 8 * gq) * 2 : kBufOOB;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) r.k[st] = bld16(rK, koff + 64 * st);
  }
  __device__ __forceinline__ void finish(const Raw& r, int /*t*/, u32x4 (&ka)[D / 32]) const {
#pragma unroll
    for (int st = 0; st < D / 32; ++st) ka[st] = r.k[st];
  }
};

// KRowsLowbit: keys rebuilt from their 2-bit codes and 8-bit residuals
// ("Faster Than Flash", Metodologia §3: the kept blocks are refined with the
// residuals), k^ = fma(code, step, lo) + r8 * rstep rounded to bf16 (nearest,
// ties to even) -- the same float32 operations, so the same value, as the
// stand-alone key rebuild.  rC / rR: buffer resources over the head's codes
// (D / 4 bytes per token: one word per 16 channels, channel 16 g + i at bit
// 8 (i % 4) + 2 (i / 4)) and residuals (D bytes per token); meta_of(t): the
// (lo, step, rstep) rows (3 x D floats, LDS) of tile t's block.
template <int D, typename MetaOf>
struct KRowsLowbit {
  __amdgpu_buffer_rsrc_t rC, rR;
  MetaOf meta_of;
  struct Raw {
    uint32_t c[D / 32];
    u32x2 r[D / 32];
  };
  __device__ __forceinline__ void issue(int tok0, int /*t*/, Raw& w) const {
    const int lane = threadIdx.x & 63, gq = lane >> 4, nn = lane & 15;
    const int row = tok0 + nn;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const int c0 = 8 * gq + 32 * st;
      w.c[st] = bld4(rC, tok0 >= 0 ? row * (D / 4) + (c0 / 16) * 4 : kBufOOB);
      w.r[st] = bld8(rR, tok0 >= 0 ? row * D + c0 : kBufOOB);
    }
  }
  __device__ __forceinline__ void finish(const Raw& w, int t, u32x4 (&ka)[D / 32]) const {
    const int lane = threadIdx.x & 63, gq = lane >> 4;
    const float* m = meta_of(t);
    const int hw = gq & 1;                 // which half of its 16-channel word
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const int c0 = 8 * gq + 32 * st;
      const f32x4 lo0 = *reinterpret_cast<const f32x4*>(m + c0);
      const f32x4 lo1 = *reinterpret_cast<const f32x4*>(m + c0 + 4);
      const f32x4 sp0 = *reinterpret_cast<const f32x4*>(m + D + c0);
      const f32x4 sp1 = *reinterpret_cast<const f32x4*>(m + D + c0 + 4);
      const f32x4 rs0 = *reinterpret_cast<const f32x4*>(m + 2 * D + c0);
      const f32x4 rs1 = *reinterpret_cast<const f32x4*>(m + 2 * D + c0 + 4);
      float kh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int code = int((w.c[st] >> (8 * (e & 3) + 2 * (2 * hw + (e >> 2)))) & 3u);
        const int r8 = int(int8_t((w.r[st][e / 4] >> (8 * (e % 4))) & 0xffu));
        const float lo = e < 4 ? lo0[e] : lo1[e - 4];
        const float sp = e < 4 ? sp0[e] : sp1[e - 4];
        const float rs = e < 4 ? rs0[e] : rs1[e - 4];
        const float tb = fmaf(float(code), sp, lo);
        kh[e] = tb + float(r8) * rs;
      }
      ka[st] = u32x4{pack_bf16x2(kh[0], kh[1]), pack_bf16x2(kh[2], kh[3]),
                     pack_bf16x2(kh[4], kh[5]), pack_bf16x2(kh[6], kh[7])};
    }
  }
};

// Tiles t = wave, wave + 4, ... < ntiles of one (b, kv head); tok_of(t) gives a
// tile's first token, or -1 to skip it (uniform across the wave).  ks: the key
// source; rV: a buffer resource over the head's V rows; sl2 = scale * log2(e).
template <int D, int G, typename KSrc, typename TokOf>
__device__ __forceinline__ void run_tiles(TileAcc<D>& ta, const u32x4 (&qb)[D / 32],
                                          const KSrc& ks, __amdgpu_buffer_rsrc_t rV,
                                          int N, float sl2, int ntiles, TokOf tok_of) {
  static_assert(2 * G <= 16, "g must be at most 8");
  constexpr int NST = D / 32;      // contraction steps of the score MFMA
  constexpr int EPL = D / 16;      // value columns per lane = PV MFMAs per tile
  constexpr int TB = kTileBatch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, nn = lane & 15;
  // the raw loads of TB tiles (tiles tb, tb + 4, ... of this wave)
  struct Batch {
    typename KSrc::Raw kr[TB];
    uint32_t vw[TB][4][EPL / 2];
    int tok0[TB];
  };
  auto issue = [&](int tb, Batch& bt) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int t = tb + 4 * u;
      const int tok0 = t < ntiles ? tok_of(t) : -1;
      bt.tok0[u] = tok0;
      ks.issue(tok0, t, bt.kr[u]);
      const int voff = tok0 >= 0 ? ((tok0 + 4 * gq) * D + EPL * nn) * 2 : kBufOOB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (EPL == 8) {
          const u32x4 w = bld16(rV, voff + j * D * 2);
          bt.vw[u][j][0] = w[0]; bt.vw[u][j][1] = w[1]; bt.vw[u][j][2] = w[2]; bt.vw[u][j][3] = w[3];
        } else {
          const u32x2 w = bld8(rV, voff + j * D * 2);
          bt.vw[u][j][0] = w[0]; bt.vw[u][j][1] = w[1];
        }
      }
    }
  };
  auto compute = [&](int tb, const Batch& bt) {
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int tok0 = bt.tok0[u];
      if (tok0 < 0) continue;  // uniform across the wave
      u32x4 ka[NST];
      ks.finish(bt.kr[u], tb + 4 * u, ka);
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st) sc = mfma16x16x32(ka[st], qb[st], sc);
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = tok0 + 4 * gq + r < N ? sc[r] * sl2 : -__builtin_inff();
      float tm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
      tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
      const float m_new = fmaxf(ta.m_run, tm);          // finite: the tile has a valid token
      const float alpha = exp2_fast(ta.m_run - m_new);  // 0 on the first tile
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = exp2_fast(sv[r] - m_new);
      ta.l_run = ta.l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      ta.m_run = m_new;
      // rescale accumulator row 4*gq+r by the factor of the head it belongs to
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * gq + r;
        const int hs = row < G ? row : (row < 2 * G ? row - G : 0);
        const float al = __shfl(alpha, hs, 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) ta.acc[e][r] *= al;
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
        if (e & 1) bv = u32x2{pack_hi(bt.vw[u][0][c], bt.vw[u][1][c]), pack_hi(bt.vw[u][2][c], bt.vw[u][3][c])};
        else       bv = u32x2{pack_lo(bt.vw[u][0][c], bt.vw[u][1][c]), pack_lo(bt.vw[u][2][c], bt.vw[u][3][c])};
        ta.acc[e] = mfma16x16x16(pa, bv, ta.acc[e]);
      }
    }
  };
  // every load of a batch is issued before its first tile is computed (issuing
  // the next batch's loads before this batch's arithmetic measured slower)
  for (int tb = wave; tb < ntiles; tb += 4 * TB) {
    Batch A;
    issue(tb, A);
    compute(tb, A);
  }
}

// LDS of the four-wave combination.
template <int D, int G>
struct CombineLds {
  __attribute__((aligned(16))) float acc[4][2 * G][D + 4];
  float m[4][G], l[4][G];
};

// Combine the four waves' states (and the hi / lo rows) into the workgroup's
// partial for each of the g heads: acc [h, D] at pacc + (h * S + s) * D and
// (m, l) at pml + 2 * (h * S + s), where pacc / pml point at the head group's
// first partial.  Stores are device-coherent (sc1) when `coh`, plain
// otherwise (visible to sc1 loads from the same XCD).  All threads call.
template <int D, int G>
__device__ __forceinline__ void store_partial(const TileAcc<D>& ta, CombineLds<D, G>& L,
                                              float* pacc, float* pml, int S, int s, bool coh) {
  constexpr int EPL = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nn = lane & 15;
  float l_tot = ta.l_run + __shfl_xor(ta.l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (gq == 0 && nn < G) { L.m[wave][nn] = ta.m_run; L.l[wave][nn] = l_tot; }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * gq + r;
    if (row < 2 * G) {
#pragma unroll
      for (int e0 = 0; e0 < EPL; e0 += 4)
        *reinterpret_cast<f32x4*>(&L.acc[wave][row][EPL * nn + e0]) =
            f32x4{ta.acc[e0][r], ta.acc[e0 + 1][r], ta.acc[e0 + 2][r], ta.acc[e0 + 3][r]};
    }
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rPw = make_rsrc(pacc, uint32_t(G) * S * D * sizeof(float));
  const __amdgpu_buffer_rsrc_t rMw = make_rsrc(pml, uint32_t(G) * S * 8);
  for (int o4 = tid; o4 < G * D / 4; o4 += 256) {
    const int h = o4 / (D / 4), d0 = (o4 % (D / 4)) * 4;
    float mw[4], lw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = L.m[w][h]; lw[w] = L.l[w][h]; }
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    float Ls = 0.f;
    f32x4 A = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2_fast(mw[w] - M);
        Ls += lw[w] * f;
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&L.acc[w][h][d0]);
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&L.acc[w][h + G][d0]);
#pragma unroll
        for (int q = 0; q < 4; ++q) A[q] += (hi[q] + lo[q]) * f;
      }
    }
    const int pi = h * S + s;   // partial within the head group
    const u32x2 ml = u32x2{__float_as_uint(M), __float_as_uint(Ls)};
    if (coh) {
      bst16c(rPw, (pi * D + d0) * int(sizeof(float)), __builtin_bit_cast(u32x4, A));
      if (d0 == 0) bst8c(rMw, pi * 8, ml);
    } else {
      bst16(rPw, (pi * D + d0) * int(sizeof(float)), __builtin_bit_cast(u32x4, A));
      if (d0 == 0) bst8(rMw, pi * 8, ml);
    }
  }
}

// Where the merged result goes: O [rows, D] (bf16 or float32) and lse [rows].
struct MergeDst {
  void* O;
  int out_bf16;
  float* lse;
};

// Merge the S partials of nh query heads, output rows row0 .. row0+nh-1 (of
// [B*Hq]), read with agent-coherent loads from pg [nh, S, D] / mg [nh, S, 2]
// (the group's first partial):
// M = max m_s, L = sum l_s 2^(m_s - M), O = sum acc_s 2^(m_s - M) / L,
// lse = (M + log2 L) ln 2 (scores are kept in log2 units).
// Thread t owns head t / (D/4) and 4 consecutive columns (nh * D / 4 <= 256).
// Its first kMergeChunk partial loads and the (m, l) pair loads are issued
// first; mid() (all threads call it) runs while they are in flight.  The
// pairs are staged in LDS, one row per head of stride Sp (S up to
// kMergeRegSplits: Sp = kMergeRegSplits, so one unrolled branch-free pass of
// 16-byte LDS reads serves every split; else S rounded up to 4), padded with
// m = -inf, l = 0.  Beyond kMergeRegSplits the rest follow 8 at a time.
// w / lv: LDS of nh * max(S rounded up to 4, kMergeRegSplits) floats each.
constexpr int kMergeChunk = 32;
constexpr int kMergeRegSplits = 32;
constexpr int kMergeMaxSplits = 128;

struct NoMid {
  __device__ void operator()() const {}
};

template <int D, typename Mid = NoMid>
__device__ void merge_tail(const float* pg, const float* mg, int S, const MergeDst& dst,
                           int row0, int nh, float* w, float* lv, Mid mid = Mid()) {
  constexpr int CH = kMergeChunk, SR = kMergeRegSplits;
  static_assert(SR == CH && CH % 4 == 0, "one chunk holds the register path");
  const int Sp = S <= SR ? SR : (S + 3) & ~3, tid = threadIdx.x;
  const bool act = tid < nh * (D / 4);
  const int h = act ? tid / (D / 4) : 0, d0 = (tid % (D / 4)) * 4;
  // the head group's partials through one buffer resource: a lane offset plus
  // a scalar offset per split
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(pg, uint32_t(nh) * S * D * sizeof(float));
  const int voff = (h * S * D + d0) * int(sizeof(float));
  u32x4 v[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) v[u] = bld16c(rP, voff, min(u, S - 1) * D * int(sizeof(float)));
  // (m, l) pairs: nh * S <= 8 * kMergeMaxSplits = 4 per thread
  static_assert(8 * kMergeMaxSplits <= 4 * 256, "pairs per thread");
  const int np = nh * S;
  const __amdgpu_buffer_rsrc_t rM = make_rsrc(mg, uint32_t(np) * 8);
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
  // threads past the nh heads' columns only take part in the barrier above
  if (act) {
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
    const size_t oi = size_t(row0 + h) * D + d0;
    if (dst.out_bf16) {
      const u32x2 pk = u32x2{pack_bf16x2(A[0] * inv, A[1] * inv), pack_bf16x2(A[2] * inv, A[3] * inv)};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst.O) + oi) = pk;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(dst.O) + oi) =
          f32x4{A[0] * inv, A[1] * inv, A[2] * inv, A[3] * inv};
    }
    if (dst.lse && d0 == 0) dst.lse[row0 + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace sa
