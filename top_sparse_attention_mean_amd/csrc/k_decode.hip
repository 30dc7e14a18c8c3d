// k_decode.hip -- split-K sparse decode attention and the log-sum-exp merge.
//
// Exact softmax attention recomputed on the selected support with the
// original q, K, V ("How Much Dense Attention is Necessary?", technical
// summary §2.1); only the chosen blocks are fetched from the retained cache
// ("Faster Than Flash", Metodologia §3 refinement stage; Quest in "The Sparse
// Frontier", Contributi §2).  Each split produces an online-softmax partial
// (m, l, sum p v) and the partials are merged exactly ("Pulsar Attention",
// Fase 2: online-softmax merge of per-shard attention).
//
// k_decode_blocks_mfma (bf16): one 256-thread workgroup per (b, kv head,
//   split).  A 16-token tile is one wave's unit of work.  Scores of the g heads
//   for 16 tokens are one chain of v_mfma_f32_16x16x32_bf16 with the key rows
//   as the A operand and the group's queries as the B operand -- both read in
//   their natural row-major layout (contraction over d), so keys go straight
//   from HBM into matrix-core registers.  The score tile comes out with lane l
//   holding head l%16 for tokens 4*(l/16)+r, which is exactly the A-operand
//   layout of v_mfma_f32_16x16x16_bf16 for P V.  V rows are loaded as 16-byte
//   row vectors and transposed in registers with v_perm_b32 so the value
//   columns land in the B operand (column d = (D/16)*n + e of MFMA e).  P is
//   split exactly as p = hi + lo (two bf16) and the lo part fills the padding
//   rows g..2g-1 of the 16-row tile, so the value product is accurate to about
//   2^-17 relative while keeping float32 accumulation.  Workgroup id % (B*Hkv)
//   selects the (b, kv head): all splits of one kv head share an XCD.
// k_decode_blocks_valu (float32): per-thread dot products, LDS softmax, and a
//   (head, column)-parallel value pass; float32 end to end.
// k_decode_tokens: per (b, query head, split) over an explicit token list
//   (threshold selection), reusing the selector's scores when given.
// k_merge: one wave per (b, query head) combines the split partials.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// ---------------------------------------------------------------- bf16 MFMA
template <int D, int G, int BLOCK>
__global__ __launch_bounds__(256) void k_decode_blocks_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int BH, int Hq, int Hkv, int N, float sl2,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int idx_stride,
    int S, float* __restrict__ pacc, float* __restrict__ pml) {
  static_assert(2 * G <= 16, "g must be at most 8");
  constexpr int NST = D / 32;      // contraction steps of the score MFMA
  constexpr int EPL = D / 16;      // value columns per lane = PV MFMAs per tile
  constexpr int TPB = BLOCK / 16;  // 16-token tiles per block
  __shared__ float s_acc[4][2 * G][D + 4];
  __shared__ float s_m[4][G], s_l[4][G];

  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / Hkv, kh = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, nn = lane & 15;

  const int cnt = count ? min(max(count[bh], 0), idx_stride) : idx_stride;
  const int bps = (cnt + S - 1) / S;
  const int blk0 = s * bps;
  const int blk1 = min(blk0 + bps, cnt);
  const int ntiles = max(blk1 - blk0, 0) * TPB;

  u32x4 qb[NST];
  if (nn < G) {
    const uint16_t* qp = Q + (size_t(b) * Hq + kh * G + nn) * D + 8 * gq;
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

  const uint16_t* Kb = K + size_t(bh) * N * D;
  const uint16_t* Vb = V + size_t(bh) * N * D;
  const int32_t* ib = idx + size_t(bh) * idx_stride;
  const int nbk = (N + BLOCK - 1) / BLOCK;

  for (int t = wave; t < ntiles; t += 4) {
    const int blk = ib[blk0 + t / TPB];
    if (blk < 0 || blk >= nbk) continue;  // uniform across the wave
    const int tok0 = blk * BLOCK + (t % TPB) * 16;
    if (tok0 >= N) continue;

    u32x4 ka[NST];
    {
      const int kr = min(tok0 + nn, N - 1);
      const uint16_t* kp = Kb + size_t(kr) * D + 8 * gq;
#pragma unroll
      for (int st = 0; st < NST; ++st) ka[st] = ld16(kp + 32 * st);
    }
    uint32_t vw[4][EPL / 2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vr = min(tok0 + 4 * gq + j, N - 1);
      const uint16_t* vp = Vb + size_t(vr) * D + EPL * nn;
      if constexpr (EPL == 8) {
        u32x4 w = ld16(vp);
        vw[j][0] = w[0]; vw[j][1] = w[1]; vw[j][2] = w[2]; vw[j][3] = w[3];
      } else {
        u32x2 w = ld8(vp);
        vw[j][0] = w[0]; vw[j][1] = w[1];
      }
    }

    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NST; ++st) sc = mfma16x16x32(ka[st], qb[st], sc);

    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = tok0 + 4 * gq + r;
      sv[r] = tk < N ? sc[r] * sl2 : -__builtin_inff();
    }
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
      const float a = __shfl(alpha, hs, 64);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e][r] *= a;
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
      if (e & 1) bv = u32x2{pack_hi(vw[0][c], vw[1][c]), pack_hi(vw[2][c], vw[3][c])};
      else       bv = u32x2{pack_lo(vw[0][c], vw[1][c]), pack_lo(vw[2][c], vw[3][c])};
      acc[e] = mfma16x16x16(pa, bv, acc[e]);
    }
  }

  // per-wave results -> LDS
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (gq == 0 && nn < G) { s_m[wave][nn] = m_run; s_l[wave][nn] = l_tot; }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * gq + r;
    if (row < 2 * G) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][row][EPL * nn + e] = acc[e][r];
    }
  }
  __syncthreads();

  // combine the 4 waves and the hi/lo rows: one (head, column) per thread
  for (int o = tid; o < G * D; o += 256) {
    const int h = o / D, d = o % D;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float Ls = 0.f, A = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2_fast(s_m[w][h] - M);
        Ls += s_l[w][h] * f;
        A += (s_acc[w][h][d] + s_acc[w][h + G][d]) * f;
      }
    }
    const size_t pi = (size_t(b) * Hq + kh * G + h) * S + s;
    pacc[pi * D + d] = A;
    if (d == 0) { pml[2 * pi] = M; pml[2 * pi + 1] = Ls; }
  }
}

// ---------------------------------------------------------------- float32 VALU
template <int D>
__global__ __launch_bounds__(256) void k_decode_blocks_valu(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    int BH, int Hq, int Hkv, int G, int N, int block, float sl2,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int idx_stride,
    int S, float* __restrict__ pacc, float* __restrict__ pml) {
  constexpr int MAXT = kValuTokensPerWG;
  __shared__ float sq[8][D];
  __shared__ float sp[8][MAXT];
  __shared__ int stok[MAXT];
  __shared__ float red[8][4];
  __shared__ float sM[8], sL[8];

  const int bh = blockIdx.x % BH, s = blockIdx.x / BH;
  const int b = bh / Hkv, kh = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cnt = count ? min(max(count[bh], 0), idx_stride) : idx_stride;
  const int bps = (cnt + S - 1) / S;
  const int blk0 = s * bps;
  const int blk1 = min(blk0 + bps, cnt);
  const int ntok = min(max(blk1 - blk0, 0) * block, MAXT);
  const int32_t* ib = idx + size_t(bh) * idx_stride;
  const float* Kb = K + size_t(bh) * N * D;
  const float* Vb = V + size_t(bh) * N * D;

  for (int o = tid; o < G * D; o += 256)
    sq[o / D][o % D] = Q[(size_t(b) * Hq + kh * G + o / D) * D + o % D];
  __syncthreads();

  for (int tt = tid; tt < ntok; tt += 256) {
    const int blk = ib[blk0 + tt / block];
    const bool okb = blk >= 0 && blk < (N + block - 1) / block;
    const int tok = okb ? blk * block + tt % block : N;
    const bool ok = okb && tok < N;
    stok[tt] = ok ? tok : -1;
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
      if (ok) {
        const float* kp = Kb + size_t(tok) * D;
        for (int d = 0; d < D; d += 4) {
          u32x4 w = ld16(kp + d);
          a += sq[h][d] * __uint_as_float(w[0]) + sq[h][d + 1] * __uint_as_float(w[1]) +
               sq[h][d + 2] * __uint_as_float(w[2]) + sq[h][d + 3] * __uint_as_float(w[3]);
        }
      }
      sp[h][tt] = ok ? a * sl2 : -__builtin_inff();
    }
  }
  __syncthreads();
  for (int h = 0; h < G; ++h) {
    float m = -__builtin_inff();
    for (int tt = tid; tt < ntok; tt += 256) m = fmaxf(m, sp[h][tt]);
    m = wave_max(m);
    if (lane == 0) red[h][wave] = m;
  }
  __syncthreads();
  if (tid < G) sM[tid] = fmaxf(fmaxf(red[tid][0], red[tid][1]), fmaxf(red[tid][2], red[tid][3]));
  __syncthreads();
  for (int h = 0; h < G; ++h) {
    const float M = sM[h];
    float l = 0.f;
    for (int tt = tid; tt < ntok; tt += 256) {
      const float pv = M == -__builtin_inff() ? 0.f : exp2_fast(sp[h][tt] - M);
      sp[h][tt] = pv;
      l += pv;
    }
    l = wave_sum(l);
    if (lane == 0) red[h][wave] = l;
  }
  __syncthreads();
  if (tid < G) sL[tid] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
  __syncthreads();
  for (int o = tid; o < G * D; o += 256) {
    const int h = o / D, d = o % D;
    float a = 0.f;
    for (int tt = 0; tt < ntok; ++tt) {
      const int tok = stok[tt];
      if (tok >= 0) a += sp[h][tt] * Vb[size_t(tok) * D + d];
    }
    const size_t pi = (size_t(b) * Hq + kh * G + h) * S + s;
    pacc[pi * D + d] = a;
    if (d == 0) { pml[2 * pi] = sM[h]; pml[2 * pi + 1] = sL[h]; }
  }
}

// ---------------------------------------------------------------- token lists
template <typename T, int D>
__global__ __launch_bounds__(256) void k_decode_tokens(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int BHq,
    int Hq, int Hkv, int N, float scale, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ count, int idx_stride, const float* __restrict__ score,
    int S, float* __restrict__ pacc, float* __restrict__ pml) {
  constexpr int MAXT = kValuTokensPerWG;
  constexpr int CPL = D / 16;                 // columns per lane in the value pass
  __shared__ float sp[MAXT];
  __shared__ int stok[MAXT];
  __shared__ float sq[D];
  __shared__ float red[4];
  __shared__ float racc[16][D + 4];

  const int bhq = blockIdx.x % BHq, s = blockIdx.x / BHq;
  const int b = bhq / Hq, h = bhq % Hq, kh = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cnt = min(max(count[bhq], 0), idx_stride);
  const int tps = (cnt + S - 1) / S;
  const int t0 = s * tps;
  const int n = min(max(min(t0 + tps, cnt) - t0, 0), MAXT);
  const T* Kb = K + (size_t(b) * Hkv + kh) * N * D;
  const T* Vb = V + (size_t(b) * Hkv + kh) * N * D;
  const float l2e = kLog2e;

  if (!score) {
    for (int d = tid; d < D; d += 256) {
      const T qv = Q[size_t(bhq) * D + d];
      if constexpr (sizeof(T) == 2) sq[d] = bf16_to_f32(qv);
      else sq[d] = qv;
    }
    __syncthreads();
  }
  for (int i = tid; i < n; i += 256) {
    const int tok = idx[size_t(bhq) * idx_stride + t0 + i];
    const bool ok = tok >= 0 && tok < N;
    float sc = -__builtin_inff();
    if (ok) {
      if (score) {
        sc = score[size_t(bhq) * idx_stride + t0 + i];
      } else {
        const T* kp = Kb + size_t(tok) * D;
        float a = 0.f;
        for (int d = 0; d < D; d += 8) {
          if constexpr (sizeof(T) == 2) {
            u32x4 w = ld16(kp + d);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              a += sq[d + 2 * c] * bf16lo(w[c]) + sq[d + 2 * c + 1] * bf16hi(w[c]);
          } else {
            u32x4 w0 = ld16(kp + d), w1 = ld16(kp + d + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              a += sq[d + c] * __uint_as_float(w0[c]) + sq[d + 4 + c] * __uint_as_float(w1[c]);
          }
        }
        sc = a * scale;
      }
    }
    sp[i] = ok ? sc * l2e : -__builtin_inff();
    stok[i] = ok ? tok : -1;
  }
  __syncthreads();
  float m = -__builtin_inff();
  for (int i = tid; i < n; i += 256) m = fmaxf(m, sp[i]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.f;
  for (int i = tid; i < n; i += 256) {
    const float pv = M == -__builtin_inff() ? 0.f : exp2_fast(sp[i] - M);
    sp[i] = pv;
    l += pv;
  }
  l = wave_sum(l);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  const float Ls = (red[0] + red[1]) + (red[2] + red[3]);

  const int rg = tid >> 4, lc = tid & 15;
  float a[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) a[c] = 0.f;
  for (int i = rg; i < n; i += 16) {
    const int tok = stok[i];
    if (tok < 0) continue;
    const float pv = sp[i];
    const T* vp = Vb + size_t(tok) * D + lc * CPL;
    if constexpr (sizeof(T) == 2) {
      if constexpr (CPL == 8) {
        u32x4 w = ld16(vp);
#pragma unroll
        for (int c = 0; c < 4; ++c) { a[2 * c] += pv * bf16lo(w[c]); a[2 * c + 1] += pv * bf16hi(w[c]); }
      } else {
        u32x2 w = ld8(vp);
#pragma unroll
        for (int c = 0; c < 2; ++c) { a[2 * c] += pv * bf16lo(w[c]); a[2 * c + 1] += pv * bf16hi(w[c]); }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        u32x4 w = ld16(vp + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) a[c + q] += pv * __uint_as_float(w[q]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) racc[rg][lc * CPL + c] = a[c];
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float A = 0.f;
    for (int g = 0; g < 16; ++g) A += racc[g][d];
    const size_t pi = size_t(bhq) * S + s;
    pacc[pi * D + d] = A;
    if (d == 0) { pml[2 * pi] = M; pml[2 * pi + 1] = Ls; }
  }
}

// ---------------------------------------------------------------- merge
template <int D>
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ pacc,
                                               const float* __restrict__ pml, int BHq, int S,
                                               void* __restrict__ O, int out_bf16,
                                               float* __restrict__ lse) {
  constexpr int CPL = D / 64;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= BHq) return;
  const int lane = threadIdx.x & 63;
  const float* ml = pml + size_t(w) * S * 2;
  float M = -__builtin_inff();
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ml[2 * s]);
  M = wave_max(M);
  float Ls = 0.f, A[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) A[c] = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float f = exp2_fast(ml[2 * s] - M);
      Ls += ml[2 * s + 1] * f;
      const float* pa = pacc + (size_t(w) * S + s) * D + lane * CPL;
#pragma unroll
      for (int c = 0; c < CPL; ++c) A[c] += pa[c] * f;
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const float o = Ls > 0.f ? A[c] / Ls : 0.f;
    const size_t oi = size_t(w) * D + lane * CPL + c;
    if (out_bf16) static_cast<uint16_t*>(O)[oi] = uint16_t(f32_to_bf16_rne(o));
    else static_cast<float*>(O)[oi] = o;
  }
  if (lse && lane == 0) lse[w] = Ls > 0.f ? (M + __log2f(Ls)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------- launchers
template <int D, int BLOCK>
static void launch_mfma_g(int G, dim3 g, hipStream_t st, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, int BH, int Hq, int Hkv, int N, float sl2,
                          const int32_t* idx, const int32_t* cnt, int stride, int S, float* pa,
                          float* pm) {
  switch (G) {
    case 1: k_decode_blocks_mfma<D, 1, BLOCK><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, N, sl2, idx, cnt, stride, S, pa, pm); break;
    case 2: k_decode_blocks_mfma<D, 2, BLOCK><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, N, sl2, idx, cnt, stride, S, pa, pm); break;
    case 4: k_decode_blocks_mfma<D, 4, BLOCK><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, N, sl2, idx, cnt, stride, S, pa, pm); break;
    default: k_decode_blocks_mfma<D, 8, BLOCK><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, N, sl2, idx, cnt, stride, S, pa, pm); break;
  }
}

hipError_t launch_decode_blocks(const void* Q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int N, int D, float scale, int block,
                                const int32_t* idx, const int32_t* count, int idx_stride,
                                const DecodeWs& w, void* ws, hipStream_t st) {
  const int BH = B * Hkv, G = Hq / Hkv;
  float* pa = reinterpret_cast<float*>(static_cast<char*>(ws) + w.acc_off);
  float* pm = reinterpret_cast<float*>(static_cast<char*>(ws) + w.ml_off);
  dim3 g(unsigned(long(BH) * w.S));
  const float sl2 = scale * kLog2e;
  if (dtype == SA_BF16) {
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
    auto v = static_cast<const uint16_t*>(V);
    if (D == 128 && block == 64) launch_mfma_g<128, 64>(G, g, st, q, k, v, BH, Hq, Hkv, N, sl2, idx, count, idx_stride, w.S, pa, pm);
    else if (D == 128)           launch_mfma_g<128, 128>(G, g, st, q, k, v, BH, Hq, Hkv, N, sl2, idx, count, idx_stride, w.S, pa, pm);
    else if (block == 64)        launch_mfma_g<64, 64>(G, g, st, q, k, v, BH, Hq, Hkv, N, sl2, idx, count, idx_stride, w.S, pa, pm);
    else                         launch_mfma_g<64, 128>(G, g, st, q, k, v, BH, Hq, Hkv, N, sl2, idx, count, idx_stride, w.S, pa, pm);
  } else {
    auto q = static_cast<const float*>(Q);
    auto k = static_cast<const float*>(K);
    auto v = static_cast<const float*>(V);
    if (D == 128) k_decode_blocks_valu<128><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, G, N, block, sl2, idx, count, idx_stride, w.S, pa, pm);
    else          k_decode_blocks_valu<64><<<g, 256, 0, st>>>(q, k, v, BH, Hq, Hkv, G, N, block, sl2, idx, count, idx_stride, w.S, pa, pm);
  }
  return hipGetLastError();
}

hipError_t launch_decode_tokens(const void* Q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int N, int D, float scale, const int32_t* idx,
                                const int32_t* count, int idx_stride, const float* score,
                                const DecodeWs& w, void* ws, hipStream_t st) {
  const int BHq = B * Hq;
  float* pa = reinterpret_cast<float*>(static_cast<char*>(ws) + w.acc_off);
  float* pm = reinterpret_cast<float*>(static_cast<char*>(ws) + w.ml_off);
  dim3 g(unsigned(long(BHq) * w.S));
  if (dtype == SA_BF16) {
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
    auto v = static_cast<const uint16_t*>(V);
    if (D == 128) k_decode_tokens<uint16_t, 128><<<g, 256, 0, st>>>(q, k, v, BHq, Hq, Hkv, N, scale, idx, count, idx_stride, score, w.S, pa, pm);
    else          k_decode_tokens<uint16_t, 64><<<g, 256, 0, st>>>(q, k, v, BHq, Hq, Hkv, N, scale, idx, count, idx_stride, score, w.S, pa, pm);
  } else {
    auto q = static_cast<const float*>(Q);
    auto k = static_cast<const float*>(K);
    auto v = static_cast<const float*>(V);
    if (D == 128) k_decode_tokens<float, 128><<<g, 256, 0, st>>>(q, k, v, BHq, Hq, Hkv, N, scale, idx, count, idx_stride, score, w.S, pa, pm);
    else          k_decode_tokens<float, 64><<<g, 256, 0, st>>>(q, k, v, BHq, Hq, Hkv, N, scale, idx, count, idx_stride, score, w.S, pa, pm);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DecodeWs& w, const void* ws, int BHq, int D, void* O, int out_dtype,
                        float* lse, hipStream_t st) {
  const float* pa = reinterpret_cast<const float*>(static_cast<const char*>(ws) + w.acc_off);
  const float* pm = reinterpret_cast<const float*>(static_cast<const char*>(ws) + w.ml_off);
  dim3 g(static_cast<unsigned>(cdiv(BHq, 4)));
  const int ob = out_dtype == SA_BF16;
  if (D == 128) k_merge<128><<<g, 256, 0, st>>>(pa, pm, BHq, w.S, O, ob, lse);
  else          k_merge<64><<<g, 256, 0, st>>>(pa, pm, BHq, w.S, O, ob, lse);
  return hipGetLastError();
}

}  // namespace sa
