// k_lowbit.hip -- 2-bit key thumbnails with 8-bit residuals, and the top-delta
// block filter that scans them.
//
// "Faster Than Flash" (Metodologia §1) keeps the key cache as 2-bit quantised
// thumbnails, which a fast scan reads to estimate the scores, plus 8-bit
// residuals that rebuild the keys close to their stored precision for the
// exact computation; its fused kernel (§3) runs a pseudo-maximum over the sink
// and local tokens, a top-delta filter of blocks over the thumbnails, and a
// refinement with residuals and values on the kept blocks.
//
// Codec (the pages give none; per channel over each token block, so outlier
// channels keep their own range):
//   lo, hi = min, max of the channel over the block;  step = (hi - lo) * fl(1/3)
//   code   = [d >= step/2] + [d >= 1.5 step] + [d >= 2.5 step],  d = k - lo
//   t      = fma(code, step, lo)                       (the thumbnail)
//   rstep  = 2^(E - 8), step = m 2^E, m in [0.5, 1)     (a power of two)
//   r8     = clamp(rint((k - t) / rstep), -127, 127);   k^ = t + r8 * rstep
// Every step is one IEEE float32 operation, so codes and residuals are a
// fixed function of the keys.  Storage per token and kv head: D/4 bytes of
// codes (one 32-bit word per 16 channels, channel 16 g + i at bit
// 8 (i % 4) + 2 (i / 4) of word g) and D bytes of residuals;
// per block: (lo, step, rstep) float32 rows of D.  The scan reads the codes
// and lo/step only: D/4 + 8 D / block bytes per token (48 B at D = 128, block
// 64) instead of 2 D (256 B).
//
// Kernels:
//   k_encode       one workgroup per (b, head, block): channel ranges, codes,
//                  residuals (run when the cache is written; a block range).
//   k_decode_keys  one workgroup per listed block (or per block of a range):
//                  k^ rounded to bf16 into a key buffer laid out as K.
//   k_thumb_scan   one wave per (b, kv head, block): provisional scores from
//                  the codes on the int8 matrix cores for the g heads (block
//                  offset q . lo plus the codes against int8 weights of
//                  q_c step_c), the block maximum per head, and the keep flag
//                  (some head reaches tau_h - margin, or a window block).
//   k_block_list   one workgroup per (b, kv head): flags -> ascending list.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr float kThird = 0.3333333432674408f;   // fl32(1/3)



template <typename T, int D>
__global__ __launch_bounds__(256) void k_encode(const T* __restrict__ K, int N, int block, int nb,
                                                int b0, int nbr, uint8_t* __restrict__ codes,
                                                int8_t* __restrict__ resid,
                                                float* __restrict__ meta) {
  constexpr int PARTS = 256 / D;              // token stripes per channel
  __shared__ float smin[PARTS][D], smax[PARTS][D];
  const int j = b0 + int(blockIdx.x % nbr), bh = blockIdx.x / nbr;
  const int t0 = j * block, nj = min(block, N - t0);
  const int c = threadIdx.x % D, part = threadIdx.x / D;
  const T* Kb = K + (size_t(bh) * N + t0) * D + c;
  auto key = [&](int r) -> float {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(Kb[size_t(r) * D]);
    else return Kb[size_t(r) * D];
  };
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int r = part; r < nj; r += PARTS) {
    const float x = key(r);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  smin[part][c] = mn;
  smax[part][c] = mx;
  __syncthreads();
  float lo = smin[0][c], hi = smax[0][c];
#pragma unroll
  for (int p = 1; p < PARTS; ++p) { lo = fminf(lo, smin[p][c]); hi = fmaxf(hi, smax[p][c]); }
  const float step = (hi - lo) * kThird;
  int E;
  (void)frexpf(step, &E);
  const float rstep = ldexpf(1.0f, E - 8), rinv = ldexpf(1.0f, 8 - E);
  if (part == 0) {
    float* mrow = meta + (size_t(bh) * nb + j) * 3 * D;
    mrow[c] = lo;
    mrow[D + c] = step;
    mrow[2 * D + c] = rstep;
  }
  const float h1 = step * 0.5f, h2 = step * 1.5f, h3 = step * 2.5f;
  const int lane = threadIdx.x & 63;
  for (int r = part; r < nj; r += PARTS) {
    const float x = key(r);
    const float d = x - lo;
    const int code = int(d >= h1) + int(d >= h2) + int(d >= h3);
    const float t = fmaf(float(code), step, lo);
    const float q = rintf((x - t) * rinv);
    const int r8 = int(fminf(fmaxf(q, -127.f), 127.f));
    const size_t row = size_t(bh) * N + t0 + r;
    resid[row * D + c] = int8_t(r8);
    // pack the codes of channels 16 g .. 16 g + 15 (consecutive lanes) into one
    // word, channel 16 g + i at bit 8 (i % 4) + 2 (i / 4)
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      word |= uint32_t(__shfl(code, (lane & ~15) + i)) << (8 * (i & 3) + 2 * (i >> 2));
    if ((c & 15) == 0) *reinterpret_cast<uint32_t*>(codes + row * (D / 4) + c / 4) = word;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_decode_keys(
    const uint8_t* __restrict__ codes, const int8_t* __restrict__ resid,
    const float* __restrict__ meta, int N, int block, int nb, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ count, int idx_stride, int b0, int nbr,
    uint16_t* __restrict__ khat) {
  constexpr int TPR = D / 8;                  // threads per token row (8 channels each)
  constexpr int RPP = 256 / TPR;
  int j, bh;
  if (idx) {
    bh = blockIdx.x / idx_stride;
    const int slot = blockIdx.x % idx_stride;
    const int n = count ? min(max(count[bh], 0), idx_stride) : idx_stride;
    if (slot >= n) return;
    j = idx[size_t(bh) * idx_stride + slot];
    if (j < 0 || j >= nb) return;
  } else {
    bh = blockIdx.x / nbr;
    j = b0 + int(blockIdx.x % nbr);
  }
  const int t0 = j * block, nj = min(block, N - t0);
  const int tr = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * 8;
  const float* mrow = meta + (size_t(bh) * nb + j) * 3 * D;
  float lo[8], st[8], rs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { lo[e] = mrow[c0 + e]; st[e] = mrow[D + c0 + e]; rs[e] = mrow[2 * D + c0 + e]; }
  for (int r = tr; r < nj; r += RPP) {
    const size_t row = size_t(bh) * N + t0 + r;
    // channels c0 .. c0 + 7 are the half h of their 16-channel word
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + row * (D / 4) + (c0 / 16) * 4);
    const int h = (c0 & 15) >> 3;
    const u32x2 rw = ld8(resid + row * D + c0);
    float kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int code = int((cw >> (8 * (e & 3) + 2 * (2 * h + (e >> 2)))) & 3u);
      const int r8 = int(int8_t((rw[e / 4] >> (8 * (e % 4))) & 0xffu));
      const float t = fmaf(float(code), st[e], lo[e]);
      kh[e] = t + float(r8) * rs[e];
    }
    uint32_t outw[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) outw[p] = pack_bf16x2(kh[2 * p], kh[2 * p + 1]);
    *reinterpret_cast<u32x4*>(khat + row * D + c0) = u32x4{outw[0], outw[1], outw[2], outw[3]};
  }
}

// One wave per (b, kv head, block); 4 waves per workgroup.
//
// The provisional score of token t in block j is the thumbnail dot product
// split into the block offset and the code term, the latter on int8 matrix
// cores:
//     s~ = scale * (q . lo_j + ws * sum_c w8_c code_t,c),
//     w_c = fl(q_c step_j,c),  ws = max_c |w_c| * fl(1/127),
//     w8_c = clamp(rint(w_c * fl(127 / max_c |w_c|)), -127, 127)
// The codes word of 16 channels holds channel i at bit 8 (i % 4) + 2 (i / 4), so
// (word >> 2m) & 0x03030303 is the 4 int8 codes of channels 4m .. 4m + 3: the
// A operand costs two operations per 4 channels.  The weights w8 (B operand)
// and the offset are built once per block.
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int D, int G>
__global__ __launch_bounds__(256) void k_thumb_scan(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ codes,
    const float* __restrict__ meta, int Hq, int Hkv, int N, int block, int nb, float scale,
    const float* __restrict__ tau, float margin, int f0, int f1, int f2, int f3,
    float* __restrict__ bmax, uint8_t* __restrict__ flag) {
  static_assert(G <= 16, "heads are the 16 columns of the score tile");
  constexpr int NST = D / 64;                 // 64 channels per int8 product
  const int nbw = (nb + 3) / 4;
  const int bh = blockIdx.x / nbw;
  const int j = (blockIdx.x % nbw) * 4 + int(threadIdx.x >> 6);
  if (j >= nb) return;                        // no barriers in this kernel
  const int b = bh / Hkv, kh = bh % Hkv;
  const int lane = threadIdx.x & 63, gq = lane >> 4, nn = lane & 15;
  const int t0 = j * block, nj = min(block, N - t0);
  const uint8_t* cb = codes + (size_t(bh) * N + t0) * (D / 4);
  // every tile's code words first (a block is at most 8 tiles; token row
  // 16 u + nn, rows past the block repeat its last row): channels
  // 64 st + 16 gq .. + 15 of the row, one word each
  constexpr int MT = 8;
  uint32_t cw[MT][NST];
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int r = min(16 * u + nn, nj - 1);
#pragma unroll
    for (int st = 0; st < NST; ++st)
      cw[u][st] = 16 * u < nj
          ? *reinterpret_cast<const uint32_t*>(cb + size_t(r) * (D / 4) + 4 * (4 * st + gq)) : 0u;
  }
  // the block's (lo, step) rows (2 D floats) through this wave's LDS slice
  __shared__ __attribute__((aligned(16))) float sm[4][2 * D];
  __shared__ __attribute__((aligned(16))) int8_t swt[4][8][D];   // int8 weights per head
  __shared__ float soff[4][8], sws[4][8];
  const int wv = threadIdx.x >> 6;
  float* mw = sm[wv];
  const float* mrow = meta + (size_t(bh) * nb + j) * 3 * D;
  if (lane < D / 2) *reinterpret_cast<u32x4*>(mw + 4 * lane) = ld16(mrow + 4 * lane);
  __builtin_amdgcn_wave_barrier();
  // weights of the group's heads, 4 heads at a time: lane (hh, cc) takes head
  // hh and channels (D / 16) cc .. + D / 16, then the 16 lanes of a head reduce
  constexpr int CPL = D / 16;
  const int hh0 = lane >> 4, cc = lane & 15;
  for (int hb = 0; hb < G; hb += 4) {
    const int hh = hb + hh0;
    const bool real = hh < G;
    const uint16_t* qh = Q + (size_t(b) * Hq + kh * G + min(hh, G - 1)) * D + CPL * cc;
    static_assert(CPL == 4 || CPL == 8, "D is 64 or 128");
    uint32_t qw[CPL / 2];
    if constexpr (CPL == 8) {
      const u32x4 v = real ? ld16(qh) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int p = 0; p < 4; ++p) qw[p] = v[p];
    } else {
      const u32x2 v = real ? ld8(qh) : u32x2{0u, 0u};
      qw[0] = v[0];
      qw[1] = v[1];
    }
    float wv8[CPL];
    float off = 0.f, wmax = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const float qf = (e & 1) ? bf16hi(qw[e >> 1]) : bf16lo(qw[e >> 1]);
      const int c = CPL * cc + e;
      off += qf * mw[c];
      wv8[e] = qf * mw[D + c];
      wmax = fmaxf(wmax, fabsf(wv8[e]));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      off += __shfl_xor(off, o);
      wmax = fmaxf(wmax, __shfl_xor(wmax, o));
    }
    const float winv = wmax > 0.f ? __fdiv_rn(127.f, wmax) : 0.f;
#pragma unroll
    for (int e0 = 0; e0 < CPL; e0 += 4) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __builtin_amdgcn_fmed3f(rintf(wv8[e0 + e] * winv), -127.f, 127.f);
        word |= uint32_t(int(x) & 0xff) << (8 * e);
      }
      if (real) *reinterpret_cast<uint32_t*>(&swt[wv][hh][CPL * cc + e0]) = word;
    }
    if (real && cc == 0) {
      soff[wv][hh] = off;
      sws[wv][hh] = wmax * 0.007874015718698502f;   // fl32(1/127)
    }
  }
  __builtin_amdgcn_wave_barrier();
  // B operand: head nn's int8 weights at channels 64 st + 16 gq .. + 15
  i32x4 wb[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    const u32x4 wq = nn < G ? *reinterpret_cast<const u32x4*>(&swt[wv][min(nn, G - 1)][64 * st + 16 * gq])
                            : u32x4{0u, 0u, 0u, 0u};
    wb[st] = i32x4{int(wq[0]), int(wq[1]), int(wq[2]), int(wq[3])};
  }
  const float off = soff[wv][min(nn, G - 1)], ws = sws[wv][min(nn, G - 1)];
  const float th = nn < G ? tau[size_t(b) * Hq + kh * G + nn] : 0.f;
  float m = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    if (16 * u >= nj) break;
    i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const uint32_t x = cw[u][st];
      const i32x4 a = i32x4{int(x & 0x03030303u), int((x >> 2) & 0x03030303u),
                            int((x >> 4) & 0x03030303u), int((x >> 6) & 0x03030303u)};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wb[st], acc, 0, 0, 0);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (16 * u + 4 * gq + rr < nj) m = fmaxf(m, float(acc[rr]));
  }
  // lanes nn, nn + 16, nn + 32, nn + 48 hold head nn's rows
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  m = scale * (off + ws * m);
  if (bmax && gq == 0 && nn < G) bmax[(size_t(b) * Hq + kh * G + nn) * nb + j] = m;
  const bool win = (j >= f0 && j < f1) || (j >= f2 && j < f3);
  const uint64_t any = __ballot(gq == 0 && nn < G && m >= th - margin);
  if (lane == 0) flag[size_t(bh) * nb + j] = (any != 0ull || win) ? 1 : 0;
}

// flags [BH, nb] -> ascending idx [BH, kcap] (-1 padded) and the true count.
__global__ __launch_bounds__(256) void k_block_list(const uint8_t* __restrict__ flag, int nb,
                                                    int kcap, int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ count) {
  __shared__ int scan[17];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int per = (nb + 255) / 256;
  const int s0 = min(tid * per, nb), s1 = min(s0 + per, nb);
  const uint8_t* f = flag + size_t(bh) * nb;
  int mine = 0;
  for (int s = s0; s < s1; ++s) mine += f[s];
  int total;
  int off = block_excl_scan<256>(mine, scan, &total);
  int32_t* o = idx + size_t(bh) * kcap;
  for (int s = s0; s < s1; ++s) {
    if (f[s]) {
      if (off < kcap) o[off] = s;
      ++off;
    }
  }
  for (int p = total + tid; p < kcap; p += 256) o[p] = -1;
  if (tid == 0) count[bh] = total;
}

hipError_t launch_encode(const void* K, int dtype, int B, int H, int N, int D, int block, int b0,
                         int b1, uint8_t* codes, int8_t* resid, float* meta, hipStream_t st) {
  const int nb = cdiv(N, block), nbr = b1 - b0;
  if (nbr <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(long(B) * H * nbr));
  if (dtype == SA_BF16) {
    auto k = static_cast<const uint16_t*>(K);
    if (D == 128) k_encode<uint16_t, 128><<<g, 256, 0, st>>>(k, N, block, nb, b0, nbr, codes, resid, meta);
    else          k_encode<uint16_t, 64><<<g, 256, 0, st>>>(k, N, block, nb, b0, nbr, codes, resid, meta);
  } else {
    auto k = static_cast<const float*>(K);
    if (D == 128) k_encode<float, 128><<<g, 256, 0, st>>>(k, N, block, nb, b0, nbr, codes, resid, meta);
    else          k_encode<float, 64><<<g, 256, 0, st>>>(k, N, block, nb, b0, nbr, codes, resid, meta);
  }
  return hipGetLastError();
}

hipError_t launch_decode_keys(const uint8_t* codes, const int8_t* resid, const float* meta, int B,
                              int H, int N, int D, int block, const int32_t* idx,
                              const int32_t* count, int idx_stride, int b0, int b1,
                              uint16_t* khat, hipStream_t st) {
  const int nb = cdiv(N, block);
  const long units = idx ? long(B) * H * idx_stride : long(B) * H * (b1 - b0);
  if (units <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(units));
  if (D == 128) k_decode_keys<128><<<g, 256, 0, st>>>(codes, resid, meta, N, block, nb, idx, count, idx_stride, b0, b1 - b0, khat);
  else          k_decode_keys<64><<<g, 256, 0, st>>>(codes, resid, meta, N, block, nb, idx, count, idx_stride, b0, b1 - b0, khat);
  return hipGetLastError();
}

hipError_t launch_thumb_scan(const uint16_t* Q, const uint8_t* codes, const float* meta, int B,
                             int Hq, int Hkv, int N, int D, int block, float scale,
                             const float* tau, float margin, int f0, int f1, int f2, int f3,
                             float* bmax, uint8_t* flag, hipStream_t st) {
  const int nb = cdiv(N, block), G = Hq / Hkv;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * cdiv(nb, 4)));
#define SA_TS(DD, GG) k_thumb_scan<DD, GG><<<g, 256, 0, st>>>(Q, codes, meta, Hq, Hkv, N, block, nb, scale, tau, margin, f0, f1, f2, f3, bmax, flag)
  if (D == 128) {
    switch (G) { case 1: SA_TS(128, 1); break; case 2: SA_TS(128, 2); break;
                 case 4: SA_TS(128, 4); break; default: SA_TS(128, 8); break; }
  } else {
    switch (G) { case 1: SA_TS(64, 1); break; case 2: SA_TS(64, 2); break;
                 case 4: SA_TS(64, 4); break; default: SA_TS(64, 8); break; }
  }
#undef SA_TS
  return hipGetLastError();
}

hipError_t launch_block_list(const uint8_t* flag, int BH, int nb, int kcap, int32_t* idx,
                             int32_t* count, hipStream_t st) {
  k_block_list<<<dim3(unsigned(BH)), 256, 0, st>>>(flag, nb, kcap, idx, count);
  return hipGetLastError();
}

}  // namespace sa
