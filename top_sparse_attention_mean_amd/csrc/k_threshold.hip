// k_threshold.hip -- half-space (threshold) selection with no false negatives.
//
// Every key k_t with q_h . k_t * scale >= tau[b, h] is returned: the half-space
// H(q, tau) of "Sparse Attention as a Range Searching Problem" (Metodologia §1),
// whose defining property is that no key inside it is missed.  With no index
// the exact check runs over every key (the index's second phase, §2, applied to
// all keys), so the kernel is a full scan of K and HBM-bound.
//
// Rigorous float32 test.  A token is kept when fl32(s) + eps_t >= tau, where
// eps_t bounds |fl32(s) - s_exact|:
//   * the dot product is one chain of bf16 matrix-core products (each product of
//     two bf16 values is exact in float32) accumulated in float32; for any
//     summation order and any accumulator that loses at most one unit of 2^-23
//     relative per addition, |err| <= gamma_D * sum_c |q_c k_c| with
//     gamma_D = D u / (1 - D u), u = 2^-23;  float32 inputs add one rounding
//     per product (gamma_{D+1});
//   * sum_c |q_c k_c| is itself computed by a second matrix-core chain on |K|
//     and |q| (a sign-bit mask), so it carries the same relative bound, which
//     the host folds into gamma;
//   * the final scaling, the comparison and tau's own float32 rounding are
//     covered by 2^-20 (|s| + |tau|).
// Hence every exactly-qualifying key is kept; extra keys lie within 2 eps_t
// below tau.
//
// Output order is ascending token position: each wave owns a 128-token
// segment, compacts its kept tokens per head with ballots (token order inside
// a 16-token tile is 4*(lane/16) + r), and stages them; k_threshold_compact
// then prefix-sums the per-segment counts of each (b, head) and copies the
// staged pairs into the capped output lists.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

template <int D, int G>
__global__ __launch_bounds__(256) void k_threshold_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int BH, int Hq, int Hkv,
    int N, float scale, float gamma, const float* __restrict__ tau, int nseg,
    const uint8_t* __restrict__ live, int pblock, int32_t* __restrict__ st_idx,
    float* __restrict__ st_val, int32_t* __restrict__ st_cnt) {
  static_assert(G <= 16, "heads are the 16 columns of the score tile");
  constexpr int NST = D / 32;
  const int bh = blockIdx.x % BH, chunk = blockIdx.x / BH;
  const int b = bh / Hkv, kh = bh % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, nn = lane & 15;
  const int seg = chunk * int(blockDim.x >> 6) + wave;
  if (seg >= nseg) return;  // no barriers below
  // Pruning by block spheres: bit i of the live byte covers the segment's
  // i-th block of `pblock` tokens; a segment with none has its counts zeroed
  // already, and tiles of dead blocks are neither loaded nor kept.
  const int lmask = live ? int(live[size_t(bh) * nseg + seg]) : 0xff;
  if (lmask == 0) return;

  u32x4 qb[NST], qa[NST];
  float th = __builtin_inff();
  if (nn < G) {
    const uint16_t* qp = Q + (size_t(b) * Hq + kh * G + nn) * D + 8 * gq;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      qb[st] = ld16(qp + 32 * st);
      qa[st] = qb[st] & 0x7fff7fffu;
    }
    th = tau[size_t(b) * Hq + kh * G + nn];
  } else {
#pragma unroll
    for (int st = 0; st < NST; ++st) { qb[st] = u32x4{0u, 0u, 0u, 0u}; qa[st] = qb[st]; }
  }
  const float gs = gamma * scale;
  const float tabs = fabsf(th);
  const uint16_t* Kb = K + size_t(bh) * N * D;
  const size_t sbase = ((size_t(b) * Hq + kh * G + min(nn, G - 1)) * nseg + seg) * kThrSeg;
  const uint64_t headmask = 0x0001000100010001ull << nn;
  const uint64_t lower = headmask & ((1ull << (16 * gq)) - 1ull);
  int run = 0;

  // a whole segment's K loads (8 tiles, 32 KiB per wave) are issued before the
  // first is used: measured 129 -> 122 us at 32K tokens x 64 heads (4 tiles: 123)
  constexpr int kTB = 8;
  for (int t0 = 0; t0 < kThrSeg / 16; t0 += kTB) {
    if (seg * kThrSeg + t0 * 16 >= N) break;
    u32x4 ka[kTB][NST];
    bool tl[kTB];
#pragma unroll
    for (int u = 0; u < kTB; ++u) {
      tl[u] = (lmask >> (((t0 + u) * 16) / pblock)) & 1;
      const int kr = min(seg * kThrSeg + (t0 + u) * 16 + nn, N - 1);
      const uint16_t* kp = Kb + size_t(kr) * D + 8 * gq;
#pragma unroll
      for (int st = 0; st < NST; ++st)
        ka[u][st] = tl[u] ? ld16(kp + 32 * st) : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kTB; ++u) {
      const int tok0 = seg * kThrSeg + (t0 + u) * 16;
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, ab = sc;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        sc = mfma16x16x32(ka[u][st], qb[st], sc);
        ab = mfma16x16x32(ka[u][st] & 0x7fff7fffu, qa[st], ab);
      }
      bool keep[4];
      float s32[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tok0 + 4 * gq + r;
        s32[r] = sc[r] * scale;
        const float eps = gs * ab[r] + (fabsf(s32[r]) + tabs) * 9.5367431640625e-07f;  // 2^-20
        keep[r] = tl[u] && nn < G && tok < N && (s32[r] + eps >= th);
      }
      uint64_t m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = __ballot(keep[r]);
      int before = 0, total = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        before += __popcll(m[r] & lower);
        total += __popcll(m[r] & headmask);
      }
      int pos = run + before;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (keep[r]) {
          st_idx[sbase + pos] = tok0 + 4 * gq + r;
          st_val[sbase + pos] = s32[r];
          ++pos;
        }
      }
      run += total;
    }
  }
  if (gq == 0 && nn < G) st_cnt[(size_t(b) * Hq + kh * G + nn) * nseg + seg] = run;
}

// float32 inputs: one token per lane, dot products on the vector ALUs.
template <int D>
__global__ __launch_bounds__(256) void k_threshold_valu(
    const float* __restrict__ Q, const float* __restrict__ K, int BH, int Hq, int Hkv, int G,
    int N, float scale, float gamma, const float* __restrict__ tau, int nseg,
    const uint8_t* __restrict__ live, int pblock, int32_t* __restrict__ st_idx,
    float* __restrict__ st_val, int32_t* __restrict__ st_cnt) {
  __shared__ float sq[16][D];
  const int bh = blockIdx.x % BH, chunk = blockIdx.x / BH;
  const int b = bh / Hkv, kh = bh % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = threadIdx.x; o < G * D; o += blockDim.x)
    sq[o / D][o % D] = Q[(size_t(b) * Hq + kh * G + o / D) * D + o % D];
  __syncthreads();
  const int seg = chunk * int(blockDim.x >> 6) + wave;
  if (seg >= nseg) return;
  const int lmask = live ? int(live[size_t(bh) * nseg + seg]) : 0xff;
  if (lmask == 0) return;
  const float* Kb = K + size_t(bh) * N * D;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int h = 0; h < G; ++h) {
    const float th = tau[size_t(b) * Hq + kh * G + h];
    const size_t sbase = ((size_t(b) * Hq + kh * G + h) * nseg + seg) * kThrSeg;
    int run = 0;
    for (int part = 0; part < kThrSeg / 64; ++part) {
      const int tok = seg * kThrSeg + part * 64 + lane;
      const bool tlive = (lmask >> ((part * 64 + lane) / pblock)) & 1;
      float s = 0.f, a = 0.f;
      if (tok < N && tlive) {
        const float* kp = Kb + size_t(tok) * D;
        for (int d = 0; d < D; d += 4) {
          u32x4 w = ld16(kp + d);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float kv = __uint_as_float(w[c]);
            s += sq[h][d + c] * kv;
            a += fabsf(sq[h][d + c] * kv);
          }
        }
      }
      const float s32 = s * scale;
      const float eps = gamma * scale * a + (fabsf(s32) + fabsf(th)) * 9.5367431640625e-07f;
      const bool keep = tok < N && tlive && (s32 + eps >= th);
      const uint64_t m = __ballot(keep);
      if (keep) {
        const int pos = run + __popcll(m & below);
        st_idx[sbase + pos] = tok;
        st_val[sbase + pos] = s32;
      }
      run += __popcll(m);
    }
    if (lane == 0) st_cnt[(size_t(b) * Hq + kh * G + h) * nseg + seg] = run;
  }
}

// ---------------------------------------------------------------- top-delta
// Threshold from a pseudo-maximum ("Faster Than Flash", Metodologia §2): per
// query head, m~ = the largest score over the sink prefix [0, sink) and the
// local window [N - local, N), and tau = m~ - delta.  One 256-thread workgroup
// per (b, kv head) scores those <= sink + local tokens for the g heads of the
// group; nothing else of the cache is read, so no reduction over the whole
// cache is needed before the scan.
//
// tau stays on the safe side of the exact value: the workgroup takes the
// maximum of fl32(s) - eps_t, a lower bound of every exact score (eps_t as in
// the scan, without the tau term), so tau <= m~_exact - delta up to its own
// float32 rounding, which the scan's comparison already covers.  Keys whose
// exact score reaches m~_exact - delta are therefore all kept.
struct PmWindow {
  int ns, t0, W;  // sink tokens [0, ns), local tokens [t0, N), W = ns + N - t0
  __device__ int token(int v) const { return v < ns ? v : t0 + (v - ns); }
};

__device__ __forceinline__ PmWindow pm_window(int N, int sink, int local) {
  PmWindow w;
  w.ns = min(sink, N);
  w.t0 = max(N - min(local, N), w.ns);
  w.W = w.ns + (N - w.t0);
  return w;
}

// bf16: 16-token tiles on the same matrix-core chains as the scan.
template <int D, int G>
__global__ __launch_bounds__(256) void k_pseudo_max_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int Hq, int Hkv, int N,
    int sink, int local, float delta, float scale, float gamma, float* __restrict__ tau) {
  static_assert(G <= 16, "heads are the 16 columns of the score tile");
  constexpr int NST = D / 32;
  __shared__ float red[4][16];
  const int bh = blockIdx.x, b = bh / Hkv, kh = bh % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, nn = lane & 15;
  const PmWindow win = pm_window(N, sink, local);
  u32x4 qb[NST], qa[NST];
  const uint16_t* qp = Q + (size_t(b) * Hq + kh * G + min(nn, G - 1)) * D + 8 * gq;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    qb[st] = nn < G ? ld16(qp + 32 * st) : u32x4{0u, 0u, 0u, 0u};
    qa[st] = qb[st] & 0x7fff7fffu;
  }
  const float gs = gamma * scale;
  const uint16_t* Kb = K + size_t(bh) * N * D;
  float lo = -__builtin_inff();
  for (int v0 = wave * 16; v0 < win.W; v0 += 64) {
    const int kr = win.token(min(v0 + nn, win.W - 1));
    const uint16_t* kp = Kb + size_t(kr) * D + 8 * gq;
    u32x4 ka[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) ka[st] = ld16(kp + 32 * st);
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, ab = sc;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      sc = mfma16x16x32(ka[st], qb[st], sc);
      ab = mfma16x16x32(ka[st] & 0x7fff7fffu, qa[st], ab);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s32 = sc[r] * scale;
      const float eps = gs * ab[r] + fabsf(s32) * 9.5367431640625e-07f;  // 2^-20
      if (v0 + 4 * gq + r < win.W) lo = fmaxf(lo, s32 - eps);
    }
  }
  // lanes nn, nn + 16, nn + 32, nn + 48 hold head nn's rows
  lo = fmaxf(lo, __shfl_xor(lo, 16));
  lo = fmaxf(lo, __shfl_xor(lo, 32));
  if (gq == 0) red[wave][nn] = lo;
  __syncthreads();
  if (wave == 0 && gq == 0 && nn < G) {
    const float m = fmaxf(fmaxf(red[0][nn], red[1][nn]), fmaxf(red[2][nn], red[3][nn]));
    tau[size_t(b) * Hq + kh * G + nn] = m - delta;
  }
}

// float32: one (token, head) pair per thread, dot products on the vector ALUs.
template <int D>
__global__ __launch_bounds__(256) void k_pseudo_max_valu(
    const float* __restrict__ Q, const float* __restrict__ K, int Hq, int Hkv, int G, int N,
    int sink, int local, float delta, float scale, float gamma, float* __restrict__ tau) {
  __shared__ float sq[8][D];
  __shared__ float red[8][4];
  const int bh = blockIdx.x, b = bh / Hkv, kh = bh % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = threadIdx.x; o < G * D; o += 256)
    sq[o / D][o % D] = Q[(size_t(b) * Hq + kh * G + o / D) * D + o % D];
  __syncthreads();
  const PmWindow win = pm_window(N, sink, local);
  const float* Kb = K + size_t(bh) * N * D;
  for (int h = 0; h < G; ++h) {
    float lo = -__builtin_inff();
    for (int v = threadIdx.x; v < win.W; v += 256) {
      const float* kp = Kb + size_t(win.token(v)) * D;
      float s = 0.f, a = 0.f;
      for (int d = 0; d < D; d += 4) {
        const u32x4 w = ld16(kp + d);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float kv = __uint_as_float(w[c]);
          s += sq[h][d + c] * kv;
          a += fabsf(sq[h][d + c] * kv);
        }
      }
      const float s32 = s * scale;
      lo = fmaxf(lo, s32 - (gamma * scale * a + fabsf(s32) * 9.5367431640625e-07f));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lo = fmaxf(lo, __shfl_xor(lo, o));
    if (lane == 0) red[h][wave] = lo;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    const float m = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
    tau[size_t(b) * Hq + kh * G + h] = m - delta;
  }
}

// One 256-thread workgroup per (b, query head): ordered copy of the staged
// segments into idx/score [cap] and the true count.  Thread t sums the counts
// of its run of `per` consecutive segments; a block scan gives each run's
// output offset.  The copy then goes by output position: position p finds its
// run by binary search over the 256 run offsets and its segment by walking at
// most `per` counts, so every position is copied independently.  With up to
// kCompactLds segments (N <= 512K) the counts sit in LDS, and each thread
// issues the loads of 4 positions before their stores: the only global reads
// on a position's path are its staged pair.
constexpr int kCompactLds = 4096;

template <bool LDS>
__global__ __launch_bounds__(256) void k_threshold_compact(
    const int32_t* __restrict__ st_idx, const float* __restrict__ st_val,
    const int32_t* __restrict__ st_cnt, int nseg, int cap, int32_t* __restrict__ idx,
    float* __restrict__ score, int32_t* __restrict__ count) {
  __shared__ int scan[17];
  __shared__ int toff[256];
  __shared__ int cl[LDS ? kCompactLds : 1];
  const int bhq = blockIdx.x, tid = threadIdx.x;
  const int per = (nseg + 255) / 256;
  const int s0 = min(tid * per, nseg), s1 = min(s0 + per, nseg);
  const int32_t* cnt = st_cnt + size_t(bhq) * nseg;
  if constexpr (LDS) {
    for (int s = tid; s < nseg; s += 256) cl[s] = cnt[s];
    __syncthreads();
  }
  auto count_of = [&](int s) { if constexpr (LDS) return cl[s]; else return cnt[s]; };
  int mine = 0;
  for (int s = s0; s < s1; ++s) mine += count_of(s);
  int total;
  toff[tid] = block_excl_scan<256>(mine, scan, &total);
  __syncthreads();
  int32_t* oi = idx + size_t(bhq) * cap;
  float* ov = score + size_t(bhq) * cap;
  const size_t sb = size_t(bhq) * nseg;
  const int lim = min(total, cap);
  auto source = [&](int p) -> size_t {
    int lo = 0, hi = 255;           // the last run whose offset is <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (toff[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    int s = lo * per, q = p - toff[lo];
    for (int c = count_of(s); q >= c; c = count_of(s)) { q -= c; ++s; }
    return (sb + s) * kThrSeg + q;
  };
  constexpr int U = 4;
  for (int p0 = tid; p0 < lim; p0 += 256 * U) {
    int32_t vi[U];
    float vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + 256 * u;
      if (p < lim) {
        const size_t src = source(p);
        vi[u] = st_idx[src];
        vv[u] = st_val[src];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + 256 * u;
      if (p < lim) {
        oi[p] = vi[u];
        ov[p] = vv[u];
      }
    }
  }
  for (int p = total + tid; p < cap; p += 256) {
    oi[p] = -1;
    ov[p] = -__builtin_inff();
  }
  if (tid == 0) count[bhq] = total;
}

// gamma of the float32 score bound: D bf16 products (exact) or D + 1 roundings
// per float32 term, and the |q|.|k| sum's own relative error, plus margin.
static float score_gamma(int dtype, int D) {
  const double u = 1.0 / 8388608.0;  // 2^-23
  const int terms = dtype == SA_BF16 ? D : D + 1;
  const double gam = terms * u / (1.0 - terms * u);
  return float(gam * (1.0 + gam) * 1.001);
}

hipError_t launch_pseudo_max(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv,
                             int N, int D, int sink, int local, float delta, float scale,
                             float* tau, hipStream_t st) {
  const int G = Hq / Hkv;
  const dim3 g(unsigned(B * Hkv));
  const float gamma = score_gamma(dtype, D);
  if (dtype == SA_BF16) {
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
#define SA_PM(DD, GG) k_pseudo_max_mfma<DD, GG><<<g, 256, 0, st>>>(q, k, Hq, Hkv, N, sink, local, delta, scale, gamma, tau)
    if (D == 128) {
      switch (G) { case 1: SA_PM(128, 1); break; case 2: SA_PM(128, 2); break;
                   case 4: SA_PM(128, 4); break; default: SA_PM(128, 8); break; }
    } else {
      switch (G) { case 1: SA_PM(64, 1); break; case 2: SA_PM(64, 2); break;
                   case 4: SA_PM(64, 4); break; default: SA_PM(64, 8); break; }
    }
#undef SA_PM
  } else {
    auto q = static_cast<const float*>(Q);
    auto k = static_cast<const float*>(K);
    if (D == 128) k_pseudo_max_valu<128><<<g, 256, 0, st>>>(q, k, Hq, Hkv, G, N, sink, local, delta, scale, gamma, tau);
    else          k_pseudo_max_valu<64><<<g, 256, 0, st>>>(q, k, Hq, Hkv, G, N, sink, local, delta, scale, gamma, tau);
  }
  return hipGetLastError();
}

hipError_t launch_threshold(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv,
                            int N, int D, const float* tau, float scale, int cap, int32_t* idx,
                            float* score, int32_t* count, const ThrWs& w, void* ws,
                            hipStream_t st, const uint8_t* live, int pblock) {
  const int BH = B * Hkv, G = Hq / Hkv;
  char* base = static_cast<char*>(ws);
  int32_t* si = reinterpret_cast<int32_t*>(base + w.idx_off);
  float* sv = reinterpret_cast<float*>(base + w.val_off);
  int32_t* sc = reinterpret_cast<int32_t*>(base + w.cnt_off);
  // Unpruned: 4 waves (4 consecutive segments) per workgroup.  Pruned: one
  // wave per workgroup, so a pruned segment frees its slot at once instead of
  // idling inside a workgroup whose other waves scan (measured: 4-wave groups
  // with a quarter of the segments live ran at a quarter of the bandwidth).
  const int wpb = live ? 1 : 4;
  const dim3 g(unsigned(long(BH) * cdiv(w.nseg, wpb))), t(unsigned(64 * wpb));
  const float gamma = score_gamma(dtype, D);
  if (dtype == SA_BF16) {
    auto q = static_cast<const uint16_t*>(Q);
    auto k = static_cast<const uint16_t*>(K);
#define SA_THR(DD, GG) k_threshold_mfma<DD, GG><<<g, t, 0, st>>>(q, k, BH, Hq, Hkv, N, scale, gamma, tau, w.nseg, live, pblock, si, sv, sc)
    if (D == 128) {
      switch (G) { case 1: SA_THR(128, 1); break; case 2: SA_THR(128, 2); break;
                   case 4: SA_THR(128, 4); break; default: SA_THR(128, 8); break; }
    } else {
      switch (G) { case 1: SA_THR(64, 1); break; case 2: SA_THR(64, 2); break;
                   case 4: SA_THR(64, 4); break; default: SA_THR(64, 8); break; }
    }
#undef SA_THR
  } else {
    auto q = static_cast<const float*>(Q);
    auto k = static_cast<const float*>(K);
    if (D == 128) k_threshold_valu<128><<<g, t, 0, st>>>(q, k, BH, Hq, Hkv, G, N, scale, gamma, tau, w.nseg, live, pblock, si, sv, sc);
    else          k_threshold_valu<64><<<g, t, 0, st>>>(q, k, BH, Hq, Hkv, G, N, scale, gamma, tau, w.nseg, live, pblock, si, sv, sc);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (w.nseg <= kCompactLds)
    k_threshold_compact<true><<<dim3(B * Hq), 256, 0, st>>>(si, sv, sc, w.nseg, cap, idx, score, count);
  else
    k_threshold_compact<false><<<dim3(B * Hq), 256, 0, st>>>(si, sv, sc, w.nseg, cap, idx, score, count);
  return hipGetLastError();
}

}  // namespace sa
