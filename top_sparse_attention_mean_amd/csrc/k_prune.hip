// k_prune.hip -- bounding spheres of key blocks and the pruned threshold scan.
//
// "Sparse Attention as a Range Searching Problem" (Metodologia §2) cuts the
// key space into S contiguous subspaces, encloses every cluster of keys in a
// sphere per subspace (centre c_s, radius rho_s) and drops a cluster when no
// sphere point can reach the half-space <q, k> >= tau; only keys of surviving
// clusters get the exact check.  Here the clusters are the contiguous token
// blocks and the centre is the block's sketch row, so one sketch serves both
// top-k scoring and pruning.
//
// For every key k of block j,  q . k = sum_s q_s . c_s + q_s . (k_s - c_s)
//                                   <= sum_s q_s . c_s + ||q_s|| rho_s,
// so a block whose bound is below tau holds no key at or above tau: pruning
// keeps the zero-false-negative guarantee.  The float32 rounding of the bound
// is covered by a margin (below), and the radius is rounded up.
//
// k_radius  one 256-thread workgroup per (b, head, block) of a block range:
//           the largest distance of the block's keys from the given centre,
//           per subspace (a range of one block refreshes the newest block's
//           sphere as keys are appended, as the sketch refresh does).
// k_prune   one workgroup per (b, kv head, 64 blocks): the bound for every
//           block and every query head of the group (one (block, head) pair
//           per thread over the sketch rows staged transposed in LDS, so the
//           dot products need no cross-lane reductions).  A block stays live
//           when it can reach the tau of any head of the group; the live byte
//           of a 128-token staging segment of the threshold scan has bit i set
//           for its live i-th block.  Segments with no live block get zero
//           staged counts for every head and are skipped; in the others the
//           scan loads only the tiles of live blocks.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

// Radius rounding: the float32 squares, sums and square root lose at most
// (D + 4) units of 2^-24 relative; scaling by 1 + 2^-16 rounds the result up.
constexpr float kRadiusUp = 1.0f + 1.52587890625e-05f;  // 1 + 2^-16

template <typename T, int D>
__global__ __launch_bounds__(256) void k_radius(const T* __restrict__ X, int H, int N, int block,
                                                int nb, int b0, int nbr, int S,
                                                const float* __restrict__ sk,
                                                float* __restrict__ rad) {
  constexpr int CPT = 8;            // columns per thread
  constexpr int TPR = D / CPT;      // threads per row
  constexpr int RPP = 256 / TPR;    // rows per pass
  __shared__ float red[RPP][TPR];
  const int j = b0 + int(blockIdx.x % nbr), bh = blockIdx.x / nbr;
  const int t0 = j * block, nj = min(block, N - t0);
  const int tr = threadIdx.x / TPR, tc = threadIdx.x % TPR;
  const int LS = (D / S) / CPT;     // threads (lanes) per subspace within a row

  float c[CPT];
  const float* cp = sk + (size_t(bh) * nb + j) * D + tc * CPT;
  {
    const u32x4 w0 = ld16(cp), w1 = ld16(cp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { c[e] = __uint_as_float(w0[e]); c[4 + e] = __uint_as_float(w1[e]); }
  }
  float mx = 0.f;
  for (int r = tr; r < nj; r += RPP) {
    const T* p = X + (size_t(bh) * N + t0 + r) * D + tc * CPT;
    float k[CPT];
    if constexpr (sizeof(T) == 2) {
      const u32x4 w = ld16(p);
#pragma unroll
      for (int e = 0; e < 4; ++e) { k[2 * e] = bf16lo(w[e]); k[2 * e + 1] = bf16hi(w[e]); }
    } else {
      const u32x4 w0 = ld16(p), w1 = ld16(p + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { k[e] = __uint_as_float(w0[e]); k[4 + e] = __uint_as_float(w1[e]); }
    }
    float d2 = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const float d = k[e] - c[e];
      d2 += d * d;
    }
    // the row's squared distance in this subspace: sum over its LS lanes
    for (int o = 1; o < LS; o <<= 1) d2 += __shfl_xor(d2, o);
    mx = fmaxf(mx, d2);
  }
  red[tr][tc] = mx;
  __syncthreads();
  if (threadIdx.x < S) {
    const int s = threadIdx.x;
    float m = 0.f;
    for (int g = 0; g < RPP; ++g) m = fmaxf(m, red[g][s * LS]);
    rad[(size_t(bh) * nb + j) * S + s] = sqrtf(m) * kRadiusUp;
  }
}

// Bound margin: the dot product q . c (at most D + 6 roundings on this
// path) is off by less than 2^-16 ||q|| ||c||, the radius term by less than
// 2^-16 of itself; the scaling and the comparison are covered by
// 2^-20 (|ub| + |tau|).
constexpr float kBoundRel = 1.52587890625e-05f;   // 2^-16
constexpr float kCmpRel = 9.5367431640625e-07f;   // 2^-20
constexpr int kPruneRows = 64;                    // blocks per workgroup

template <typename T, int D>
__global__ __launch_bounds__(256) void k_prune(
    const T* __restrict__ Q, const float* __restrict__ sk, const float* __restrict__ rad,
    const float* __restrict__ tau, int Hq, int Hkv, int G, int nb, int block, int S, int nseg,
    float scale, uint8_t* __restrict__ live, int32_t* __restrict__ st_cnt) {
  constexpr int LPR = D / 4;               // lanes per sketch row in the load (4 floats each)
  constexpr int RPS = 256 / LPR;           // rows per workgroup load step
  constexpr int NSTEP = kPruneRows / RPS;
  __shared__ float cT[D][kPruneRows + 1];  // sketch rows, transposed (row index fastest)
  __shared__ float rT[16][kPruneRows];     // radii, transposed
  __shared__ __attribute__((aligned(16))) float sq[8][D];   // the group's queries
  __shared__ float part[8 * D / 8];        // squares of 8-column pieces
  __shared__ float qn[8][16];              // ||q_h,s||
  __shared__ float qnorm[8], th[8];
  __shared__ int segf[kPruneRows];
  const int nchunk = (nb + kPruneRows - 1) / kPruneRows;
  const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const int b = bh / Hkv, kh = bh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* Qg = Q + (size_t(b) * Hq + kh * G) * D;
  const int j0 = chunk * kPruneRows;

  // the query loads (4 columns per thread) and tau first, then the sketch
  // rows (coalesced, 16 bytes per lane) and the radii, all in flight together
  const bool qt = tid < G * D / 4;
  float q4[4];
  if constexpr (sizeof(T) == 2) {
    const u32x2 w = qt ? ld8(Qg + 4 * tid) : u32x2{0u, 0u};
    q4[0] = bf16lo(w[0]); q4[1] = bf16hi(w[0]); q4[2] = bf16lo(w[1]); q4[3] = bf16hi(w[1]);
  } else {
    const u32x4 w = qt ? ld16(Qg + 4 * tid) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) q4[e] = __uint_as_float(w[e]);
  }
  const float tv = tid < G ? tau[size_t(b) * Hq + kh * G + tid] : 0.f;
  const int lr = tid / LPR, lc = tid % LPR;
  u32x4 cr[NSTEP];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    const int j = min(j0 + st * RPS + lr, nb - 1);
    cr[st] = ld16(sk + (size_t(bh) * nb + j) * D + lc * 4);
  }
  float rv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {            // S * 64 <= 1024 radii, 4 per thread
    const int o = tid + 256 * u, r = o / S, sub = o % S;
    rv[u] = o < S * kPruneRows ? rad[(size_t(bh) * nb + min(j0 + r, nb - 1)) * S + sub] : 0.f;
  }
  if (qt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sq[(4 * tid) / D][(4 * tid) % D + e] = q4[e];
  }
  if (tid < G) th[tid] = tv;
  if (tid < kPruneRows) segf[tid] = 0;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
#pragma unroll
    for (int e = 0; e < 4; ++e) cT[lc * 4 + e][st * RPS + lr] = __uint_as_float(cr[st][e]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int o = tid + 256 * u;
    if (o < S * kPruneRows) rT[o % S][o / S] = rv[u];
  }
  __syncthreads();
  if (tid < G * D / 8) {
    const int h = tid / (D / 8), c0 = (tid % (D / 8)) * 8;
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a += sq[h][c0 + e] * sq[h][c0 + e];
    part[tid] = a;
  }
  __syncthreads();
  const int W8 = D / S / 8;                // 8-column pieces per subspace
  if (tid < G * S) {
    const int h = tid / S, sub = tid % S;
    float a = 0.f;
    for (int i = 0; i < W8; ++i) a += part[h * (D / 8) + sub * W8 + i];
    qn[h][sub] = sqrtf(a);
  }
  if (tid < G) {
    float a = 0.f;
    for (int i = 0; i < D / 8; ++i) a += part[tid * (D / 8) + i];
    qnorm[tid] = sqrtf(a);
  }
  __syncthreads();

  // one (block row, head) per thread: row = lane, head = wave (+ 4 per pass)
  const int bps = kThrSeg / block;         // blocks per staging segment
  const int r = lane, j = j0 + r;
  float cc = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) cc += cT[c][r] * cT[c][r];
  const float cn = sqrtf(cc);
  bool alive = false;
  for (int h = wave; h < G; h += 4) {
    float dot = 0.f;
#pragma unroll 8
    for (int c = 0; c < D; ++c) dot += sq[h][c] * cT[c][r];
    float R = 0.f;
    for (int sub = 0; sub < S; ++sub) R += qn[h][sub] * rT[sub][r];
    const float ub = scale * (dot + R);
    const float hi = ub + scale * kBoundRel * (qnorm[h] * cn + R) +
                     kCmpRel * (fabsf(ub) + fabsf(th[h]));
    alive |= !(hi < th[h]);                // a NaN bound stays alive
  }
  if (alive && j < nb) atomicOr(&segf[r / bps], 1 << (r % bps));
  __syncthreads();
  const int s0 = j0 / bps, ns = min(kPruneRows / bps, nseg - s0);
  for (int i = tid; i < ns; i += 256) {
    const int seg = s0 + i;
    const int on = segf[i];
    live[size_t(bh) * nseg + seg] = uint8_t(on);
    if (!on) {
      for (int h = 0; h < G; ++h) st_cnt[(size_t(b) * Hq + kh * G + h) * nseg + seg] = 0;
    }
  }
}

hipError_t launch_radius(const void* X, int dtype, int B, int H, int N, int D, int block, int S,
                         int b0, int b1, const float* sketch, float* radius, hipStream_t st) {
  const int nb = cdiv(N, block), nbr = b1 - b0;
  if (nbr <= 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(long(B) * H * nbr));
  if (dtype == SA_BF16) {
    auto x = static_cast<const uint16_t*>(X);
    if (D == 128) k_radius<uint16_t, 128><<<g, 256, 0, st>>>(x, H, N, block, nb, b0, nbr, S, sketch, radius);
    else          k_radius<uint16_t, 64><<<g, 256, 0, st>>>(x, H, N, block, nb, b0, nbr, S, sketch, radius);
  } else {
    auto x = static_cast<const float*>(X);
    if (D == 128) k_radius<float, 128><<<g, 256, 0, st>>>(x, H, N, block, nb, b0, nbr, S, sketch, radius);
    else          k_radius<float, 64><<<g, 256, 0, st>>>(x, H, N, block, nb, b0, nbr, S, sketch, radius);
  }
  return hipGetLastError();
}

hipError_t launch_prune(const void* Q, int dtype, int B, int Hq, int Hkv, int N, int D, int block,
                        int S, const float* sketch, const float* radius, const float* tau,
                        float scale, int nseg, uint8_t* live, int32_t* st_cnt, hipStream_t st) {
  const int nb = cdiv(N, block);
  const int G = Hq / Hkv;
  const dim3 g(static_cast<unsigned>(long(B) * Hkv * cdiv(nb, kPruneRows)));
  if (dtype == SA_BF16) {
    auto q = static_cast<const uint16_t*>(Q);
    if (D == 128) k_prune<uint16_t, 128><<<g, 256, 0, st>>>(q, sketch, radius, tau, Hq, Hkv, G, nb, block, S, nseg, scale, live, st_cnt);
    else          k_prune<uint16_t, 64><<<g, 256, 0, st>>>(q, sketch, radius, tau, Hq, Hkv, G, nb, block, S, nseg, scale, live, st_cnt);
  } else {
    auto q = static_cast<const float*>(Q);
    if (D == 128) k_prune<float, 128><<<g, 256, 0, st>>>(q, sketch, radius, tau, Hq, Hkv, G, nb, block, S, nseg, scale, live, st_cnt);
    else          k_prune<float, 64><<<g, 256, 0, st>>>(q, sketch, radius, tau, Hq, Hkv, G, nb, block, S, nseg, scale, live, st_cnt);
  }
  return hipGetLastError();
}

}  // namespace sa
