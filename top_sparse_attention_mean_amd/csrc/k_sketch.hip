// k_sketch.hip -- per-block mean sketch of keys (or pooled query blocks).
//
// The sketch is the compact key summary that is scanned before any full key
// is fetched ("Faster Than Flash", Metodologia §1), realised as the per-block
// centre of the keys (the range-search index's cluster centres, "Sparse
// Attention as a Range Searching Problem", Metodologia §2).  Pooling over the
// heads of a KV group as well gives the pooled query block that ranks key
// blocks in block-sparse prefill ("The Sparse Frontier", Contributi §2).
//
// HBM-bound streaming reduction: one 256-thread workgroup per output row
// (b, pooled head, block); every thread reads 16-byte vectors of one input row
// (coalesced across the row), accumulates 8 columns in float32, then the
// row groups are summed in a fixed order through LDS (deterministic).
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_sketch(const T* __restrict__ X, int H, int N,
                                                int block, int hp, int b0, int nbr,
                                                int nb, float* __restrict__ out) {
  constexpr int CPT = 8;            // columns per thread
  constexpr int TPR = D / CPT;      // threads per row
  constexpr int RPP = 256 / TPR;    // rows per pass
  __shared__ float red[RPP][D + 4];

  int id = blockIdx.x;
  const int jj = id % nbr;
  id /= nbr;
  const int Hh = H / hp;
  const int hh = id % Hh;
  const int b = id / Hh;
  const int j = b0 + jj;
  const int t0 = j * block;
  const int nj = min(block, N - t0);
  const int rows = hp * nj;
  const int tr = threadIdx.x / TPR, tc = threadIdx.x % TPR;

  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;

  for (int r = tr; r < rows; r += RPP) {
    const int h = hh * hp + r / nj;
    const int t = t0 + r % nj;
    const T* p = X + ((size_t(b) * H + h) * N + t) * D + tc * CPT;
    if constexpr (sizeof(T) == 2) {
      u32x4 w = ld16(p);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] += bf16lo(w[c]);
        acc[2 * c + 1] += bf16hi(w[c]);
      }
    } else {
      u32x4 w0 = ld16(p), w1 = ld16(p + 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[c] += __uint_as_float(w0[c]);
        acc[4 + c] += __uint_as_float(w1[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) red[tr][tc * CPT + c] = acc[c];
  __syncthreads();
  const float n = float(rows);
  for (int col = threadIdx.x; col < D; col += 256) {
    float s = 0.f;
    for (int g = 0; g < RPP; ++g) s += red[g][col];
    out[((size_t(b) * Hh + hh) * nb + j) * D + col] = s / n;
  }
}

hipError_t launch_sketch(const void* X, int dtype, int B, int H, int N, int D,
                         int block, int hp, int b0, int b1, float* out, hipStream_t st) {
  const int nb = cdiv(N, block);
  const int nbr = b1 - b0;
  if (nbr <= 0) return hipSuccess;
  const long grid = long(B) * (H / hp) * nbr;
  dim3 g(static_cast<unsigned>(grid)), t(256);
  if (dtype == SA_BF16) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    if (D == 128) k_sketch<uint16_t, 128><<<g, t, 0, st>>>(x, H, N, block, hp, b0, nbr, nb, out);
    else          k_sketch<uint16_t, 64><<<g, t, 0, st>>>(x, H, N, block, hp, b0, nbr, nb, out);
  } else {
    const float* x = static_cast<const float*>(X);
    if (D == 128) k_sketch<float, 128><<<g, t, 0, st>>>(x, H, N, block, hp, b0, nbr, nb, out);
    else          k_sketch<float, 64><<<g, t, 0, st>>>(x, H, N, block, hp, b0, nbr, nb, out);
  }
  return hipGetLastError();
}

}  // namespace sa
