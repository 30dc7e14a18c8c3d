// k_mass.hip -- the attention-mass top-k selector on the GPU.
//
// "How Much Dense Attention is Necessary?" (technical summary §2.1) ranks the
// blocks of a query block by their exact attention mass: dense causal softmax
// for every row, the probability summed over each key block, averaged over
// the block's rows and the heads of the KV group; the top-k of the earlier
// blocks [1, i-1] form the support.  The pages call it a reference (it needs
// the dense attention it is meant to avoid); here it makes the recall of the
// sketch selector measurable over every query block.
//
// The dense passes reuse the block-sparse prefill kernel's staging and score
// tiles with every earlier block listed and no value product: one pass
// writes each row's softmax statistics (its maximum m and sum l over all of
// its keys); then, per chunk of 128 key blocks, a second pass recomputes the
// scores of the chunk's blocks and writes each row's mass on each of them,
// the sum over the block's keys of 2^(s log2e scale - m) / l, in float32.
// Both passes compute each score the same way, so a row's masses over all
// blocks sum to 1 up to float32 rounding.
//
//   k_dense_list   idx [B, Hkv, M, M] = 0..i for query block i (dense causal)
//   k_mass_reduce  one workgroup per (b, kv head, query block): the chunk's
//                  columns summed over the block's rows and the group's heads
//   k_mass_select  one workgroup per (b, kv head, query block): the k largest
//                  masses of blocks 1..i-1 (ties to the lower block), ascending
//   k_row_mass     per-query supports (b_sel = 1): each row's own masses,
//                  averaged over the group's heads, then k_mass_select per row
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

__global__ __launch_bounds__(256) void k_dense_list(int M, long rows, int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ count) {
  const long o = long(blockIdx.x) * 256 + threadIdx.x;   // (b, kv head, i, slot)
  if (o >= rows * M) return;
  const long r = o / M;
  const int s = int(o % M), i = int(r % M);
  idx[o] = s <= i ? s : -1;
  if (s == 0) count[r] = i + 1;
}

// mass[b, kh, i, 128 c + col] = mean over rows of block i and heads of the
// group of O[b, h, row, col].
__global__ __launch_bounds__(256) void k_mass_reduce(const float* __restrict__ O, int Hq, int Hkv,
                                                     int L, int block, int M, int c,
                                                     float* __restrict__ mass) {
  __shared__ float part[2][128];
  const int i = blockIdx.x % M, bh = blockIdx.x / M;
  const int b = bh / Hkv, kh = bh % Hkv, G = Hq / Hkv;
  const int col = threadIdx.x & 127, half = threadIdx.x >> 7;
  const int r0 = i * block, nr = min(block, L - r0);
  float acc = 0.f;
  for (int h = kh * G; h < (kh + 1) * G; ++h) {
    const float* Ob = O + ((size_t(b) * Hq + h) * L + r0) * 128 + col;
    for (int r = half; r < nr; r += 2) acc += Ob[size_t(r) * 128];
  }
  part[half][col] = acc;
  __syncthreads();
  const int j = 128 * c + col;
  if (half == 0 && j < M)
    mass[(size_t(bh) * M + i) * M + j] = j <= i ? (part[0][col] + part[1][col]) / float(nr * G) : 0.f;
}

// The k largest masses among blocks 1..i-1, ties to the lower block index,
// listed ascending.  Masses are >= 0, so their float bits order them; the key
// (bits << 32 | ~j) makes the lower j win a tie.
// Per query block (rows of [B, Hkv, M] mass rows, i = r % M) or per query
// row (rows of [B, Hkv, L], i = (r % L) / block when L > 0).
__global__ __launch_bounds__(256) void k_mass_select(const float* __restrict__ mass, int M,
                                                     int k, int L, int block,
                                                     int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ count) {
  __shared__ uint64_t wbest[4];
  __shared__ int chosen[64];
  const int r = blockIdx.x, i = L > 0 ? (r % L) / block : r % M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* mrow = mass + size_t(r) * M;
  const int n = min(k, max(i - 1, 0));
  for (int round = 0; round < n; ++round) {
    uint64_t best = 0;
    for (int j = 1 + tid; j < i; j += 256) {
      bool taken = false;
      for (int q = 0; q < round; ++q) taken |= chosen[q] == j;
      if (!taken) {
        const uint64_t key = (uint64_t(__float_as_uint(mrow[j])) << 32) | uint32_t(~uint32_t(j));
        best = key > best ? key : best;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t other = (uint64_t(uint32_t(__shfl_xor(int(best >> 32), o))) << 32) |
                             uint32_t(__shfl_xor(int(uint32_t(best)), o));
      best = other > best ? other : best;
    }
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t bb = wbest[0];
      for (int w = 1; w < 4; ++w) bb = wbest[w] > bb ? wbest[w] : bb;
      chosen[round] = int(~uint32_t(bb));
    }
    __syncthreads();
  }
  if (tid == 0) {
    for (int a = 1; a < n; ++a) {                 // insertion sort, ascending
      const int v = chosen[a];
      int b2 = a - 1;
      while (b2 >= 0 && chosen[b2] > v) { chosen[b2 + 1] = chosen[b2]; --b2; }
      chosen[b2 + 1] = v;
    }
    count[r] = n;
  }
  __syncthreads();
  for (int q = tid; q < k; q += 256) idx[size_t(r) * k + q] = q < n ? chosen[q] : -1;
}

// row_mass[b, kh, t, 128 c + col] = mean over the group's heads of O[b, h, t, col]
// (0 for blocks after the row's own).
__global__ __launch_bounds__(256) void k_row_mass(const float* __restrict__ O, int Hq, int Hkv,
                                                  int L, int block, int M, int c, long rows,
                                                  float* __restrict__ row_mass) {
  const long o = long(blockIdx.x) * 256 + threadIdx.x;   // (b, kv head, t, col)
  const long bt = o >> 7;                                // row of [B, Hkv, L]
  if (bt >= rows) return;
  const int col = int(o & 127);
  const int t = int(bt % L);
  const int bh = int(bt / L), b = bh / Hkv, kh = bh % Hkv, G = Hq / Hkv;
  const int j = 128 * c + col;
  if (j >= M) return;
  float acc = 0.f;
  for (int h = kh * G; h < (kh + 1) * G; ++h) acc += O[((size_t(b) * Hq + h) * L + t) * 128 + col];
  row_mass[(size_t(bh) * L + t) * M + j] = j <= t / block ? acc / float(G) : 0.f;
}

hipError_t launch_mass_select(const void* Q, const void* K, int B, int Hq, int Hkv, int L, int D,
                              float scale, int block, int kfree, float* mass, int32_t* idx,
                              int32_t* count, float* row_mass, int32_t* row_idx,
                              int32_t* row_count, const MassWs& w, void* ws, hipStream_t st) {
  char* base = static_cast<char*>(ws);
  float* stats = reinterpret_cast<float*>(base + w.stats_off);
  float* O = reinterpret_cast<float*>(base + w.o_off);
  int32_t* lst = reinterpret_cast<int32_t*>(base + w.list_off);
  int32_t* lcnt = reinterpret_cast<int32_t*>(base + w.lcnt_off);
  float* ms = mass ? mass : reinterpret_cast<float*>(base + w.mass_off);
  const int M = cdiv(L, block);
  const long lrows = long(B) * Hkv * M;
  k_dense_list<<<dim3(unsigned(cdiv(lrows * M, 256))), 256, 0, st>>>(M, lrows, lst, lcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long vrows = long(B) * Hkv * L;
  e = launch_prefill_mass(Q, K, B, Hq, Hkv, L, scale, lst, lcnt, M, O, stats, 0, true, st);
  if (e != hipSuccess) return e;
  for (int c = 0; c * 128 < M; ++c) {
    e = launch_prefill_mass(Q, K, B, Hq, Hkv, L, scale, lst, lcnt, M, O, stats, 128 * c, false,
                            st);
    if (e != hipSuccess) return e;
    k_mass_reduce<<<dim3(unsigned(lrows)), 256, 0, st>>>(O, Hq, Hkv, L, block, M, c, ms);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (row_mass) {
      k_row_mass<<<dim3(unsigned(cdiv(vrows * 128, 256))), 256, 0, st>>>(O, Hq, Hkv, L, block, M,
                                                                         c, vrows, row_mass);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  k_mass_select<<<dim3(unsigned(lrows)), 256, 0, st>>>(ms, M, kfree, 0, block, idx, count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (row_mass) {
    k_mass_select<<<dim3(unsigned(vrows)), 256, 0, st>>>(row_mass, M, kfree, L, block, row_idx,
                                                          row_count);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sa
