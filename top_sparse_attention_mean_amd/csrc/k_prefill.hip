// k_prefill.hip -- block-sparse causal prefill attention on bf16 matrix cores.
//
// Query block i attends to the tokens of its listed key blocks (block 0, the
// diagonal block and the selected earlier blocks), causally masked: the
// block-by-block selection of Block-Sparse prefill ("The Sparse Frontier",
// Contributi §2) with one support shared by the block's queries and the
// group's heads ("How Much Dense Attention is Necessary?", technical summary
// §2.1, block-shared support), computed exactly on that support with the
// original Q, K, V.  This is the dense contraction of the path, so it runs on
// v_mfma_f32_32x32x16_bf16 with float32 accumulation.
//
// Workgroup = 4 waves = one (b, head, 128-row query block); each wave owns 32
// query rows.  Per listed key block the workgroup stages K (row-major, rows
// padded to 272 B) and V^T (transposed in registers with v_perm_b32, rows
// padded to 264 B) in LDS.  Scores are computed transposed, S^T = K Q^T
// (M = keys, N = query rows, contraction over d, both operands in natural
// row-major layout), so every lane holds the scores of ONE query row: the
// online softmax and the rescale of the O^T = V^T P^T accumulators are
// lane-local apart from one exchange with the lane 32 apart.  The score tile's
// output layout is the B-operand layout of the value product, so P goes from
// registers straight into the matrix cores (as bf16; query block 0, whose rows
// see at most 128 keys, splits P into two bf16 parts hi + lo instead, about 16
// significant bits, and so does every block when the caller asks for it).
// Workgroup ids are ordered so that all heads of one (kv head, query block)
// land on the same XCD (id % 8) and are dispatched together: their shared K/V
// tiles are fetched into that XCD's L2 once.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
struct f32x2_pair {
  float a, b;
};

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int PF_BLK = 128;         // query and key block
constexpr int PF_D = 128;
constexpr int PF_KS = PF_D + 8;     // K tile row stride (elements)
constexpr int PF_VS = PF_BLK + 4;   // V^T tile row stride (elements)
constexpr int PF_KT = 2;            // 32-key tiles per exponent + value-product step (4: spills)

// The two lanes of a query row (l and l ^ 32) combine their values with
// v_permlane32_swap: swapping lanes 32..63 of the first operand with lanes
// 0..31 of the second, both holding x, leaves every lane with x of itself and
// of its partner, in a register and without an LDS round trip.
__device__ __forceinline__ f32x2_pair pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_pair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

template <bool SPLITP, int NKT>
__device__ __forceinline__ void pv_tiles(const uint16_t* __restrict__ vt, const f32x16* sfr,
                                         int kt0, f32x16* acc, int lane) {
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int kk = 0; kk < NKT; ++kk) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 pb, pl;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = sfr[kk][8 * half + 2 * w], p1 = sfr[kk][8 * half + 2 * w + 1];
        const uint32_t hw = pack_bf16x2(p0, p1);
        pb[w] = hw;
        if constexpr (SPLITP) pl[w] = pack_bf16x2(p0 - bf16lo(hw), p1 - bf16hi(hw));
      }
      const int key = (kt0 + kk) * 32 + 16 * half + 4 * h;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* row = vt + (dt * 32 + col) * PF_VS + key;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(row);
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(row + 8);
        const u32x4 av = u32x4{a0[0], a0[1], a1[0], a1[1]};
        acc[dt] = mfma32x32x16(av, pb, acc[dt]);
        if constexpr (SPLITP) acc[dt] = mfma32x32x16(av, pl, acc[dt]);
      }
    }
  }
}

// MODE 0: every query block but the first, P in bf16 (the sparse prefill's
//         bulk); MODE 2: only the first query block of each (b, kv head), P as
//         bf16 hi + lo (its rows see at most 128 keys); MODE 1: every block
//         with P as hi + lo.  Keeping the hi + lo path out of MODE 0 keeps that
//         kernel within its registers (one inlined copy of the value product).
template <int MODE>
__global__ __launch_bounds__(256, 2) void k_prefill_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int Hq, int Hkv, int L, int M, int units, float sl2,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int kmax,
    void* __restrict__ O, int out_bf16, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[PF_BLK * PF_KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[PF_D * PF_VS];

  const int G = Hq / Hkv;
  const int id = blockIdx.x;
  const int grp = id / (8 * G), rem = id % (8 * G);
  const int hh = rem / 8;
  int u = grp * 8 + rem % 8;
  if (u >= units) return;  // uniform, before any barrier
  if constexpr (MODE == 2) u *= M;
  const int i = u % M, bkh = u / M;
  if constexpr (MODE == 0) {
    if (i == 0) return;
  }
  const int b = bkh / Hkv, kh = bkh % Hkv;
  const int h = kh * G + hh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qrow = i * PF_BLK + wave * 32 + col;     // this lane's query position

  // Q^T operand: query row qrow, d = 16*st + 8*half .. +7
  u32x4 qf[PF_D / 16];
  {
    const int qr = min(qrow, L - 1);
    const uint16_t* qp = Q + ((size_t(b) * Hq + h) * L + qr) * PF_D + 8 * half;
#pragma unroll
    for (int st = 0; st < PF_D / 16; ++st) qf[st] = ld16(qp + 16 * st);
  }

  const size_t kvbase = (size_t(b) * Hkv + kh) * size_t(L) * PF_D;
  const int32_t* lst = idx + (size_t(bkh) * M + i) * kmax;
  const int cnt = min(max(count[size_t(bkh) * M + i], 0), kmax);

  float m = -__builtin_inff(), l = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  const int ldc = tid & 15, ldr = tid >> 4;   // K loaders: 16-byte chunk, row group
  // V^T loaders: key group vk (4 rows) and column group vc (8 columns); they
  // write 8 V^T rows x 4 keys.  The 16 lanes of one LDS write phase differ in
  // vk, so their 8-byte stores fall 2 dwords apart in distinct banks (with the
  // column group varying inside a phase, rows 8 apart at a stride of 66
  // dwords met in two bank pairs: an 8-way conflict).
  const int vk = tid & 15, vc = tid >> 4;

  for (int e = 0; e < cnt; ++e) {
    const int jb = lst[e];
    if (jb < 0 || jb > i) continue;          // uniform
    const int key0 = jb * PF_BLK;
    // ---- stage K (row-major) and V^T; all 16 loads of a thread are in flight
    //      at once.  The block's rows go through resources based at its first
    //      row (scalar work), so each load's lane offset is the same for every
    //      block; rows past L lie beyond the resource's range and read as 0.
    const size_t boff = kvbase + size_t(key0) * PF_D;
    const uint32_t bbytes = uint32_t(L - key0) * PF_D * 2;
    const __amdgpu_buffer_rsrc_t rKb = make_rsrc(K + boff, bbytes);
    const __amdgpu_buffer_rsrc_t rVb = make_rsrc(V + boff, bbytes);
#pragma unroll
    for (int p0 = 0; p0 < 8; p0 += 4) {
      u32x4 w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        w[p] = bld16(rKb, ((ldr + 16 * (p0 + p)) * PF_D + 8 * ldc) * 2);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<u32x4*>(&kt_lds[(ldr + 16 * (p0 + p)) * PF_KS + 8 * ldc]) = w[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int k0 = 4 * vk + 64 * p;
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = bld16(rVb, ((k0 + j) * PF_D + 8 * vc) * 2);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2 ev = u32x2{pack_lo(w[0][c], w[1][c]), pack_lo(w[2][c], w[3][c])};
        const u32x2 od = u32x2{pack_hi(w[0][c], w[1][c]), pack_hi(w[2][c], w[3][c])};
        *reinterpret_cast<u32x2*>(&vt_lds[(8 * vc + 2 * c) * PF_VS + k0]) = ev;
        *reinterpret_cast<u32x2*>(&vt_lds[(8 * vc + 2 * c + 1) * PF_VS + k0]) = od;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for the block, online softmax, O^T += V^T P^T in steps of
    //      32 PF_KT keys
    const bool diag = jb == i;
    const bool tail = key0 + PF_BLK > L;
    // all scores of the block first: the masking, the row maximum and the
    // rescale then run once per block, and the second half's exponents run on
    // the vector ALUs while the matrix cores do the first half's value product
    f32x16 sall[4 / PF_KT][PF_KT];
#pragma unroll
    for (int sb = 0; sb < 4 / PF_KT; ++sb)
#pragma unroll
      for (int kk = 0; kk < PF_KT; ++kk) {
        const uint16_t* kr = kt_lds + ((PF_KT * sb + kk) * 32 + col) * PF_KS + 8 * half;
        sall[sb][kk] = mfma32x32x16(*reinterpret_cast<const u32x4*>(kr), qf[0], f32x16{});
#pragma unroll
        for (int st = 1; st < PF_D / 16; ++st) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(kr + 16 * st);
          sall[sb][kk] = mfma32x32x16(a, qf[st], sall[sb][kk]);
        }
      }
    // one maximum, rescale and exponent base for the whole block
    float mraw = -__builtin_inff();
    if (diag || tail) {  // uniform: mask keys past this row or past L
      // key offset (PF_KT sb + kk) 32 + 8 (r/4) + (r%4) is kept when <= lim
      const int lim = min(qrow, L - 1) - key0 - 4 * half;
#pragma unroll
      for (int sb = 0; sb < 4 / PF_KT; ++sb)
#pragma unroll
        for (int kk = 0; kk < PF_KT; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = (PF_KT * sb + kk) * 32 + 8 * (r >> 2) + (r & 3);
            sall[sb][kk][r] = ko <= lim ? sall[sb][kk][r] : -__builtin_inff();
            mraw = fmaxf(mraw, sall[sb][kk][r]);
          }
    } else {
#pragma unroll
      for (int sb = 0; sb < 4 / PF_KT; ++sb)
#pragma unroll
        for (int kk = 0; kk < PF_KT; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, sall[sb][kk][r]);
    }
    {
      const f32x2_pair pr = pair32(mraw);
      mraw = fmaxf(pr.a, pr.b);
    }
    const float m_new = fmaxf(m, mraw * sl2);
    // with no key seen yet (m_new = -inf) every p and alpha below is 0
    const float m_use = m_new != -__builtin_inff() ? m_new : 0.f;
    const float alpha = exp2_fast(m - m_use);
    l *= alpha;
    m = m_new;
    // the accumulators change only where a row's maximum moved
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
#pragma unroll
    for (int sb = 0; sb < 4 / PF_KT; ++sb) {
      f32x16* sfr = sall[sb];
      float ls = 0.f;
#pragma unroll
      for (int kk = 0; kk < PF_KT; ++kk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(__builtin_fmaf(sfr[kk][r], sl2, -m_use));
          sfr[kk][r] = p;
          ls += p;
        }
      }
      l += ls;
      pv_tiles<MODE != 0, PF_KT>(vt_lds, sfr, PF_KT * sb, acc, lane);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[d = 32 dt + 8 (r/4) + 4 half + r%4][qrow]
  const f32x2_pair lp = pair32(l);
  const float lt = lp.a + lp.b;
  if (qrow < L) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t ob = ((size_t(b) * Hq + h) * L + qrow) * PF_D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + 8 * a + 4 * half;
        float o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = acc[dt][4 * a + c] * inv;
        if (out_bf16) {
          const u32x2 pk = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(O) + ob + d) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(O) + ob + d) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    if (lse && half == 0)
      lse[(size_t(b) * Hq + h) * L + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -__builtin_inff();
  }
}

hipError_t launch_prefill(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                          int L, int D, float scale, int block, const int32_t* idx,
                          const int32_t* count, int kmax, void* O, int out_dtype, float* lse,
                          hipStream_t st, bool split_p) {
  (void)D;
  (void)block;
  const int M = cdiv(L, PF_BLK);
  const int G = Hq / Hkv;
  const int units = B * Hkv * M, firsts = B * Hkv;
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  const float sl2 = scale * kLog2e;
  const int ob = out_dtype == SA_BF16;
  if (split_p) {
    const long grid = long(cdiv(units, 8)) * 8 * G;
    k_prefill_bf16<1><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, st>>>(
        q, k, v, Hq, Hkv, L, M, units, sl2, idx, count, kmax, O, ob, lse);
    return hipGetLastError();
  }
  const long grid = long(cdiv(units, 8)) * 8 * G;
  k_prefill_bf16<0><<<dim3(static_cast<unsigned>(grid)), dim3(256), 0, st>>>(
      q, k, v, Hq, Hkv, L, M, units, sl2, idx, count, kmax, O, ob, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long grid0 = long(cdiv(firsts, 8)) * 8 * G;
  k_prefill_bf16<2><<<dim3(static_cast<unsigned>(grid0)), dim3(256), 0, st>>>(
      q, k, v, Hq, Hkv, L, M, firsts, sl2, idx, count, kmax, O, ob, lse);
  return hipGetLastError();
}

}  // namespace sa
