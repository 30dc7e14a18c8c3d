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
// Workgroup = one (b, kv head, query block) and one or two heads of the
// group (two at D 128 with 128-row blocks); each wave owns 32 query rows of
// one head.  Per listed key block the workgroup stages K (streamed from HBM
// into LDS by buffer loads with the LDS flag, no registers involved) and V^T
// (transposed in registers with v_perm_b32, rows padded to 264 B) in LDS; the
// next block's loads are in flight while the current block's value products
// run, and both heads read the same staged block.  Scores are computed
// transposed, S^T = K Q^T (M = keys, N = query rows, contraction over d, both
// operands in natural row-major layout), so every lane holds the scores of
// ONE query row: the
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
struct f32x2_pair {
  float a, b;
};

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int PF_KT = 2;            // 32-key tiles per exponent + value-product step (4: spills)
// Two heads of a group per workgroup (D 128, blocks of 128): they share each
// staged K / V^T block.
constexpr bool kPrefillHeadPairs = true;

// Tile geometry of one (D, BLK) instance: BLK query rows per workgroup, one
// wave per 32 rows.
//
// K goes from HBM to LDS without registers (buffer loads with the LDS flag):
// one wave instruction moves 1 KiB of consecutive K rows, a "group" of RG
// rows, to consecutive LDS bytes, and groups sit GB = 1 KiB + 16 B apart.  A
// row inside a group is then 2 D bytes from the next, which would put the
// rows that 16 lanes read together in one bank; so the score tile's row
// positions are permuted: position p holds key perm(p) = RG (p mod NG) +
// p / NG (NG groups per block), and the 16 lanes of a read phase, reading
// positions p..p+15, meet 16 different groups whose 16-byte pad staggers them
// across the banks.  V^T columns follow the same permutation (position p holds
// key perm(p)), which leaves every product unchanged: a block's keys are only
// relabelled.  V^T rows are padded to BLK + 4.
template <int D, int BLK, int HPW>
struct PfGeom {
  static constexpr int NT = 2 * BLK * HPW;    // threads: HPW heads x BLK / 32 waves
  static constexpr int ROWB = 2 * D;          // bytes per K row
  static constexpr int RG = 1024 / ROWB;      // K rows per group
  static constexpr int NG = BLK / RG;         // groups per block
  static constexpr int GB = 1024 + 16;        // LDS bytes per group
  static constexpr int GPW = NG / (NT / 64);  // groups loaded per wave
  static constexpr int VS = BLK + 4;          // V^T tile row stride (elements)
  static constexpr int CG = D / 8;            // V^T column groups (8 columns each)
  static constexpr int KG = NT / CG;          // V^T key groups (4 positions each) per pass
  static constexpr int VP = BLK / (4 * KG);   // V^T staging passes
  static constexpr int NKT = BLK / 32;        // 32-key score tiles per block
  static constexpr int perm(int p) { return RG * (p % NG) + p / NG; }
  static_assert(GPW >= 1 && NG * RG == BLK && 32 % NG == 0 && VP >= 1 && NKT % PF_KT == 0,
                "tile geometry");
};

// The two lanes of a query row (l and l ^ 32) combine their values with
// v_permlane32_swap: swapping lanes 32..63 of the first operand with lanes
// 0..31 of the second, both holding x, leaves every lane with x of itself and
// of its partner, in a register and without an LDS round trip.
__device__ __forceinline__ f32x2_pair pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_pair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

template <bool SPLITP, int NKT, int D, int VS>
__device__ __forceinline__ void pv_tiles(const uint16_t* __restrict__ vt, const f32x16* sfr,
                                         int kt0, f32x16* acc, int lane) {
  const int h = lane >> 5, col = lane & 31;
  // V^T operand of (key step ks = 2 kk + half, d tile dt); the next step's
  // operands are read while this step's products run
  auto read = [&](int ks, int dt) {
    const uint16_t* row = vt + (dt * 32 + col) * VS + (kt0 * 32 + 16 * ks + 4 * h);
    const u32x2 a0 = *reinterpret_cast<const u32x2*>(row);
    const u32x2 a1 = *reinterpret_cast<const u32x2*>(row + 8);
    return u32x4{a0[0], a0[1], a1[0], a1[1]};
  };
  u32x4 av[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) av[dt] = read(0, dt);
#pragma unroll
  for (int ks = 0; ks < 2 * NKT; ++ks) {
    const int kk = ks / 2, half = ks % 2;
    u32x4 pb, pl;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = sfr[kk][8 * half + 2 * w], p1 = sfr[kk][8 * half + 2 * w + 1];
      const uint32_t hw = pack_bf16x2(p0, p1);
      pb[w] = hw;
      if constexpr (SPLITP) pl[w] = pack_bf16x2(p0 - bf16lo(hw), p1 - bf16hi(hw));
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      acc[dt] = mfma32x32x16(av[dt], pb, acc[dt]);
      if constexpr (SPLITP) acc[dt] = mfma32x32x16(av[dt], pl, acc[dt]);
      if (ks + 1 < 2 * NKT) av[dt] = read(ks + 1, dt);
      __builtin_amdgcn_sched_barrier(0);     // keep the read ahead where it is
    }
  }
}

// MODE 0: every query block but the first, P in bf16 (the sparse prefill's
//         bulk); MODE 2: only the first query block of each (b, kv head), P as
//         bf16 hi + lo (its rows see at most BLK keys); MODE 1: every block
//         with P as hi + lo.  Keeping the hi + lo path out of MODE 0 keeps that
//         kernel within its registers (one inlined copy of the value product).
// MODE 3 and 4 serve the attention-mass selector and stage no V: MODE 3
//         writes each row's softmax statistics over its listed blocks, stats
//         [b, h, row] = (m, l) (m the row maximum in log2 units, l the sum of
//         2^(s log2e scale - m)); MODE 4 takes them and writes, for each
//         listed block j in [c0, c0 + 128), the row's probability mass on
//         block j, sum over its keys of 2^(s log2e scale - m) / l, to
//         O [b, h, row, j - c0] (float32; other columns untouched).
template <int MODE, int D, int BLK, int HPW>
__global__ __launch_bounds__(2 * BLK * HPW, 2 / HPW) void k_prefill_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, int Hq, int Hkv, int L, int M, int units, float sl2,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int kmax,
    void* __restrict__ O, int out_bf16, float* __restrict__ lse, float* __restrict__ stats,
    int c0) {
  using Gm = PfGeom<D, BLK, HPW>;
  __shared__ __attribute__((aligned(16))) unsigned char kt_lds[Gm::NG * Gm::GB];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * Gm::VS];

  const int G = Hq / Hkv, GH = G / HPW;         // head slots of a group
  const int id = blockIdx.x;
  const int grp = id / (8 * GH), rem = id % (8 * GH);
  const int hs = rem / 8;
  int u = grp * 8 + rem % 8;
  if (u >= units) return;  // uniform, before any barrier
  if constexpr (MODE == 2) u *= M;
  const int i = u % M, bkh = u / M;
  if constexpr (MODE == 0) {
    if (i == 0) return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  constexpr int WPH = BLK / 32;                      // waves per head
  const int b = bkh / Hkv, kh = bkh % Hkv;
  const int h = kh * G + hs * HPW + wave / WPH;      // this wave's head
  const int qrow = i * BLK + (wave % WPH) * 32 + col;  // this lane's query position

  // Q^T operand: query row qrow, d = 16*st + 8*half .. +7
  u32x4 qf[D / 16];
  {
    const int qr = min(qrow, L - 1);
    const uint16_t* qp = Q + ((size_t(b) * Hq + h) * L + qr) * D + 8 * half;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) qf[st] = ld16(qp + 16 * st);
  }

  const size_t kvbase = (size_t(b) * Hkv + kh) * size_t(L) * D;
  const int32_t* lst = idx + (size_t(bkh) * M + i) * kmax;
  const int cnt = min(max(count[size_t(bkh) * M + i], 0), kmax);

  float m = -__builtin_inff(), l = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  // V^T loaders: key-position group vk (4 positions) and column group vc (8
  // columns); they write 8 V^T rows x 4 positions.  With 16 or more position
  // groups the 16 lanes of one LDS write phase differ in vk, so their 8-byte
  // stores fall 2 dwords apart in distinct banks (with the column group
  // varying inside a phase, rows 8 apart at a stride of 66 dwords met in two
  // bank pairs: an 8-way conflict).  Positions k0..k0+3 hold keys perm(k0) +
  // RG j, one group apart.
  const int vk = tid % Gm::KG, vc = tid / Gm::KG;
  const int vrow = Gm::RG * ((4 * vk) % Gm::NG) + (4 * vk) / Gm::NG;  // perm(4 vk)
  const int wid = __builtin_amdgcn_readfirstlane(wave);

  // A key block's rows go through resources based at its first row (scalar
  // work), so each load's lane offset is the same for every block; rows past
  // L lie beyond the resource's range (their scores are masked; V reads them
  // as 0).
  auto load_k = [&](int jb) {
    const int key0 = jb * BLK;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(K + kvbase + size_t(key0) * D, uint32_t(L - key0) * D * 2);
#pragma unroll
    for (int n = 0; n < Gm::GPW; ++n) {
      const int g = wid * Gm::GPW + n;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(kt_lds + g * Gm::GB), 16,
          g * 1024 + 16 * lane, 0, 0, 0);
    }
  };
  auto load_v = [&](int jb, u32x4 (&w)[Gm::VP][4]) {
    const int key0 = jb * BLK;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(V + kvbase + size_t(key0) * D, uint32_t(L - key0) * D * 2);
#pragma unroll
    for (int p = 0; p < Gm::VP; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // position 4 vk + 4 KG p + j holds key vrow + (4 KG p / NG) + RG j
        const int key = vrow + (4 * Gm::KG * p) / Gm::NG + Gm::RG * j;
        w[p][j] = bld16(r, (key * D + 8 * vc) * 2);
      }
  };
  auto store_v = [&](const u32x4 (&w)[Gm::VP][4]) {
#pragma unroll
    for (int p = 0; p < Gm::VP; ++p) {
      const int k0 = 4 * vk + 4 * Gm::KG * p;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2 ev = u32x2{pack_lo(w[p][0][c], w[p][1][c]), pack_lo(w[p][2][c], w[p][3][c])};
        const u32x2 od = u32x2{pack_hi(w[p][0][c], w[p][1][c]), pack_hi(w[p][2][c], w[p][3][c])};
        *reinterpret_cast<u32x2*>(&vt_lds[(8 * vc + 2 * c) * Gm::VS + k0]) = ev;
        *reinterpret_cast<u32x2*>(&vt_lds[(8 * vc + 2 * c + 1) * Gm::VS + k0]) = od;
      }
    }
  };
  // listed blocks outside 0..i (in MODE 4 also outside [c0, c0 + 128)) are
  // skipped (uniform)
  auto next_listed = [&](int e) {
    while (e < cnt) {
      const int jb = lst[e];
      if (jb >= 0 && jb <= i && (MODE != 4 || (jb >= c0 && jb < c0 + 128))) break;
      ++e;
    }
    return e;
  };
  // this lane's K read address for score tile 0: position col, bytes 16 half
  // of each 32-byte step; tile t reads position 32 t + col, 32 t / NG rows on
  const unsigned char* kbase =
      kt_lds + (col % Gm::NG) * Gm::GB + (col / Gm::NG) * Gm::ROWB + 16 * half;

  // Software pipeline over the listed blocks, two barriers per block: after
  // the first (every wave done reading K) the next block's K streams into LDS
  // and its V into registers while this block's value products run; after the
  // second (every wave done reading V^T, every load of the next block landed)
  // V^T is written, ordered before its reads by the next block's first
  // barrier.
  int e = next_listed(0);
  if (e < cnt) {
    load_k(lst[e]);
    if constexpr (MODE < 3) {
      u32x4 wv[Gm::VP][4];
      load_v(lst[e], wv);
      store_v(wv);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // MODE 4: the row's statistics from MODE 3
  float m_fin = 0.f, inv_l = 0.f;
  if constexpr (MODE == 4) {
    const int qr = min(qrow, L - 1);
    const f32x2 st2 = *reinterpret_cast<const f32x2*>(stats + 2 * ((size_t(b) * Hq + h) * L + qr));
    m_fin = st2[0];
    inv_l = st2[1] > 0.f ? 1.f / st2[1] : 0.f;
  }

  while (e < cnt) {
    const int jb = lst[e];
    const int en = next_listed(e + 1);
    const bool more = en < cnt;              // uniform
    const int key0 = jb * BLK;

    // ---- S^T = K Q^T for the block, online softmax, O^T += V^T P^T in steps of
    //      32 PF_KT keys
    const bool diag = jb == i;
    const bool tail = key0 + BLK > L;
    // all scores of the block first: the masking, the row maximum and the
    // rescale then run once per block, and the later steps' exponents run on
    // the vector ALUs while the matrix cores do the earlier value products
    constexpr int NSB = Gm::NKT / PF_KT;
    f32x16 sall[NSB][PF_KT];
    {
      // the next tile's K operands are read while this tile's products run
      // (one LDS latency per block rather than per product pair)
      u32x4 ka[D / 16];
#pragma unroll
      for (int st = 0; st < D / 16; ++st) ka[st] = *reinterpret_cast<const u32x4*>(kbase + 32 * st);
#pragma unroll
      for (int t = 0; t < Gm::NKT; ++t) {
        const unsigned char* kn = kbase + (32 * (t + 1) / Gm::NG) * Gm::ROWB;
        f32x16& sc = sall[t / PF_KT][t % PF_KT];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          sc = mfma32x32x16(ka[st], qf[st], st ? sc : f32x16{});
          if (t + 1 < Gm::NKT) ka[st] = *reinterpret_cast<const u32x4*>(kn + 32 * st);
          __builtin_amdgcn_sched_barrier(0);   // keep the read ahead where it is
        }
      }
    }
    __syncthreads();                         // every wave is done reading K
    u32x4 wv[Gm::VP][4];
    if (more) {
      load_k(lst[en]);
      if constexpr (MODE < 3) load_v(lst[en], wv);
    }
    // one maximum, rescale and exponent base for the whole block
    float mraw = -__builtin_inff();
    if (diag || tail) {  // uniform: mask keys past this row or past L
      // position (PF_KT sb + kk) 32 + 8 (r/4) + 4 half + (r%4) holds key
      // perm(that with half = 0) + 4 RG half, kept when <= the row's limit
      const int lim = min(qrow, L - 1) - key0 - 4 * Gm::RG * half;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int kk = 0; kk < PF_KT; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = Gm::perm((PF_KT * sb + kk) * 32 + 8 * (r >> 2) + (r & 3));
            sall[sb][kk][r] = ko <= lim ? sall[sb][kk][r] : -__builtin_inff();
            mraw = fmaxf(mraw, sall[sb][kk][r]);
          }
    } else {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int kk = 0; kk < PF_KT; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, sall[sb][kk][r]);
    }
    if constexpr (MODE == 4) {
      // the block's probability mass for this row, with the row's final
      // maximum and sum (masked keys give 2^-inf = 0)
      float ps = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int kk = 0; kk < PF_KT; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r) ps += exp2_fast(__builtin_fmaf(sall[sb][kk][r], sl2, -m_fin));
      const f32x2_pair pp = pair32(ps);
      if (qrow < L && half == 0)
        static_cast<float*>(O)[((size_t(b) * Hq + h) * L + qrow) * 128 + (jb - c0)] =
            (pp.a + pp.b) * inv_l;
      __builtin_amdgcn_s_waitcnt(0);         // this wave's loads of the next block
      __syncthreads();
      e = en;
      continue;
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
    if (MODE < 3 && __ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
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
      if constexpr (MODE < 3)
        pv_tiles<MODE != 0, PF_KT, D, Gm::VS>(vt_lds, sfr, PF_KT * sb, acc, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);           // this wave's loads of the next block
    __syncthreads();                         // every wave is done reading V^T
    if constexpr (MODE < 3) {
      if (more) store_v(wv);
    }
    e = en;
  }
  if constexpr (MODE == 4) return;
  if constexpr (MODE == 3) {
    const f32x2_pair lp = pair32(l);
    if (qrow < L && half == 0)
      *reinterpret_cast<f32x2*>(stats + 2 * ((size_t(b) * Hq + h) * L + qrow)) =
          f32x2{m, lp.a + lp.b};
    return;
  }

  // ---- epilogue: lane holds O^T[d = 32 dt + 8 (r/4) + 4 half + r%4][qrow]
  const f32x2_pair lp = pair32(l);
  const float lt = lp.a + lp.b;
  if (qrow < L) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const size_t ob = ((size_t(b) * Hq + h) * L + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
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

template <int D, int BLK, int HPW>
static hipError_t launch_prefill_db(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    int B, int Hq, int Hkv, int L, float sl2, const int32_t* idx,
                                    const int32_t* count, int kmax, void* O, int ob, float* lse,
                                    hipStream_t st, bool split_p) {
  const int M = cdiv(L, BLK);
  const int GH = Hq / Hkv / HPW;
  const int units = B * Hkv * M, firsts = B * Hkv;
  const dim3 blk(2 * BLK * HPW);
  if (split_p) {
    const long grid = long(cdiv(units, 8)) * 8 * GH;
    k_prefill_bf16<1, D, BLK, HPW><<<dim3(static_cast<unsigned>(grid)), blk, 0, st>>>(
        q, k, v, Hq, Hkv, L, M, units, sl2, idx, count, kmax, O, ob, lse, nullptr, 0);
    return hipGetLastError();
  }
  const long grid = long(cdiv(units, 8)) * 8 * GH;
  k_prefill_bf16<0, D, BLK, HPW><<<dim3(static_cast<unsigned>(grid)), blk, 0, st>>>(
      q, k, v, Hq, Hkv, L, M, units, sl2, idx, count, kmax, O, ob, lse, nullptr, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long grid0 = long(cdiv(firsts, 8)) * 8 * GH;
  k_prefill_bf16<2, D, BLK, HPW><<<dim3(static_cast<unsigned>(grid0)), blk, 0, st>>>(
      q, k, v, Hq, Hkv, L, M, firsts, sl2, idx, count, kmax, O, ob, lse, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_prefill(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                          int L, int D, float scale, int block, const int32_t* idx,
                          const int32_t* count, int kmax, void* O, int out_dtype, float* lse,
                          hipStream_t st, bool split_p) {
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  auto v = static_cast<const uint16_t*>(V);
  const float sl2 = scale * kLog2e;
  const int ob = out_dtype == SA_BF16;
  const bool pair = kPrefillHeadPairs && (Hq / Hkv) % 2 == 0;
  if (D == 128 && block == 128)
    return pair ? launch_prefill_db<128, 128, 2>(q, k, v, B, Hq, Hkv, L, sl2, idx, count, kmax, O,
                                                 ob, lse, st, split_p)
                : launch_prefill_db<128, 128, 1>(q, k, v, B, Hq, Hkv, L, sl2, idx, count, kmax, O,
                                                 ob, lse, st, split_p);
  if (D == 128)
    return launch_prefill_db<128, 64, 1>(q, k, v, B, Hq, Hkv, L, sl2, idx, count, kmax, O, ob, lse,
                                         st, split_p);
  if (block == 128)
    return launch_prefill_db<64, 128, 1>(q, k, v, B, Hq, Hkv, L, sl2, idx, count, kmax, O, ob, lse,
                                         st, split_p);
  return launch_prefill_db<64, 64, 1>(q, k, v, B, Hq, Hkv, L, sl2, idx, count, kmax, O, ob, lse,
                                      st, split_p);
}

template <int MODE, int HPW>
static hipError_t launch_mass_mode(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv,
                                   int L, float sl2, const int32_t* idx, const int32_t* count,
                                   int kmax, float* O, float* stats, int c0, hipStream_t st) {
  const int M = cdiv(L, 128);
  const int GH = Hq / Hkv / HPW;
  const int units = B * Hkv * M;
  const long grid = long(cdiv(units, 8)) * 8 * GH;
  k_prefill_bf16<MODE, 128, 128, HPW><<<dim3(static_cast<unsigned>(grid)), dim3(256 * HPW), 0,
                                        st>>>(q, k, nullptr, Hq, Hkv, L, M, units, sl2, idx, count,
                                              kmax, O, 0, nullptr, stats, c0);
  return hipGetLastError();
}

hipError_t launch_prefill_mass(const void* Q, const void* K, int B, int Hq, int Hkv, int L,
                               float scale, const int32_t* idx, const int32_t* count, int kmax,
                               float* O, float* stats, int c0, bool stats_pass, hipStream_t st) {
  auto q = static_cast<const uint16_t*>(Q);
  auto k = static_cast<const uint16_t*>(K);
  const float sl2 = scale * kLog2e;
  // one head per workgroup: with no value product a wave takes 144-152
  // VGPRs, so three 4-wave workgroups share a compute unit (38.9 ms per call
  // at L = 64K against 45.2 ms for two heads in one 8-wave workgroup)
  if (stats_pass)
    return launch_mass_mode<3, 1>(q, k, B, Hq, Hkv, L, sl2, idx, count, kmax, O, stats, c0, st);
  return launch_mass_mode<4, 1>(q, k, B, Hq, Hkv, L, sl2, idx, count, kmax, O, stats, c0, st);
}

}  // namespace sa
