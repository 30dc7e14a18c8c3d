// sa_device.h -- device helpers shared by the gfx950 kernels of this library.
//
// Wave64 only.  Values stored as bf16 travel as raw 16-bit patterns packed two
// per 32-bit word (the even element in the low half).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ bf16 <-> f32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16 with IEEE round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// ------------------------------------------------------------ math
// 2^x on the hardware exponential unit; 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ loads
template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
template <typename T>
__device__ __forceinline__ u32x2 ld8(const T* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// ------------------------------------------------------------ matrix cores
// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies row l%16 of
// A and column l%16 of B, 8 contraction elements each (the same contraction
// slots in both operands); D row 4*(l/16)+r, column l%16 lands in element r.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// Same with a 16-element contraction (4 elements per lane).
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Byte permute: result byte i = byte sel_i of the 8-byte value (hi:lo).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low halves of two words -> one word (a.lo | b.lo << 16); high halves likewise.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

// ------------------------------------------------------------ buffer loads
// A raw buffer resource over [base, base + bytes) (bytes <= 0x7f000000).  Loads
// at byte offsets past `bytes` return zeros instead of touching memory, so a
// tile that is invalid or runs past the end needs no branch: it gets the offset
// kBufOOB.  Each load takes one 32-bit offset register; constant parts of the
// offset go into the instruction's immediate field.
constexpr int kBufOOB = 0x7fff0000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 bld8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bld4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// Plain buffer stores: they land in this XCD's L2, where sc1 loads from the
// same XCD see them (but not loads from another XCD).
__device__ __forceinline__ void bst16(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void bst8(__amdgpu_buffer_rsrc_t r, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
// Agent-coherent accesses (cache policy sc1, the policy the compiler gives
// agent-scope atomic loads and stores): a completed sc1 store is visible to
// sc1 loads from every compute unit of the device, whatever its L2 holds.
// Loads take a wave-uniform part of the offset in a scalar register (soff),
// so a run of loads shares one offset VGPR.
constexpr int kCoherent = 16;
__device__ __forceinline__ u32x4 bld16c(__amdgpu_buffer_rsrc_t r, int off, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kCoherent));
}
__device__ __forceinline__ u32x2 bld8c(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent));
}
__device__ __forceinline__ void bst16c(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCoherent);
}
__device__ __forceinline__ void bst8c(__amdgpu_buffer_rsrc_t r, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCoherent);
}

// ------------------------------------------------------------ wave scans (DPP)
// A 64-lane inclusive scan in six register-to-register steps, no LDS: row
// shifts by 1, 2, 4 and 8 scan each 16-lane row, then row broadcasts add lane
// 15 of rows 0 and 2 into rows 1 and 3, and lane 31 into rows 2 and 3 (GFX9
// DPP row_shr / row_bcast controls).  A lane whose source falls outside its row
// or whose row is masked off reads `id`, the identity of the operation.  The
// whole wave must be converged.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t id, uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(id), int(v), CTRL, ROWMASK, 0xf, false));
}
template <typename Op>
__device__ __forceinline__ uint32_t dpp_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_u32<0x111>(id, v));
  v = op(v, dpp_u32<0x112>(id, v));
  v = op(v, dpp_u32<0x114>(id, v));
  v = op(v, dpp_u32<0x118>(id, v));
  v = op(v, dpp_u32<0x142, 0xa>(id, v));
  v = op(v, dpp_u32<0x143, 0xc>(id, v));
  return v;
}
__device__ __forceinline__ uint32_t lane63(uint32_t v) {
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
// Sum over aligned groups of L consecutive lanes (L = 16 or 32) by DPP; the
// group's total lands in its last lane (the other lanes hold partial sums).
template <int L>
__device__ __forceinline__ float group_sum_to_last(float v) {
  static_assert(L == 16 || L == 32, "groups of 16 or 32 lanes");
  auto add = [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  };
  uint32_t x = __float_as_uint(v);
  x = add(x, dpp_u32<0x111>(0u, x));
  x = add(x, dpp_u32<0x112>(0u, x));
  x = add(x, dpp_u32<0x114>(0u, x));
  x = add(x, dpp_u32<0x118>(0u, x));
  if constexpr (L == 32) x = add(x, dpp_u32<0x142, 0xa>(0u, x));
  return __uint_as_float(x);
}
// Integer sum over each group of 8 adjacent lanes, landing in the group's
// last lane (the other lanes hold partial sums).
__device__ __forceinline__ int group_isum8_to_last(int v) {
  uint32_t x = uint32_t(v);
  x += dpp_u32<0x111>(0u, x);
  x += dpp_u32<0x112>(0u, x);
  x += dpp_u32<0x114>(0u, x);
  return int(x);
}
// Inclusive prefix sum over the 64 lanes (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  return int(dpp_scan(uint32_t(v), 0u, [](uint32_t a, uint32_t b) { return a + b; }));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  return lane63(dpp_scan(v, ~0u, [](uint32_t a, uint32_t b) { return a < b ? a : b; }));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  return lane63(dpp_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; }));
}
__device__ __forceinline__ float wave_max(float v) {
  const uint32_t r = dpp_scan(__float_as_uint(v), __float_as_uint(-__builtin_inff()),
                              [](uint32_t a, uint32_t b) {
                                return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                              });
  return __uint_as_float(lane63(r));
}
__device__ __forceinline__ float wave_sum(float v) {
  const uint32_t r = dpp_scan(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float(lane63(r));
}

// Exclusive prefix sum over a whole workgroup of NT threads (thread order).
// `tmp` must hold NT/64 ints of LDS.  Returns the exclusive prefix and the
// total through *total.  Contains barriers: every thread must call it.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = tmp[i];
    base += i < w ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();   // tmp may be rewritten right after the call
  return base + incl - v;
}

// Order-preserving 32-bit key of a float score: larger score -> larger key.
// -0 ranks as +0; NaN ranks as -inf.  max(f, -inf) maps NaN to -inf (IEEE
// maxNum returns the non-NaN operand), adding +0 turns -0 into +0, and the
// sign-driven xor flips negative patterns and sets the top bit of positive
// ones: five plain VALU operations.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(fmaxf(f, -__builtin_inff()) + 0.0f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}

}  // namespace sa
