// sa_api.hip -- the extern "C" entry points declared in include/sa.h.
//
// Every argument check runs on the host before anything is enqueued and
// before any HIP runtime call, so invalid calls fail the same way with or
// without a GPU.  Launches are asynchronous on the caller's stream.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "sa_internal.h"

using namespace sa;

namespace {

thread_local char g_err[512] = "";

sa_status fail(sa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

sa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return SA_OK;
  return fail(SA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int dt) { return dt == SA_F32 || dt == SA_BF16; }
float eff_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / sqrtf(float(D)); }
bool pow2_le8(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Knob SA_STEP_MODE of sa_decode_step: 0 (default) the two-kernel step
// (scoring kernel, then the selecting split-K decode); 1 the one-launch step
// (k_step.hip) with plain stores inside an XCD team, 2 the same with
// device-coherent stores throughout, 3 the same with every workgroup acting as
// if it ran off its team's XCD.  The one-launch step is slower at the long
// decode shape (its cross-workgroup selection costs more than the kernel
// boundary it removes), so it is kept for measurement and tests only.
int step_mode() {
  const char* e = getenv("SA_STEP_MODE");
  if (!e) return 0;
  const int m = atoi(e);
  return m >= 0 && m <= 3 ? m : 0;
}

#define REQ(cond, ...)                                   \
  do {                                                   \
    if (!(cond)) return fail(SA_ERR_INVALID, __VA_ARGS__); \
  } while (0)
#define SUP(cond, ...)                                       \
  do {                                                       \
    if (!(cond)) return fail(SA_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)
#define PTR(p) REQ((p) != nullptr && al16(p), #p " must be a non-null 16-byte aligned device pointer")

sa_status check_heads(int B, int Hq, int Hkv) {
  REQ(B >= 1 && Hq >= 1 && Hkv >= 1, "B, Hq, Hkv must be >= 1 (got %d, %d, %d)", B, Hq, Hkv);
  REQ(Hq % Hkv == 0, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  return SA_OK;
}

// --------------------------------------------------------------- validation
sa_status v_sketch(const void* X, int dtype, int B, int H, int N, int D, int block, int hp,
                   int b0, int b1, const float* sk) {
  PTR(X);
  PTR(sk);
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  REQ(B >= 1 && H >= 1 && N >= 1, "B, H, N must be >= 1");
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(block >= 1, "block must be >= 1");
  REQ(hp >= 1 && H % hp == 0, "head_pool (%d) must divide H (%d)", hp, H);
  const int nb = cdiv(N, block);
  REQ(0 <= b0 && b0 <= b1 && b1 <= nb, "block range [%d, %d) outside [0, %d]", b0, b1, nb);
  REQ(long(B) * (H / hp) * (b1 - b0) < (1L << 31), "too many output rows");
  return SA_OK;
}

sa_status v_select(const void* Q, int dtype, int B, int Hq, int Hkv, int Lq, int D, int q_block,
                   const float* ksk, int nb, int k, unsigned flags, int32_t* idx,
                   int32_t* count, float* score, void* ws, size_t ws_bytes) {
  PTR(Q);
  PTR(ksk);
  PTR(idx);
  PTR(count);
  if (score) PTR(score);
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(nb >= 1 && k >= 1, "nb and k must be >= 1 (got %d, %d)", nb, k);
  REQ((flags & ~7u) == 0, "unknown flag bits 0x%x", flags);
  const int nF = int((flags & SA_FORCE_SINK) != 0) + int((flags & SA_FORCE_LOCAL) != 0);
  if (flags & SA_CAUSAL) {
    REQ(Lq >= 1 && q_block >= 1, "Lq and q_block must be >= 1");
    const int M = cdiv(Lq, q_block);
    REQ(nb >= M, "the key sketch has %d blocks but the queries need %d", nb, M);
    SUP(M <= kMaxNbPrefill, "at most %d query blocks per selection row", kMaxNbPrefill);
    REQ(k >= nF, "k (%d) smaller than the %d forced blocks", k, nF);
    REQ(long(B) * Hkv * M < (1L << 31), "too many selection rows");
  } else {
    REQ(Lq == 1 && q_block == 1, "decode selection takes one query position (Lq = q_block = 1)");
    SUP(nb <= kMaxNbDecode, "at most %d blocks per decode selection row", kMaxNbDecode);
    REQ(nb == 1 || k >= nF, "k (%d) smaller than the %d forced blocks", k, nF);
  }
  const size_t need = select_ws_bytes(B, Hkv, (flags & SA_CAUSAL) ? Lq : 1, D, q_block, nb);
  if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  PTR(ws);
  const long grid = long(B) * Hkv * select_plan(B * Hkv, nb).C + long(B) * Hkv;
  REQ(grid < (1L << 31), "too many scoring workgroups");
  return SA_OK;
}

sa_status v_decode(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                   int Hkv, int N, int D, int mode, int block, const int32_t* idx,
                   const int32_t* count, int idx_stride, const float* score, const void* O,
                   int out_dtype, const float* lse, const void* ws, size_t ws_bytes) {
  PTR(Q);
  PTR(K);
  PTR(V);
  PTR(idx);
  PTR(O);
  if (count) PTR(count);
  if (score) PTR(score);
  if (lse) PTR(lse);
  REQ(dtype_ok(dtype) && dtype_ok(out_dtype), "unknown dtype");
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(N >= 1 && idx_stride >= 1, "N and idx_stride must be >= 1");
  const int G = Hq / Hkv;
  if (mode == SA_IDX_BLOCKS) {
    REQ(block >= 1, "block must be >= 1");
    if (dtype == SA_BF16) {
      SUP(block == 64 || block == 128, "bf16 block-mode decode needs block 64 or 128");
      SUP(pow2_le8(G), "bf16 block-mode decode needs g in {1, 2, 4, 8} (got %d)", G);
      SUP(long(N) * D * 2 <= 0x7f000000L, "bf16 block-mode decode reads one kv head through a "
          "buffer resource of at most 0x7f000000 bytes (N * D * 2 = %ld)", long(N) * D * 2);
    } else {
      SUP(G <= 8, "float32 decode needs g <= 8 (got %d)", G);
    }
  } else if (mode == SA_IDX_TOKENS) {
    REQ(count != nullptr, "token mode needs count");
  } else {
    return fail(SA_ERR_INVALID, "unknown mode %d", mode);
  }
  const DecodeWs w = decode_ws(B, Hq, Hkv, D, mode, block, idx_stride);
  const int Sg = mode == SA_IDX_BLOCKS ? std::max({w.S, decode_sel_splits(B * Hkv, idx_stride, block),
                                                   decode_valu_splits(idx_stride, block)})
                                       : w.S;
  REQ(long(B) * (mode == SA_IDX_BLOCKS ? Hkv : Hq) * Sg < (1L << 31), "grid too large");
  if (ws_bytes < w.bytes) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, ws_bytes);
  PTR(ws);
  return SA_OK;
}

}  // namespace

// Checks of the low-bit selection's arguments (nothing enqueued).
static sa_status v_lowbit(const void* Q, const uint8_t* codes, const int8_t* resid,
                          const float* meta, int B, int Hq, int Hkv, int N, int D, int block,
                          int sink, int local, float delta, float margin, int kcap,
                          int32_t* idx, int32_t* count, float* tau, float* bmax, void* khat,
                          void* ws, size_t ws_bytes) {
  PTR(Q);
  PTR(codes);
  PTR(resid);
  PTR(meta);
  PTR(idx);
  PTR(count);
  PTR(khat);
  if (tau) PTR(tau);
  if (bmax) PTR(bmax);
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  SUP(block == 64 || block == 128, "block must be 64 or 128 (got %d)", block);
  SUP(pow2_le8(Hq / Hkv), "the low-bit filter needs g in {1, 2, 4, 8}");
  REQ(N >= 1 && kcap >= 1, "N and kcap must be >= 1");
  REQ(sink >= 0 && local >= 0, "sink and local must be >= 0 (got %d, %d)", sink, local);
  REQ(sink > 0 || local > 0, "the sink and local windows are both empty");
  REQ(delta >= 0.f, "delta must be >= 0 (got %g)", double(delta));
  REQ(margin >= 0.f, "margin must be >= 0 (got %g)", double(margin));
  const int nb = cdiv(N, block);
  REQ(long(B) * Hkv * cdiv(nb, 4) < (1L << 31), "grid too large");
  const size_t need = lowbit_ws_bytes(B, Hq, Hkv, N, block);
  if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  PTR(ws);
  return SA_OK;
}

// The low-bit selection's launches: the window's refined keys into khat, the
// pseudo-maximum and tau, the thumbnail scan and the block list; then, when
// refine_kept, the refined keys of the kept blocks into khat.
static sa_status run_lowbit_select(const void* Q, const uint8_t* codes, const int8_t* resid,
                                   const float* meta, int B, int Hq, int Hkv, int N, int D,
                                   int block, int sink, int local, float delta, float margin,
                                   float scale, int kcap, int32_t* idx, int32_t* count,
                                   float* tau, float* bmax, void* khat, void* ws,
                                   bool refine_kept, hipStream_t st, const char* what) {
  const int nb = cdiv(N, block);
  const float sc = eff_scale(scale, D);
  char* base = static_cast<char*>(ws);
  uint8_t* flag = reinterpret_cast<uint8_t*>(base);
  float* t = tau ? tau : reinterpret_cast<float*>(base + align256(size_t(B) * Hkv * nb));
  uint16_t* kh = static_cast<uint16_t*>(khat);
  // the window's blocks: [0, f1) holds the sink tokens, [f2, nb) the local ones
  const int ns = sink < N ? sink : N;
  const int lt = N - (local < N ? local : N);
  const int tw = lt > ns ? lt : ns;
  const int f1 = cdiv(ns, block), f2 = tw < N ? tw / block : nb;
  hipError_t e = launch_decode_keys(codes, resid, meta, B, Hkv, N, D, block, nullptr, nullptr, 0,
                                    0, f1, kh, st);
  if (e == hipSuccess)
    e = launch_decode_keys(codes, resid, meta, B, Hkv, N, D, block, nullptr, nullptr, 0, f2, nb,
                           kh, st);
  if (e != hipSuccess) return hip_status(e, what);
  e = launch_pseudo_max(Q, kh, SA_BF16, B, Hq, Hkv, N, D, sink, local, delta, sc, t, st);
  if (e != hipSuccess) return hip_status(e, what);
  e = launch_thumb_scan(static_cast<const uint16_t*>(Q), codes, meta, B, Hq, Hkv, N, D, block, sc,
                        t, margin, 0, f1, f2, nb, bmax, flag, st);
  if (e != hipSuccess) return hip_status(e, what);
  e = launch_block_list(flag, B * Hkv, nb, kcap, idx, count, st);
  if (e != hipSuccess || !refine_kept) return hip_status(e, what);
  return hip_status(launch_decode_keys(codes, resid, meta, B, Hkv, N, D, block, idx, count, kcap,
                                       0, 0, kh, st),
                    what);
}

// Selection from a score row fused with the split-K decode where a fused
// kernel exists (bf16, D = 128, k <= kMaxKFused); otherwise the selection
// kernel followed by the block decode.
static sa_status run_select_decode(const void* Q, const void* K, const void* V, int dtype, int B,
                                   int Hq, int Hkv, int N, int D, int block, const float* scores,
                                   int nb, int k, unsigned flags, float sc, int32_t* idx,
                                   int32_t* count, void* O, int out_dtype, float* lse, void* dws,
                                   hipStream_t st, const char* what) {
  if (dtype == SA_BF16 && D == 128 && k <= kMaxKFused) {
    // same workspace size as the block decode; its own split count
    const DecodeWs w = decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k, true);
    return hip_status(launch_decode_select_blocks(Q, K, V, B, Hq, Hkv, N, D, sc, block, scores, nb,
                                                  k, flags, idx, count, w, dws, O, out_dtype, lse,
                                                  st),
                      what);
  }
  const DecodeWs w = decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k);
  if (dtype == SA_F32 && nb <= 256 * kValuSelKpt && k <= kValuSelMaxK)
    return hip_status(launch_decode_select_valu(Q, K, V, B, Hq, Hkv, N, D, sc, block, scores, nb,
                                                k, flags, idx, count, w, dws, O, out_dtype, lse,
                                                st),
                      what);
  const hipError_t e = launch_select_rows(scores, B * Hkv, nb, k, flags, idx, count, st);
  if (e != hipSuccess) return hip_status(e, what);
  return hip_status(launch_decode_blocks(Q, K, V, dtype, B, Hq, Hkv, N, D, sc, block, idx, count,
                                         k, w, dws, O, out_dtype, lse, st),
                    what);
}

namespace {

// Fills n 32-bit words with zero (a kernel, not a memset, so that the call can
// be captured into a HIP graph).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

}  // namespace

namespace sa {

sa_status report(sa_status s, const char* what) { return fail(s, "%s", what); }

sa_status decode_step(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                      int Hkv, int N, int D, int block, float* ksketch, int update_block, int k,
                      float scale, int32_t* idx, int32_t* count, float* score, void* O,
                      int out_dtype, float* lse, void* ws, size_t ws_bytes, hipStream_t st,
                      StepPhase phase) {
  PTR(ksketch);
  REQ(block >= 1, "block must be >= 1");
  const int nb = cdiv(N, block);
  REQ(update_block >= -1 && update_block < nb, "update_block %d outside [-1, %d)", update_block, nb);
  const size_t sel = select_ws_bytes(B, Hkv, 1, D, 1, nb);
  sa_status s = v_select(Q, dtype, B, Hq, Hkv, 1, D, 1, ksketch, nb, k,
                         SA_FORCE_SINK | SA_FORCE_LOCAL, idx, count, score, ws, ws_bytes);
  if (s) return s;
  if (ws_bytes < sel) return fail(SA_ERR_WORKSPACE, "workspace too small");
  void* dws = static_cast<char*>(ws) + sel;
  s = v_decode(Q, K, V, dtype, B, Hq, Hkv, N, D, SA_IDX_BLOCKS, block, idx, count, k, nullptr, O,
               out_dtype, lse, dws, ws_bytes - sel);
  if (s) return s;
  if (update_block >= 0) {
    s = v_sketch(K, dtype, B, Hkv, N, D, block, 1, update_block, update_block + 1, ksketch);
    if (s) return s;
  }
  const int mode = step_mode();
  const bool one = mode != 0 && step_fusable(dtype, B, Hq, Hkv, N, D, block, k);
  if (one) {
    const size_t need = step_ws(B, Hq, Hkv, D).bytes;
    if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  }
  if (phase == StepPhase::kCheck) return SA_OK;
  const float sc = eff_scale(scale, D);
  if (phase == StepPhase::kClearAndLaunch) {
    // the words that must read zero when a step starts: the one-launch step's
    // error word and counters, or the selecting decode's arrival counters
    const size_t off = one ? 0 : sel + decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k).cnt_off;
    const size_t bytes = one ? step_ws(B, Hq, Hkv, D).pub_off
                             : size_t(B) * Hq * kCounterStride * sizeof(uint32_t);
    const int n = int(bytes / sizeof(uint32_t));
    k_zero_words<<<dim3(std::min(cdiv(n, 256), 64)), 256, 0, st>>>(
        reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + off), n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "sa_decode_step (workspace clear)");
  }
  if (one)
    return hip_status(launch_decode_step(Q, K, V, B, Hq, Hkv, N, D, block, ksketch, update_block,
                                         k, SA_FORCE_SINK | SA_FORCE_LOCAL, sc, idx, count, score,
                                         O, out_dtype, lse, ws, mode - 1, st),
                      "sa_decode_step");
  const SelectWs sw = select_ws(B, Hkv, 1, D, 1, nb);
  float* scores = score ? score : reinterpret_cast<float*>(static_cast<char*>(ws) + sw.score_off);
  if (dtype == SA_F32 && nb <= 256 * kValuSelKpt && k <= kValuSelMaxK) {
    // float32 rows of up to 512 blocks: the whole step in the decode kernel
    const DecodeWs w = decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k);
    return hip_status(launch_decode_step_valu(Q, K, V, B, Hq, Hkv, N, D, sc, block, ksketch,
                                              update_block, scores, nb, k,
                                              SA_FORCE_SINK | SA_FORCE_LOCAL, idx, count, w, dws,
                                              O, out_dtype, lse, st),
                      "sa_decode_step (one-launch float32 step)");
  }
  hipError_t e = launch_score(Q, dtype, B, Hq, Hkv, D, ksketch, nb, K, N, block, update_block, sc,
                              scores, st);
  if (e != hipSuccess) return hip_status(e, "sa_decode_step (score)");
  return run_select_decode(Q, K, V, dtype, B, Hq, Hkv, N, D, block, scores, nb, k,
                           SA_FORCE_SINK | SA_FORCE_LOCAL, sc, idx, count, O, out_dtype, lse, dws,
                           st, "sa_decode_step (select + decode)");
}

}  // namespace sa

extern "C" {

int sa_version(void) { return 100; }

const char* sa_last_error(void) { return g_err; }

const char* sa_status_str(int s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SA_ERR_WORKSPACE: return "workspace too small";
    case SA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t sa_workspace_bytes(int op, int B, int Hq, int Hkv, int N, int D, int block, int k) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1) return SIZE_MAX;
  switch (op) {
    case SA_OP_SELECT_TOPK:          // N = Lq, block = q_block, k = nb
      if (k < 1 || block < 1) return SIZE_MAX;
      return select_ws_bytes(B, Hkv, N, D, block, k);
    case SA_OP_SELECT_THRESHOLD:
      return threshold_ws(B, Hq, N).bytes;
    case SA_OP_SELECT_TOPDELTA:
      return topdelta_ws_bytes(B, Hq, N);
    case SA_OP_SELECT_PRUNED:
      return pruned_ws_bytes(B, Hq, Hkv, N);
    case SA_OP_MASS_SELECT:          // N = L, block = the block size
      if (block < 1) return SIZE_MAX;
      return mass_ws(B, Hq, Hkv, N, block).bytes;
    case SA_OP_SELECT_LOWBIT:        // block = the block size
      if (block < 1) return SIZE_MAX;
      return lowbit_ws_bytes(B, Hq, Hkv, N, block);
    case SA_OP_DECODE_LOWBIT:        // block = the block size, k = kcap
      if (block < 1 || k < 1) return SIZE_MAX;
      return lowbit_ws_bytes(B, Hq, Hkv, N, block) +
             decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k).bytes;
    case SA_OP_SPARSE_DECODE:        // k = idx_stride; block = 0 for token mode
      if (k < 1) return SIZE_MAX;
      return decode_ws(B, Hq, Hkv, D, block > 0 ? SA_IDX_BLOCKS : SA_IDX_TOKENS, block, k).bytes;
    case SA_OP_DECODE_STEP: {
      // room for both paths (the one-launch step serves bf16 shapes only; the
      // dtype is not an argument here)
      if (k < 1 || block < 1) return SIZE_MAX;
      const int nb = cdiv(N, block);
      const size_t two = select_ws_bytes(B, Hkv, 1, D, 1, nb) +
                         decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, k).bytes;
      const size_t one = step_fusable(SA_BF16, B, Hq, Hkv, N, D, block, k)
                             ? step_ws(B, Hq, Hkv, D).bytes : 0;
      return std::max(two, one);
    }
    default:
      return SIZE_MAX;
  }
}

sa_status sa_build_sketch(const void* X, int dtype, int B, int H, int N, int D, int block,
                          int head_pool, int blk_begin, int blk_end, float* sketch,
                          void* stream) {
  sa_status s = v_sketch(X, dtype, B, H, N, D, block, head_pool, blk_begin, blk_end, sketch);
  if (s) return s;
  return hip_status(launch_sketch(X, dtype, B, H, N, D, block, head_pool, blk_begin, blk_end,
                                  sketch, static_cast<hipStream_t>(stream)),
                    "sa_build_sketch");
}

sa_status sa_select_topk(const void* Q, int dtype, int B, int Hq, int Hkv, int Lq, int D,
                         int q_block, const float* ksketch, int nb, int k, unsigned flags,
                         float scale, int32_t* idx, int32_t* count, float* score, void* ws,
                         size_t ws_bytes, void* stream) {
  sa_status s = v_select(Q, dtype, B, Hq, Hkv, Lq, D, q_block, ksketch, nb, k, flags, idx, count,
                         score, ws, ws_bytes);
  if (s) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = eff_scale(scale, D);
  if (flags & SA_CAUSAL) {
    const int M = cdiv(Lq, q_block);
    float* qbar = static_cast<float*>(ws);
    hipError_t e = launch_sketch(Q, dtype, B, Hq, Lq, D, q_block, Hq / Hkv, 0, M, qbar, st);
    if (e != hipSuccess) return hip_status(e, "sa_select_topk (pool)");
    return hip_status(launch_prefill_select(qbar, ksketch, B * Hkv, M, nb, D, k, flags, sc, idx,
                                            count, score, st),
                      "sa_select_topk (prefill)");
  }
  const SelectWs w = select_ws(B, Hkv, 1, D, 1, nb);
  float* scores = score ? score : reinterpret_cast<float*>(static_cast<char*>(ws) + w.score_off);
  hipError_t e = launch_score(Q, dtype, B, Hq, Hkv, D, const_cast<float*>(ksketch), nb, nullptr,
                              0, 1, -1, sc, scores, st);
  if (e != hipSuccess) return hip_status(e, "sa_select_topk (score)");
  return hip_status(launch_select_rows(scores, B * Hkv, nb, k, flags, idx, count, st),
                    "sa_select_topk (select)");
}

static sa_status v_threshold(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv,
                             int N, int D, int cap, int32_t* idx, float* score, int32_t* count) {
  PTR(Q);
  PTR(K);
  PTR(idx);
  PTR(score);
  PTR(count);
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(N >= 1 && cap >= 1, "N and cap must be >= 1");
  const int G = Hq / Hkv;
  if (dtype == SA_BF16) SUP(pow2_le8(G), "bf16 threshold selection needs g in {1, 2, 4, 8}");
  else SUP(G <= 8, "float32 threshold selection needs g <= 8");
  const ThrWs w = threshold_ws(B, Hq, N);
  REQ(long(B) * Hkv * w.nseg < (1L << 31), "grid too large");
  return SA_OK;
}

sa_status sa_select_threshold(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv,
                              int N, int D, const float* tau, float scale, int cap, int32_t* idx,
                              float* score, int32_t* count, void* ws, size_t ws_bytes,
                              void* stream) {
  sa_status s = v_threshold(Q, K, dtype, B, Hq, Hkv, N, D, cap, idx, score, count);
  if (s) return s;
  PTR(tau);
  const ThrWs w = threshold_ws(B, Hq, N);
  if (ws_bytes < w.bytes) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, ws_bytes);
  PTR(ws);
  return hip_status(launch_threshold(Q, K, dtype, B, Hq, Hkv, N, D, tau, eff_scale(scale, D), cap,
                                     idx, score, count, w, ws, static_cast<hipStream_t>(stream)),
                    "sa_select_threshold");
}

sa_status sa_select_topdelta(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv,
                             int N, int D, int sink, int local, float delta, float scale,
                             int cap, int32_t* idx, float* score, int32_t* count, float* tau,
                             void* ws, size_t ws_bytes, void* stream) {
  sa_status s = v_threshold(Q, K, dtype, B, Hq, Hkv, N, D, cap, idx, score, count);
  if (s) return s;
  REQ(sink >= 0 && local >= 0, "sink and local must be >= 0 (got %d, %d)", sink, local);
  REQ(sink > 0 || local > 0, "the sink and local windows are both empty");
  REQ(delta >= 0.f, "delta must be >= 0 (got %g)", double(delta));   // NaN fails too
  if (tau) PTR(tau);
  const ThrWs w = threshold_ws(B, Hq, N);
  const size_t need = topdelta_ws_bytes(B, Hq, N);
  if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  PTR(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = eff_scale(scale, D);
  float* t = tau ? tau : reinterpret_cast<float*>(static_cast<char*>(ws) + w.bytes);
  hipError_t e = launch_pseudo_max(Q, K, dtype, B, Hq, Hkv, N, D, sink, local, delta, sc, t, st);
  if (e != hipSuccess) return hip_status(e, "sa_select_topdelta (pseudo-max)");
  return hip_status(launch_threshold(Q, K, dtype, B, Hq, Hkv, N, D, t, sc, cap, idx, score, count,
                                     w, ws, st),
                    "sa_select_topdelta (scan)");
}

static bool subspaces_ok(int D, int S) {
  return S >= 1 && S <= 16 && D % S == 0 && (D / S) % 8 == 0;
}

sa_status sa_build_radius(const void* X, int dtype, int B, int H, int N, int D, int block, int S,
                          int blk_begin, int blk_end, const float* sketch, float* radius,
                          void* stream) {
  PTR(X);
  PTR(sketch);
  PTR(radius);
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  REQ(B >= 1 && H >= 1 && N >= 1, "B, H, N must be >= 1");
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(block >= 1, "block must be >= 1");
  SUP(subspaces_ok(D, S), "S (%d) must divide D (%d) into subspaces of a multiple of 8 "
      "channels, S <= 16", S, D);
  const int nb = cdiv(N, block);
  REQ(0 <= blk_begin && blk_begin <= blk_end && blk_end <= nb,
      "block range [%d, %d) outside [0, %d]", blk_begin, blk_end, nb);
  REQ(long(B) * H * (blk_end - blk_begin) < (1L << 31), "too many blocks");
  return hip_status(launch_radius(X, dtype, B, H, N, D, block, S, blk_begin, blk_end, sketch,
                                  radius, static_cast<hipStream_t>(stream)),
                    "sa_build_radius");
}

sa_status sa_select_threshold_pruned(const void* Q, const void* K, int dtype, int B, int Hq,
                                     int Hkv, int N, int D, int block, int S,
                                     const float* sketch, const float* radius, const float* tau,
                                     float scale, int cap, int32_t* idx, float* score,
                                     int32_t* count, uint8_t* live, void* ws, size_t ws_bytes,
                                     void* stream) {
  sa_status s = v_threshold(Q, K, dtype, B, Hq, Hkv, N, D, cap, idx, score, count);
  if (s) return s;
  PTR(tau);
  PTR(sketch);
  PTR(radius);
  if (live) PTR(live);
  SUP(block == 32 || block == 64 || block == 128, "block must be 32, 64 or 128 (got %d)", block);
  SUP(subspaces_ok(D, S), "S (%d) must divide D (%d) into subspaces of a multiple of 8 "
      "channels, S <= 16", S, D);
  const ThrWs w = threshold_ws(B, Hq, N);
  const size_t need = pruned_ws_bytes(B, Hq, Hkv, N);
  if (ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  PTR(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = eff_scale(scale, D);
  char* base = static_cast<char*>(ws);
  uint8_t* lv = live ? live : reinterpret_cast<uint8_t*>(base + w.bytes);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + w.cnt_off);
  hipError_t e = launch_prune(Q, dtype, B, Hq, Hkv, N, D, block, S, sketch, radius, tau, sc,
                              w.nseg, lv, cnt, st);
  if (e != hipSuccess) return hip_status(e, "sa_select_threshold_pruned (bounds)");
  return hip_status(launch_threshold(Q, K, dtype, B, Hq, Hkv, N, D, tau, sc, cap, idx, score,
                                     count, w, ws, st, lv, block),
                    "sa_select_threshold_pruned (scan)");
}

sa_status sa_encode_keys(const void* K, int dtype, int B, int H, int N, int D, int block,
                         int blk_begin, int blk_end, uint8_t* codes, int8_t* resid, float* meta,
                         void* stream) {
  PTR(K);
  PTR(codes);
  PTR(resid);
  PTR(meta);
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  REQ(B >= 1 && H >= 1 && N >= 1, "B, H, N must be >= 1");
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(block >= 1, "block must be >= 1");
  const int nb = cdiv(N, block);
  REQ(0 <= blk_begin && blk_begin <= blk_end && blk_end <= nb,
      "block range [%d, %d) outside [0, %d]", blk_begin, blk_end, nb);
  REQ(long(B) * H * (blk_end - blk_begin) < (1L << 31), "too many blocks");
  return hip_status(launch_encode(K, dtype, B, H, N, D, block, blk_begin, blk_end, codes, resid,
                                  meta, static_cast<hipStream_t>(stream)),
                    "sa_encode_keys");
}

sa_status sa_decode_keys(const uint8_t* codes, const int8_t* resid, const float* meta, int B,
                         int H, int N, int D, int block, const int32_t* idx,
                         const int32_t* count, int idx_stride, int blk_begin, int blk_end,
                         void* khat, void* stream) {
  PTR(codes);
  PTR(resid);
  PTR(meta);
  PTR(khat);
  REQ(B >= 1 && H >= 1 && N >= 1, "B, H, N must be >= 1");
  SUP(D == 64 || D == 128, "D must be 64 or 128 (got %d)", D);
  REQ(block >= 1, "block must be >= 1");
  const int nb = cdiv(N, block);
  if (idx) {
    PTR(idx);
    if (count) PTR(count);
    REQ(idx_stride >= 1, "idx_stride must be >= 1");
    REQ(long(B) * H * idx_stride < (1L << 31), "too many list entries");
  } else {
    REQ(0 <= blk_begin && blk_begin <= blk_end && blk_end <= nb,
        "block range [%d, %d) outside [0, %d]", blk_begin, blk_end, nb);
  }
  return hip_status(launch_decode_keys(codes, resid, meta, B, H, N, D, block, idx, count,
                                       idx_stride, blk_begin, blk_end,
                                       static_cast<uint16_t*>(khat),
                                       static_cast<hipStream_t>(stream)),
                    "sa_decode_keys");
}

sa_status sa_select_topdelta_lowbit(const void* Q, const uint8_t* codes, const int8_t* resid,
                                    const float* meta, int B, int Hq, int Hkv, int N, int D,
                                    int block, int sink, int local, float delta, float margin,
                                    float scale, int kcap, int32_t* idx, int32_t* count,
                                    float* tau, float* bmax, void* khat, void* ws,
                                    size_t ws_bytes, void* stream) {
  sa_status s = v_lowbit(Q, codes, resid, meta, B, Hq, Hkv, N, D, block, sink, local, delta,
                         margin, kcap, idx, count, tau, bmax, khat, ws, ws_bytes);
  if (s) return s;
  return run_lowbit_select(Q, codes, resid, meta, B, Hq, Hkv, N, D, block, sink, local, delta,
                           margin, scale, kcap, idx, count, tau, bmax, khat, ws, true,
                           static_cast<hipStream_t>(stream), "sa_select_topdelta_lowbit");
}

sa_status sa_decode_topdelta_lowbit(const void* Q, const uint8_t* codes, const int8_t* resid,
                                    const float* meta, const void* V, int B, int Hq, int Hkv,
                                    int N, int D, int block, int sink, int local, float delta,
                                    float margin, float scale, int kcap, int32_t* idx,
                                    int32_t* count, float* tau, float* bmax, void* khat, void* O,
                                    int out_dtype, float* lse, void* ws, size_t ws_bytes,
                                    void* stream) {
  PTR(V);
  PTR(O);
  if (lse) PTR(lse);
  REQ(dtype_ok(out_dtype), "unknown output dtype %d", out_dtype);
  const size_t lws = lowbit_ws_bytes(B, Hq, Hkv, N, block);
  sa_status s = v_lowbit(Q, codes, resid, meta, B, Hq, Hkv, N, D, block, sink, local, delta,
                         margin, kcap, idx, count, tau, bmax, khat, ws, ws_bytes);
  if (s) return s;
  SUP(kcap <= kMaxSplits * (kLowbitMetaBlocks - 1),
      "the thumbnail-key decode lists at most %d blocks (kcap = %d)",
      kMaxSplits * (kLowbitMetaBlocks - 1), kcap);
  SUP(long(N) * D * 2 <= 0x7f000000L, "the thumbnail-key decode reads one kv head through a "
      "buffer resource of at most 0x7f000000 bytes (N * D * 2 = %ld)", long(N) * D * 2);
  const DecodeWs dw = decode_ws(B, Hq, Hkv, D, SA_IDX_BLOCKS, block, kcap);
  if (ws_bytes < lws + dw.bytes)
    return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", lws + dw.bytes, ws_bytes);
  REQ(long(B) * Hkv * decode_lowbit_splits(kcap, block) < (1L << 31), "grid too large");
  hipStream_t st = static_cast<hipStream_t>(stream);
  s = run_lowbit_select(Q, codes, resid, meta, B, Hq, Hkv, N, D, block, sink, local, delta,
                        margin, scale, kcap, idx, count, tau, bmax, khat, ws, false, st,
                        "sa_decode_topdelta_lowbit");
  if (s) return s;
  return hip_status(launch_decode_lowbit(Q, codes, resid, meta, V, B, Hq, Hkv, N, D,
                                         eff_scale(scale, D), block, idx, count, kcap, dw,
                                         static_cast<char*>(ws) + lws, O, out_dtype, lse, st),
                    "sa_decode_topdelta_lowbit (decode)");
}

sa_status sa_mass_select(const void* Q, const void* K, int dtype, int B, int Hq, int Hkv, int L,
                         int D, int block, int k_free, float scale, float* mass, int32_t* idx,
                         int32_t* count, float* row_mass, int32_t* row_idx,
                         int32_t* row_count, void* ws, size_t ws_bytes, void* stream) {
  PTR(Q);
  PTR(K);
  PTR(idx);
  PTR(count);
  if (mass) PTR(mass);
  REQ((row_mass == nullptr) == (row_idx == nullptr) && (row_idx == nullptr) == (row_count == nullptr),
      "row_mass, row_idx and row_count go together (all NULL or none)");
  if (row_mass) {
    PTR(row_mass);
    PTR(row_idx);
    PTR(row_count);
  }
  REQ(dtype_ok(dtype), "unknown dtype %d", dtype);
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  SUP(dtype == SA_BF16, "the dense pass runs on bf16 matrix cores: dtype must be SA_BF16");
  SUP(D == 128, "the mass selector supports D = 128");
  SUP(block == 128, "the mass selector supports 128-token blocks");
  SUP(long(L) * D * 2 <= 0x7f000000L, "the dense pass reads one kv head through a buffer "
      "resource of at most 0x7f000000 bytes (L * D * 2 = %ld)", long(L) * D * 2);
  REQ(L >= 1, "L must be >= 1");
  REQ(k_free >= 1 && k_free <= 64, "k_free must be in [1, 64] (got %d)", k_free);
  const long units = long(B) * Hkv * cdiv(L, block);
  REQ(cdiv(units, 8) * 8L * (Hq / Hkv) < (1L << 31), "grid too large");
  const MassWs w = mass_ws(B, Hq, Hkv, L, block);
  if (ws_bytes < w.bytes) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, ws_bytes);
  PTR(ws);
  return hip_status(launch_mass_select(Q, K, B, Hq, Hkv, L, D, eff_scale(scale, D), block, k_free,
                                       mass, idx, count, row_mass, row_idx, row_count, w, ws,
                                       static_cast<hipStream_t>(stream)),
                    "sa_mass_select");
}

sa_status sa_sparse_decode(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                           int Hkv, int N, int D, float scale, int mode, int block,
                           const int32_t* idx, const int32_t* count, int idx_stride,
                           const float* score, void* O, int out_dtype, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
  sa_status s = v_decode(Q, K, V, dtype, B, Hq, Hkv, N, D, mode, block, idx, count, idx_stride,
                         score, O, out_dtype, lse, ws, ws_bytes);
  if (s) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float sc = eff_scale(scale, D);
  const DecodeWs w = decode_ws(B, Hq, Hkv, D, mode, block, idx_stride);
  hipError_t e = mode == SA_IDX_BLOCKS
                     ? launch_decode_blocks(Q, K, V, dtype, B, Hq, Hkv, N, D, sc, block, idx,
                                            count, idx_stride, w, ws, O, out_dtype, lse, st)
                     : launch_decode_tokens(Q, K, V, dtype, B, Hq, Hkv, N, D, sc, idx, count,
                                            idx_stride, score, w, ws, O, out_dtype, lse, st);
  return hip_status(e, "sa_sparse_decode");
}

sa_status sa_sparse_prefill(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                            int Hkv, int L, int D, float scale, int block, const int32_t* idx,
                            const int32_t* count, int kmax, void* O, int out_dtype, float* lse,
                            void* stream) {
  PTR(Q);
  PTR(K);
  PTR(V);
  PTR(idx);
  PTR(count);
  PTR(O);
  if (lse) PTR(lse);
  REQ(dtype_ok(dtype) && dtype_ok(out_dtype), "unknown dtype");
  sa_status s = check_heads(B, Hq, Hkv);
  if (s) return s;
  REQ(L >= 1 && kmax >= 1 && block >= 1, "L, kmax and block must be >= 1");
  SUP(dtype == SA_BF16, "prefill runs on bf16 matrix cores: dtype must be SA_BF16");
  SUP(D == 64 || D == 128, "prefill supports D = 64 or 128 (got %d)", D);
  SUP(block == 64 || block == 128, "prefill supports blocks of 64 or 128 tokens (got %d)", block);
  SUP(long(L) * D * 2 <= 0x7f000000L, "prefill reads one kv head through a buffer resource of "
      "at most 0x7f000000 bytes (L * D * 2 = %ld)", long(L) * D * 2);
  const long units = long(B) * Hkv * cdiv(L, block);
  REQ(cdiv(units, 8) * 8L * (Hq / Hkv) < (1L << 31), "grid too large");
  return hip_status(launch_prefill(Q, K, V, B, Hq, Hkv, L, D, eff_scale(scale, D), block, idx,
                                   count, kmax, O, out_dtype, lse,
                                   static_cast<hipStream_t>(stream)),
                    "sa_sparse_prefill");
}

sa_status sa_decode_step(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                         int Hkv, int N, int D, int block, float* ksketch, int update_block,
                         int k, float scale, int32_t* idx, int32_t* count, float* score,
                         void* O, int out_dtype, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  return decode_step(Q, K, V, dtype, B, Hq, Hkv, N, D, block, ksketch, update_block, k, scale,
                     idx, count, score, O, out_dtype, lse, ws, ws_bytes,
                     static_cast<hipStream_t>(stream), StepPhase::kLaunch);
}

sa_status sa_select_decode(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                           int Hkv, int N, int D, int block, const float* score, int k,
                           unsigned flags, float scale, int32_t* idx, int32_t* count, void* O,
                           int out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  PTR(score);
  PTR(count);
  REQ(block >= 1, "block must be >= 1");
  REQ(N >= 1 && k >= 1, "N and k must be >= 1 (got %d, %d)", N, k);
  REQ((flags & ~3u) == 0, "decode selection takes SA_FORCE_SINK / SA_FORCE_LOCAL only (0x%x)",
      flags);
  const int nb = cdiv(N, block);
  const int nF = int((flags & SA_FORCE_SINK) != 0) + int((flags & SA_FORCE_LOCAL) != 0);
  REQ(nb == 1 || k >= nF, "k (%d) smaller than the %d forced blocks", k, nF);
  SUP(nb <= kMaxNbDecode, "at most %d blocks per decode selection row", kMaxNbDecode);
  sa_status s = v_decode(Q, K, V, dtype, B, Hq, Hkv, N, D, SA_IDX_BLOCKS, block, idx, count, k,
                         nullptr, O, out_dtype, lse, ws, ws_bytes);
  if (s) return s;
  return run_select_decode(Q, K, V, dtype, B, Hq, Hkv, N, D, block, score, nb, k, flags,
                           eff_scale(scale, D), idx, count, O, out_dtype, lse, ws,
                           static_cast<hipStream_t>(stream), "sa_select_decode");
}

}  // extern "C"
