// sa_internal.h -- host-side plumbing shared by the C ABI and the kernel
// launchers: workspace layouts, split plans and launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa.h"

namespace sa {

constexpr int kTargetWGs = 1024;      // 256 CUs x 4: enough workgroups to fill the chip
constexpr int kMaxNbDecode = 8192;    // LDS-resident keys of one decode selection row (32 KiB)
constexpr int kMaxNbPrefill = 8192;   // LDS-resident keys of one prefill selection row
constexpr int kValuTokensPerWG = 1024;
constexpr int kThrSeg = 128;          // tokens per threshold staging segment

inline int cdiv(long a, long b) { return int((a + b - 1) / b); }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kMaxSplits = 128;       // partials merged by one workgroup
constexpr int kMaxKFused = 1024;      // k of the decode step that selects inside the decode kernel
// The float32 decode selects its own blocks for rows of up to 256 kValuSelKpt
// blocks and k up to kValuSelMaxK; longer rows go through k_select_rows.
constexpr int kValuSelKpt = 2;
constexpr int kValuSelMaxK = 512;
constexpr int kTokensPerSplit = 256;  // block-mode split target: 16 tiles of 16 tokens
constexpr int kCounterStride = 64;    // arrival counters 256 B apart (own cache lines)
constexpr int kScoreRows = 32;        // sketch rows per scoring workgroup

// Number of splits per (b, kv head) for the block-mode split-K decode: about
// 256 selected tokens per workgroup (4 waves x 4 tiles of 16 tokens, all loads
// in flight at once).  The kernel divides the actual selected-block count
// evenly over the splits; the last split to finish merges them.
inline int decode_block_splits(int idx_stride, int block) {
  int S = cdiv(long(idx_stride) * block, kTokensPerSplit);
  if (S > idx_stride) S = idx_stride;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return S;
}
// Splits per (b, kv head) of the float32 block decode: one compute unit pulls
// only a few tens of GB/s, so each split takes about one 64-token block.
constexpr int kValuTokensPerSplit = 64;
inline int decode_valu_splits(int idx_stride, int block) {
  int S = cdiv(long(idx_stride) * block, kValuTokensPerSplit);
  if (S > idx_stride) S = idx_stride;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return S;
}
// Splits per (b, kv head) of the thumbnail-key decode (k_decode_lowbit): the
// block decode's, raised so that a split's tiles touch at most
// kLowbitMetaBlocks list entries (their block rows are staged in LDS).  Never
// above decode_valu_splits, so decode_ws already sizes its partials.
constexpr int kLowbitMetaBlocks = 16;
inline int decode_lowbit_splits(int idx_stride, int block) {
  int S = decode_block_splits(idx_stride, block);
  const int smin = cdiv(idx_stride, kLowbitMetaBlocks - 1);
  if (S < smin) S = smin;
  if (S > idx_stride) S = idx_stride;
  if (S > kMaxSplits) S = kMaxSplits;
  return S;
}
// Splits per (b, query head) for token-mode decode.
inline int decode_token_splits(int BHq, int idx_stride) {
  int S = cdiv(kTargetWGs, BHq);
  const int smax = cdiv(idx_stride, 16);
  if (S > smax) S = smax;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return S;
}

constexpr int kCUs = 256;             // compute units of the gfx950 part
constexpr int kSelEntCap = 520;       // entries of a selecting-decode row: 2 forced + 512 candidates

// Splits per (b, kv head) of the decode that selects its own blocks: one
// workgroup per compute unit when the heads are few (the gather is then bound
// by the busiest unit's bytes, so the work is spread as evenly as the heads
// allow), capped where a split would get less than about half a batch of tiles.
inline int decode_sel_splits(int BH, int k, int block) {
  int S = cdiv(kCUs, BH);
  const int cap = decode_block_splits(2 * k, block);
  if (S > cap) S = cap;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return S;
}

// Workspace of the split-K decode: partial accumulators, (m, l) pairs, one
// arrival counter per head group (zero between calls) and, in block mode, the
// per-entry kept blocks of the selecting decode ([B*Hkv, kSelEntCap] int32,
// rewritten by every call).  Block mode sizes the partials for the larger
// split count of the two block-mode kernels, so one workspace serves both;
// `fused` picks the split count S of the selecting kernel.
struct DecodeWs {
  size_t acc_off, ml_off, cnt_off, ent_off, bytes;
  int S;
};
inline DecodeWs decode_ws(int B, int Hq, int Hkv, int D, int mode, int block,
                          int idx_stride, bool fused = false) {
  DecodeWs w{};
  const bool blocks = mode == SA_IDX_BLOCKS;
  int Ssz;
  if (blocks) {
    const int Sp = decode_block_splits(idx_stride, block);
    const int Sf = decode_sel_splits(B * Hkv, idx_stride, block);
    const int Sv = decode_valu_splits(idx_stride, block);
    w.S = fused ? Sf : Sp;
    Ssz = Sp > Sf ? Sp : Sf;
    if (Sv > Ssz) Ssz = Sv;
  } else {
    w.S = Ssz = decode_token_splits(B * Hq, idx_stride);
  }
  const size_t parts = size_t(B) * Hq * Ssz;
  w.acc_off = 0;
  w.ml_off = align256(parts * D * sizeof(float));
  w.cnt_off = w.ml_off + align256(parts * 2 * sizeof(float));
  w.ent_off = w.cnt_off + align256(size_t(B) * Hq * kCounterStride * sizeof(uint32_t));
  w.bytes = w.ent_off + (blocks ? align256(size_t(B) * Hkv * kSelEntCap * sizeof(int32_t)) : 0);
  return w;
}

// The one-launch decode step (k_step.hip): one team of kStepTeam workgroups
// per XCD (one per compute unit), kv head bh on team bh % 8 with S = team /
// (heads of the team) splits; split s scores the sketch rows s, s + S, ...
// (at most kStepMaxRows of them) and publishes up to kStepPubCap candidates.
constexpr int kStepTeam = 32;
constexpr int kStepMaxRows = 256;
constexpr int kStepPubWords = 64;                 // 2 header words + the candidates
constexpr int kStepPubCap = kStepPubWords - 2;
constexpr int kStepSpinLimit = 1 << 21;           // polls of one wait (seconds)
constexpr int kStepMaxCand = 512;                 // bracketed candidates ranked per head
constexpr int kStepMergeEnt = 320;                // (split, 4-column chunk) entries of a merge share

// Workspace of the one-launch step: an error word at offset 0 (nonzero once a
// wait ran out; never cleared by the library), three counters per head (two
// barriers and the merge arrivals, zero between calls) in a region sized for
// the most heads any shape can have (so the same buffer serves every shape:
// the rest is always written before it is read), the published candidates
// [BH, team, kStepPubWords] u64, the scores in slot order [BH, team,
// kStepMaxRows], and the partials [B*Hq, team, D] + (m, l) [B*Hq, team, 2].
constexpr int kStepMaxHeads = 8 * kStepTeam;
constexpr size_t kStepCtrBytes = size_t(kStepMaxHeads) * 3 * kCounterStride * sizeof(uint32_t);
struct StepWs {
  size_t ctr_off, pub_off, srow_off, acc_off, ml_off, bytes;
};
inline StepWs step_ws(int B, int Hq, int Hkv, int D) {
  const size_t BH = size_t(B) * Hkv, W = kStepTeam;
  StepWs w{};
  w.ctr_off = 256;
  w.pub_off = w.ctr_off + kStepCtrBytes;
  w.srow_off = w.pub_off + align256(BH * W * kStepPubWords * sizeof(uint64_t));
  w.acc_off = w.srow_off + align256(BH * W * kStepMaxRows * sizeof(float));
  w.ml_off = w.acc_off + align256(size_t(B) * Hq * W * D * sizeof(float));
  w.bytes = w.ml_off + align256(size_t(B) * Hq * W * 2 * sizeof(float));
  return w;
}
// Shapes the one-launch step covers (bf16, D 64 or 128, g in {1, 2, 4, 8},
// blocks of 64 or 128, at most kStepTeam heads per XCD, at most kStepMaxRows
// sketch rows per split, k <= kMaxKFused).
inline bool step_fusable(int dtype, int B, int Hq, int Hkv, int N, int D, int block, int k) {
  if (dtype != SA_BF16 || !(D == 64 || D == 128) || !(block == 64 || block == 128)) return false;
  if (Hkv < 1 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return false;
  const long BH = long(B) * Hkv;
  const long Hx = (BH + 7) / 8;
  if (Hx > kStepTeam) return false;
  const int S = kStepTeam / int(Hx);
  const int nb = cdiv(N, block);
  if (cdiv(nb, S) > kStepMaxRows || nb > kMaxNbDecode) return false;
  if (k < 1 || k > kMaxKFused) return false;
  return long(N) * D * 2 <= 0x7f000000L;
}

// Workspace of the top-k selection.  Decode: the block scores.
// Prefill: the pooled query blocks.
struct SelectWs {
  size_t score_off, bytes;
};
inline SelectWs select_ws(int B, int Hkv, int Lq, int D, int q_block, int nb) {
  SelectWs w{};
  if (Lq <= 1) {
    const size_t BH = size_t(B) * Hkv;
    w.score_off = 0;
    w.bytes = align256(BH * nb * sizeof(float));
  } else {
    const int M = cdiv(Lq, q_block);
    w.bytes = align256(size_t(B) * Hkv * M * D * sizeof(float));
  }
  return w;
}
inline size_t select_ws_bytes(int B, int Hkv, int Lq, int D, int q_block, int nb) {
  return select_ws(B, Hkv, Lq, D, q_block, nb).bytes;
}

// Workspace of the threshold selection: per 128-token segment staging of the
// kept (index, score) pairs and their counts.
struct ThrWs {
  size_t idx_off, val_off, cnt_off, bytes;
  int nseg;
};
inline ThrWs threshold_ws(int B, int Hq, int N) {
  ThrWs w{};
  w.nseg = cdiv(N, kThrSeg);
  size_t slots = size_t(B) * Hq * w.nseg * kThrSeg;
  w.idx_off = 0;
  w.val_off = align256(slots * sizeof(int32_t));
  w.cnt_off = w.val_off + align256(slots * sizeof(float));
  w.bytes = w.cnt_off + align256(size_t(B) * Hq * w.nseg * sizeof(int32_t));
  return w;
}
// Top-delta adds the per-head thresholds [B, Hq] after the threshold workspace.
inline size_t topdelta_ws_bytes(int B, int Hq, int N) {
  return threshold_ws(B, Hq, N).bytes + align256(size_t(B) * Hq * sizeof(float));
}
// The low-bit top-delta filter: one keep flag per (b, kv head, block), then
// the per-head thresholds [B, Hq].
inline size_t lowbit_ws_bytes(int B, int Hq, int Hkv, int N, int block) {
  return align256(size_t(B) * Hkv * cdiv(N, block)) + align256(size_t(B) * Hq * sizeof(float));
}
// The attention-mass selector: the rows' softmax statistics [B, Hq, L, 2] f32,
// the mass pass's output [B, Hq, L, 128] f32, the dense causal block lists
// [B, Hkv, M, M] and counts, and the masses [B, Hkv, M, M] f32 (unless the
// caller takes them).
struct MassWs {
  size_t stats_off, o_off, list_off, lcnt_off, mass_off, bytes;
};
inline MassWs mass_ws(int B, int Hq, int Hkv, int L, int block) {
  MassWs w{};
  const size_t M = size_t(cdiv(L, block));
  w.stats_off = 0;
  w.o_off = align256(size_t(B) * Hq * L * 2 * 4);
  w.list_off = w.o_off + align256(size_t(B) * Hq * L * 128 * 4);
  w.lcnt_off = w.list_off + align256(size_t(B) * Hkv * M * M * 4);
  w.mass_off = w.lcnt_off + align256(size_t(B) * Hkv * M * 4);
  w.bytes = w.mass_off + align256(size_t(B) * Hkv * M * M * 4);
  return w;
}
// The sphere-pruned threshold adds one live flag per (b, kv head, segment).
inline size_t pruned_ws_bytes(int B, int Hq, int Hkv, int N) {
  const ThrWs w = threshold_ws(B, Hq, N);
  return w.bytes + align256(size_t(B) * Hkv * w.nseg);
}

// ---------------------------------------------------------------- launchers
struct SelectPlan {
  int C;    // scoring workgroups per (b, kv head)
  int RPW;  // sketch rows per scoring workgroup
};
SelectPlan select_plan(int BH, int nb);

hipError_t launch_sketch(const void* X, int dtype, int B, int H, int N, int D,
                         int block, int head_pool, int blk_begin, int blk_end,
                         float* out, hipStream_t st);
// Decode block scores (upd >= 0 also rebuilds that block's sketch from K).
hipError_t launch_score(const void* Q, int dtype, int B, int Hq, int Hkv, int D, float* sk,
                        int nb, const void* K, int N, int block, int upd, float scale,
                        float* scores, hipStream_t st);
// Top-k per score row (decode rules: forced sink/local, ties to lower index).
hipError_t launch_select_rows(const float* scores, int rows, int nb, int k, unsigned flags,
                              int32_t* idx, int32_t* count, hipStream_t st);
// bf16 split-K decode whose workgroups select their blocks from the scores.
hipError_t launch_decode_select_blocks(const void* Q, const void* K, const void* V, int B, int Hq,
                                       int Hkv, int N, int D, float scale, int block,
                                       const float* scores, int nb, int k, unsigned flags,
                                       int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                       void* O, int out_dtype, float* lse, hipStream_t st);
// The same for float32 (k_decode_blocks_valu selecting its own blocks): rows of
// nb <= 256 kValuSelKpt blocks, k <= kValuSelMaxK.
hipError_t launch_decode_select_valu(const void* Q, const void* K, const void* V, int B, int Hq,
                                     int Hkv, int N, int D, float scale, int block,
                                     const float* scores, int nb, int k, unsigned flags,
                                     int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                     void* O, int out_dtype, float* lse, hipStream_t st);
// The whole float32 decode step in one launch (the same shapes): every split
// scores its kv head's sketch row itself (row update_block rebuilt from K
// first; -1: none), split 0 storing that sketch row and the scores.
hipError_t launch_decode_step_valu(const void* Q, const void* K, const void* V, int B, int Hq,
                                   int Hkv, int N, int D, float scale, int block, float* sketch,
                                   int update_block, float* scores, int nb, int k, unsigned flags,
                                   int32_t* idx, int32_t* count, const DecodeWs& w, void* ws,
                                   void* O, int out_dtype, float* lse, hipStream_t st);
// The one-launch decode step (bf16; step_fusable shapes).  coh_mode: 0 plain
// stores inside an XCD team, 1 device-coherent stores throughout, 2 every
// workgroup acts as if it ran off its team's XCD (both for tests).
hipError_t launch_decode_step(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                              int N, int D, int block, float* sk, int upd, int k, unsigned flags,
                              float scale, int32_t* idx, int32_t* count, float* score, void* O,
                              int out_dtype, float* lse, void* ws, int coh_mode, hipStream_t st);
// sa_decode_step in phases: kCheck runs only the host-side argument checks
// (nothing is enqueued and no HIP call is made); kLaunch enqueues the step;
// kClearAndLaunch first zeroes, on the stream, the workspace words that must
// read zero when a step starts (arrival counters, the error word).
enum class StepPhase { kCheck, kLaunch, kClearAndLaunch };
sa_status decode_step(const void* Q, const void* K, const void* V, int dtype, int B, int Hq,
                      int Hkv, int N, int D, int block, float* ksketch, int update_block, int k,
                      float scale, int32_t* idx, int32_t* count, float* score, void* O,
                      int out_dtype, float* lse, void* ws, size_t ws_bytes, hipStream_t st,
                      StepPhase phase);
// Records `what` as the calling thread's sa_last_error() message; returns s.
sa_status report(sa_status s, const char* what);
// The block-mode split-K decode over keys rebuilt from 2-bit codes and 8-bit
// residuals (bf16 V; D 64 or 128; blocks of 64 or 128; g in {1, 2, 4, 8}).
// Needs decode_lowbit_splits(idx_stride, block) <= kMaxSplits splits whose
// tiles span at most kLowbitMetaBlocks entries (idx_stride <=
// kMaxSplits * (kLowbitMetaBlocks - 1)).
hipError_t launch_decode_lowbit(const void* Q, const uint8_t* codes, const int8_t* resid,
                                const float* meta, const void* V, int B, int Hq, int Hkv, int N,
                                int D, float scale, int block, const int32_t* idx,
                                const int32_t* count, int idx_stride, const DecodeWs& w, void* ws,
                                void* O, int out_dtype, float* lse, hipStream_t st);
hipError_t launch_prefill_select(const float* qbar, const float* ksk, int BH,
                                 int M, int nb, int D, int k, unsigned flags,
                                 float scale, int32_t* idx, int32_t* count,
                                 float* score, hipStream_t st);
hipError_t launch_decode_blocks(const void* Q, const void* K, const void* V,
                                int dtype, int B, int Hq, int Hkv, int N, int D,
                                float scale, int block, const int32_t* idx,
                                const int32_t* count, int idx_stride,
                                const DecodeWs& w, void* ws, void* O, int out_dtype,
                                float* lse, hipStream_t st);
hipError_t launch_decode_tokens(const void* Q, const void* K, const void* V,
                                int dtype, int B, int Hq, int Hkv, int N, int D,
                                float scale, const int32_t* idx,
                                const int32_t* count, int idx_stride,
                                const float* score, const DecodeWs& w, void* ws,
                                void* O, int out_dtype, float* lse, hipStream_t st);
hipError_t launch_pseudo_max(const void* Q, const void* K, int dtype, int B,
                             int Hq, int Hkv, int N, int D, int sink, int local,
                             float delta, float scale, float* tau, hipStream_t st);
hipError_t launch_threshold(const void* Q, const void* K, int dtype, int B,
                            int Hq, int Hkv, int N, int D, const float* tau,
                            float scale, int cap, int32_t* idx, float* score,
                            int32_t* count, const ThrWs& w, void* ws,
                            hipStream_t st, const uint8_t* live = nullptr,
                            int pblock = kThrSeg);
hipError_t launch_encode(const void* K, int dtype, int B, int H, int N, int D,
                         int block, int b0, int b1, uint8_t* codes, int8_t* resid,
                         float* meta, hipStream_t st);
hipError_t launch_decode_keys(const uint8_t* codes, const int8_t* resid,
                              const float* meta, int B, int H, int N, int D,
                              int block, const int32_t* idx, const int32_t* count,
                              int idx_stride, int b0, int b1, uint16_t* khat,
                              hipStream_t st);
hipError_t launch_thumb_scan(const uint16_t* Q, const uint8_t* codes,
                             const float* meta, int B, int Hq, int Hkv, int N,
                             int D, int block, float scale, const float* tau,
                             float margin, int f0, int f1, int f2, int f3,
                             float* bmax, uint8_t* flag, hipStream_t st);
hipError_t launch_block_list(const uint8_t* flag, int BH, int nb, int kcap,
                             int32_t* idx, int32_t* count, hipStream_t st);
hipError_t launch_mass_select(const void* Q, const void* K, int B, int Hq, int Hkv,
                              int L, int D, float scale, int block, int kfree,
                              float* mass, int32_t* idx, int32_t* count,
                              float* row_mass, int32_t* row_idx, int32_t* row_count,
                              const MassWs& w, void* ws, hipStream_t st);
hipError_t launch_radius(const void* X, int dtype, int B, int H, int N, int D,
                         int block, int S, int b0, int b1, const float* sketch,
                         float* radius, hipStream_t st);
hipError_t launch_prune(const void* Q, int dtype, int B, int Hq, int Hkv, int N,
                        int D, int block, int S, const float* sketch,
                        const float* radius, const float* tau, float scale,
                        int nseg, uint8_t* live, int32_t* st_cnt, hipStream_t st);
hipError_t launch_prefill(const void* Q, const void* K, const void* V, int B,
                          int Hq, int Hkv, int L, int D, float scale, int block,
                          const int32_t* idx, const int32_t* count, int kmax,
                          void* O, int out_dtype, float* lse, hipStream_t st,
                          bool split_p = false);
// The attention-mass selector's dense passes (D = 128, blocks of 128): the
// rows' softmax statistics stats [B, Hq, L, 2] over their listed blocks
// (stats_pass), or each row's probability mass on its listed blocks in
// [c0, c0 + 128), written to O [B, Hq, L, 128] float32.
hipError_t launch_prefill_mass(const void* Q, const void* K, int B, int Hq, int Hkv, int L,
                               float scale, const int32_t* idx, const int32_t* count, int kmax,
                               float* O, float* stats, int c0, bool stats_pass, hipStream_t st);

}  // namespace sa
