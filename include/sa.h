/*
 * sa.h -- C ABI of the MI355X (gfx950) top-k block-sparse attention library.
 *
 * The library computes query-aware sparse attention over a GQA KV cache:
 *   1. compress the keys into per-block mean sketches        (sa_build_sketch)
 *   2. score blocks against the query heads of each KV group
 *      and keep the top-k, always including sink and local     (sa_select_topk)
 *      -- or keep every key above a score threshold            (sa_select_threshold)
 *   3. exact softmax attention over the kept keys only         (sa_sparse_decode,
 *                                                               sa_sparse_prefill)
 *
 * Pages the operations follow (title, section):
 *   [ORACLE]  "How Much Dense Attention is Necessary? Oracle-Guided Sparse
 *             Prefill for Full/GQA Layers in Hybrid Long-Context Models",
 *             technical summary §2.1: choose a top-k support from head-averaged
 *             importance, then recompute attention on that support with the
 *             original Q, K, V; supports may be shared by a block of queries.
 *   [FRONTIER] "The Sparse Frontier: Sparse Attention Trade-offs in Transformer
 *             LLMs", Metodologia §1 and Contributi §2: block/page units, full
 *             cache retained and loaded selectively (Quest decode), block-by-block
 *             selection in prefill (Block-Sparse).
 *   [FFD]     "Faster Than Flash: Exploiting Attention Sparsity for Efficient
 *             Long-Context Decoding", Metodologia §1-§3: scan a compact key
 *             summary first, fetch exact data only for the chosen parts; sink and
 *             local tokens dominate attention.
 *   [PULSAR]  "Pulsar Attention", Fase 1 (64-token attention-sink prefix) and
 *             Fase 2 (online-softmax merge of partial attention is exact).
 *   [RANGE]   "Sparse Attention as a Range Searching Problem: Towards an
 *             Inference-Efficient Index for KV Cache", Metodologia §1: return
 *             every key in the half-space <q, k> >= tau (no false negatives).
 *
 * Conventions shared by every entry point
 *   - Layouts are row-major with D innermost:
 *       K, V  [B, Hkv, N, D]      Q  [B, Hq, D] (decode) or [B, Hq, L, D] (prefill)
 *     Query head h reads kv head h / g, g = Hq / Hkv (Hq % Hkv == 0).
 *   - Every pointer is DEVICE memory owned by the caller.  Inputs are const.
 *     The library allocates nothing and keeps no state between calls apart
 *     from a cached device-property query and the per-GPU scratch array of
 *     sa_decode_step_noalloc.
 *   - `ws` is a caller-provided device workspace of at least
 *     sa_workspace_bytes(...) bytes.  It holds partial results plus arrival
 *     counters and histograms that must read zero when a call starts: zero-fill
 *     it once when it is allocated; every completed call leaves that state at
 *     zero again, so the same workspace can serve later calls of the same
 *     operation and shapes.  Calls of another operation or shape, or calls
 *     that run concurrently, need their own workspace (or a re-zeroed one).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises the host.
 *   - dtype codes: SA_F32 (float) or SA_BF16 (raw bfloat16 bits, uint16).
 *   - scale <= 0 means 1/sqrt(D).
 *   - Pointers must be 16-byte aligned.  D must be 64 or 128.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     return SA_ERR_INVALID; shapes/dtypes with no compiled kernel return
 *     SA_ERR_UNSUPPORTED; a too-small workspace returns SA_ERR_WORKSPACE; a
 *     failed launch returns SA_ERR_HIP.  sa_last_error() describes the last
 *     failure of the calling thread.
 *   - Same inputs, same device, same build -> bitwise identical outputs (no
 *     floating-point atomics; every reduction has a fixed order).
 *   - Index lists are ascending; unused slots are written as -1.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID = 1,
  SA_ERR_UNSUPPORTED = 2,
  SA_ERR_WORKSPACE = 3,
  SA_ERR_HIP = 4
} sa_status;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* selection flags */
enum {
  SA_FORCE_SINK = 1u,  /* always keep block 0 (the attention-sink prefix, [PULSAR] Fase 1) */
  SA_FORCE_LOCAL = 2u, /* always keep the newest block (decode) / the diagonal block (prefill) */
  SA_CAUSAL = 4u       /* prefill: query block i ranks key blocks 1..i-1 only */
};

/* sparse_decode modes */
enum { SA_IDX_BLOCKS = 0, SA_IDX_TOKENS = 1 };

/* operations for sa_workspace_bytes */
enum {
  SA_OP_SELECT_TOPK = 0,
  SA_OP_SELECT_THRESHOLD = 1,
  SA_OP_SPARSE_DECODE = 2,
  SA_OP_DECODE_STEP = 3,
  SA_OP_SELECT_TOPDELTA = 4,
  SA_OP_SELECT_PRUNED = 5,
  SA_OP_SELECT_LOWBIT = 6,
  SA_OP_MASS_SELECT = 7,
  SA_OP_DECODE_LOWBIT = 8
};

/*
 * sa_build_sketch -- per-block mean sketch ([FFD] Metodologia §1: the compact
 * key summary scanned before any full key is fetched; a per-block centre as in
 * [RANGE] Metodologia §2).
 *
 *   X        [B, H, N, D] dtype           input rows (keys, or queries to pool)
 *   block    tokens per block; nb = ceil(N / block); the last block may be
 *            partial and is averaged over its valid rows only
 *   head_pool  1 for keys; g to also average each group of g consecutive heads
 *            (the pooled query block of block-sparse prefill); H % head_pool == 0
 *   blk_begin, blk_end  block range to (re)write, 0 <= begin <= end <= nb; a
 *            decode step rewrites only the newest block
 *   sketch   [B, H / head_pool, nb, D] float32, output (only the range is written)
 *
 * Entry s[b, hh, j, :] = mean over heads hh*head_pool .. +head_pool-1 and
 * tokens of block j of X[b, h, t, :], accumulated in float32.
 */
sa_status sa_build_sketch(const void* X, int dtype, int B, int H, int N, int D,
                          int block, int head_pool, int blk_begin, int blk_end,
                          float* sketch, void* stream);

/*
 * sa_select_topk -- block scores and top-k block selection ([ORACLE] §2.1,
 * [FRONTIER] Contributi §2, [FFD] Metodologia §2).
 *
 * Decode (Lq == 1, q_block == 1, no SA_CAUSAL):
 *   Q        [B, Hq, D] dtype
 *   ksketch  [B, Hkv, nb, D] float32 (sa_build_sketch of K)
 *   score[b, kh, j] = (mean over the g query heads of kv head kh of q_h) . s_j * scale
 *   Forced blocks (SA_FORCE_SINK: block 0; SA_FORCE_LOCAL: block nb-1) are kept
 *   and count toward k; the other slots go to the best remaining scores, ties
 *   to the lower block index; NaN scores rank below every number.  k >= nb
 *   keeps all blocks.
 *   idx      [B, Hkv, k] int32 out (ascending; slots past count are -1)
 *   count    [B, Hkv]    int32 out (= min(k, nb))
 *
 * Causal prefill (SA_CAUSAL, q_block == the key block size, Lq == N):
 *   Q        [B, Hq, Lq, D] dtype; pooled per query block i over its q_block
 *            tokens and the group's g heads into Qbar_i (float32)
 *   ksketch  [B, Hkv, nb, D] float32 with nb >= M = ceil(Lq / q_block)
 *   r_ij = Qbar_i . s_j * scale for j in 1..i-1; query block i keeps block 0
 *   (SA_FORCE_SINK), block i (SA_FORCE_LOCAL) and the top k - 2 of 1..i-1.
 *   One list per (b, kv head, query block), shared by its queries and heads
 *   ([ORACLE] §2.1 block-shared support).
 *   idx      [B, Hkv, M, k] int32 out;  count [B, Hkv, M] int32 out (min(i + 1, k))
 *
 *   score    optional float32 out (NULL to skip): [B, Hkv, nb] (decode) or
 *            [B, Hkv, M, nb] (prefill; entries outside 1..i-1 are -inf)
 *   ws       workspace of sa_workspace_bytes(SA_OP_SELECT_TOPK, B, Hq, Hkv, Lq, D, q_block, nb)
 *
 * Errors: SA_ERR_INVALID if k < number of forced blocks, k <= 0 or nb <= 0;
 * SA_ERR_UNSUPPORTED if nb > 8192 (decode) or M > 8192 (prefill).
 */
sa_status sa_select_topk(const void* Q, int dtype, int B, int Hq, int Hkv,
                         int Lq, int D, int q_block, const float* ksketch,
                         int nb, int k, unsigned flags, float scale,
                         int32_t* idx, int32_t* count, float* score, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * sa_select_threshold -- every key in the half-space ([RANGE] Metodologia §1):
 * keep token t for query head (b, h) when q_h . k_t * scale >= tau[b, h].
 *
 *   Q [B, Hq, D], K [B, Hkv, N, D] dtype;  tau [B, Hq] float32 (-inf keeps all)
 *   cap      capacity of each list
 *   idx      [B, Hq, cap] int32 out, ascending token positions (unused: -1)
 *   score    [B, Hq, cap] float32 out, the scaled scores of those tokens
 *   count    [B, Hq] int32 out, the TRUE number of kept tokens; when it exceeds
 *            cap only the first cap (lowest positions) are written -- the
 *            caller checks count > cap (reported in band, so the call stays
 *            asynchronous).
 *
 * No false negatives: scores are computed in float32 and a token is kept when
 * its float32 score plus a rigorous bound on the float32 rounding error of
 * that score reaches tau, so every key whose exact score reaches tau is kept;
 * the only extra keys are those within that bound below tau.
 * ws: sa_workspace_bytes(SA_OP_SELECT_THRESHOLD, B, Hq, Hkv, N, D, 0, cap).
 */
sa_status sa_select_threshold(const void* Q, const void* K, int dtype, int B,
                              int Hq, int Hkv, int N, int D, const float* tau,
                              float scale, int cap, int32_t* idx, float* score,
                              int32_t* count, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * sa_select_topdelta -- top-delta selection with a pseudo-maximum ([FFD]
 * Metodologia §2): keep token t of query head (b, h) when
 *     s_t >= m~ - delta,   s_t = q_h . k_t * scale,
 * where m~ is the largest score over the sink prefix [0, sink) and the local
 * window [N - local, N) (both clipped to the cache).  The estimate reads only
 * those tokens, so the threshold needs no reduction over the whole cache;
 * the scan, compaction and outputs are those of sa_select_threshold with
 * tau = m~ - delta.  Follow with sa_sparse_decode in SA_IDX_TOKENS mode.
 *
 *   Q [B, Hq, D], K [B, Hkv, N, D] dtype
 *   sink, local  window sizes in tokens, >= 0, not both 0
 *   delta        >= 0 (the pages use 5 and 7); +inf keeps every token
 *   cap, idx, score, count   as sa_select_threshold (count > cap is reported
 *            in band; the first cap positions are written)
 *   tau      [B, Hq] float32 out: the threshold used (NULL: kept in ws)
 *
 * No false negatives against the exact rule: tau is computed from lower
 * bounds fl32(s) - eps of the window scores, so it never exceeds
 * m~_exact - delta beyond its own float32 rounding, and the scan keeps every
 * key whose exact score reaches it (see sa_select_threshold).  The extra keys
 * lie within a few float32 rounding bounds below the exact threshold.  The
 * token attaining m~ always passes, so no list is empty.  NaN window scores
 * are ignored by the maximum.
 * ws: sa_workspace_bytes(SA_OP_SELECT_TOPDELTA, B, Hq, Hkv, N, D, 0, cap).
 */
sa_status sa_select_topdelta(const void* Q, const void* K, int dtype, int B,
                             int Hq, int Hkv, int N, int D, int sink, int local,
                             float delta, float scale, int cap, int32_t* idx,
                             float* score, int32_t* count, float* tau, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * sa_build_radius -- bounding spheres of the key blocks per subspace ([RANGE]
 * Metodologia §2: the key space is cut into S contiguous subspaces and every
 * cluster gets a centre and a radius in each; here the clusters are the
 * token blocks and the centres the block sketch rows).
 *
 *   X        [B, H, N, D] dtype (the keys)
 *   sketch   [B, H, nb, D] float32 in: the centres (sa_build_sketch's output)
 *   radius   [B, H, nb, S] float32 out: rho[j, s] >= the largest distance
 *            ||x_t,s - c_j,s|| over the valid tokens t of block j (rounded up
 *            by a relative 2^-16, so it never falls below the exact value)
 *   S        subspaces of D/S consecutive channels; D/S a multiple of 8,
 *            S <= 16 (else SA_ERR_UNSUPPORTED)
 *   [blk_begin, blk_end)  the blocks to (re)compute; the others are left as
 *            they are (decode refreshes only the newest block, after its
 *            sketch row, as keys are appended)
 * NaN keys are skipped by the maximum (their block's centre is NaN anyway).
 */
sa_status sa_build_radius(const void* X, int dtype, int B, int H, int N, int D,
                          int block, int S, int blk_begin, int blk_end,
                          const float* sketch, float* radius, void* stream);

/*
 * sa_select_threshold_pruned -- the half-space selection of
 * sa_select_threshold with whole blocks pruned first ([RANGE] Metodologia §2,
 * the two-phase filter).  Block j is dropped for query head h when
 *     scale * sum_s (q_s . c_j,s + ||q_s|| rho_j,s) < tau[b, h],
 * a rigorous upper bound of every score in the block (Cauchy-Schwarz per
 * subspace), evaluated in float32 with a margin that covers its rounding.
 * A block is scanned when it survives for any head of the kv group; the
 * scan, the exact check and the outputs are those of sa_select_threshold on
 * the scanned blocks, so there are no false negatives.
 *
 *   block    32, 64 or 128 (the blocks of sketch and radius)
 *   S, sketch, radius   as built by sa_build_sketch and sa_build_radius on K
 *   tau, cap, idx, score, count   as sa_select_threshold
 *   live     [B, Hkv, ceil(N/128)] uint8 out, one byte per 128-token segment:
 *            bit i set when the segment's i-th block was scanned (NULL: kept
 *            in ws)
 * ws: sa_workspace_bytes(SA_OP_SELECT_PRUNED, B, Hq, Hkv, N, D, block, cap).
 */
sa_status sa_select_threshold_pruned(const void* Q, const void* K, int dtype,
                                     int B, int Hq, int Hkv, int N, int D,
                                     int block, int S, const float* sketch,
                                     const float* radius, const float* tau,
                                     float scale, int cap, int32_t* idx,
                                     float* score, int32_t* count, uint8_t* live,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * sa_encode_keys -- 2-bit key thumbnails with 8-bit residuals ([FFD]
 * Metodologia §1: thumbnails are scanned to estimate scores, residuals rebuild
 * the keys for the exact computation).  Per channel c over each block j:
 *     lo, hi = min, max;  step = (hi - lo) * fl32(1/3);  d = k - lo
 *     code = [d >= step/2] + [d >= 1.5 step] + [d >= 2.5 step]   (0..3)
 *     t = fma(code, step, lo);  rstep = 2^(E - 8) where step = m 2^E, m in [0.5, 1)
 *     r8 = clamp(rint((k - t) / rstep), -127, 127)
 * all in IEEE float32, so the output is a fixed function of K.
 *
 *   K        [B, H, N, D] dtype (finite values)
 *   codes    [B, H, N, D/4] uint8 out: one little-endian 32-bit word per 16
 *            channels; channel 16 g + i of a token sits at bit 8 (i % 4) +
 *            2 (i / 4) of word g (so a shift and a mask give the codes of 4
 *            consecutive channels as 4 bytes)
 *   resid    [B, H, N, D] int8 out
 *   meta     [B, H, nb, 3, D] float32 out: (lo, step, rstep) rows per block
 *   [blk_begin, blk_end)  the blocks to (re)encode (decode appends re-encode
 *            the newest block)
 */
sa_status sa_encode_keys(const void* K, int dtype, int B, int H, int N, int D,
                         int block, int blk_begin, int blk_end, uint8_t* codes,
                         int8_t* resid, float* meta, void* stream);

/*
 * sa_decode_keys -- the refined keys k^ = t + r8 * rstep, rounded to bf16
 * (nearest, ties to even), written into khat [B, H, N, D] (bf16, laid out as
 * K) for the listed blocks only: idx [B, H, idx_stride] block ids with count
 * [B, H] valid (NULL: all idx_stride; entries < 0 are skipped), or, when idx
 * is NULL, the block range [blk_begin, blk_end).  Other rows are untouched.
 */
sa_status sa_decode_keys(const uint8_t* codes, const int8_t* resid,
                         const float* meta, int B, int H, int N, int D,
                         int block, const int32_t* idx, const int32_t* count,
                         int idx_stride, int blk_begin, int blk_end, void* khat,
                         void* stream);

/*
 * sa_select_topdelta_lowbit -- the three stages of [FFD]'s fused decode
 * (Metodologia §3) up to the attention: (1) the refined keys of the blocks
 * holding the sink prefix [0, sink) and the local window [N - local, N) are
 * rebuilt into khat and give tau = m~ - delta as sa_select_topdelta does;
 * (2) every token's provisional score comes from its 2-bit thumbnail: the
 * block offset q . lo plus ws * sum_c w8_c code_c, with int8 weights w8 of
 * q_c step_c (scale ws) on the int8 matrix cores,
 * and block j is kept for a kv head when a head h of its group has a
 * provisional score >= tau_h - margin, or when it holds window tokens;
 * (3) the refined keys of the kept blocks are written into khat.  Follow
 * with sa_sparse_decode(Q, khat, V, idx, count, SA_IDX_BLOCKS, block,
 * idx_stride = kcap).
 *
 *   Q        [B, Hq, D] bf16; codes, resid, meta as sa_encode_keys built them
 *            from K [B, Hkv, N, D]
 *   block    64 or 128 (the encoding's block); g in {1, 2, 4, 8}
 *   delta, margin  >= 0
 *   idx      [B, Hkv, kcap] int32 out, ascending kept block ids (-1 padded)
 *   count    [B, Hkv] int32 out, the TRUE number kept (may exceed kcap; only
 *            the first kcap are listed and rebuilt)
 *   tau      [B, Hq] float32 out (NULL: kept in ws);  bmax [B, Hq, nb]
 *            float32 out, each block's largest provisional score (NULL: none)
 *   khat     [B, Hkv, N, D] bf16: rows of window and kept blocks written
 * Selection is not exact against the full-precision keys: the thumbnail
 * error decides which blocks reach the filter (margin trades bytes for
 * recall); attention over the kept blocks uses the refined keys.
 * ws: sa_workspace_bytes(SA_OP_SELECT_LOWBIT, B, Hq, Hkv, N, D, block, kcap).
 */
sa_status sa_select_topdelta_lowbit(const void* Q, const uint8_t* codes,
                                    const int8_t* resid, const float* meta, int B,
                                    int Hq, int Hkv, int N, int D, int block,
                                    int sink, int local, float delta, float margin,
                                    float scale, int kcap, int32_t* idx,
                                    int32_t* count, float* tau, float* bmax,
                                    void* khat, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * sa_decode_topdelta_lowbit -- [FFD]'s fused decode (Metodologia §3) in full:
 * stages (1) and (2) of sa_select_topdelta_lowbit (the window's refined keys
 * into khat, tau, the thumbnail filter and the kept-block list), then (3) the
 * refinement and the attention in one pass: a block-mode split-K decode over
 * the kept blocks whose key rows are rebuilt inside the kernel from their codes
 * and residuals (the value sa_decode_keys writes) and whose values come from
 * V.  Same idx, count, tau and bmax as sa_select_topdelta_lowbit, and bitwise
 * the output of sa_select_topdelta_lowbit followed by sa_sparse_decode over
 * khat on the same lists, except that only the window's rows of khat are
 * written.
 *
 *   Q, codes, resid, meta, block, sink, local, delta, margin, scale, kcap,
 *            idx, count, tau, bmax: as sa_select_topdelta_lowbit
 *            (kcap <= 1920)
 *   V        [B, Hkv, N, D] bf16 (N * D * 2 <= 0x7f000000)
 *   khat     [B, Hkv, N, D] bf16 scratch: the window blocks' rows are written
 *   O        [B, Hq, D] out_dtype;  lse [B, Hq] float32 (NULL to skip)
 * ws: sa_workspace_bytes(SA_OP_DECODE_LOWBIT, B, Hq, Hkv, N, D, block, kcap).
 */
sa_status sa_decode_topdelta_lowbit(const void* Q, const uint8_t* codes,
                                    const int8_t* resid, const float* meta,
                                    const void* V, int B, int Hq, int Hkv, int N,
                                    int D, int block, int sink, int local,
                                    float delta, float margin, float scale,
                                    int kcap, int32_t* idx, int32_t* count,
                                    float* tau, float* bmax, void* khat, void* O,
                                    int out_dtype, float* lse, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * sa_mass_select -- the attention-mass top-k oracle of [ORACLE] §2.1 on the
 * GPU, at block granularity with a block-shared support: for query block i
 * of kv head kh, dense causal softmax for each of its rows and each head of
 * the group, each row's probability summed over every key block j, averaged
 * over the rows and heads -> mass[i][j]; the k_free blocks j in [1, i-1] with
 * the largest mass (ties to the lower j) are listed ascending.  A reference
 * for the recall of the sketch selector, not a fast path: it runs the dense
 * causal scores twice, once for each row's softmax maximum and sum and once
 * (per chunk of 128 key blocks) for its probability mass on each block,
 * summed over the block's keys in float32.
 *
 *   Q [B, Hq, L, D], K [B, Hkv, L, D] bf16; D = 128, block = 128,
 *            L * D * 2 <= 0x7f000000 (else SA_ERR_UNSUPPORTED)
 *   mass     [B, Hkv, M, M] float32 out (M = ceil(L / 128); entries j > i are
 *            0), or NULL (kept in ws)
 *   idx      [B, Hkv, M, k_free] int32 out, ascending (-1 padded)
 *   count    [B, Hkv, M] int32 out, min(k_free, max(i - 1, 0))
 *   row_mass, row_idx, row_count  per-query supports (b_sel = 1), all three or
 *            none (NULL): row_mass [B, Hkv, L, M] float32 out, each row's own
 *            masses averaged over the group's heads; row_idx [B, Hkv, L, k_free]
 *            its k_free largest of blocks [1, i - 1], i = t / 128, ascending;
 *            row_count [B, Hkv, L]
 *   k_free   1..64
 * ws: sa_workspace_bytes(SA_OP_MASS_SELECT, B, Hq, Hkv, L, D, block, k_free):
 *     about L * Hq * 520 bytes per batch row plus the lists.
 */
sa_status sa_mass_select(const void* Q, const void* K, int dtype, int B, int Hq,
                         int Hkv, int L, int D, int block, int k_free,
                         float scale, float* mass, int32_t* idx, int32_t* count,
                         float* row_mass, int32_t* row_idx, int32_t* row_count,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * sa_sparse_decode -- exact attention restricted to the selected keys, as
 * split-K flash decoding with a log-sum-exp merge of the partials ([ORACLE]
 * §2.1 recompute on the support; [PULSAR] Fase 2 online-softmax merge).
 *
 *   Q [B, Hq, D], K, V [B, Hkv, N, D] dtype
 *   mode SA_IDX_BLOCKS:  idx [B, Hkv, idx_stride] ascending block ids of size
 *            `block` (the last block of the cache may be partial), count
 *            [B, Hkv] valid entries (NULL: all idx_stride); the g heads of a
 *            group share the list.
 *   mode SA_IDX_TOKENS:  idx [B, Hq, idx_stride] token positions, count [B, Hq]
 *            (required; values above idx_stride are clamped to it), score
 *            [B, Hq, idx_stride] the scaled scores of those tokens as written
 *            by sa_select_threshold (NULL: recomputed from Q and K).
 *   O        [B, Hq, D] out_dtype;  lse [B, Hq] float32 (NULL to skip)
 *            O = sum_t softmax(s)_t v_t over the kept tokens, lse = log sum exp s;
 *            an empty selection gives O = 0, lse = -inf.
 * Accumulation is float32 throughout.
 * bf16 block mode reads each kv head through a 32-bit buffer range:
 * N * D * 2 <= 0x7f000000 (else SA_ERR_UNSUPPORTED).
 * ws: sa_workspace_bytes(SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, block, idx_stride)
 *     (for SA_IDX_TOKENS pass block = 0).
 */
sa_status sa_sparse_decode(const void* Q, const void* K, const void* V,
                           int dtype, int B, int Hq, int Hkv, int N, int D,
                           float scale, int mode, int block,
                           const int32_t* idx, const int32_t* count,
                           int idx_stride, const float* score, void* O,
                           int out_dtype, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * sa_sparse_prefill -- block-sparse causal attention ([FRONTIER] Contributi §2
 * Block-Sparse prefill; [ORACLE] §2.1 block-shared support).
 *
 *   Q [B, Hq, L, D], K, V [B, Hkv, L, D] dtype (SA_BF16 only: this is the
 *            path's one dense contraction and runs on the bf16 matrix cores;
 *            float32 inputs return SA_ERR_UNSUPPORTED.  D = 64 or 128; each kv
 *            head is read through a 32-bit buffer range: L * D * 2 <=
 *            0x7f000000, else SA_ERR_UNSUPPORTED)
 *   block    query and key block size (64 or 128)
 *   idx      [B, Hkv, M, kmax] int32 ascending key blocks per query block
 *            (M = ceil(L / block)), count [B, Hkv, M]; entries must be <= i
 *   Row t of query block i attends to every token of its listed blocks at
 *   position <= t.
 *   O        [B, Hq, L, D] out_dtype;  lse [B, Hq, L] float32 (NULL to skip)
 * Accumulation is float32.  The probabilities enter the value product as
 * bf16 (relative rounding <= 2^-8), so a row's output lies within
 * 2^-8 * sum_t p_t |v_t| of the exact one plus float32 rounding; rows of the
 * first query block use a bf16 hi + lo split of P (about 2^-16).
 */
sa_status sa_sparse_prefill(const void* Q, const void* K, const void* V,
                            int dtype, int B, int Hq, int Hkv, int L, int D,
                            float scale, int block, const int32_t* idx,
                            const int32_t* count, int kmax, void* O,
                            int out_dtype, float* lse, void* stream);

/*
 * sa_decode_step -- one whole decode step for one layer, fused where the
 * hardware allows: rewrite the sketch of block `update_block` (pass -1 to
 * skip), score and select the top-k blocks (forced sink + local), then the
 * split-K sparse attention and merge.  Same result as calling
 * sa_build_sketch, sa_select_topk (decode) and sa_sparse_decode (blocks) in
 * sequence (the same selection; the attention output up to float32 rounding,
 * since the fused kernel splits the blocks over workgroups differently);
 * idx/count/score (score may be NULL) receive the selection.
 * ws: sa_workspace_bytes(SA_OP_DECODE_STEP, B, Hq, Hkv, N, D, block, k).
 */
sa_status sa_decode_step(const void* Q, const void* K, const void* V,
                         int dtype, int B, int Hq, int Hkv, int N, int D,
                         int block, float* ksketch, int update_block, int k,
                         float scale, int32_t* idx, int32_t* count,
                         float* score, void* O, int out_dtype, float* lse,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * sa_decode_step_noalloc -- sa_decode_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc).  Arguments, layouts and
 * results are those of sa_decode_step (bitwise the same outputs).  The
 * workspace is a scratch array of 16 MiB that the library holds on each GPU
 * it runs on, until the process ends; it calls no allocator.  Each call first
 * zeroes the scratch words the step needs at zero (a small fill kernel on
 * `stream`, capturable), so consecutive calls may use different shapes.
 * Calls that overlap in time on one GPU (other streams or threads) share the
 * scratch and race: serialise them.  A shape whose workspace
 * (sa_workspace_bytes(SA_OP_DECODE_STEP, ...)) exceeds 16 MiB returns
 * SA_ERR_WORKSPACE; the scratch lookup failing returns SA_ERR_HIP.
 */
sa_status sa_decode_step_noalloc(const void* Q, const void* K, const void* V,
                                 int dtype, int B, int Hq, int Hkv, int N, int D,
                                 int block, float* ksketch, int update_block,
                                 int k, float scale, int32_t* idx,
                                 int32_t* count, float* score, void* O,
                                 int out_dtype, float* lse, void* stream);

/*
 * sa_select_decode -- the selection and attention half of a decode step, as
 * one kernel: top-k blocks per (b, kv head) from given block scores (the
 * selection rule of sa_select_topk, decode), then the split-K sparse attention
 * over the selected blocks and the merge (the decode steps of "The Sparse
 * Frontier", Contributi §2 Quest; split-K merge, "Pulsar Attention", Fase 2).
 * Each attention workgroup repeats the selection pre-filter of its kv head from
 * the score row instead of waiting on another workgroup, then ranks only the
 * candidates of its own slice of tiles and attends to the kept ones; the last
 * workgroup of the head merges the partials and writes idx and count.
 *
 *   Q [B, Hq, D], K, V [B, Hkv, N, D] dtype
 *   score    [B, Hkv, nb] float32 block scores (input; nb = ceil(N / block));
 *            NaN ranks as -inf
 *   k        blocks per (b, kv head), forced ones included; flags: any of
 *            SA_FORCE_SINK | SA_FORCE_LOCAL
 *   idx      [B, Hkv, k] int32 out, ascending, -1 padded; count [B, Hkv] out
 *   O        [B, Hq, D] out_dtype;  lse [B, Hq] float32 (NULL to skip)
 * Same selection as sa_select_topk's; the attention equals that of
 * sa_sparse_decode (blocks) on it up to float32 rounding, and repeated calls
 * give bitwise the same output.  nb <= 8192.
 * ws: sa_workspace_bytes(SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, block, k).
 */
sa_status sa_select_decode(const void* Q, const void* K, const void* V,
                           int dtype, int B, int Hq, int Hkv, int N, int D,
                           int block, const float* score, int k,
                           unsigned flags, float scale, int32_t* idx,
                           int32_t* count, void* O, int out_dtype, float* lse,
                           void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by an operation (0 if none; SIZE_MAX on bad input). */
size_t sa_workspace_bytes(int op, int B, int Hq, int Hkv, int N, int D,
                          int block, int k);

/* Static description of a status code. */
const char* sa_status_str(int status);

/* Description of the calling thread's last failure ("" if none). */
const char* sa_last_error(void);

/* Library ABI version (major * 100 + minor). */
int sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
