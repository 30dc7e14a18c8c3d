"""Float64 definitions of every step of the sparse-attention hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, float64,
one function per step, in the order the method runs:

  O0 dense            textbook softmax attention (the reference every sparse
                      result reduces to when nothing is dropped)
  O1 sketch           per-block mean of the keys (the compact key summary)
  O2 block_scores     group-averaged query . sketch, times the softmax scale
  O3 select_topk      forced sink + local blocks, then the best-scoring rest
  O4 attend_blocks    exact attention restricted to the selected blocks
  O5 threshold        tau from the exact scores; keep every key at or above it
  O6 prefill_select   pooled-query-block . pooled-key-block ranking, causal
  O7 prefill_attend   causal attention of each query row over its block list
  O8 mass_oracle      exact per-block attention mass, for recall reporting
  O9 select_topdelta  pseudo-max over sink + local tokens; keep s >= m~ - delta
  O10 select_threshold_pruned  block spheres per subspace prune, exact check after
  O11 select_topdelta_lowbit   2-bit thumbnails filter blocks, 8-bit residuals refine
     lse_merge        exact merge of attention partials over a split support

Arrays: q [B, Hq, D]; Q [B, Hq, L, D]; K, V [B, Hkv, N, D]; query head h uses
kv head h // g with g = Hq // Hkv.  bf16 inputs arrive as uint16 bit patterns
and are widened exactly.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


# ------------------------------------------------------------------ inputs
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 copy of a stored array ("f32" floats or "bf16" bits)."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _default_scale(D: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)


def _attend(s: np.ndarray, Vrows: np.ndarray) -> Tuple[np.ndarray, float]:
    """Softmax of the scores s [n] applied to the rows Vrows [n, D].

    Returns (o, lse).  An empty support gives o = 0 and lse = -inf.
    """
    if s.size == 0:
        return np.zeros(Vrows.shape[-1]), NEG_INF
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ Vrows) / l, m + math.log(l)


# ------------------------------------------------------------------ O0
def dense(q: np.ndarray, K: np.ndarray, V: np.ndarray,
          scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O0: full softmax attention of one decode query per head over all N keys.

    The decode query sees every cached key, unmasked (its own key is already
    in the cache).  The dense result is what the attention-mass oracle of
    "How Much Dense Attention is Necessary?" (§2.1) starts from and what any
    sparse support must reproduce when it keeps everything.
    """
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    O = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            s = (K[b, kh] @ q[b, h]) * sc
            O[b, h], lse[b, h] = _attend(s, V[b, kh])
    return O, lse


def dense_causal_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                      rows: Sequence[Tuple[int, int, int]],
                      scale: Optional[float] = None):
    """O0 for prefill rows: row (b, h, t) attends to keys 0..t (causal)."""
    D = Q.shape[-1]
    g = Q.shape[1] // K.shape[1]
    sc = _default_scale(D, scale)
    O = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    for r, (b, h, t) in enumerate(rows):
        kh = h // g
        s = (K[b, kh, :t + 1] @ Q[b, h, t]) * sc
        O[r], lse[r] = _attend(s, V[b, kh, :t + 1])
    return O, lse


# ------------------------------------------------------------------ O1
def sketch(X: np.ndarray, block: int, head_pool: int = 1) -> np.ndarray:
    """O1: per-block mean sketch of X [B, H, N, D] -> [B, H/head_pool, nb, D].

    Block j covers tokens [j*block, min((j+1)*block, N)); the last block may be
    partial and is averaged over its valid tokens only.  With head_pool > 1 the
    mean also runs over each group of head_pool consecutive heads (the pooled
    query block of block-sparse prefill).  The mean is our reading of
    the "compact summary of the keys" that is scanned before any full key is
    fetched ("Faster Than Flash", Metodologia §1) -- a per-block centre, like
    the cluster centres of the range-search index ("Sparse Attention as a Range
    Searching Problem", Metodologia §2).
    """
    B, H, N, D = X.shape
    if H % head_pool:
        raise ValueError("H must be a multiple of head_pool")
    nb = -(-N // block)
    Xg = X.reshape(B, H // head_pool, head_pool, N, D)
    out = np.zeros((B, H // head_pool, nb, D))
    for j in range(nb):
        lo, hi = j * block, min((j + 1) * block, N)
        out[:, :, j] = Xg[:, :, :, lo:hi, :].sum(axis=(2, 3)) / (head_pool * (hi - lo))
    return out


# ------------------------------------------------------------------ O2
def block_scores(q: np.ndarray, sk: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """O2: score[b, kh, j] = mean over the group's query heads of (q_h . s_j) * scale.

    Averaging over the query heads of a KV group follows the head-averaged
    token importance of "How Much Dense Attention is Necessary?" (§2.1).
    """
    B, Hq, D = q.shape
    Hkv = sk.shape[1]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    out = np.zeros((B, Hkv, sk.shape[2]))
    for b in range(B):
        for kh in range(Hkv):
            per_head = np.stack([sk[b, kh] @ q[b, h] for h in range(kh * g, (kh + 1) * g)])
            out[b, kh] = per_head.mean(axis=0) * sc
    return out


# ------------------------------------------------------------------ O3
def _rank_key(scores: np.ndarray) -> np.ndarray:
    """Scores as ranking keys: NaN counts as -inf (never preferred)."""
    s = np.array(scores, dtype=np.float64)
    s[np.isnan(s)] = NEG_INF
    return s


def select_topk(scores: np.ndarray, k: int, forced: Iterable[int] = None) -> np.ndarray:
    """O3: the kept blocks of one (b, kv head), ascending.

    Forced blocks (default: the sink block 0 and the local block nb-1) are
    always kept and count toward k.  The other k - |forced| slots go to the
    remaining blocks by score, higher first, ties to the lower block index.
    k >= nb keeps everything.  The sink follows the fixed attention-sink prefix
    of "Pulsar Attention" (Fase 1; 64 tokens = one 64-token block); sink and
    local tokens dominating the distribution is the observation of "Faster
    Than Flash" (Metodologia §2); per-page selection from the full cache is
    Quest as described in "The Sparse Frontier" (Contributi §2).
    """
    s = _rank_key(scores)
    nb = s.size
    if forced is None:
        forced = {0, nb - 1}
    F = sorted({int(j) for j in forced if 0 <= j < nb})
    if k >= nb:
        return np.arange(nb)
    if k < len(F):
        raise ValueError("k smaller than the number of forced blocks")
    cand = np.array([j for j in range(nb) if j not in set(F)], dtype=np.int64)
    order = cand[np.lexsort((cand, -s[cand]))]   # score desc, then index asc
    return np.sort(np.concatenate([np.array(F, dtype=np.int64), order[:k - len(F)]]))


def select_topk_all(scores: np.ndarray, k: int) -> np.ndarray:
    """O3 over every (b, kv head): scores [B, Hkv, nb] -> idx [B, Hkv, min(k, nb)]."""
    B, Hkv, nb = scores.shape
    kk = min(k, nb)
    idx = np.zeros((B, Hkv, kk), dtype=np.int64)
    for b in range(B):
        for kh in range(Hkv):
            idx[b, kh] = select_topk(scores[b, kh], k)
    return idx


# ------------------------------------------------------------------ O4
def block_tokens(blocks: Iterable[int], block: int, N: int) -> np.ndarray:
    """Token positions of the given blocks, in block order."""
    parts = [np.arange(j * block, min((j + 1) * block, N)) for j in blocks]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def attend_blocks(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
                  block: int, scale: Optional[float] = None,
                  count: Optional[np.ndarray] = None):
    """O4: exact attention of each query head over the tokens of its group's blocks.

    idx [B, Hkv, k] lists blocks (ascending; entries past count[b, kh] are
    ignored).  The recomputation uses the original q, K, V on the support
    only, as the oracle of "How Much Dense Attention is Necessary?" (§2.1)
    does after choosing its support.
    """
    B, Hq, D = q.shape
    Hkv, N = K.shape[1], K.shape[2]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    O = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for kh in range(Hkv):
            n = idx.shape[2] if count is None else int(count[b, kh])
            toks = block_tokens(idx[b, kh, :n], block, N)
            for h in range(kh * g, (kh + 1) * g):
                s = (K[b, kh, toks] @ q[b, h]) * sc
                O[b, h], lse[b, h] = _attend(s, V[b, kh, toks])
    return O, lse


def attend_tokens(q: np.ndarray, K: np.ndarray, V: np.ndarray,
                  lists: Sequence[Sequence[np.ndarray]],
                  scale: Optional[float] = None):
    """O4 over per-head token lists: lists[b][h] holds token positions."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    O = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            toks = np.asarray(lists[b][h], dtype=np.int64)
            s = (K[b, h // g, toks] @ q[b, h]) * sc
            O[b, h], lse[b, h] = _attend(s, V[b, h // g, toks])
    return O, lse


def lse_merge(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Exact merge of attention partials (o_i normalised, lse_i) over disjoint supports.

    With weights w_i = exp(lse_i - max lse), the union's output is
    sum_i w_i o_i / sum_i w_i and its lse is max lse + log(sum_i w_i): the
    online-softmax merge that "Pulsar Attention" (Fase 2) uses to recover exact
    global attention from per-shard results.  Empty parts (lse = -inf) drop out.
    """
    live = [(o, l) for o, l in parts if l != NEG_INF]
    if not live:
        D = parts[0][0].shape[-1]
        return np.zeros(D), NEG_INF
    m = max(l for _, l in live)
    w = np.array([math.exp(l - m) for _, l in live])
    o = sum(wi * oi for wi, (oi, _) in zip(w, live)) / w.sum()
    return o, m + math.log(w.sum())


# ------------------------------------------------------------------ O5
def exact_scores(q: np.ndarray, K: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """s[b, h, t] = q_h . k_t * scale for every cached token (float64)."""
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    s = np.zeros((B, Hq, K.shape[2]))
    for b in range(B):
        for h in range(Hq):
            s[b, h] = (K[b, h // g] @ q[b, h]) * sc
    return s


def threshold_tau(q: np.ndarray, K: np.ndarray, percentile: float = 99.0,
                  scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """tau[b, h] = the given percentile of the exact scores of head (b, h).

    NumPy's default (linear interpolation) percentile, in float64; also
    returned rounded toward -inf to float32, which is what a float32 caller
    passes (it can only add keys, never drop one).
    """
    s = exact_scores(q, K, scale)
    tau64 = np.percentile(s, percentile, axis=-1)
    tau32 = tau64.astype(np.float32)
    over = tau32.astype(np.float64) > tau64
    tau32[over] = np.nextafter(tau32[over], np.float32(-np.inf))
    return tau64, tau32


def select_threshold(q: np.ndarray, K: np.ndarray, tau: np.ndarray,
                     scale: Optional[float] = None):
    """O5: every token whose exact score is >= tau[b, h], ascending, with scores.

    This is the half-space H(q, tau) of "Sparse Attention as a Range Searching
    Problem" (Metodologia §1) on the scaled dot product; returning every key
    inside it is what makes the selection free of false negatives.
    Returns (lists[b][h] -> int64 array, scores[b][h] -> float64 array).
    """
    s = exact_scores(q, K, scale)
    B, Hq, _ = s.shape
    lists = [[None] * Hq for _ in range(B)]
    vals = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            t = np.nonzero(s[b, h] >= tau[b, h])[0]
            lists[b][h] = t
            vals[b][h] = s[b, h, t]
    return lists, vals


# ------------------------------------------------------------------ O6
def prefill_pool_queries(Q: np.ndarray, block: int, g: int) -> np.ndarray:
    """Pooled query blocks: mean of Q over each block's tokens and the group's heads."""
    return sketch(Q, block, head_pool=g)


def prefill_select(Qbar: np.ndarray, Kbar: np.ndarray, k: int,
                   scale: Optional[float] = None, rows: Optional[Iterable[int]] = None):
    """O6: per (b, kv head, query block i) the kept key blocks, ascending.

    Block 0 (sink) and the diagonal block i are always kept; the remaining
    min(k - 2, i - 1) slots go to the earlier blocks j in [1, i-1] ranked by
    r_ij = Qbar_i . Kbar_j * scale (higher first, ties to the lower j).  One
    list is shared by all queries of the block and all heads of the group --
    the block-shared support granularity of "How Much Dense Attention is
    Necessary?" (§2.1) and the block-by-block selection of Block-Sparse
    prefill ("The Sparse Frontier", Contributi §2).
    Returns idx [B, Hkv, M, k] (unused slots -1) and count [B, Hkv, M].
    """
    if k < 2:
        raise ValueError("prefill keeps at least the sink and the diagonal block")
    B, Hkv, M, D = Qbar.shape
    sc = _default_scale(D, scale)
    idx = -np.ones((B, Hkv, M, k), dtype=np.int64)
    cnt = np.zeros((B, Hkv, M), dtype=np.int64)
    rows = range(M) if rows is None else rows
    for b in range(B):
        for kh in range(Hkv):
            for i in rows:
                if i == 0:
                    S = np.array([0])
                else:
                    cand = np.arange(1, i)
                    r = _rank_key((Kbar[b, kh, 1:i] @ Qbar[b, kh, i]) * sc)
                    top = cand[np.lexsort((cand, -r))][:min(k - 2, i - 1)]
                    S = np.sort(np.concatenate([[0, i], top]))
                idx[b, kh, i, :S.size] = S
                cnt[b, kh, i] = S.size
    return idx, cnt


# ------------------------------------------------------------------ O7
def prefill_attend_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray,
                        idx: np.ndarray, count: np.ndarray, block: int,
                        rows: Sequence[Tuple[int, int, int]],
                        scale: Optional[float] = None):
    """O7 for chosen rows (b, h, t): causal attention over the tokens of S(t // block).

    Keys after position t are masked; every other token of the listed blocks
    is used with the original Q, K, V.
    """
    D = Q.shape[-1]
    L = K.shape[2]
    g = Q.shape[1] // K.shape[1]
    sc = _default_scale(D, scale)
    O = np.zeros((len(rows), D))
    lse = np.zeros(len(rows))
    for r, (b, h, t) in enumerate(rows):
        kh, i = h // g, t // block
        blocks = idx[b, kh, i, :int(count[b, kh, i])]
        toks = block_tokens(blocks, block, L)
        toks = toks[toks <= t]
        s = (K[b, kh, toks] @ Q[b, h, t]) * sc
        O[r], lse[r] = _attend(s, V[b, kh, toks])
    return O, lse


def prefill_attend(Q, K, V, idx, count, block, scale=None):
    """O7 for every row (small sizes only): O [B, Hq, L, D], lse [B, Hq, L]."""
    B, Hq, L, D = Q.shape
    rows = [(b, h, t) for b in range(B) for h in range(Hq) for t in range(L)]
    O, lse = prefill_attend_rows(Q, K, V, idx, count, block, rows, scale)
    return O.reshape(B, Hq, L, D), lse.reshape(B, Hq, L)


# ------------------------------------------------------------------ O8
def mass_oracle(Q: np.ndarray, K: np.ndarray, block: int, k_free: int = 8,
                scale: Optional[float] = None,
                qblocks: Optional[Iterable[int]] = None):
    """O8: attention-mass block ranking (recall reference for prefill selection).

    For query block i of kv head kh: run dense causal softmax for every row t of
    the block and every head of the group, sum each row's probability over the
    tokens of key block j, and average over the rows and heads.  The k_free
    earlier blocks j in [1, i-1] with the largest mass (ties to lower j) form
    S_mass(i).  This is the attention-mass top-k oracle of "How Much Dense
    Attention is Necessary?" (§2.1) at block granularity, with the head average
    of its token-importance distribution and a block-shared support.
    Returns {(b, kh, i): (mass [nb], S_mass ascending)}.
    """
    B, Hq, L, D = Q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    nb = -(-L // block)
    sc = _default_scale(D, scale)
    qblocks = range(nb) if qblocks is None else qblocks
    out = {}
    for b in range(B):
        for kh in range(Hkv):
            for i in qblocks:
                lo, hi = i * block, min((i + 1) * block, L)
                mass = np.zeros(nb)
                nrows = 0
                for h in range(kh * g, (kh + 1) * g):
                    S = (Q[b, h, lo:hi] @ K[b, kh, :hi].T) * sc      # [rows, hi]
                    t = np.arange(lo, hi)[:, None]
                    u = np.arange(hi)[None, :]
                    S = np.where(u <= t, S, NEG_INF)
                    P = np.exp(S - S.max(axis=1, keepdims=True))
                    P /= P.sum(axis=1, keepdims=True)
                    for j in range(i + 1):
                        mass[j] += P[:, j * block:min((j + 1) * block, hi)].sum()
                    nrows += hi - lo
                mass /= nrows
                if i >= 2:
                    cand = np.arange(1, i)
                    top = cand[np.lexsort((cand, -mass[1:i]))][:min(k_free, i - 1)]
                    sel = np.sort(top)
                else:
                    sel = np.zeros(0, dtype=np.int64)
                out[(b, kh, i)] = (mass, sel)
    return out


# ------------------------------------------------------------------ whole step
def decode_step(q, K, V, block: int, k: int, scale: Optional[float] = None,
                sk: Optional[np.ndarray] = None):
    """Sketch -> scores -> top-k -> attention, all float64.  Returns a dict."""
    if sk is None:
        sk = sketch(K, block)
    sc = block_scores(q, sk, scale)
    idx = select_topk_all(sc, k)
    O, lse = attend_blocks(q, K, V, idx, block, scale)
    return {"sketch": sk, "scores": sc, "idx": idx, "O": O, "lse": lse}


# ------------------------------------------------------------------ O9
def window_tokens(N: int, sink: int, local: int) -> np.ndarray:
    """Ascending positions of the sink prefix [0, sink) and the local window
    [N - local, N), both clipped to the cache (their union when they meet)."""
    head = np.arange(min(max(sink, 0), N))
    tail = np.arange(max(N - max(local, 0), 0), N)
    return np.union1d(head, tail).astype(np.int64)


def pseudo_max(q: np.ndarray, K: np.ndarray, sink: int, local: int,
               scale: Optional[float] = None) -> np.ndarray:
    """O9a: m~[b, h], the largest exact score over the sink and local tokens.

    "Faster Than Flash" (Metodologia §2) estimates the row maximum of the
    scores from the initial (sink) tokens and the recent local context only,
    so no reduction over the whole cache is needed.  Reading taken: the
    estimate is the plain maximum of the exact scaled scores of those tokens.
    An empty window (sink = local = 0) has no estimate and is rejected.
    """
    N = K.shape[2]
    win = window_tokens(N, sink, local)
    if win.size == 0:
        raise ValueError("the sink and local windows are both empty")
    s = exact_scores(q, K, scale)
    return s[:, :, win].max(axis=-1)


def select_topdelta(q: np.ndarray, K: np.ndarray, sink: int, local: int, delta: float,
                    scale: Optional[float] = None):
    """O9: top-delta selection: keep token j when s_j >= m~ - delta.

    The criterion of "Faster Than Flash" (Metodologia §2): a token stays when
    its score is within delta of the pseudo-maximum m~ (O9a), i.e. when its
    unnormalised softmax weight exp(s_j) is at least exp(-delta) times that of
    the estimated peak.  delta >= 0 (the pages use 5 and 7); +inf keeps every
    token.  Reading taken: only this criterion decides; the sink and local
    tokens are not forced in beyond it (the token that attains m~ always
    passes, so the list is never empty).
    Returns (lists, vals, tau) with tau[b, h] = m~ - delta and lists/vals as
    select_threshold (O5) returns them.
    """
    if not delta >= 0:
        raise ValueError("delta must be >= 0")
    tau = pseudo_max(q, K, sink, local, scale) - float(delta)
    lists, vals = select_threshold(q, K, tau, scale)
    return lists, vals, tau


# ------------------------------------------------------------------ O10
def subspaces(D: int, S: int):
    """Channel ranges of the S contiguous subspaces of a D-dim key space."""
    if S < 1 or D % S:
        raise ValueError("S must divide D")
    w = D // S
    return [(s * w, (s + 1) * w) for s in range(S)]


def subspace_radius(K: np.ndarray, sk: np.ndarray, block: int, S: int) -> np.ndarray:
    """O10a: rho[b, h, j, s] = max over the tokens t of block j of ||k_t,s - c_j,s||.

    The bounding sphere of a cluster in one subspace ("Sparse Attention as a
    Range Searching Problem", Metodologia §2: centre and radius per cluster,
    one index per contiguous subspace).  Reading taken: the clusters are the
    contiguous token blocks and the centre is the block's sketch row c_j (O1);
    the radius is the exact largest distance of the block's keys from it.
    """
    B, H, N, D = K.shape
    nb = -(-N // block)
    out = np.zeros((B, H, nb, S))
    for j in range(nb):
        lo, hi = j * block, min((j + 1) * block, N)
        dev = K[:, :, lo:hi, :] - sk[:, :, j][:, :, None, :]
        for s, (c0, c1) in enumerate(subspaces(D, S)):
            out[:, :, j, s] = np.sqrt((dev[..., c0:c1] ** 2).sum(axis=-1)).max(axis=-1)
    return out


def block_upper_bound(q: np.ndarray, sk: np.ndarray, rad: np.ndarray,
                      scale: Optional[float] = None) -> np.ndarray:
    """O10b: ub[b, h, j] = scale * sum_s (q_s . c_j,s + ||q_s|| rho_j,s).

    For every key k in the block, q . k = sum_s q_s . c_s + q_s . (k_s - c_s),
    and Cauchy-Schwarz bounds each q_s . (k_s - c_s) by ||q_s|| rho_s, so ub is
    at least every exact score of the block: the sphere-versus-half-space test
    of the two-phase filter (same page, Metodologia §2) summed over the
    subspaces.  scale > 0 keeps the direction of the inequality.
    """
    B, Hq, D = q.shape
    Hkv, nb, S = sk.shape[1], sk.shape[2], rad.shape[3]
    g = Hq // Hkv
    sc = _default_scale(D, scale)
    out = np.zeros((B, Hq, nb))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for s, (c0, c1) in enumerate(subspaces(D, S)):
                qs = q[b, h, c0:c1]
                out[b, h] += sk[b, kh, :, c0:c1] @ qs + np.linalg.norm(qs) * rad[b, kh, :, s]
    return out * sc


def select_threshold_pruned(q: np.ndarray, K: np.ndarray, tau: np.ndarray, block: int,
                            S: int, scale: Optional[float] = None):
    """O10: the half-space selection (O5) with whole blocks pruned first.

    Phase one drops every block whose upper bound (O10b) is below tau[b, h];
    phase two checks the exact score of every key of the surviving blocks
    ("Sparse Attention as a Range Searching Problem", Metodologia §2, the
    two-phase filter; its zero-false-negative guarantee holds because the
    bound is rigorous).  The result equals select_threshold's.
    Returns (lists, vals, survivors) with survivors[b][h] the ascending kept
    block ids.
    """
    B, Hq, D = q.shape
    N = K.shape[2]
    sk = sketch(K, block)
    rad = subspace_radius(K, sk, block, S)
    ub = block_upper_bound(q, sk, rad, scale)
    s = exact_scores(q, K, scale)
    g = Hq // K.shape[1]
    lists = [[None] * Hq for _ in range(B)]
    vals = [[None] * Hq for _ in range(B)]
    surv = [[None] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            alive = np.nonzero(ub[b, h] >= tau[b, h])[0]
            toks = block_tokens(alive, block, N)
            keep = toks[s[b, h, toks] >= tau[b, h]]
            surv[b][h] = alive
            lists[b][h] = keep
            vals[b][h] = s[b, h, keep]
    return lists, vals, surv


# ------------------------------------------------------------------ O11
_THIRD32 = np.float32(1.0) / np.float32(3.0)


def lowbit_encode(K: np.ndarray, block: int):
    """O11a: 2-bit key thumbnails with 8-bit residuals.

    "Faster Than Flash" (Metodologia §1) splits the key cache into 2-bit
    quantised thumbnails, scanned to estimate scores, and 8-bit residuals
    that rebuild the keys close to their stored precision for the exact
    computation.  The pages fix no codec; reading taken (asymmetric per
    channel over each token block, which keeps outlier channels from
    flattening the others):
      lo, hi  = min and max of channel c over the block's tokens,
      step    = (hi - lo) * fl32(1/3)            (four levels lo + i*step),
      code    = [d >= step/2] + [d >= 1.5 step] + [d >= 2.5 step], d = k - lo,
      t       = fma(code, step, lo)              (the thumbnail value),
      rstep   = 2^(E - 8) with step = m 2^E, m in [0.5, 1)  (a power of two,
                so r / rstep and r8 * rstep are exact),
      r8      = clip(rint((k - t) / rstep), -127, 127).
    Every operation is one IEEE float32 operation, so the codes are a fixed
    function of the stored keys; fma is evaluated exactly in float64 and
    rounded once.  Keys must be finite.
    Returns codes uint8 [B, H, N, D] (0..3), resid int8 [B, H, N, D] and
    meta float32 [B, H, nb, 3, D] = (lo, step, rstep).
    """
    X = np.asarray(K, dtype=np.float64).astype(np.float32)
    B, H, N, D = X.shape
    nb = -(-N // block)
    codes = np.zeros((B, H, N, D), dtype=np.uint8)
    resid = np.zeros((B, H, N, D), dtype=np.int8)
    meta = np.zeros((B, H, nb, 3, D), dtype=np.float32)
    for j in range(nb):
        lo_t, hi_t = j * block, min((j + 1) * block, N)
        xb = X[:, :, lo_t:hi_t, :]
        lo = xb.min(axis=2)
        hi = xb.max(axis=2)
        step = (hi - lo) * _THIRD32
        d = xb - lo[:, :, None, :]
        s2 = step[:, :, None, :]
        code = ((d >= s2 * np.float32(0.5)).astype(np.uint8)
                + (d >= s2 * np.float32(1.5)).astype(np.uint8)
                + (d >= s2 * np.float32(2.5)).astype(np.uint8))
        t = (code.astype(np.float64) * s2.astype(np.float64)
             + lo[:, :, None, :].astype(np.float64)).astype(np.float32)
        E = np.frexp(step)[1]
        rstep = np.ldexp(np.float32(1.0), E - 8).astype(np.float32)
        r = xb - t
        r8 = np.clip(np.rint(r / rstep[:, :, None, :]), -127, 127).astype(np.int8)
        codes[:, :, lo_t:hi_t] = code
        resid[:, :, lo_t:hi_t] = r8
        meta[:, :, j, 0], meta[:, :, j, 1], meta[:, :, j, 2] = lo, step, rstep
    return codes, resid, meta


def lowbit_thumbnail(codes: np.ndarray, meta: np.ndarray, block: int) -> np.ndarray:
    """O11b: the thumbnail keys t = fma(code, step, lo), float32."""
    B, H, N, D = codes.shape
    tok_blk = np.arange(N) // block
    lo = meta[:, :, tok_blk, 0, :].astype(np.float64)
    step = meta[:, :, tok_blk, 1, :].astype(np.float64)
    return (codes.astype(np.float64) * step + lo).astype(np.float32)


def lowbit_reconstruct(codes: np.ndarray, resid: np.ndarray, meta: np.ndarray,
                       block: int) -> np.ndarray:
    """O11c: the refined keys k^ = t + r8 * rstep (one float32 rounding)."""
    N = codes.shape[2]
    t = lowbit_thumbnail(codes, meta, block)
    rstep = meta[:, :, np.arange(N) // block, 2, :]
    return (t + resid.astype(np.float32) * rstep).astype(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float64.

    The plain IEEE rule on the bit pattern: add half a bf16 unit minus one,
    plus the lowest kept bit (so exact halves go to the even neighbour), and
    drop the low 16 bits.  Finite values past the largest bf16 round to
    infinity, infinities stay, and a NaN stays a NaN (quiet, sign kept).
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    nan = np.isnan(f)
    r = np.where(nan, (u & 0xFFFF0000) | 0x00400000, r)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def select_topdelta_lowbit(q: np.ndarray, codes: np.ndarray, resid: np.ndarray,
                           meta: np.ndarray, block: int, sink: int, local: int,
                           delta: float, margin: float, scale: Optional[float] = None):
    """O11: top-delta block filter over the thumbnails, refined keys for the rest.

    The three stages of the fused kernel of "Faster Than Flash" (Metodologia
    §3): (1) the pseudo-maximum m~ over the sink and local tokens (O9a), here
    with the refined keys; (2) provisional scores of every token from the
    2-bit thumbnails, and a block is kept for a kv head when some head h of
    its group has a provisional score >= tau_h - margin, tau = m~ - delta;
    the blocks holding sink or local tokens are always kept (they set m~);
    (3) exact attention over the kept blocks with the refined keys (O4).
    Readings taken: the provisional score of token t is the plain thumbnail
    dot product scale * q . t_t, in float64, with t = fma(code, step, lo) the
    float32 thumbnail of the codec (O11b); the refined key is k^ rounded to
    bf16, the precision of the cache it stands for; `margin` (>= 0) widens
    the filter against the thumbnail error.
    Returns (idx, count, tau, bmax): idx [B, Hkv, nb] ascending block ids
    (count valid), tau [B, Hq], bmax [B, Hq, nb] the largest provisional
    score of each block.
    """
    B, Hq, D = q.shape
    _, Hkv, N, _ = codes.shape
    g = Hq // Hkv
    nb = -(-N // block)
    sc = _default_scale(D, scale)
    khat = bf16_round(lowbit_reconstruct(codes, resid, meta, block))
    thumb = lowbit_thumbnail(codes, meta, block).astype(np.float64)
    win = window_tokens(N, sink, local)
    if win.size == 0:
        raise ValueError("the sink and local windows are both empty")
    forced = np.unique(win // block)
    tau = np.zeros((B, Hq))
    bmax = np.full((B, Hq, nb), -np.inf)
    idx = np.full((B, Hkv, nb), -1, dtype=np.int64)
    count = np.zeros((B, Hkv), dtype=np.int64)
    for b in range(B):
        for kh in range(Hkv):
            keep = np.zeros(nb, dtype=bool)
            keep[forced] = True
            for h in range(kh * g, (kh + 1) * g):
                tau[b, h] = (khat[b, kh, win] @ q[b, h]).max() * sc - float(delta)
                prov = (thumb[b, kh] @ q[b, h]) * sc
                for j in range(nb):
                    bmax[b, h, j] = prov[j * block:min((j + 1) * block, N)].max()
                keep |= bmax[b, h] >= tau[b, h] - float(margin)
            sel = np.nonzero(keep)[0]
            idx[b, kh, :sel.size] = sel
            count[b, kh] = sel.size
    return idx, count, tau, bmax


def mass_oracle_rows(Q: np.ndarray, K: np.ndarray, block: int, k_free: int = 8,
                     scale: Optional[float] = None, rows: Optional[Iterable[int]] = None):
    """O8 with a per-query support (b_sel = 1): row t of kv head kh ranks the
    key blocks by its own attention mass, averaged over the group's heads,
    and keeps the k_free largest of blocks [1, i - 1], i = t // block (ties
    to the lower block); the sink block 0 and the row's own block are the
    forced ones, as in the block-shared rule.  "How Much Dense Attention is
    Necessary?" (§2.1) compares this per-query support with supports shared
    by b_sel consecutive queries.
    Returns {(b, kh, t): (mass [nb], S ascending)}.
    """
    B, Hq, L, D = Q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    nb = -(-L // block)
    sc = _default_scale(D, scale)
    rows = range(L) if rows is None else rows
    out = {}
    for b in range(B):
        for kh in range(Hkv):
            for t in rows:
                mass = np.zeros(nb)
                for h in range(kh * g, (kh + 1) * g):
                    s = (K[b, kh, :t + 1] @ Q[b, h, t]) * sc
                    p = np.exp(s - s.max())
                    p /= p.sum()
                    for j in range(t // block + 1):
                        mass[j] += p[j * block:min((j + 1) * block, t + 1)].sum()
                mass /= g
                i = t // block
                if i >= 2:
                    cand = np.arange(1, i)
                    sel = np.sort(cand[np.lexsort((cand, -mass[1:i]))][:min(k_free, i - 1)])
                else:
                    sel = np.zeros(0, dtype=np.int64)
                out[(b, kh, t)] = (mass, sel)
    return out
