"""CPU oracle for query-aware top-k block-sparse attention over a GQA KV cache.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 statement
of what the hot path computes.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the library and its Python
binding never do, and it shares no code with the HIP kernels (it imports
nothing from them, nor they from it).

Pages cited (by title, section):
  * "How Much Dense Attention is Necessary? Oracle-Guided Sparse Prefill for
    Full/GQA Layers in Hybrid Long-Context Models" -- technical summary §2.1
    (attention-mass top-k oracle: dense attention, head-averaged importance,
    top-k support, recompute on the support with the original Q, K, V;
    per-query vs block-shared support granularity).
  * "The Sparse Frontier: Sparse Attention Trade-offs in Transformer LLMs" --
    Metodologia §1 (block/page units, full-cache retention) and Contributi §2
    (Block-Sparse prefill selects block by block; Quest-style decode selects
    pages from the retained cache).
  * "Faster Than Flash: Exploiting Attention Sparsity for Efficient
    Long-Context Decoding" -- Metodologia §1 (scan a compact key summary, then
    fetch exact data for the chosen parts; 2-bit thumbnails with 8-bit
    residuals), §3 (pseudo-max, top-delta over thumbnails, refinement) and §2 (sink and local tokens
    dominate the attention distribution, so a pseudo-maximum from them sets
    the top-delta threshold m~ - delta).
  * "Pulsar Attention" -- Fase 1 (64-token attention-sink prefix) and Fase 2
    (online-softmax merge of per-shard partial attention is exact).
  * "Sparse Attention as a Range Searching Problem: Towards an
    Inference-Efficient Index for KV Cache" -- Metodologia §1 (the half-space
    H(q, tau) = {p : <q, p> >= tau}; every key inside it is returned, so the
    selection has no false negatives) and §2 (subspace decomposition, bounding
    spheres of clusters, the two-phase filter: prune by sphere, then check
    the survivors exactly).

Where the pages are silent or ambiguous, each function's docstring states the
reading it takes.

Parity status: every function is pinned by tests/test_oracle.py (``mass_oracle``
(O8) against per-row softmax from scipy and brute-force top-k, besides its
invariants).
"""
from .attention import (
    widen, dense, dense_causal_rows, sketch, block_scores, select_topk,
    select_topk_all, attend_blocks, attend_tokens, lse_merge,
    threshold_tau, select_threshold, prefill_pool_queries, prefill_select,
    prefill_attend_rows, prefill_attend, mass_oracle, decode_step,
    window_tokens, pseudo_max, select_topdelta, subspaces, subspace_radius,
    block_upper_bound, select_threshold_pruned, lowbit_encode, lowbit_thumbnail,
    lowbit_reconstruct, bf16_round, select_topdelta_lowbit, mass_oracle_rows,
)

__all__ = [
    "widen", "dense", "dense_causal_rows", "sketch", "block_scores",
    "select_topk", "select_topk_all", "attend_blocks", "attend_tokens",
    "lse_merge", "threshold_tau", "select_threshold", "prefill_pool_queries",
    "prefill_select", "prefill_attend_rows", "prefill_attend", "mass_oracle",
    "decode_step", "window_tokens", "pseudo_max", "select_topdelta", "subspaces",
    "subspace_radius", "block_upper_bound", "select_threshold_pruned", "lowbit_encode",
    "lowbit_thumbnail", "lowbit_reconstruct", "bf16_round", "select_topdelta_lowbit",
    "mass_oracle_rows",
]
