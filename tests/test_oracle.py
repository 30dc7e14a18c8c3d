"""Pins for the float64 CPU oracle (runs without a GPU).

Each test ties an oracle function to something other than itself: a
hand-derived worked example (tests/golden), a closed form, a library routine
that computes the same mathematical object differently, or brute-force
enumeration on tiny inputs.  The cases are chosen so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails one of them.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from oracle import attention as A
from tests.conftest import read_golden
from workloads import (bf16_bits_to_f32, f32_to_bf16_bits, get_workload,
                       make_inputs)


def rnd(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------ O0 / O4
def test_golden_two_key_softmax():
    g = dict((k, v) for k, v in read_golden("softmax_two_keys.txt") if k not in ("k", "v"))
    rows = read_golden("softmax_two_keys.txt")
    K = np.array([[float(x) for x in v] for k, v in rows if k == "k"])
    V = np.array([[float(x) for x in v] for k, v in rows if k == "v"])
    q = np.array([float(x) for x in g["q"]])
    scale = float(g["scale"][0])
    O, lse = oracle.dense(q[None, None], K[None, None], V[None, None], scale)
    np.testing.assert_allclose(O[0, 0], [float(x) for x in g["o"]], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - float(g["lse"][0])) < 1e-14
    # the same support through the block path (one 2-token block)
    O2, lse2 = oracle.attend_blocks(q[None, None], K[None, None], V[None, None],
                                    np.array([[[0]]]), block=2, scale=scale)
    np.testing.assert_allclose(O2, O, atol=1e-15)


def test_dense_matches_scipy_softmax():
    B, Hq, Hkv, N, D = 2, 4, 2, 37, 8
    q, K, V = rnd(B, Hq, D, seed=1), rnd(B, Hkv, N, D, seed=2), rnd(B, Hkv, N, D, seed=3)
    O, lse = oracle.dense(q, K, V)
    for b in range(B):
        for h in range(Hq):
            s = K[b, h // 2] @ q[b, h] / math.sqrt(D)
            np.testing.assert_allclose(O[b, h], softmax(s) @ V[b, h // 2], rtol=1e-12, atol=1e-13)
            assert abs(lse[b, h] - logsumexp(s)) < 1e-12


def test_dense_closed_forms():
    B, Hq, Hkv, N, D = 1, 2, 1, 9, 4
    q, K = rnd(B, Hq, D, seed=4), rnd(B, Hkv, N, D, seed=5)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    Vc = np.broadcast_to(c, (B, Hkv, N, D)).copy()
    O, _ = oracle.dense(q, K, Vc)
    np.testing.assert_allclose(O[0, 0], c, atol=1e-14)           # constant V -> V
    Ksame = np.broadcast_to(K[:, :, :1], K.shape).copy()
    V = rnd(B, Hkv, N, D, seed=6)
    O, lse = oracle.dense(q, Ksame, V)
    np.testing.assert_allclose(O[0, 1], V[0, 0].mean(axis=0), atol=1e-14)   # equal keys -> mean
    s0 = K[0, 0, 0] @ q[0, 1] / 2.0
    assert abs(lse[0, 1] - (s0 + math.log(N))) < 1e-13
    O1, lse1 = oracle.dense(q, K[:, :, :1], V[:, :, :1])
    np.testing.assert_allclose(O1[0, 0], V[0, 0, 0], atol=0)      # one token -> its value
    assert abs(lse1[0, 0] - K[0, 0, 0] @ q[0, 0] / 2.0) < 1e-15


def test_attend_all_blocks_is_dense_and_split_merge_is_exact():
    B, Hq, Hkv, N, D, blk = 2, 8, 2, 200, 16, 32      # last block partial (8 tokens)
    q, K, V = rnd(B, Hq, D, seed=7), rnd(B, Hkv, N, D, seed=8), rnd(B, Hkv, N, D, seed=9)
    nb = -(-N // blk)
    idx = np.broadcast_to(np.arange(nb), (B, Hkv, nb)).copy()
    O, lse = oracle.attend_blocks(q, K, V, idx, blk)
    Od, lsed = oracle.dense(q, K, V)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, rtol=0, atol=1e-13)
    # any partition of the support merges back to the unsplit result
    parts = [[0, 3], [1], [2, 4, 5, 6]]
    for b in range(B):
        for h in range(Hq):
            pp = []
            for blocks in parts:
                o, l = oracle.attend_blocks(q[b:b + 1, h:h + 1], K[b:b + 1, h // 4:h // 4 + 1],
                                            V[b:b + 1, h // 4:h // 4 + 1],
                                            np.array([[blocks]]), blk)
                pp.append((o[0, 0], l[0, 0]))
            om, lm = oracle.lse_merge(pp + [(np.zeros(D), -math.inf)])
            np.testing.assert_allclose(om, Od[b, h], atol=1e-12)
            assert abs(lm - lsed[b, h]) < 1e-12


def test_attend_restricts_to_selected_tokens():
    """Dropping a block must equal dense attention on the remaining keys."""
    B, Hq, Hkv, N, D, blk = 1, 4, 1, 96, 8, 32
    q, K, V = rnd(B, Hq, D, seed=10), rnd(B, Hkv, N, D, seed=11), rnd(B, Hkv, N, D, seed=12)
    O, lse = oracle.attend_blocks(q, K, V, np.array([[[0, 2]]]), blk)
    keep = np.r_[0:32, 64:96]
    Od, lsed = oracle.dense(q, K[:, :, keep], V[:, :, keep])
    np.testing.assert_allclose(O, Od, atol=1e-14)
    np.testing.assert_allclose(lse, lsed, atol=1e-14)


# ------------------------------------------------------------------ O1 / O2
def test_sketch_closed_forms():
    B, H, D, blk = 1, 2, 3, 4
    N = 10                                   # blocks of 4, 4, 2 tokens
    X = np.zeros((B, H, N, D))
    for t in range(N):
        X[0, 0, t] = [t, 2 * t, -t]          # arithmetic progression
        X[0, 1, t] = [7.0, -1.0, 0.5]        # constant
    s = oracle.sketch(X, blk)
    assert s.shape == (1, 2, 3, 3)
    np.testing.assert_allclose(s[0, 0, :, 0], [1.5, 5.5, 8.5])    # midpoints; last block 8,9
    np.testing.assert_allclose(s[0, 0, :, 1], [3.0, 11.0, 17.0])
    np.testing.assert_allclose(s[0, 1], np.tile([7.0, -1.0, 0.5], (3, 1)))
    # head pooling: mean over both heads and the block's tokens
    sp = oracle.sketch(X, blk, head_pool=2)
    np.testing.assert_allclose(sp[0, 0, 2], ((X[0, 0, 8:10] + X[0, 1, 8:10]) / 2).mean(axis=0))
    # full blocks equal numpy's mean of the reshaped array
    Y = rnd(2, 3, 64, 5, seed=13)
    np.testing.assert_allclose(oracle.sketch(Y, 16), Y.reshape(2, 3, 4, 16, 5).mean(axis=3), atol=1e-15)


def test_block_scores_head_average_and_needle_boost():
    wl = get_workload("tiny_decode_f32")
    planted = make_inputs(wl)
    clean = make_inputs(wl.scaled(needle_gain=0.0))      # same draws, no needles
    q = A.widen(planted.Q, "f32")
    s_p = oracle.block_scores(q, oracle.sketch(A.widen(planted.K, "f32"), wl.block))
    s_c = oracle.block_scores(q, oracle.sketch(A.widen(clean.K, "f32"), wl.block))
    qbar = q[0].mean(axis=0)
    boost = 3.0 * np.linalg.norm(qbar) / math.sqrt(wl.D)
    diff = s_p[0, 0] - s_c[0, 0]
    needles = set(planted.needles[0, 0].tolist())
    for j in range(wl.nb):
        # keys are stored in fp32 after planting: allow that rounding only
        expect = boost if j in needles else 0.0
        assert abs(diff[j] - expect) < 2e-6, (j, diff[j], expect)
    # head average equals the mean query's score, and g = 1 is a plain dot
    sk = rnd(1, 1, 10, wl.D, seed=14)
    np.testing.assert_allclose(oracle.block_scores(q, sk)[0, 0], sk[0, 0] @ qbar / 8.0, atol=1e-14)
    np.testing.assert_allclose(oracle.block_scores(q[:, :1], sk)[0, 0], sk[0, 0] @ q[0, 0] / 8.0,
                               atol=1e-14)


# ------------------------------------------------------------------ O3
def test_golden_topk_pipeline_with_tie():
    g = {}
    sel = {}
    for k, v in read_golden("topk_tie_pipeline.txt"):
        if k == "select":
            sel[int(v[0])] = [int(x) for x in v[1:]]
        else:
            g[k] = v
    keys = np.array([float(x) for x in g["keys"]]).reshape(1, 1, -1, 1)
    blk = int(g["block"][0])
    sk = oracle.sketch(keys, blk)
    sc = oracle.block_scores(np.ones((1, 1, 1)), sk, scale=1.0)
    np.testing.assert_allclose(sc[0, 0], [float(x) for x in g["scores"]], atol=1e-15)
    assert sc[0, 0, 1] == sc[0, 0, 3]
    for k, want in sel.items():
        assert oracle.select_topk(sc[0, 0], k).tolist() == want


def _brute_topk(s, k, forced):
    """Maximum total score over all subsets of the free blocks, ties to the
    lexicographically smallest ascending list."""
    nb = len(s)
    F = sorted(set(forced))
    C = [j for j in range(nb) if j not in F]
    # NaN ranks below every real score (finite stand-in keeps sums comparable)
    finite = [x for x in s if not math.isnan(x)]
    low = (min(finite) if finite else 0.0) - 1000.0
    val = [low if math.isnan(x) else x for x in s]
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(C, k - len(F)):
        tot = sum(val[j] for j in sub)
        cand = sorted(F + list(sub))
        if tot > best_sum or (tot == best_sum and cand < best):
            best, best_sum = cand, tot
    return best


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(3, 12))
    # small integers force many exact ties; a few NaNs test the NaN reading
    s = rng.integers(-3, 4, size=nb).astype(float)
    if seed % 3 == 0:
        s[rng.integers(0, nb)] = np.nan
    if seed % 4 == 0:
        s[rng.integers(0, nb)] = -0.0
    for k in range(2, nb + 1):
        got = oracle.select_topk(s, k).tolist()
        want = list(range(nb)) if k >= nb else _brute_topk(s, k, [0, nb - 1])
        assert got == want, (s, k, got, want)


def test_topk_edge_cases():
    assert oracle.select_topk(np.array([5.0]), 1).tolist() == [0]          # nb = 1
    assert oracle.select_topk(np.array([1.0, 9.0, 9.0, 0.0]), 2).tolist() == [0, 3]
    assert oracle.select_topk(np.array([1.0, 2.0, 3.0]), 99).tolist() == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.select_topk(np.zeros(8), 1)
    # +0 and -0 are the same score: the lower index wins
    assert oracle.select_topk(np.array([0.0, 0.0, -0.0, 0.0, 1.0]), 3).tolist() == [0, 1, 4]


# ------------------------------------------------------------------ O5
def test_threshold_count_and_zero_false_negatives():
    wl = get_workload("threshold_decode_bf16", B=1)
    inp = make_inputs(wl)
    q, K, V = (A.widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    q = q[:, :8]                                   # two kv heads' worth of queries
    K, V = K[:, :2], V[:, :2]
    tau64, tau32 = oracle.threshold_tau(q, K, 99.0)
    assert np.all(tau32.astype(np.float64) <= tau64)
    assert np.all(np.nextafter(tau32, np.float32(np.inf)).astype(np.float64) > tau64)
    lists, vals = oracle.select_threshold(q, K, tau64)
    s = A.exact_scores(q, K)
    for h in range(8):
        # the linear-interpolated 99th percentile sits strictly between the
        # order statistics i0 = floor(0.99 (N - 1)) and i0 + 1 whenever those
        # two differ, so exactly N - i0 - 1 = 328 scores reach it
        srt = np.sort(s[0, h])
        i0 = int(math.floor(0.99 * (wl.N - 1)))
        assert srt[i0] < srt[i0 + 1]
        assert srt[i0] < tau64[0, h] < srt[i0 + 1]
        assert len(lists[0][h]) == wl.N - i0 - 1 == 328
        # zero false negatives against a plain loop over every token
        brute = [t for t in range(wl.N) if s[0, h, t] >= tau64[0, h]]
        assert lists[0][h].tolist() == brute
        np.testing.assert_array_equal(vals[0][h], s[0, h, brute])
    # tau = -inf keeps everything and reproduces dense attention
    allk, _ = oracle.select_threshold(q[:, :4, :], K[:, :1], np.full((1, 4), -np.inf))
    O, lse = oracle.attend_tokens(q[:, :4], K[:, :1], V[:, :1], allk)
    Od, lsed = oracle.dense(q[:, :4], K[:, :1], V[:, :1])
    np.testing.assert_allclose(O, Od, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


def test_threshold_brute_force_tiny():
    q, K = rnd(1, 2, 4, seed=20), rnd(1, 1, 50, 4, seed=21)
    tau = np.array([[0.3, -0.1]])
    lists, _ = oracle.select_threshold(q, K, tau)
    for h in range(2):
        want = [t for t in range(50)
                if sum(q[0, h, c] * K[0, 0, t, c] for c in range(4)) / 2.0 >= tau[0, h]]
        assert lists[0][h].tolist() == want
    # a key exactly on the boundary <q, k> * scale == tau is inside the half-space
    q1 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    K1 = np.zeros((1, 1, 3, 4))
    K1[0, 0, :, 0] = [0.25, 0.5, 0.75]           # scores 0.125, 0.25, 0.375 exactly
    lists, vals = oracle.select_threshold(q1, K1, np.array([[0.25]]))
    assert lists[0][0].tolist() == [1, 2] and vals[0][0].tolist() == [0.25, 0.375]


# ------------------------------------------------------------------ O6 / O7
def test_prefill_select_sizes_and_brute_force():
    rng = np.random.default_rng(30)
    M, D = 512, 16
    Qb, Kb = rng.standard_normal((1, 1, M, D)), rng.standard_normal((1, 1, M, D))
    idx, cnt = oracle.prefill_select(Qb, Kb, 10)
    assert cnt[0, 0].tolist() == [min(i + 1, 10) for i in range(M)]
    assert int(cnt.sum()) == 5075
    for i in (0, 1, 2, 5, 9, 10, 11, 100, 511):
        S = idx[0, 0, i, :cnt[0, 0, i]].tolist()
        assert S == sorted(S) and S[0] == 0 and S[-1] == i and len(set(S)) == len(S)
        if i >= 2:
            r = (Kb[0, 0, :i] @ Qb[0, 0, i]) / 4.0
            if i <= 12:   # the free part by subset enumeration
                want = _brute_topk(np.r_[r[:i], 0.0], min(10, i + 1), [0, i])
            else:         # ... or by Python's stable sort on (-r, j)
                free = sorted(range(1, i), key=lambda j: (-r[j], j))[:8]
                want = sorted([0, i] + free)
            assert S == want


def test_prefill_attend_widened_is_dense_causal():
    B, Hq, Hkv, L, D, blk = 1, 4, 2, 96, 8, 16
    Q, K, V = rnd(B, Hq, L, D, seed=31), rnd(B, Hkv, L, D, seed=32), rnd(B, Hkv, L, D, seed=33)
    M = L // blk
    Qb, Kb = oracle.prefill_pool_queries(Q, blk, 2), oracle.sketch(K, blk)
    idx, cnt = oracle.prefill_select(Qb, Kb, M + 1)      # every earlier block
    O, lse = oracle.prefill_attend(Q, K, V, idx, cnt, blk)
    rows = [(0, h, t) for h in range(Hq) for t in range(L)]
    Od, lsed = oracle.dense_causal_rows(Q, K, V, rows)
    np.testing.assert_allclose(O.reshape(-1, D), Od, atol=1e-13)
    np.testing.assert_allclose(lse.reshape(-1), lsed, atol=1e-13)
    np.testing.assert_array_equal(O[0, :, 0], V[0, [0, 0, 1, 1], 0])   # row 0 -> v_0
    # with k = 3 the rows of block 3 see blocks {0, best of 1..2, 3} only
    idx3, cnt3 = oracle.prefill_select(Qb, Kb, 3)
    S = idx3[0, 0, 3, :3]
    toks = np.concatenate([np.arange(j * blk, (j + 1) * blk) for j in S])
    t = 3 * blk + 5
    o, l = oracle.prefill_attend_rows(Q, K, V, idx3, cnt3, blk, [(0, 1, t)])
    keep = toks[toks <= t]
    Od2, lsed2 = oracle.dense(Q[:, 1:2, t], K[:, :1, keep], V[:, :1, keep])
    np.testing.assert_allclose(o[0], Od2[0, 0], atol=1e-14)


def test_prefill_pooling_head_group():
    Q = rnd(1, 4, 8, 3, seed=34)
    Qb = oracle.prefill_pool_queries(Q, 4, 2)
    np.testing.assert_allclose(Qb[0, 1, 1], Q[0, 2:4, 4:8].mean(axis=(0, 1)), atol=1e-15)


# ------------------------------------------------------------------ O8
def test_mass_oracle_invariants_and_identical_keys():
    B, Hq, Hkv, L, D, blk = 1, 2, 1, 64, 4, 8
    Q, K = rnd(B, Hq, L, D, seed=40), rnd(B, Hkv, L, D, seed=41)
    res = oracle.mass_oracle(Q, K, blk, k_free=3)
    for (b, kh, i), (mass, sel) in res.items():
        assert abs(mass[:i + 1].sum() - 1.0) < 1e-12 and np.all(mass[i + 1:] == 0)
        assert len(sel) == min(3, max(i - 1, 0))
    # identical keys: uniform causal attention, block j gets |j-block ∩ [0, t]| / (t+1)
    Ks = np.broadcast_to(K[:, :, :1], K.shape).copy()
    res = oracle.mass_oracle(Q, Ks, blk, k_free=3)
    for i in range(L // blk):
        rows = np.arange(i * blk, (i + 1) * blk)
        want = [np.mean([max(0, min(t + 1, (j + 1) * blk) - j * blk) / (t + 1) for t in rows])
                for j in range(i + 1)]
        mass, sel = res[(0, 0, i)]
        np.testing.assert_allclose(mass[:i + 1], want, atol=1e-13)
        # earlier full blocks tie exactly in mass -> lowest indices win
        assert sel.tolist() == list(range(1, 1 + min(3, max(i - 1, 0))))


@pytest.mark.parametrize("seed", range(3))
def test_mass_oracle_equals_row_softmax_by_scipy(seed):
    """Per-row causal softmax from scipy, summed per key block, averaged over
    the block's rows and the group's heads; top-k of [1, i-1] by brute force
    over all subsets (largest total mass, ties to the smallest indices)."""
    rng = np.random.default_rng(600 + seed)
    B, Hq, Hkv, blk = 1, 4, 2, 6
    L = int(rng.integers(20, 40))
    D = 8
    Q = rng.standard_normal((B, Hq, L, D)) * 1.5
    K = rng.standard_normal((B, Hkv, L, D))
    kf = 2
    res = oracle.mass_oracle(Q, K, blk, k_free=kf)
    nb = -(-L // blk)
    for kh in range(Hkv):
        for i in range(nb):
            rows = range(i * blk, min((i + 1) * blk, L))
            want = np.zeros(nb)
            n = 0
            for h in (2 * kh, 2 * kh + 1):
                for t in rows:
                    s = np.array([Q[0, h, t] @ K[0, kh, u] for u in range(t + 1)]) / math.sqrt(D)
                    p = softmax(s)
                    for u in range(t + 1):
                        want[u // blk] += p[u]
                    n += 1
            want /= n
            mass, sel = res[(0, kh, i)]
            np.testing.assert_allclose(mass, want, atol=1e-12)
            cand = list(range(1, i))
            best = None
            for sub in itertools.combinations(cand, min(kf, len(cand))):
                key = (-sum(want[j] for j in sub), list(sub))
                if best is None or key < best:
                    best = key
            assert sel.tolist() == (best[1] if best else [])


def test_mass_oracle_rows_by_scipy_and_block_average():
    """Per-row masses from scipy's softmax (head-averaged); their mean over a
    block's rows is the block-shared mass of mass_oracle."""
    rng = np.random.default_rng(610)
    B, Hq, Hkv, blk, L, D = 1, 4, 2, 5, 23, 8
    Q = rng.standard_normal((B, Hq, L, D)) * 1.5
    K = rng.standard_normal((B, Hkv, L, D))
    res = oracle.mass_oracle_rows(Q, K, blk, k_free=2)
    shared = oracle.mass_oracle(Q, K, blk, k_free=2)
    nb = -(-L // blk)
    for kh in range(Hkv):
        for t in range(L):
            want = np.zeros(nb)
            for h in (2 * kh, 2 * kh + 1):
                p = softmax(np.array([Q[0, h, t] @ K[0, kh, u] for u in range(t + 1)]) / math.sqrt(D))
                for u in range(t + 1):
                    want[u // blk] += p[u] / 2
            mass, sel = res[(0, kh, t)]
            np.testing.assert_allclose(mass, want, atol=1e-12)
            i = t // blk
            cand = list(range(1, i))
            top = sorted(sorted(cand, key=lambda j: (-want[j], j))[:min(2, len(cand))])
            assert sel.tolist() == top
        for i in range(nb):
            rows = range(i * blk, min((i + 1) * blk, L))
            avg = np.mean([res[(0, kh, t)][0] for t in rows], axis=0)
            np.testing.assert_allclose(avg, shared[(0, kh, i)][0], atol=1e-12)


# ------------------------------------------------------------------ needles
@pytest.mark.parametrize("name,over", [
    ("tiny_decode_f32", {}),
    ("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2}),
    ("long_decode_bf16", {"Hq": 16, "Hkv": 2, "N": 65536}),
])
def test_needle_recovery_decode(name, over):
    wl = get_workload(name, **over)
    inp = make_inputs(wl)
    q, K = A.widen(inp.Q, wl.dtype), A.widen(inp.K, wl.dtype)
    sc = oracle.block_scores(q, oracle.sketch(K, wl.block))
    idx = oracle.select_topk_all(sc, wl.k)
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            assert set(inp.needles[b, kh].tolist()) <= set(idx[b, kh].tolist())
            assert idx[b, kh, 0] == 0 and idx[b, kh, -1] == wl.nb - 1


def test_needle_recovery_prefill():
    wl = get_workload("sparse_prefill_bf16", Hq=8, Hkv=1, N=8192, needles=16)
    inp = make_inputs(wl)
    Q, K = A.widen(inp.Q, "bf16"), A.widen(inp.K, "bf16")
    idx, cnt = oracle.prefill_select(oracle.prefill_pool_queries(Q, wl.block, wl.g),
                                     oracle.sketch(K, wl.block), wl.k)
    for j, i in zip(inp.needles[0, 0], inp.partners[0, 0]):
        assert j in idx[0, 0, i, :cnt[0, 0, i]]


# ------------------------------------------------------------------ inputs
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(50).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]    # exact ties
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), A.widen(ours, "bf16").astype(np.float32))


def test_golden_bf16_round():
    """oracle.bf16_round against hand-derived bit patterns (ties to even,
    subnormals, overflow, signed zeros, infinities)."""
    rows = [v for k, v in read_golden("bf16_round.txt") if k == "case"]
    assert len(rows) >= 15
    src = np.array([int(a, 16) for a, _ in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(b, 16) << 16 for _, b in rows], dtype=np.uint32)
    got = A.bf16_round(src).astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(got, want)


def test_bf16_round_matches_torch():
    """oracle.bf16_round equals torch's float32 -> bfloat16 conversion on
    random values of every magnitude, on exact ties, on subnormals and on the
    non-finite values (a NaN stays a NaN)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(51)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2 ** 16, size=4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    sub = rng.integers(0, 0x00800000, size=4000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                        0xFFFFFFFF, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000000, 0x80000000],
                       dtype=np.uint32)
    x = np.concatenate([bits, ties, sub, sub | 0x80000000, special]).view(np.float32)
    got = A.bf16_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))


def test_inputs_are_seeded():
    a = make_inputs("tiny_decode_f32")
    b = make_inputs("tiny_decode_f32")
    np.testing.assert_array_equal(a.K, b.K)
    c = make_inputs("tiny_decode_f32", seed=7)
    assert not np.array_equal(a.K, c.K)


# ------------------------------------------------------------------ O9
def _golden_topdelta():
    keys, cases = None, []
    for k, v in read_golden("topdelta_window.txt"):
        if k == "keys":
            keys = np.array([float(x) for x in v])
        elif k == "case":
            sink, local, delta, _, tau, _, *kept = v
            cases.append((int(sink), int(local), float(delta), float(tau),
                          [int(x) for x in kept]))
    return keys, cases


def test_golden_topdelta_window():
    keys, cases = _golden_topdelta()
    assert len(cases) == 6
    q = np.ones((1, 1, 1))
    K = keys.reshape(1, 1, -1, 1)
    for sink, local, delta, tau, kept in cases:
        lists, vals, t = oracle.select_topdelta(q, K, sink, local, delta, scale=1.0)
        assert t[0, 0] == tau, (sink, local, delta)
        assert lists[0][0].tolist() == kept, (sink, local, delta)
        np.testing.assert_array_equal(vals[0][0], keys[kept])


def test_window_tokens_cases():
    assert A.window_tokens(10, 2, 3).tolist() == [0, 1, 7, 8, 9]
    assert A.window_tokens(10, 0, 1).tolist() == [9]
    assert A.window_tokens(10, 6, 6).tolist() == list(range(10))     # windows meet
    assert A.window_tokens(3, 64, 64).tolist() == [0, 1, 2]          # clipped
    assert A.window_tokens(10, 0, 0).size == 0
    with pytest.raises(ValueError):
        oracle.pseudo_max(np.ones((1, 1, 2)), np.ones((1, 1, 5, 2)), 0, 0)
    with pytest.raises(ValueError):
        oracle.select_topdelta(np.ones((1, 1, 2)), np.ones((1, 1, 5, 2)), 1, 1, -1.0)


@pytest.mark.parametrize("seed", range(4))
def test_topdelta_is_the_relative_weight_rule(seed):
    """Keep j iff its softmax weight is at least e^-delta times the largest
    weight in the sink/local window: the same rule stated on probabilities
    (scipy softmax), with the window maximum found by a plain loop."""
    rng = np.random.default_rng(300 + seed)
    B, Hq, Hkv, N, D = 2, 4, 2, 90, 8
    q = rng.standard_normal((B, Hq, D)) * 1.5
    K = rng.standard_normal((B, Hkv, N, D))
    sink, local, delta = [(4, 8, 5.0), (0, 16, 2.0), (16, 0, 3.5), (1, 1, 0.5)][seed]
    lists, _, tau = oracle.select_topdelta(q, K, sink, local, delta)
    win = [t for t in range(N) if t < sink or t >= N - local]
    for b in range(B):
        for h in range(Hq):
            s = np.array([sum(q[b, h, c] * K[b, h // 2, t, c] for c in range(D)) for t in range(N)])
            s /= math.sqrt(D)
            p = softmax(s)
            pw = max(p[t] for t in win)
            r = p / pw
            want = [t for t in range(N) if r[t] >= math.exp(-delta)]
            # no score sits within rounding of the boundary on these draws
            assert np.all(np.abs(np.log(r) + delta) > 1e-9)
            assert lists[b][h].tolist() == want
            assert abs(tau[b, h] - (max(s[t] for t in win) - delta)) < 1e-12


def test_topdelta_special_cases():
    rng = np.random.default_rng(310)
    B, Hq, Hkv, N, D = 1, 4, 1, 70, 8
    q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, N, D))
    V = rng.standard_normal((B, Hkv, N, D))
    s = np.einsum("hd,nd->hn", q[0], K[0, 0]) / math.sqrt(D)
    # window = whole cache: the pseudo-max is the true max; delta = 0 keeps
    # exactly the arg-max
    lists, _, tau = oracle.select_topdelta(q, K, N, 0, 0.0)
    for h in range(Hq):
        assert lists[0][h].tolist() == [int(np.argmax(s[h]))]
        assert abs(tau[0, h] - s[h].max()) < 1e-12
    # delta = +inf keeps every token: attention over the list is dense attention
    lists, _, _ = oracle.select_topdelta(q, K, 1, 1, math.inf)
    assert all(len(lists[0][h]) == N for h in range(Hq))
    O, lse = oracle.attend_tokens(q, K, V, lists)
    Od, lsed = oracle.dense(q, K, V)
    np.testing.assert_allclose(O, Od, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


@pytest.mark.parametrize("delta", [2.0, 5.0, 7.0])
def test_topdelta_dropped_mass_bound(delta):
    """Each dropped token weighs under e^-delta of the window peak, which is
    kept, so the dropped share of the softmax mass is below n_drop e^-delta and
    the attention output moves by at most twice that times max |v|."""
    rng = np.random.default_rng(320 + int(delta))
    B, Hq, Hkv, N, D = 1, 8, 2, 400, 16
    q = rng.standard_normal((B, Hq, D)) * 2.0
    K = rng.standard_normal((B, Hkv, N, D))
    V = rng.standard_normal((B, Hkv, N, D))
    lists, _, _ = oracle.select_topdelta(q, K, 8, 8, delta)
    O, _ = oracle.attend_tokens(q, K, V, lists)
    Od, _ = oracle.dense(q, K, V)
    for h in range(Hq):
        s = K[0, h // 4] @ q[0, h] / math.sqrt(D)
        p = softmax(s)
        n_drop = N - len(lists[0][h])
        f = 1.0 - p[lists[0][h]].sum()
        bound = n_drop * math.exp(-delta)
        assert f <= bound + 1e-15
        assert np.abs(O[0, h] - Od[0, h]).max() <= 2 * f * np.abs(V[0, h // 4]).max() + 1e-12
    assert any(len(lists[0][h]) < N for h in range(Hq))          # something was dropped


def test_topdelta_workload_concentrates_on_anchors():
    """The top-delta workload plants sink/local anchors and needles: on its
    draws the selection keeps a few percent of the cache, almost all of it
    planted tokens."""
    wl = get_workload("topdelta_decode_bf16", B=1, Hq=8, Hkv=2, N=8192, needles=4)
    inp = make_inputs(wl)
    q, K = A.widen(inp.Q, "bf16"), A.widen(inp.K, "bf16")
    lists, _, _ = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
    win = A.window_tokens(wl.N, wl.sink, wl.local)
    fr = [len(lists[0][h]) / wl.N for h in range(wl.Hq)]
    assert max(fr) < 0.08 and np.mean(fr) < 0.04
    for h in range(wl.Hq):
        need = np.concatenate([np.arange(j * 64, (j + 1) * 64) for j in inp.needles[0, h // wl.g]])
        assert np.isin(lists[0][h], np.union1d(win, need)).mean() > 0.95


# ------------------------------------------------------------------ O10
def test_golden_sphere_bound():
    g = {}
    for k, v in read_golden("sphere_bound.txt"):
        g.setdefault(k, []).append(v)
    K = np.array([float(x) for x in g["keys"][0]]).reshape(1, 1, 4, 4)
    q = np.array([float(x) for x in g["q"][0]]).reshape(1, 1, 4)
    sk = oracle.sketch(K, 2)
    np.testing.assert_array_equal(sk[0, 0, 0], [float(x) for x in g["centre0"][0]])
    for row in g["rho"]:
        S = int(row[0][1:])
        rad = oracle.subspace_radius(K, sk, 2, S)
        np.testing.assert_allclose(rad[0, 0, 0], [float(x) for x in row[1:]], atol=1e-15)
        assert np.all(rad[0, 0, 1] == 0)
    for row in g["ub"]:
        S = int(row[0][1:])
        rad = oracle.subspace_radius(K, sk, 2, S)
        ub = oracle.block_upper_bound(q, sk, rad, scale=1.0)
        np.testing.assert_allclose(ub[0, 0], [float(x) for x in row[1:]], atol=1e-14)
    # tau = 5.1: only the box bound (S = 4) prunes block 0; nothing is kept
    for S, alive in ((1, [0]), (2, [0]), (4, [])):
        lists, _, surv = oracle.select_threshold_pruned(q, K, np.array([[5.1]]), 2, S, scale=1.0)
        assert surv[0][0].tolist() == alive and lists[0][0].size == 0
    lists, _, surv = oracle.select_threshold_pruned(q, K, np.array([[0.0]]), 2, 2, scale=1.0)
    assert surv[0][0].tolist() == [0, 1] and lists[0][0].tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("seed", range(6))
def test_sphere_bound_dominates_every_score(seed):
    """ub_j >= every exact score of block j, brute force, for every S dividing D,
    partial last blocks and clustered or isotropic keys."""
    rng = np.random.default_rng(400 + seed)
    B, Hq, Hkv, D = 1, 4, 2, 16
    N = int(rng.integers(20, 90))
    block = int(rng.choice([4, 8, 16]))
    K = rng.standard_normal((B, Hkv, N, D))
    if seed % 2:
        nb = -(-N // block)
        mu = rng.standard_normal((B, Hkv, nb, D)) * 3
        K = np.repeat(mu, block, axis=2)[:, :, :N] + 0.1 * K
    q = rng.standard_normal((B, Hq, D))
    s = A.exact_scores(q, K)
    sk = oracle.sketch(K, block)
    for S in (1, 2, 4, 8, 16):
        rad = oracle.subspace_radius(K, sk, block, S)
        ub = oracle.block_upper_bound(q, sk, rad)
        for j in range(-(-N // block)):
            lo, hi = j * block, min((j + 1) * block, N)
            # the radius is a maximum over the block's keys, by a plain loop
            for sub, (c0, c1) in enumerate(oracle.subspaces(D, S)):
                r = max(math.sqrt(sum((K[0, 0, t, c] - sk[0, 0, j, c]) ** 2 for c in range(c0, c1)))
                        for t in range(lo, hi))
                assert abs(rad[0, 0, j, sub] - r) < 1e-12
            assert np.all(ub[:, :, j] >= s[:, :, lo:hi].max(axis=-1) - 1e-12)
    # the box bound (S = D) is sum_i |q_i| max_t |k_t,i - c_i|
    rad = oracle.subspace_radius(K, sk, block, D)
    box = (sk[0, 0] @ q[0, 0] + np.abs(q[0, 0]) @ rad[0, 0].T) / math.sqrt(D)
    np.testing.assert_allclose(oracle.block_upper_bound(q, sk, rad)[0, 0], box, atol=1e-12)


def test_sphere_bound_equality_case():
    """Keys c +- rho q/||q|| attain the S = 1 bound: ub = max score exactly."""
    D, rho = 8, 0.75
    q = np.random.default_rng(410).standard_normal((1, 1, D))
    u = q[0, 0] / np.linalg.norm(q[0, 0])
    c = np.random.default_rng(411).standard_normal(D)
    K = np.stack([c + rho * u, c - rho * u]).reshape(1, 1, 2, D)
    sk = oracle.sketch(K, 2)
    rad = oracle.subspace_radius(K, sk, 2, 1)
    assert abs(rad[0, 0, 0, 0] - rho) < 1e-12
    ub = oracle.block_upper_bound(q, sk, rad)
    assert abs(ub[0, 0, 0] - A.exact_scores(q, K).max()) < 1e-12


@pytest.mark.parametrize("S", [1, 4])
def test_pruned_selection_equals_threshold(S):
    """Zero false negatives: pruning changes nothing in the kept lists, on
    isotropic keys (nothing pruned) and on the clustered workload (most
    blocks pruned)."""
    for name, over in (("threshold_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 4096}),
                       ("clustered_threshold_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 8192})):
        wl = get_workload(name, **over)
        inp = make_inputs(wl)
        q, K = A.widen(inp.Q, "bf16"), A.widen(inp.K, "bf16")
        tau64, _ = oracle.threshold_tau(q, K, wl.percentile)
        want, wv = oracle.select_threshold(q, K, tau64)
        got, gv, surv = oracle.select_threshold_pruned(q, K, tau64, wl.block, S)
        alive = np.mean([len(surv[0][h]) / wl.nb for h in range(wl.Hq)])
        for h in range(wl.Hq):
            assert got[0][h].tolist() == want[0][h].tolist()
            np.testing.assert_array_equal(gv[0][h], wv[0][h])
        if name.startswith("clustered"):
            assert alive < 0.2          # the spheres prune most blocks
        else:
            assert alive > 0.95         # isotropic keys: nothing to prune


# ------------------------------------------------------------------ O11
def test_golden_lowbit_codec():
    g = {k: v for k, v in read_golden("lowbit_codec.txt")}
    K = np.array([float(x) for x in g["keys"]]).reshape(1, 1, 4, 2)
    codes, resid, meta = oracle.lowbit_encode(K, 4)
    assert codes[0, 0, :, 0].tolist() == [int(x) for x in g["codes0"]]
    assert codes[0, 0, :, 1].tolist() == [int(x) for x in g["codes1"]]
    assert resid[0, 0, :, 0].tolist() == [int(x) for x in g["resid0"]]
    assert resid[0, 0, :, 1].tolist() == [int(x) for x in g["resid1"]]
    for row, name in enumerate(("lo", "step", "rstep")):
        np.testing.assert_array_equal(meta[0, 0, 0, row], np.float32([float(x) for x in g[name]]))
    khat = oracle.lowbit_reconstruct(codes, resid, meta, 4)
    np.testing.assert_array_equal(khat[0, 0, :, 0], [0, 1, 2, 3])
    assert np.abs(khat - K).max() <= 0.0078125 / 2


@pytest.mark.parametrize("seed", range(4))
def test_lowbit_codes_are_nearest_levels_and_errors_bounded(seed):
    rng = np.random.default_rng(500 + seed)
    B, H, N, D, block = 1, 2, 200, 16, 64
    K = rng.standard_normal((B, H, N, D)).astype(np.float32) * np.float32(rng.uniform(0.1, 10))
    K[0, 0, :, 3] = 1.5                                   # a constant channel: step 0
    codes, resid, meta = oracle.lowbit_encode(K, block)
    t = oracle.lowbit_thumbnail(codes, meta, block).astype(np.float64)
    khat = oracle.lowbit_reconstruct(codes, resid, meta, block).astype(np.float64)
    blk = np.arange(N) // block
    lo, step, rstep = (meta[:, :, blk, i, :].astype(np.float64) for i in range(3))
    X = K.astype(np.float64)
    # nearest of the four levels, by a plain search (ties up), away from the
    # thresholds' own float32 rounding
    d = X - lo
    lev = np.stack([np.abs(d - i * step) for i in range(4)], -1)
    near = np.argmin(lev + 1e-12 * np.arange(4)[::-1], -1)   # ties to the upper level
    clear = np.min(np.abs(d[..., None] - (np.arange(3) + 0.5) * step[..., None]), -1) > 1e-5 * (step + 1e-30)
    assert np.array_equal(codes[clear], near[clear])
    assert np.all(np.abs(t - X) <= step / 2 * (1 + 1e-5) + 1e-6)
    # the refined key: within half a residual step unless the residual clipped,
    # within one step always
    unclipped = np.abs(resid) < 127
    tol = 2.0 ** -23 * np.abs(X)
    assert np.all(np.abs(khat - X)[unclipped] <= (rstep / 2 + tol)[unclipped])
    assert np.all(np.abs(khat - X) <= rstep + tol)
    # step 0: every threshold is 0 and d = 0 passes all three (any code decodes to lo)
    assert np.all(khat[0, 0, :, 3] == 1.5) and np.all(codes[0, 0, :, 3] == 3)
    # rstep is the power of two 2^(E - 8) of step
    m, E = np.frexp(meta[:, :, :, 1, :])
    np.testing.assert_array_equal(meta[:, :, :, 2, :], np.ldexp(np.float32(1), E - 8))


def test_lowbit_on_grid_keys_is_exact_top_delta():
    """Keys already on each block's four levels: thumbnails equal the keys,
    residuals vanish, and with margin 0 the filter keeps exactly the blocks
    holding a token at or above m~ - delta (plus the window's blocks).  Every
    value is dyadic, so the float64 provisional maxima are the exact ones."""
    rng = np.random.default_rng(520)
    B, Hq, Hkv, N, D, block = 1, 4, 2, 512, 8, 64
    nb = N // block
    lo = rng.integers(-8, 8, size=(B, Hkv, nb, D)) / 4.0
    s = 2.0 ** rng.integers(-3, 1, size=(B, Hkv, nb, D))
    lev = rng.integers(0, 4, size=(B, Hkv, N, D))
    lev[:, :, ::block, :] = 0                      # every level range spans 0..3
    lev[:, :, 1::block, :] = 3
    K = np.repeat(lo, block, 2) + lev * np.repeat(s, block, 2)
    q = rng.integers(-4, 5, size=(B, Hq, D)) / 2.0
    codes, resid, meta = oracle.lowbit_encode(K, block)
    assert np.array_equal(codes, lev) and not resid.any()
    np.testing.assert_array_equal(oracle.lowbit_reconstruct(codes, resid, meta, block), K)
    sink, local, delta = 8, 8, 3.0
    idx, cnt, tau, bmax = oracle.select_topdelta_lowbit(q, codes, resid, meta, block, sink, local,
                                                        delta, 0.0)
    _, _, tau_x = oracle.select_topdelta(q, K, sink, local, delta)
    np.testing.assert_allclose(tau, tau_x, atol=1e-12)
    sx = A.exact_scores(q, K)
    for kh in range(Hkv):
        want = {0, nb - 1}
        for h in range(kh * 2, kh * 2 + 2):
            want |= {t // block for t in np.nonzero(sx[0, h] >= tau_x[0, h])[0]}
            np.testing.assert_allclose(bmax[0, h], sx[0, h].reshape(nb, block).max(-1), atol=1e-12)
        assert idx[0, kh, :cnt[0, kh]].tolist() == sorted(want)
    # an infinite margin keeps every block
    _, cnt, _, _ = oracle.select_topdelta_lowbit(q, codes, resid, meta, block, sink, local, delta,
                                                 np.inf)
    assert np.all(cnt == nb)


def test_lowbit_provisional_scores_are_thumbnail_products():
    """Off the grid: each block's provisional maximum is the largest scaled
    product of the query with a thumbnail row, the thumbnail being the codec's
    level lo + code * step (rounded to float32, so within half a float32 unit
    of that level), checked by a plain loop over tokens and channels."""
    rng = np.random.default_rng(521)
    B, Hq, Hkv, N, D, block = 1, 2, 1, 150, 16, 64
    K = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D))
    codes, resid, meta = oracle.lowbit_encode(K, block)
    _, _, _, bmax = oracle.select_topdelta_lowbit(q, codes, resid, meta, block, 4, 4, 5.0, 0.0)
    sc = 1.0 / math.sqrt(D)
    for h in range(Hq):
        for j in range(-(-N // block)):
            best = -np.inf
            for t in range(j * block, min((j + 1) * block, N)):
                acc = 0.0
                for c in range(D):
                    lo_c, st_c = float(meta[0, 0, j, 0, c]), float(meta[0, 0, j, 1, c])
                    level = lo_c + int(codes[0, 0, t, c]) * st_c
                    acc += q[0, h, c] * level
                best = max(best, acc * sc)
            # float32 thumbnails: each level moves by at most half a unit
            slack = sc * sum(abs(q[0, h, c]) * 2.0 ** -24 *
                             (abs(float(meta[0, 0, j, 0, c])) + 3 * float(meta[0, 0, j, 1, c]))
                             for c in range(D)) + 1e-12
            assert abs(bmax[0, h, j] - best) <= slack, (h, j, bmax[0, h, j], best)


def test_lowbit_recall_on_the_top_delta_workload():
    """Selection-quality study on the anchored workload: the thumbnail filter
    keeps the blocks of (nearly) every token the exact top-delta rule keeps."""
    wl = get_workload("lowbit_topdelta_bf16", B=1, Hq=8, Hkv=2, N=8192, needles=4)
    inp = make_inputs(wl)
    q, K = A.widen(inp.Q, "bf16"), A.widen(inp.K, "bf16")
    codes, resid, meta = oracle.lowbit_encode(K, wl.block)
    lists, _, _ = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
    for margin, floor in ((0.0, 0.99), (wl.margin, 1.0)):
        idx, cnt, _, _ = oracle.select_topdelta_lowbit(q, codes, resid, meta, wl.block, wl.sink,
                                                       wl.local, wl.delta, margin)
        rec = []
        for h in range(wl.Hq):
            kept = set(idx[0, h // wl.g, :cnt[0, h // wl.g]].tolist())
            rec.append(np.mean([t // wl.block in kept for t in lists[0][h]]))
        assert np.mean(rec) >= floor, (margin, rec)
        assert cnt.mean() / wl.nb < 0.3
