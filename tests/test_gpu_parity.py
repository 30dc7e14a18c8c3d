"""GPU parity of every entry point against the float64 oracle.

Sizes here finish on the CPU oracle in seconds and still span several tiles,
splits and ragged tails; tests/test_gpu_fullsize.py covers the full workloads.
Tolerances: selections as in tests/parity_util.py (1e-5 relative tie band);
outputs max-abs 2e-3 for bf16 inputs and 1e-5 for float32 inputs, compared in
the float32-output mode against the oracle evaluated on the GPU's own index
lists; the bf16-output mode must equal the round-to-nearest-even bf16 of the
float32-output mode bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.attention import block_tokens, exact_scores, widen
from tests.parity_util import (bf16_rne_of_f32, check_topk_row, lowbit_bmax_bound,
                                 lowbit_kept_band, max_abs, to_dev)
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import top_sparse_attention_mean_amd as sa  # noqa: E402  (fails loudly if not built)

OUT_TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    yield


def _decode_case(name, over, seed=None):
    wl = get_workload(name, **over)
    inp = make_inputs(wl, seed=seed)
    d = wl.dtype
    return wl, inp, widen(inp.Q, d), widen(inp.K, d), widen(inp.V, d)


DECODE_CASES = [
    ("tiny_decode_f32", {}),
    ("tiny_decode_f32", {"N": 4096 - 23}),                                   # ragged last block
    ("tiny_decode_f32", {"k": 64}),                                          # k = nb -> dense
    ("tiny_decode_f32", {"N": 50, "k": 8}),                                  # nb = 1
    ("gqa_decode_bf16", {"B": 2}),
    ("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 5000}),             # ragged
    ("gqa_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 2, "D": 64, "N": 3001}),    # g = 2, D = 64
    ("gqa_decode_bf16", {"B": 1, "Hq": 2, "Hkv": 2, "N": 4100, "k": 9, "needles": 5}),   # g = 1
    ("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 9000, "block": 128, "k": 12,
                         "needles": 8}),
    ("long_decode_bf16", {"N": 65536 + 100}),                                # g = 8
]


@pytest.mark.parametrize("name,over", DECODE_CASES)
def test_decode_pipeline_parity(name, over):
    wl, inp, q, K, V = _decode_case(name, over)
    dt = wl.dtype
    Qd, Kd, Vd = to_dev(inp.Q, dt), to_dev(inp.K, dt), to_dev(inp.V, dt)
    # a1 sketch
    sk = sa.sa_build_sketch(Kd, wl.block)
    sk_ref = oracle.sketch(K, wl.block)
    assert max_abs(sk.cpu().numpy(), sk_ref) <= 2e-6 * max(1.0, np.abs(sk_ref).max())
    # a2 + a3 scores and selection
    idx, cnt, score = sa.sa_select_topk(Qd, sk, wl.k, want_score=True)
    sc_ref = oracle.block_scores(q, sk_ref)
    assert max_abs(score.cpu().numpy(), sc_ref) <= 1e-5 * max(1e-3, np.abs(sc_ref).max())
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    nb = wl.nb
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            n = int(cnt_h[b, kh])
            assert n == min(wl.k, nb)
            assert np.all(idx_h[b, kh, n:] == -1)
            if wl.k >= nb:
                assert idx_h[b, kh, :n].tolist() == list(range(nb))
                continue
            check_topk_row(idx_h[b, kh, :n], sc_ref[b, kh], wl.k, [0, nb - 1],
                           np.arange(1, nb - 1), where=f"b{b} kh{kh}")
            assert set(inp.needles[b, kh].tolist()) <= set(idx_h[b, kh, :n].tolist())
    # a5 + a6 attention on the GPU's own lists, float32 and bf16 outputs
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx_h, wl.block, count=cnt_h)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= OUT_TOL[dt], err
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    O16, _ = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.bfloat16)
    bits = O16.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, bf16_rne_of_f32(O32.cpu().numpy()))
    if wl.k >= nb:  # keeping every block is dense attention
        Od, lsed = oracle.dense(q, K, V)
        assert max_abs(O32.cpu().numpy(), Od) <= OUT_TOL[dt]
    print(f"{name} {over}: max-abs O error {err:.2e}")


def test_decode_step_equals_separate_calls():
    wl, inp, q, K, V = _decode_case("gqa_decode_bf16", {"B": 2, "N": 8192 + 40})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk_full = sa.sa_build_sketch(Kd, wl.block)
    # stale sketch of the newest block, refreshed inside the step
    sk = sk_full.clone()
    sk[:, :, -1] = 0
    O, lse, idx, cnt = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                         update_block=wl.nb - 1, out_dtype=torch.float32)
    assert torch.equal(sk, sk_full)
    idx2, cnt2, _ = sa.sa_select_topk(Qd, sk_full, wl.k)
    O2, lse2 = sa.sa_sparse_decode(Qd, Kd, Vd, idx2, cnt2, block=wl.block, out_dtype=torch.float32)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    # the fused step splits the same blocks differently, which changes the
    # running maxima the probabilities are scaled by and so their rounding (P
    # keeps 16 significant bits as bf16 hi + lo): agreement to ~2^-16
    assert max_abs(O.cpu().numpy(), O2.cpu().numpy()) <= 1e-5
    assert max_abs(lse.cpu().numpy(), lse2.cpu().numpy()) <= 1e-5
    O3, lse3, idx3, cnt3 = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                             out_dtype=torch.float32)
    assert torch.equal(idx, idx3) and torch.equal(cnt, cnt3)
    assert torch.equal(O, O3) and torch.equal(lse, lse3)          # bitwise repeatable


F32_STEP_CASES = [
    {},
    {"N": 4096 - 23},                                  # ragged last block
    {"k": 64},                                         # k = nb: every block
    {"N": 50, "k": 8},                                 # nb = 1
    {"Hq": 8, "Hkv": 2, "D": 128, "N": 3000},          # g = 4, D = 128
    {"Hq": 6, "Hkv": 2, "N": 2500, "k": 11},           # g = 3
    {"N": 64 * 600, "k": 12},                          # nb = 600: the list from k_select_rows
]


@pytest.mark.parametrize("over", F32_STEP_CASES)
def test_decode_step_f32_equals_separate_calls(over):
    """The float32 step (its decode kernel selecting its own blocks up to 512
    blocks per row) against the separate selection and decode: the same lists
    and, the split of the blocks being the same, the same outputs bit for bit;
    sa_select_decode on the step's scores likewise."""
    wl, inp, q, K, V = _decode_case("tiny_decode_f32", over)
    Qd, Kd, Vd = to_dev(inp.Q, "f32"), to_dev(inp.K, "f32"), to_dev(inp.V, "f32")
    sk_full = sa.sa_build_sketch(Kd, wl.block)
    sk = sk_full.clone()
    sk[:, :, -1] = 0                                   # stale newest block, refreshed in the step
    score = torch.empty(wl.B, wl.Hkv, wl.nb, dtype=torch.float32, device="cuda")
    O, lse, idx, cnt = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                         update_block=wl.nb - 1, score=score,
                                         out_dtype=torch.float32)
    assert torch.equal(sk, sk_full)
    idx2, cnt2, _ = sa.sa_select_topk(Qd, sk_full, wl.k)
    O2, lse2 = sa.sa_sparse_decode(Qd, Kd, Vd, idx2, cnt2, block=wl.block, out_dtype=torch.float32)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
    O3, lse3, idx3, cnt3 = sa.sa_select_decode(Qd, Kd, Vd, score, wl.k, block=wl.block,
                                               out_dtype=torch.float32)
    assert torch.equal(idx3, idx) and torch.equal(cnt3, cnt)
    assert torch.equal(O3, O) and torch.equal(lse3, lse)
    # and against the oracle on the lists
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx.cpu().numpy(), wl.block,
                                          count=cnt.cpu().numpy())
    assert max_abs(O.cpu().numpy(), O_ref) <= OUT_TOL["f32"]
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4


@pytest.mark.parametrize("D,upd", [(128, 5), (128, -1), (64, 7)])
def test_decode_step_scores_and_paths(D, upd):
    """The decode step's scores equal the standalone selection's bit for bit
    (the refreshed block, anywhere in the row, to rounding), for D = 128 and
    D = 64, with the newest-block refresh anywhere in the row or skipped."""
    wl, inp, q, K, V = _decode_case("gqa_decode_bf16", {"B": 2, "Hq": 8, "Hkv": 2, "D": D,
                                                        "N": 6000})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk_full = sa.sa_build_sketch(Kd, wl.block)
    sk = sk_full.clone()
    if upd >= 0:
        sk[:, :, upd] = 0
    score = torch.empty(wl.B, wl.Hkv, wl.nb, dtype=torch.float32, device="cuda")
    O, lse, idx, cnt = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block, update_block=upd,
                                         score=score, out_dtype=torch.float32)
    assert torch.equal(sk, sk_full)
    idx2, cnt2, score2 = sa.sa_select_topk(Qd, sk_full, wl.k, want_score=True)
    sc, sc2 = score.cpu().numpy(), score2.cpu().numpy()
    if upd >= 0:
        # the rebuilt block is scored right from its new sketch row, summed in
        # another order than a sketch-row pass: equal up to float32 rounding
        assert max_abs(sc[:, :, upd], sc2[:, :, upd]) <= 1e-6 * max(1.0, np.abs(sc2).max())
        sc[:, :, upd] = sc2[:, :, upd] = 0
    np.testing.assert_array_equal(sc, sc2)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    O2, lse2 = sa.sa_sparse_decode(Qd, Kd, Vd, idx2, cnt2, block=wl.block, out_dtype=torch.float32)
    assert max_abs(O.cpu().numpy(), O2.cpu().numpy()) <= 1e-5
    assert max_abs(lse.cpu().numpy(), lse2.cpu().numpy()) <= 1e-5
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx.cpu().numpy(), wl.block, count=cnt.cpu().numpy())
    assert max_abs(O.cpu().numpy(), O_ref) <= OUT_TOL["bf16"]


def _scores_for(mode, nb, rng):
    if mode == "ties":
        return (np.arange(nb) % 7).astype(np.float32)
    if mode in ("rank_all", "direct"):
        return np.full(nb, 0.25, dtype=np.float32)
    s = rng.standard_normal(nb).astype(np.float32)
    s[rng.choice(nb, 3, replace=False)] = np.nan
    s[rng.choice(nb, 3, replace=False)] = -np.inf
    return s


# (mode, nb, k, flags, Hq, Hkv): "cand" and "ties" take the per-split slices
# of the candidate list; "rank_all" (slices over 64 entries) and "direct" (list
# over capacity) select the whole row in every split; k >= nb and k = forced
# skip the ranking.
SD_MODES = [
    ("cand", 700, 40, 3, 8, 2),
    ("ties", 900, 60, 1, 8, 2),
    ("rank_all", 300, 8, 3, 8, 2),
    ("direct", 1500, 16, 0, 8, 2),
    ("cand", 20, 30, 3, 4, 1),
    ("cand", 100, 2, 3, 4, 1),
    ("cand", 5000, 100, 3, 8, 1),
]


@pytest.mark.parametrize("mode,nb,k,flags,Hq,Hkv", SD_MODES)
def test_select_decode_selection_modes(mode, nb, k, flags, Hq, Hkv):
    """Every selection route of the selecting decode, twice on one workspace
    (the kept-block bitmaps must be clear again), against the oracle."""
    block, D = 64, 128
    N = nb * block - 13
    rng = np.random.default_rng(nb * 31 + k)
    q = bf16_rne_of_f32(rng.standard_normal((1, Hq, D)).astype(np.float32))
    K = bf16_rne_of_f32(rng.standard_normal((1, Hkv, N, D)).astype(np.float32))
    V = bf16_rne_of_f32(rng.standard_normal((1, Hkv, N, D)).astype(np.float32))
    Qd, Kd, Vd = to_dev(q, "bf16"), to_dev(K, "bf16"), to_dev(V, "bf16")
    qw, Kw, Vw = widen(q, "bf16"), widen(K, "bf16"), widen(V, "bf16")
    forced = ([0] if flags & sa.SA_FORCE_SINK else []) + \
             ([nb - 1] if flags & sa.SA_FORCE_LOCAL and nb > 1 else [])
    outs = []
    for rep in range(2):
        sc = np.stack([_scores_for(mode, nb, rng) for _ in range(Hkv)])[None]
        O, lse, idx, cnt = sa.sa_select_decode(Qd, Kd, Vd, to_dev(sc, "f32"), k, block=block,
                                               flags=flags, out_dtype=torch.float32)
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        for kh in range(Hkv):
            want = oracle.select_topk(sc[0, kh].astype(np.float64), k, forced)
            n = int(cnt_h[0, kh])
            assert n == want.size, f"{mode} rep {rep} kh {kh}: count {n}, want {want.size}"
            assert idx_h[0, kh, :n].tolist() == want.tolist(), f"{mode} rep {rep} kh {kh}"
            assert np.all(idx_h[0, kh, n:] == -1)
        O_ref, lse_ref = oracle.attend_blocks(qw, Kw, Vw, idx_h, block, count=cnt_h)
        assert max_abs(O.cpu().numpy(), O_ref) <= OUT_TOL["bf16"]
        assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
        outs.append((sc, O, idx))
    # same scores again: bitwise the same result
    O2, _, idx2, _ = sa.sa_select_decode(Qd, Kd, Vd, to_dev(outs[1][0], "f32"), k, block=block,
                                         flags=flags, out_dtype=torch.float32)
    assert torch.equal(idx2, outs[1][2]) and torch.equal(O2, outs[1][1])


def test_select_decode_matches_step_and_flags():
    wl, inp, q, K, V = _decode_case("gqa_decode_bf16", {"B": 2, "N": 8192 + 40})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    _, _, score = sa.sa_select_topk(Qd, sk, wl.k, want_score=True)
    O, lse, idx, cnt = sa.sa_select_decode(Qd, Kd, Vd, score, wl.k, block=wl.block,
                                           out_dtype=torch.float32)
    O2, lse2, idx2, cnt2 = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                             out_dtype=torch.float32)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
    # other forced-block choices, against the oracle
    sc_ref = oracle.block_scores(q, oracle.sketch(K, wl.block))
    nb = wl.nb
    for flags, forced in ((sa.SA_FORCE_SINK, [0]), (0, [])):
        O, lse, idx, cnt = sa.sa_select_decode(Qd, Kd, Vd, score, wl.k, block=wl.block,
                                               flags=flags, out_dtype=torch.float32)
        idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
        cand = np.array([j for j in range(nb) if j not in forced])
        for b in range(wl.B):
            for kh in range(wl.Hkv):
                n = int(cnt_h[b, kh])
                assert n == wl.k and np.all(idx_h[b, kh, n:] == -1)
                check_topk_row(idx_h[b, kh, :n], sc_ref[b, kh], wl.k, forced, cand,
                               where=f"flags {flags} b{b} kh{kh}")
        O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx_h, wl.block, count=cnt_h)
        assert max_abs(O.cpu().numpy(), O_ref) <= OUT_TOL["bf16"]
        assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4


def test_decode_step_long_rows():
    # 4500 blocks per row: the 32-keys-per-thread selection tier (4096 < nb <= 8192)
    wl, inp, q, K, V = _decode_case("long_decode_bf16", {"Hq": 8, "Hkv": 1, "N": 4500 * 64 - 7})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    O, lse, idx, cnt = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                         out_dtype=torch.float32)
    sc_ref = oracle.block_scores(q, oracle.sketch(K, wl.block))
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    nb = wl.nb
    assert int(cnt_h[0, 0]) == wl.k
    check_topk_row(idx_h[0, 0], sc_ref[0, 0], wl.k, [0, nb - 1], np.arange(1, nb - 1),
                   where="long row")
    assert set(inp.needles[0, 0].tolist()) <= set(idx_h[0, 0].tolist())
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx_h, wl.block, count=cnt_h)
    assert max_abs(O.cpu().numpy(), O_ref) <= OUT_TOL["bf16"]
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4


def test_decode_split_invariance_and_determinism():
    wl, inp, q, K, V = _decode_case("long_decode_bf16", {"N": 32768})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    idx, cnt, _ = sa.sa_select_topk(Qd, sk, wl.k)
    O1, l1 = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    O1b, l1b = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    assert torch.equal(O1, O1b) and torch.equal(l1, l1b)          # bitwise repeatable
    # a wider index buffer changes the number of splits; results agree to rounding
    for stride in (wl.k * 3, 1000):
        wide = torch.full((wl.B, wl.Hkv, stride), -1, dtype=torch.int32, device="cuda")
        wide[:, :, :wl.k] = idx
        O2, l2 = sa.sa_sparse_decode(Qd, Kd, Vd, wide, cnt, block=wl.block, out_dtype=torch.float32)
        assert max_abs(O1.cpu().numpy(), O2.cpu().numpy()) <= 2e-6
        assert max_abs(l1.cpu().numpy(), l2.cpu().numpy()) <= 2e-6
    # an empty selection gives O = 0 and lse = -inf
    zero = torch.zeros_like(cnt)
    O3, l3 = sa.sa_sparse_decode(Qd, Kd, Vd, idx, zero, block=wl.block, out_dtype=torch.float32)
    assert torch.all(O3 == 0) and torch.all(torch.isinf(l3)) and torch.all(l3 < 0)


def test_sketch_block_range_update():
    wl, inp, q, K, V = _decode_case("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 1000})
    Kd = to_dev(inp.K, "bf16")
    sk = torch.full((1, 2, wl.nb, wl.D), 7.0, device="cuda")
    sa.sa_build_sketch(Kd, wl.block, blk_begin=3, blk_end=5, out=sk)
    ref = oracle.sketch(K, wl.block)
    got = sk.cpu().numpy()
    assert np.all(got[:, :, :3] == 7.0) and np.all(got[:, :, 5:] == 7.0)
    assert max_abs(got[:, :, 3:5], ref[:, :, 3:5]) <= 1e-6


def test_select_nan_and_ties():
    """NaN scores rank last; equal scores resolve to the lower block index."""
    B, Hq, Hkv, D, nb = 1, 1, 1, 64, 40
    sk = torch.zeros(B, Hkv, nb, D, device="cuda")
    sk[0, 0, :, 0] = torch.tensor([float(j % 5) for j in range(nb)])
    sk[0, 0, 7, 0] = float("nan")
    sk[0, 0, 12, 0] = 100.0
    q = torch.zeros(B, Hq, D, device="cuda")
    q[0, 0, 0] = 1.0
    idx, cnt, score = sa.sa_select_topk(q, sk, 10, want_score=True)
    s = score.cpu().numpy()[0, 0].astype(np.float64)
    check_topk_row(idx.cpu().numpy()[0, 0], s, 10, [0, nb - 1], np.arange(1, nb - 1))
    got = idx.cpu().numpy()[0, 0].tolist()
    assert 12 in got and 7 not in got
    assert got == oracle.select_topk(s, 10).tolist()


THRESH_CASES = [
    ("threshold_decode_bf16", {"B": 2}),
    ("threshold_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 5000}),
    ("threshold_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 4, "D": 64, "N": 3000}),
    ("threshold_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "D": 64, "N": 4096, "dtype": "f32",
                               "outlier_channels": 0}),
    # long caches: several staging segments per compaction thread, then more
    # segments than the compaction keeps in LDS
    ("threshold_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "D": 64, "N": 300000, "needles": 8,
                               "percentile": 99.8}),
    ("threshold_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "D": 64, "N": 4099 * 128 - 51,
                               "needles": 8, "percentile": 99.9}),
]


def _eps_bound(q, K, wl):
    """A loose float32 rounding bound of each score (for the false-positive band)."""
    g = wl.Hq // wl.Hkv
    sc = 1.0 / math.sqrt(wl.D)
    A = np.stack([np.abs(K[:, h // g]) @ np.abs(q[:, h])[..., None] for h in range(wl.Hq)], 1)[..., 0]
    return 4.0 * (wl.D + 1) * 2.0 ** -23 * A * sc + 2.0 ** -18 * (1 + np.abs(exact_scores(q, K)))


@pytest.mark.parametrize("name,over", THRESH_CASES)
def test_threshold_parity(name, over):
    wl, inp, q, K, V = _decode_case(name, over)
    dt = wl.dtype
    Qd, Kd, Vd = to_dev(inp.Q, dt), to_dev(inp.K, dt), to_dev(inp.V, dt)
    tau64, tau32 = oracle.threshold_tau(q, K, wl.percentile)
    s = exact_scores(q, K)
    eps = _eps_bound(q, K, wl)
    cap = wl.cap
    idx, score, cnt = sa.sa_select_threshold(Qd, Kd, torch.from_numpy(tau32).cuda(), cap)
    idx_h, sc_h, cnt_h = idx.cpu().numpy(), score.cpu().numpy(), cnt.cpu().numpy()
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    extra = 0
    for b in range(wl.B):
        for h in range(wl.Hq):
            n = int(cnt_h[b, h])
            assert n <= cap
            got = idx_h[b, h, :n]
            assert np.all(idx_h[b, h, n:] == -1)
            assert np.all(np.diff(got) > 0)
            exact = np.nonzero(s[b, h] >= tau64[b, h])[0]
            missing = set(exact.tolist()) - set(got.tolist())
            assert not missing, f"false negatives at b{b} h{h}: {sorted(missing)[:5]}"
            ex = np.setdiff1d(got, exact)
            assert np.all(s[b, h, ex] >= tau64[b, h] - 2 * eps[b, h, ex])
            extra += ex.size
            assert max_abs(sc_h[b, h, :n], s[b, h, got]) <= 1e-4
            lists[b][h] = got
    # token-mode attention on the GPU's lists, with and without the stored scores
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    for use_scores in (True, False):
        O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS,
                                       score=score if use_scores else None,
                                       out_dtype=torch.float32)
        err = max_abs(O32.cpu().numpy(), O_ref)
        assert err <= OUT_TOL[dt], err
        assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    print(f"{name} {over}: extra keys {extra}, max-abs O error {err:.2e}")


def test_threshold_capacity_and_minus_inf():
    wl, inp, q, K, V = _decode_case("threshold_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "N": 3000})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    tau = torch.full((1, 4), -float("inf"), device="cuda")
    idx, score, cnt = sa.sa_select_threshold(Qd, Kd, tau, 3000)
    assert torch.all(cnt == 3000)
    O32, _ = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                 out_dtype=torch.float32)
    Od, _ = oracle.dense(q, K, V)
    assert max_abs(O32.cpu().numpy(), Od) <= 2e-3
    # capacity overflow: true count reported, first `cap` positions written
    tau64, tau32 = oracle.threshold_tau(q, K, 90.0)
    idx, score, cnt = sa.sa_select_threshold(Qd, Kd, torch.from_numpy(tau32).cuda(), 50)
    s = exact_scores(q, K)
    for h in range(4):
        n = int(cnt[0, h])
        assert n >= int((s[0, h] >= tau64[0, h]).sum()) > 50
        full, _, _ = sa.sa_select_threshold(Qd, Kd, torch.from_numpy(tau32).cuda(), 3000)
        assert torch.equal(idx[0, h], full[0, h, :50])


TOPDELTA_CASES = [
    ("topdelta_decode_bf16", {"B": 2, "N": 8192, "needles": 4}),                  # g = 4
    ("topdelta_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 1, "N": 5000, "needles": 3,  # g = 8, ragged
                              "delta": 7.0, "cap": 5000}),
    ("topdelta_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 4, "D": 64, "N": 3001, "needles": 2,
                              "sink": 16, "local": 100}),                          # g = 1, D = 64
    ("topdelta_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 2, "N": 2048, "needles": 2,  # g = 2
                              "sink": 0, "local": 1, "delta": 2.0, "cap": 2048}),
    ("topdelta_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "D": 64, "N": 4096 - 13, "dtype": "f32",
                              "outlier_channels": 0, "needles": 2, "cap": 4096}),
    ("topdelta_decode_bf16", {"B": 1, "Hq": 6, "Hkv": 1, "D": 128, "N": 3000, "dtype": "f32",
                              "needles": 2, "sink": 5, "local": 37, "cap": 3000}),  # f32 g = 6
    ("topdelta_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 100, "needles": 0,   # window = cache
                              "delta": 0.0, "cap": 100}),
    ("topdelta_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 7, "needles": 0,     # N < one tile
                              "sink": 2, "local": 2, "delta": 1.0, "cap": 16}),
]


def _check_topdelta(wl, q, K, idx_h, sc_h, cnt_h, tau_h, where=""):
    """Selection checks of one top-delta call against the oracle; returns the
    GPU lists and the number of extra (boundary) keys."""
    s = exact_scores(q, K)
    eps = _eps_bound(q, K, wl)
    _, _, tau_x = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
    win = oracle.window_tokens(wl.N, wl.sink, wl.local)
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    extra = 0
    for b in range(wl.B):
        for h in range(wl.Hq):
            # the threshold: never above the exact one beyond its own rounding,
            # below it by at most the window scores' error bounds
            t = float(tau_h[b, h])
            assert t <= tau_x[b, h] + 2.0 ** -21 * abs(tau_x[b, h]), (where, b, h)
            assert t >= tau_x[b, h] - 2 * eps[b, h, win].max() - 1e-6, (where, b, h)
            n = int(cnt_h[b, h])
            cap = idx_h.shape[-1]
            got = idx_h[b, h, :min(n, cap)]
            assert n <= cap, (where, b, h, n)
            assert np.all(idx_h[b, h, n:] == -1)
            assert np.all(np.diff(got) > 0)
            exact = np.nonzero(s[b, h] >= tau_x[b, h])[0]
            missing = set(exact.tolist()) - set(got.tolist())
            assert not missing, f"{where} false negatives at b{b} h{h}: {sorted(missing)[:5]}"
            ex = np.setdiff1d(got, exact)
            assert np.all(s[b, h, ex] >= t - 2 * eps[b, h, ex]), (where, b, h)
            extra += ex.size
            assert max_abs(sc_h[b, h, :n], s[b, h, got]) <= 1e-4 * max(1.0, np.abs(s[b, h]).max())
            lists[b][h] = got
    return lists, extra


@pytest.mark.parametrize("name,over", TOPDELTA_CASES)
def test_topdelta_parity(name, over):
    wl, inp, q, K, V = _decode_case(name, over)
    dt = wl.dtype
    Qd, Kd, Vd = to_dev(inp.Q, dt), to_dev(inp.K, dt), to_dev(inp.V, dt)
    idx, score, cnt, tau = sa.sa_select_topdelta(Qd, Kd, wl.sink, wl.local, wl.delta, wl.cap)
    lists, extra = _check_topdelta(wl, q, K, idx.cpu().numpy(), score.cpu().numpy(),
                                   cnt.cpu().numpy(), tau.cpu().numpy(), f"{name} {over}")
    # token-mode attention over the GPU's lists, with and without the stored scores
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    for use_scores in (True, False):
        O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS,
                                       score=score if use_scores else None,
                                       out_dtype=torch.float32)
        err = max_abs(O32.cpu().numpy(), O_ref)
        assert err <= OUT_TOL[dt], err
        assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    if extra == 0:
        # the same lists as the oracle's rule: the oracle's top-delta attention
        ol, _, _ = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
        O_x, _ = oracle.attend_tokens(q, K, V, ol)
        assert max_abs(O32.cpu().numpy(), O_x) <= OUT_TOL[dt]
    # bitwise repeatable
    idx2, score2, cnt2, tau2 = sa.sa_select_topdelta(Qd, Kd, wl.sink, wl.local, wl.delta, wl.cap)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2) and torch.equal(tau, tau2)
    kept = int(cnt.sum())
    print(f"{name} {over}: kept {kept} ({kept / (wl.B * wl.Hq * wl.N):.3%}), extra keys {extra}, "
          f"max-abs O error {err:.2e}")


def test_topdelta_infinite_delta_is_dense_and_capacity():
    wl, inp, q, K, V = _decode_case("topdelta_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1,
                                                             "N": 3000, "needles": 2})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    idx, score, cnt, tau = sa.sa_select_topdelta(Qd, Kd, 64, 64, math.inf, 3000)
    assert torch.all(cnt == 3000) and torch.all(torch.isinf(tau) & (tau < 0))
    O32, _ = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                 out_dtype=torch.float32)
    Od, _ = oracle.dense(q, K, V)
    assert max_abs(O32.cpu().numpy(), Od) <= 2e-3
    # capacity overflow: the true count is reported, the first `cap` written
    full, _, cfull, _ = sa.sa_select_topdelta(Qd, Kd, 64, 64, 7.0, 3000)
    small, _, csmall, _ = sa.sa_select_topdelta(Qd, Kd, 64, 64, 7.0, 40)
    assert torch.equal(cfull, csmall) and int(cfull.min()) > 40
    assert torch.equal(small, full[..., :40])
    # the caller's threshold output may be omitted (kept in the workspace)
    ws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_TOPDELTA, 1, 4, 1, 3000, 128, 0, 3000),
                     dtype=torch.uint8, device="cuda")
    i3 = torch.empty_like(full)
    s3 = torch.empty(1, 4, 3000, dtype=torch.float32, device="cuda")
    c3 = torch.empty_like(cfull)
    st = sa._select_topdelta(sa._ptr(Qd), sa._ptr(Kd), sa.SA_BF16, 1, 4, 1, 3000, 128, 64, 64, 7.0,
                             0.0, 3000, sa._ptr(i3), sa._ptr(s3), sa._ptr(c3), None, sa._ptr(ws),
                             ws.numel(), sa._stream())
    assert st == 0
    assert torch.equal(i3, full) and torch.equal(c3, cfull)


PRUNE_CASES = [
    ("clustered_threshold_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 8192, "needles": 4}, 1),
    ("clustered_threshold_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 8192 - 77, "needles": 4}, 4),
    ("clustered_threshold_bf16", {"B": 2, "Hq": 4, "Hkv": 4, "D": 64, "N": 3000, "needles": 2,
                                  "block": 32}, 2),
    ("clustered_threshold_bf16", {"B": 1, "Hq": 8, "Hkv": 1, "N": 5000, "needles": 3,
                                  "block": 128}, 16),
    ("clustered_threshold_bf16", {"B": 1, "Hq": 6, "Hkv": 1, "D": 64, "N": 4096 - 5,
                                  "dtype": "f32", "needles": 2}, 8),
    ("threshold_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 5000}, 1),      # nothing to prune
]


def _radius_check(K, sk_gpu, rad_gpu, block, S):
    """The GPU radius bounds every key's distance from the GPU's own centre and
    exceeds it by at most the stated rounding allowance."""
    B, H, N, D = K.shape
    sk = sk_gpu.astype(np.float64)
    W = D // S
    for j in range(-(-N // block)):
        lo, hi = j * block, min((j + 1) * block, N)
        dev = K[:, :, lo:hi, :] - sk[:, :, j][:, :, None, :]
        r = np.sqrt((dev.reshape(B, H, hi - lo, S, W) ** 2).sum(-1)).max(axis=2)   # [B, H, S]
        got = rad_gpu[:, :, j, :].astype(np.float64)
        assert np.all(got >= r), j
        assert np.all(got <= r * (1 + 1e-4) + 1e-30), j


@pytest.mark.parametrize("name,over,S", PRUNE_CASES)
def test_pruned_threshold_parity(name, over, S):
    wl, inp, q, K, V = _decode_case(name, over)
    dt, blk = wl.dtype, wl.block
    Qd, Kd, Vd = to_dev(inp.Q, dt), to_dev(inp.K, dt), to_dev(inp.V, dt)
    sk = sa.sa_build_sketch(Kd, blk)
    rad = sa.sa_build_radius(Kd, sk, blk, S)
    sk_h, rad_h = sk.cpu().numpy(), rad.cpu().numpy()
    _radius_check(K, sk_h, rad_h, blk, S)
    # a range rebuild (the decode refresh of the newest blocks) writes only its blocks
    part = torch.full_like(rad, -1.0)
    sa.sa_build_radius(Kd, sk, blk, S, blk_begin=wl.nb - 2, blk_end=wl.nb, out=part)
    assert torch.equal(part[:, :, wl.nb - 2:], rad[:, :, wl.nb - 2:])
    assert torch.all(part[:, :, :wl.nb - 2] == -1.0)
    # against the oracle's own spheres (float64 centres)
    sk_x = oracle.sketch(K, blk)
    rad_x = oracle.subspace_radius(K, sk_x, blk, S)
    assert max_abs(rad_h, rad_x) <= 1e-4 * max(1.0, np.abs(rad_x).max())
    tau64, tau32 = oracle.threshold_tau(q, K, wl.percentile)
    tau = torch.from_numpy(tau32).cuda()
    idx, score, cnt, live = sa.sa_select_threshold_pruned(Qd, Kd, sk, rad, tau, wl.cap, blk)
    idx_h, sc_h, cnt_h, live_h = (t.cpu().numpy() for t in (idx, score, cnt, live))
    # the unpruned scan on the same inputs: identical on every scanned segment
    idx0, score0, cnt0 = sa.sa_select_threshold(Qd, Kd, tau, wl.cap)
    idx0_h, sc0_h, cnt0_h = idx0.cpu().numpy(), score0.cpu().numpy(), cnt0.cpu().numpy()
    s = exact_scores(q, K)
    eps = _eps_bound(q, K, wl)
    ub = oracle.block_upper_bound(q, sk_x, rad_x)
    g, nseg, bps = wl.g, -(-wl.N // 128), 128 // blk
    # per-block scanned flags from the segment bytes
    bits = np.stack([(live_h >> i) & 1 for i in range(bps)], -1).reshape(wl.B, wl.Hkv, -1)
    assert np.all(live_h >> bps == 0)
    assert np.all(bits[:, :, wl.nb:] == 0)
    scanned = bits[:, :, :wl.nb] == 1
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            hs = range(kh * g, (kh + 1) * g)
            need = np.any([ub[b, h] >= tau64[b, h] for h in hs], axis=0)
            near = np.any([ub[b, h] >= tau64[b, h] - 1e-3 * (1 + abs(tau64[b, h])) for h in hs],
                          axis=0)
            assert np.all(scanned[b, kh][need]), (b, kh)
            assert np.all(near[scanned[b, kh]]), (b, kh)
        for h in range(wl.Hq):
            n = int(cnt_h[b, h])
            got = idx_h[b, h, :n]
            assert n <= wl.cap and np.all(idx_h[b, h, n:] == -1) and np.all(np.diff(got) > 0)
            exact = np.nonzero(s[b, h] >= tau64[b, h])[0]
            missing = set(exact.tolist()) - set(got.tolist())
            assert not missing, f"false negatives at b{b} h{h}: {sorted(missing)[:5]}"
            ex = np.setdiff1d(got, exact)
            assert np.all(s[b, h, ex] >= tau64[b, h] - 2 * eps[b, h, ex])
            ref = idx0_h[b, h, :cnt0_h[b, h]]
            on = scanned[b, h // g][ref // blk]
            assert np.array_equal(got, ref[on])
            np.testing.assert_array_equal(sc_h[b, h, :n], sc0_h[b, h, :cnt0_h[b, h]][on])
            lists[b][h] = got
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                   out_dtype=torch.float32)
    assert max_abs(O32.cpu().numpy(), O_ref) <= OUT_TOL[dt]
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    print(f"{name} {over} S={S}: {scanned.mean():.1%} of blocks scanned")


def _unpack_codes(packed):
    """[..., D/4] uint8 -> [..., D] codes: one little-endian 32-bit word per 16
    channels, channel 16 g + i at bit 8 (i % 4) + 2 (i / 4) of word g."""
    w = np.ascontiguousarray(packed).view(np.uint32)
    i = np.arange(16)
    shift = (8 * (i % 4) + 2 * (i // 4)).astype(np.uint32)
    return ((w[..., None] >> shift) & 3).astype(np.uint8).reshape(*packed.shape[:-1], -1)


LOWBIT_CODEC_CASES = [
    ("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 5000, "needles": 4}, 64),  # outliers
    ("tiny_decode_f32", {"N": 3001}, 37),                                           # fp32, odd block
    ("long_decode_bf16", {"Hq": 8, "Hkv": 1, "N": 4096 + 100}, 128),                 # drift
]


@pytest.mark.parametrize("name,over,block", LOWBIT_CODEC_CASES)
def test_lowbit_codec_parity(name, over, block):
    wl, inp, q, K, V = _decode_case(name, over)
    Kd = to_dev(inp.K, wl.dtype)
    codes, resid, meta = sa.sa_encode_keys(Kd, block)
    c_x, r_x, m_x = oracle.lowbit_encode(K, block)
    assert np.array_equal(_unpack_codes(codes.cpu().numpy()), c_x)
    assert np.array_equal(resid.cpu().numpy(), r_x)
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), m_x.view(np.uint32))
    # refined keys of a block list, bit for bit; other rows untouched
    nb = -(-wl.N // block)
    rng = np.random.default_rng(7)
    lst = np.full((wl.B, wl.Hkv, 6), -1, dtype=np.int32)
    cnt = np.zeros((wl.B, wl.Hkv), dtype=np.int32)
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            sel = np.sort(rng.choice(nb, size=min(5, nb), replace=False))
            sel[-1] = nb - 1                                      # the partial last block
            sel = np.unique(sel)
            lst[b, kh, :sel.size] = sel
            cnt[b, kh] = sel.size
    kh_d = sa.sa_decode_keys(codes, resid, meta, block, idx=torch.from_numpy(lst).cuda(),
                             count=torch.from_numpy(cnt).cuda())
    got = kh_d.float().cpu().numpy().astype(np.float64)
    want = oracle.bf16_round(oracle.lowbit_reconstruct(c_x, r_x, m_x, block))
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            rows = block_tokens(lst[b, kh, :cnt[b, kh]], block, wl.N)
            assert np.array_equal(got[b, kh, rows], want[b, kh, rows])
            other = np.setdiff1d(np.arange(wl.N), rows)
            assert not got[b, kh, other].any()
    # a re-encode of a block range leaves the rest as it was
    c2, r2, m2 = sa.sa_encode_keys(Kd, block, blk_begin=nb - 1, blk_end=nb)
    last = slice((nb - 1) * block, wl.N)
    assert np.array_equal(_unpack_codes(c2.cpu().numpy())[:, :, last], c_x[:, :, last])
    assert not c2.cpu().numpy()[:, :, :(nb - 1) * block].any()
    print(f"{name} {over} block {block}: max |k^ - k| {np.abs(want - K).max():.3g}")


LOWBIT_CASES = [
    ("lowbit_topdelta_bf16", {"B": 2, "N": 8192, "needles": 4, "cap": 128}),            # g = 4
    ("lowbit_topdelta_bf16", {"B": 1, "Hq": 8, "Hkv": 1, "N": 5000, "needles": 3,        # g = 8, ragged
                              "cap": 79, "margin": 0.0}),
    ("lowbit_topdelta_bf16", {"B": 1, "Hq": 4, "Hkv": 4, "D": 64, "N": 3001, "needles": 2,
                              "sink": 16, "local": 100, "cap": 47}),                     # g = 1, D = 64
    ("lowbit_topdelta_bf16", {"B": 1, "Hq": 4, "Hkv": 2, "N": 6000, "needles": 2, "block": 128,
                              "cap": 47, "delta": 7.0}),                                 # g = 2, block 128
    ("lowbit_topdelta_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 4096, "needles": 2, "cap": 8,
                              "margin": 3.0}),                                           # capacity overflow
]


@pytest.mark.parametrize("name,over", LOWBIT_CASES)
def test_lowbit_topdelta_parity(name, over):
    wl, inp, q, K, V = _decode_case(name, over)
    blk = wl.block
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    codes, resid, meta = sa.sa_encode_keys(Kd, blk)
    idx, cnt, tau, bmax, khat = sa.sa_select_topdelta_lowbit(
        Qd, codes, resid, meta, blk, wl.sink, wl.local, wl.delta, wl.margin, wl.cap,
        want_bmax=True)
    c_x, r_x, m_x = oracle.lowbit_encode(K, blk)
    i_x, n_x, t_x, b_x = oracle.select_topdelta_lowbit(q, c_x, r_x, m_x, blk, wl.sink, wl.local,
                                                       wl.delta, wl.margin)
    tau_h, bmax_h = tau.cpu().numpy(), bmax.cpu().numpy()
    tau_up = 1e-6 * (1 + np.abs(t_x))
    tau_down = 1e-3 * (1 + np.abs(t_x))
    assert np.all(tau_h <= t_x + tau_up)
    assert np.all(tau_h >= t_x - tau_down)
    # the int8 weights of the matrix-core scan move each block maximum by at
    # most the derived bound
    delta, _ = lowbit_bmax_bound(q, c_x, m_x, blk, 1.0 / math.sqrt(wl.D))
    dev = np.abs(bmax_h - b_x)
    assert np.all(dev <= delta), float((dev - delta).max())
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    g, nb = wl.g, wl.nb
    win = np.unique(oracle.window_tokens(wl.N, wl.sink, wl.local) // blk)
    khat_x = oracle.bf16_round(oracle.lowbit_reconstruct(c_x, r_x, m_x, blk))
    khat_h = khat.float().cpu().numpy().astype(np.float64)
    band = 0
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            n = int(cnt_h[b, kh])
            got = idx_h[b, kh, :min(n, wl.cap)]
            assert np.all(np.diff(got) > 0) and np.all(idx_h[b, kh, min(n, wl.cap):] == -1)
            hs = list(range(kh * g, (kh + 1) * g))
            must, may = lowbit_kept_band(b_x[b], t_x[b], delta[b], wl.margin, win, hs,
                                         tau_up[b], tau_down[b])
            full = np.nonzero(must)[0]
            assert n >= full.size and n <= int(may.sum())
            if n <= wl.cap:
                assert set(full.tolist()) <= set(got.tolist())
                assert np.all(may[got])
            band += int(may.sum() - must.sum())
            rows = block_tokens(got, blk, wl.N)
            assert np.array_equal(khat_h[b, kh, rows], khat_x[b, kh, rows])
    # refinement: attention over the kept blocks with the refined keys
    O32, lse = sa.sa_sparse_decode(Qd, khat, Vd, idx, cnt, block=blk, out_dtype=torch.float32)
    O_ref, lse_ref = oracle.attend_blocks(q, khat_x, V, idx_h, blk, count=np.minimum(cnt_h, wl.cap))
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= OUT_TOL["bf16"], err
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    # the fused decode (keys rebuilt inside the attention kernel): the same
    # selection, and bitwise the output of the two-pass path above
    O2, lse2, idx2, cnt2, tau2, bmax2 = sa.sa_decode_topdelta_lowbit(
        Qd, codes, resid, meta, Vd, blk, wl.sink, wl.local, wl.delta, wl.margin, wl.cap,
        out_dtype=torch.float32, want_bmax=True)
    assert torch.equal(idx2, idx) and torch.equal(cnt2, cnt)
    assert torch.equal(tau2, tau) and torch.equal(bmax2, bmax)
    assert torch.equal(O2, O32) and torch.equal(lse2, lse)
    print(f"{name} {over}: {cnt_h.mean() / nb:.1%} of blocks kept, {band} blocks in the bound's "
          f"band, max |bmax - oracle| {dev.max():.2e} (bound {delta.min():.2e}..{delta.max():.2e}), "
          f"max-abs O error {err:.2e}")


MASS_TOL = 5e-5

MASS_CASES = [
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 2, "N": 2048, "needles": 4}, None),
    ("sparse_prefill_bf16", {"Hq": 4, "Hkv": 1, "N": 128 * 130 + 37, "needles": 6},   # 2 chunks
     [0, 1, 2, 63, 127, 128, 129, 130]),
]


@pytest.mark.parametrize("name,over,qblocks", MASS_CASES)
def test_mass_select_parity(name, over, qblocks):
    wl, inp, Q, K, V = _decode_case(name, over)
    Qd, Kd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16")
    kf = 8
    idx, cnt, mass, rows = sa.sa_mass_select(Qd, Kd, kf, want_mass=True, per_row=True)
    idx_h, cnt_h, mass_h = idx.cpu().numpy(), cnt.cpu().numpy(), mass.cpu().numpy()
    M = wl.nb
    res = oracle.mass_oracle(Q, K, wl.block, k_free=kf, qblocks=qblocks)
    worst = 0.0
    for (b, kh, i), (m_x, sel_x) in res.items():
        m_g = mass_h[b, kh, i]
        worst = max(worst, float(np.abs(m_g[:M] - m_x).max()))
        # the masses are float32 sums of float32 probabilities: the rounding of
        # the float32 scores (128-term dot products), of their exponents and of
        # the sums, far inside the bar
        assert np.abs(m_g - m_x).max() <= MASS_TOL, (b, kh, i)
        n = int(cnt_h[b, kh, i])
        assert n == min(kf, max(i - 1, 0))
        got = idx_h[b, kh, i, :n]
        assert np.all(np.diff(got) > 0) and np.all(idx_h[b, kh, i, n:] == -1)
        if n:
            cand = np.arange(1, i)
            order = cand[np.lexsort((cand, -m_x[1:i]))]
            cut = m_x[order[n - 1]]
            band = 2 * MASS_TOL
            must = set(cand[m_x[1:i] > cut + band].tolist())
            may = set(cand[m_x[1:i] >= cut - band].tolist())
            assert must <= set(got.tolist()) <= may, (b, kh, i)
            if not (set(got.tolist()) ^ set(sel_x.tolist())):
                continue
            # a differing choice lies inside the tie band
            for j in set(got.tolist()) ^ set(sel_x.tolist()):
                assert abs(m_x[j] - cut) <= band, (b, kh, i, j)
    # per-query supports on sampled rows (block edges included)
    ri, rc, rm = (t.cpu().numpy() for t in rows)
    L, blk = wl.N, wl.block
    sample = sorted({0, 1, blk - 1, blk, 2 * blk + 5, 3 * blk - 1, L // 2, L - blk - 1, L - 1}
                    | set(np.random.default_rng(3).integers(0, L, 8).tolist()))
    rres = oracle.mass_oracle_rows(Q, K, blk, k_free=kf, rows=sample)
    rworst = 0.0
    for (b, kh, t), (m_x, sel_x) in rres.items():
        rworst = max(rworst, float(np.abs(rm[b, kh, t] - m_x).max()))
        assert np.abs(rm[b, kh, t] - m_x).max() <= MASS_TOL, (b, kh, t)
        i = t // blk
        n = int(rc[b, kh, t])
        assert n == min(kf, max(i - 1, 0))
        got = ri[b, kh, t, :n]
        assert np.all(np.diff(got) > 0) and np.all(ri[b, kh, t, n:] == -1)
        for j in set(got.tolist()) ^ set(sel_x.tolist()):
            cand = np.arange(1, i)
            cut = np.sort(m_x[1:i])[::-1][n - 1]
            assert abs(m_x[j] - cut) <= 2 * MASS_TOL, (b, kh, t, j)
    print(f"{name} {over}: max |mass - oracle| {worst:.2e} over {len(res)} query blocks, "
          f"per-row {rworst:.2e} over {len(rres)} rows")


PREFILL_CASES = [
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 2, "N": 2048, "needles": 4}),
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 1, "N": 2048 + 77, "needles": 4}),   # ragged
    ("sparse_prefill_bf16", {"Hq": 4, "Hkv": 4, "N": 1536, "needles": 2, "k": 4}),
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 2, "N": 1024 + 33, "D": 64, "block": 64, "needles": 4}),
    ("sparse_prefill_bf16", {"Hq": 4, "Hkv": 1, "N": 1024, "block": 64, "needles": 4}),
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 2, "N": 1536 + 5, "D": 64, "needles": 4}),
    # shorter than one block; one token past a block edge; an odd group (one
    # head per workgroup at D 128 with blocks of 128, two heads otherwise)
    ("sparse_prefill_bf16", {"Hq": 8, "Hkv": 2, "N": 37, "needles": 0}),
    ("sparse_prefill_bf16", {"Hq": 4, "Hkv": 2, "N": 129, "D": 64, "block": 64, "needles": 1}),
    ("sparse_prefill_bf16", {"Hq": 6, "Hkv": 2, "N": 300, "needles": 1}),
]


@pytest.mark.parametrize("name,over", PREFILL_CASES)
def test_prefill_parity(name, over):
    wl = get_workload(name, **over)
    inp = make_inputs(wl)
    Q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    M = wl.nb
    sk = sa.sa_build_sketch(Kd, wl.block)
    flags = sa.SA_FORCE_SINK | sa.SA_FORCE_LOCAL | sa.SA_CAUSAL
    idx, cnt, score = sa.sa_select_topk(Qd, sk, wl.k, flags=flags, q_block=wl.block, want_score=True)
    Qb, Kb = oracle.prefill_pool_queries(Q, wl.block, wl.g), oracle.sketch(K, wl.block)
    scale = 1.0 / math.sqrt(wl.D)
    idx_h, cnt_h, sc_h = idx.cpu().numpy(), cnt.cpu().numpy(), score.cpu().numpy()
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            for i in range(M):
                n = int(cnt_h[b, kh, i])
                assert n == min(i + 1, wl.k)
                assert np.all(idx_h[b, kh, i, n:] == -1)
                r = np.full(M, -np.inf)
                r[1:i] = (Kb[b, kh, 1:i] @ Qb[b, kh, i]) * scale
                if i >= 2:
                    assert max_abs(sc_h[b, kh, i, 1:i], r[1:i]) <= 1e-5 * max(1e-3, np.abs(r[1:i]).max())
                forced = [0] if i == 0 else [0, i]
                check_topk_row(idx_h[b, kh, i, :n], r, wl.k, forced, np.arange(1, max(i, 1)),
                               where=f"kh{kh} i{i}")
    for j, i in zip(inp.needles[0, 0], inp.partners[0, 0]):
        assert j in idx_h[0, 0, i, :cnt_h[0, 0, i]]
    O32, lse = sa.sa_sparse_prefill(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    O_ref, lse_ref = oracle.prefill_attend(Q, K, V, idx_h, cnt_h, wl.block)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3, err
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    O16, _ = sa.sa_sparse_prefill(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.bfloat16)
    bits = O16.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, bf16_rne_of_f32(O32.cpu().numpy()))
    print(f"{name} {over}: max-abs O error {err:.2e}")


@pytest.mark.parametrize("D,block", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_prefill_all_blocks_is_dense_causal(D, block):
    wl = get_workload("sparse_prefill_bf16", Hq=4, Hkv=2, N=1024, needles=2, D=D, block=block)
    inp = make_inputs(wl)
    Q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    M = wl.nb
    idx = torch.full((1, 2, M, M), -1, dtype=torch.int32)
    for i in range(M):
        idx[0, :, i, :i + 1] = torch.arange(i + 1, dtype=torch.int32)
    cnt = torch.arange(1, M + 1, dtype=torch.int32).repeat(1, 2, 1)
    O32, lse = sa.sa_sparse_prefill(Qd, Kd, Vd, idx.cuda(), cnt.cuda().contiguous(), block=block,
                                    out_dtype=torch.float32)
    rows = [(0, h, t) for h in range(4) for t in range(0, wl.N, 7)]
    Od, lsed = oracle.dense_causal_rows(Q, K, V, rows)
    got = O32.cpu().numpy()
    assert max_abs(np.stack([got[b, h, t] for b, h, t in rows]), Od) <= 2e-3
    gl = lse.cpu().numpy()
    assert max_abs(np.array([gl[b, h, t] for b, h, t in rows]), lsed) <= 1e-4


def test_prefill_peaked_rows_within_bf16_p_bound():
    """Rows whose attention sits on three keys of a middle block with values
    of +-4.  The bulk prefill kernel rounds each probability to bf16 before
    the value product (relative error <= 2^-8), so a row's output may move by
    at most 2^-8 * sum_t p_t |v_t| from the exact one (plus float32
    accumulation); that bound, not 2e-3, is what such rows are held to.  Rows
    of the first query block, and every row's lse, keep the tight bars."""
    from workloads import f32_to_bf16_bits
    wl = get_workload("sparse_prefill_bf16", Hq=4, Hkv=1, N=1024, needles=2, k=8)
    inp = make_inputs(wl)
    rng = np.random.default_rng(11)
    w = rng.standard_normal(wl.D)
    w /= np.linalg.norm(w)
    Qf = widen(inp.Q, "bf16").astype(np.float32) + (3.0 * w).astype(np.float32)
    Kf = widen(inp.K, "bf16").astype(np.float32)
    Vf = widen(inp.V, "bf16").astype(np.float32)
    hot = [256 + 5, 256 + 40, 256 + 90]
    for j, t in enumerate(hot):
        Kf[0, 0, t] = (40.0 * w).astype(np.float32) + 0.5 * Kf[0, 0, t]
        Vf[0, 0, t] = 4.0 * np.sign(rng.standard_normal(wl.D)).astype(np.float32)
    Qb, Kb, Vb = (f32_to_bf16_bits(x) for x in (Qf, Kf, Vf))
    Q, K, V = (widen(x, "bf16") for x in (Qb, Kb, Vb))
    Qd, Kd, Vd = to_dev(Qb, "bf16"), to_dev(Kb, "bf16"), to_dev(Vb, "bf16")
    M = wl.nb
    idx = torch.full((1, 1, M, M), -1, dtype=torch.int32)
    for i in range(M):
        idx[0, 0, i, :i + 1] = torch.arange(i + 1, dtype=torch.int32)
    cnt = torch.arange(1, M + 1, dtype=torch.int32).reshape(1, 1, M).contiguous()
    O, lse = sa.sa_sparse_prefill(Qd, Kd, Vd, idx.cuda(), cnt.cuda(), block=wl.block,
                                  out_dtype=torch.float32)
    rows = [(0, h, t) for h in range(wl.Hq) for t in range(0, wl.N, 3)]
    Od, lsed = oracle.dense_causal_rows(Q, K, V, rows)
    got, gl = O.cpu().numpy(), lse.cpu().numpy()
    scale = 1.0 / math.sqrt(wl.D)
    peaked, worst, ratio = 0, 0.0, 0.0
    for r, (b, h, t) in enumerate(rows):
        s_row = (K[b, 0, :t + 1] @ Q[b, h, t]) * scale
        p = np.exp(s_row - s_row.max())
        p /= p.sum()
        bound = 2.0 ** -8 * float(p @ np.abs(V[b, 0, :t + 1]).max(axis=1)) + 1e-5
        err = float(np.abs(got[b, h, t] - Od[r]).max())
        if t < wl.block:
            assert err <= 1e-4, (h, t, err)                # first block: P as bf16 hi + lo
        else:
            assert err <= bound, (h, t, err, bound)
            worst, ratio = max(worst, err), max(ratio, err / bound)
        peaked += t >= hot[-1] and p[hot].sum() > 0.9
        assert abs(gl[b, h, t] - lsed[r]) <= 1e-4
    assert peaked > 100                                    # the case is what it claims
    print(f"peaked prefill rows: {peaked}; max-abs O error {worst:.2e} "
          f"(at most {ratio:.2f} of the bf16-P bound)")


def test_decode_step_graph_replay_matches_eager():
    """The fused step captured in a HIP graph gives the eager result on every
    replay (its arrival counters and histograms reset themselves in-kernel)."""
    wl, inp, q, K, V = _decode_case("long_decode_bf16", {"N": 32768 + 64})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    ws = torch.zeros(sa.workspace_bytes(sa.SA_OP_DECODE_STEP, wl.B, wl.Hq, wl.Hkv, wl.N, wl.D,
                                        wl.block, wl.k), dtype=torch.uint8, device="cuda")
    idx = torch.empty(wl.B, wl.Hkv, wl.k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(wl.B, wl.Hkv, dtype=torch.int32, device="cuda")
    O = torch.empty(wl.B, wl.Hq, wl.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device="cuda")

    def step():
        sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block, update_block=wl.nb - 1,
                          idx=idx, count=cnt, O=O, lse=lse, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), O.clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        idx.zero_()
        O.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(O, ref[1]) and torch.equal(lse, ref[2]), rep
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(O, ref[1])


def test_selectors_graph_replay_match_eager():
    """Top-delta (with its token decode), the sphere-pruned threshold and the
    low-bit filter (with its block decode), captured together in one HIP graph,
    give the eager results on every replay, with eager calls between replays."""
    wl, inp, q, K, V = _decode_case("topdelta_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 4096,
                                                             "needles": 2, "cap": 1024})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    B, Hq, Hkv, D, N, blk = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N, wl.block
    dev = "cuda"
    z = lambda n: torch.zeros(n, dtype=torch.uint8, device=dev)  # noqa: E731
    # top-delta + token decode
    t_idx = torch.empty(B, Hq, wl.cap, dtype=torch.int32, device=dev)
    t_sc = torch.empty(B, Hq, wl.cap, dtype=torch.float32, device=dev)
    t_cnt = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    t_tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    t_O = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    t_ws = z(sa.workspace_bytes(sa.SA_OP_SELECT_TOPDELTA, B, Hq, Hkv, N, D, 0, wl.cap))
    t_dws = z(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, 0, wl.cap))
    # sphere-pruned threshold
    sk = sa.sa_build_sketch(Kd, blk)
    rad = sa.sa_build_radius(Kd, sk, blk, 2)
    tau = torch.full((B, Hq), 1.5, device=dev)
    p_idx = torch.empty(B, Hq, wl.cap, dtype=torch.int32, device=dev)
    p_sc = torch.empty(B, Hq, wl.cap, dtype=torch.float32, device=dev)
    p_cnt = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    p_live = torch.empty(B, Hkv, -(-N // 128), dtype=torch.uint8, device=dev)
    p_ws = z(sa.workspace_bytes(sa.SA_OP_SELECT_PRUNED, B, Hq, Hkv, N, D, blk, wl.cap))
    # low-bit filter + block decode
    codes, resid, meta = sa.sa_encode_keys(Kd, blk)
    nb = wl.nb
    l_idx = torch.empty(B, Hkv, nb, dtype=torch.int32, device=dev)
    l_cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    l_tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    khat = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device=dev)
    l_O = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    l_ws = z(sa.workspace_bytes(sa.SA_OP_SELECT_LOWBIT, B, Hq, Hkv, N, D, blk, nb))
    l_dws = z(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, blk, nb))

    def run():
        sa.sa_select_topdelta(Qd, Kd, wl.sink, wl.local, wl.delta, wl.cap, idx=t_idx, score=t_sc,
                              count=t_cnt, tau=t_tau, ws=t_ws)
        sa.sa_sparse_decode(Qd, Kd, Vd, t_idx, t_cnt, mode=sa.SA_IDX_TOKENS, score=t_sc, O=t_O,
                            out_dtype=torch.float32, ws=t_dws)
        sa.sa_select_threshold_pruned(Qd, Kd, sk, rad, tau, wl.cap, blk, idx=p_idx, score=p_sc,
                                      count=p_cnt, live=p_live, ws=p_ws)
        sa.sa_select_topdelta_lowbit(Qd, codes, resid, meta, blk, wl.sink, wl.local, wl.delta, 1.0,
                                     nb, khat=khat, idx=l_idx, count=l_cnt, tau=l_tau, ws=l_ws)
        sa.sa_sparse_decode(Qd, khat, Vd, l_idx, l_cnt, block=blk, O=l_O, out_dtype=torch.float32,
                            ws=l_dws)

    outs = (t_idx, t_sc, t_cnt, t_tau, t_O, p_idx, p_sc, p_cnt, p_live, l_idx, l_cnt, l_tau, l_O)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b_ in zip(outs, ref):
            assert torch.equal(a, b_), rep
        run()                                    # eager work between replays
        torch.cuda.synchronize()
        for a, b_ in zip(outs, ref):
            assert torch.equal(a, b_), rep
