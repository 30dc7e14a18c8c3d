"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Decode workloads are checked completely (every selection row,
every head); the 64K-token prefill checks every selection row and a sample of
output rows (every query block's first and last row for two heads, plus rows
spread over all heads), which the oracle computes one by one."""
import math
import time

import numpy as np
import pytest

import oracle
from oracle.attention import exact_scores, widen
from tests.parity_util import (check_topk_row, lowbit_bmax_bound, lowbit_kept_band, max_abs,
                                 to_dev)
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import top_sparse_attention_mean_amd as sa  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gqa_decode_bf16", "long_decode_bf16"])
def test_full_decode(name):
    t0 = time.time()
    wl = get_workload(name)
    inp = make_inputs(wl)
    q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    idx, cnt, score = sa.sa_select_topk(Qd, sk, wl.k, want_score=True)
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    # same step through the fused entry point, updating the newest block's sketch
    O2, lse2, idx2, cnt2 = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block,
                                             update_block=wl.nb - 1, out_dtype=torch.float32)
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    # the fused kernel splits the same blocks differently, which changes the
    # running maxima the probabilities are scaled by and so their rounding (P
    # keeps 16 significant bits as bf16 hi + lo): agreement to ~2^-16
    assert max_abs(O32.cpu().numpy(), O2.cpu().numpy()) <= 1e-5
    assert max_abs(lse.cpu().numpy(), lse2.cpu().numpy()) <= 1e-5
    sk_ref = oracle.sketch(K, wl.block)
    assert max_abs(sk.cpu().numpy(), sk_ref) <= 2e-6 * max(1.0, np.abs(sk_ref).max())
    sc_ref = oracle.block_scores(q, sk_ref)
    assert max_abs(score.cpu().numpy(), sc_ref) <= 1e-5 * np.abs(sc_ref).max()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    ties = 0
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            ties += check_topk_row(idx_h[b, kh], sc_ref[b, kh], wl.k, [0, wl.nb - 1],
                                   np.arange(1, wl.nb - 1), where=f"b{b} kh{kh}")
            assert set(inp.needles[b, kh].tolist()) <= set(idx_h[b, kh].tolist())
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx_h, wl.block, count=cnt_h)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    print(f"{name}: ties in band {ties}, max-abs O error {err:.2e}, {time.time() - t0:.1f}s")


def test_full_threshold():
    t0 = time.time()
    wl = get_workload("threshold_decode_bf16")
    inp = make_inputs(wl)
    q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    tau64, tau32 = oracle.threshold_tau(q, K, wl.percentile)
    idx, score, cnt = sa.sa_select_threshold(Qd, Kd, torch.from_numpy(tau32).cuda(), wl.cap)
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                   out_dtype=torch.float32)
    s = exact_scores(q, K)
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    extra = 0
    for b in range(wl.B):
        for h in range(wl.Hq):
            got = idx_h[b, h, :cnt_h[b, h]]
            exact = np.nonzero(s[b, h] >= tau64[b, h])[0]
            assert exact.size >= 328
            assert set(exact.tolist()) <= set(got.tolist()), f"false negative at b{b} h{h}"
            ex = np.setdiff1d(got, exact)
            assert np.all(s[b, h, ex] >= tau64[b, h] - 1e-3)
            extra += ex.size
            lists[b][h] = got
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    print(f"threshold: extra keys {extra} over {wl.B * wl.Hq} heads, max-abs O error {err:.2e}, "
          f"{time.time() - t0:.1f}s")


def test_full_topdelta():
    """The top-delta workload whole: the GPU's tau against the pseudo-max rule,
    zero false negatives against the exact rule, attention over the lists."""
    t0 = time.time()
    wl = get_workload("topdelta_decode_bf16")
    inp = make_inputs(wl)
    q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    idx, score, cnt, tau = sa.sa_select_topdelta(Qd, Kd, wl.sink, wl.local, wl.delta, wl.cap)
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                   out_dtype=torch.float32)
    lists_x, _, tau_x = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
    s = exact_scores(q, K)
    tau_h, idx_h, cnt_h = tau.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    assert np.all(tau_h <= tau_x + 1e-6 * (1 + np.abs(tau_x)))
    assert np.all(tau_h >= tau_x - 1e-3)
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    extra = 0
    for b in range(wl.B):
        for h in range(wl.Hq):
            n = int(cnt_h[b, h])
            assert n <= wl.cap
            got = idx_h[b, h, :n]
            assert set(lists_x[b][h].tolist()) <= set(got.tolist()), f"false negative at b{b} h{h}"
            ex = np.setdiff1d(got, lists_x[b][h])
            assert np.all(s[b, h, ex] >= tau_x[b, h] - 1e-3)
            extra += ex.size
            lists[b][h] = got
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    kept = int(cnt_h.sum())
    print(f"top-delta: kept {kept} ({kept / (wl.B * wl.Hq * wl.N):.2%}), extra keys {extra}, "
          f"max-abs O error {err:.2e}, {time.time() - t0:.1f}s")


def test_full_pruned_threshold():
    """The clustered threshold workload whole: bounding spheres built on the GPU,
    the pruned scan against the exact rule (zero false negatives) and against
    the unpruned scan on every scanned segment."""
    t0 = time.time()
    wl = get_workload("clustered_threshold_bf16")
    inp = make_inputs(wl)
    q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    tau64, tau32 = oracle.threshold_tau(q, K, wl.percentile)
    tau = torch.from_numpy(tau32).cuda()
    sk = sa.sa_build_sketch(Kd, wl.block)
    rad = sa.sa_build_radius(Kd, sk, wl.block, wl.subspaces)
    idx, score, cnt, live = sa.sa_select_threshold_pruned(Qd, Kd, sk, rad, tau, wl.cap, wl.block)
    idx0, _, cnt0 = sa.sa_select_threshold(Qd, Kd, tau, wl.cap)
    O32, lse = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, mode=sa.SA_IDX_TOKENS, score=score,
                                   out_dtype=torch.float32)
    s = exact_scores(q, K)
    idx_h, cnt_h, live_h = idx.cpu().numpy(), cnt.cpu().numpy(), live.cpu().numpy()
    idx0_h, cnt0_h = idx0.cpu().numpy(), cnt0.cpu().numpy()
    bps = 128 // wl.block
    scanned = np.stack([(live_h >> i) & 1 for i in range(bps)], -1).reshape(
        wl.B, wl.Hkv, -1)[:, :, :wl.nb] == 1
    lists = [[None] * wl.Hq for _ in range(wl.B)]
    for b in range(wl.B):
        for h in range(wl.Hq):
            got = idx_h[b, h, :cnt_h[b, h]]
            exact = np.nonzero(s[b, h] >= tau64[b, h])[0]
            assert set(exact.tolist()) <= set(got.tolist()), f"false negative at b{b} h{h}"
            assert np.all(s[b, h, np.setdiff1d(got, exact)] >= tau64[b, h] - 1e-3)
            ref = idx0_h[b, h, :cnt0_h[b, h]]
            assert np.array_equal(got, ref[scanned[b, h // wl.g][ref // wl.block]])
            lists[b][h] = got
    O_ref, lse_ref = oracle.attend_tokens(q, K, V, lists)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    frac = scanned.mean()
    assert frac < 0.3
    print(f"pruned threshold: {frac:.1%} of blocks scanned, max-abs O error {err:.2e}, "
          f"{time.time() - t0:.1f}s")


def test_full_lowbit_topdelta():
    """The low-bit top-delta workload whole: codec bit-exact, the thumbnail
    filter against the oracle's within its band, recall of the exact top-delta
    rule on the full-precision keys, attention over the refined keys."""
    t0 = time.time()
    wl = get_workload("lowbit_topdelta_bf16")
    inp = make_inputs(wl)
    q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    codes, resid, meta = sa.sa_encode_keys(Kd, wl.block)
    idx, cnt, tau, bmax, khat = sa.sa_select_topdelta_lowbit(
        Qd, codes, resid, meta, wl.block, wl.sink, wl.local, wl.delta, wl.margin, wl.cap,
        want_bmax=True)
    O32, lse = sa.sa_sparse_decode(Qd, khat, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    # the fused decode: the same lists and bitwise the same attention
    O2, lse2, idx2, cnt2, _, _ = sa.sa_decode_topdelta_lowbit(
        Qd, codes, resid, meta, Vd, wl.block, wl.sink, wl.local, wl.delta, wl.margin, wl.cap,
        out_dtype=torch.float32)
    assert torch.equal(idx2, idx) and torch.equal(cnt2, cnt)
    assert torch.equal(O2, O32) and torch.equal(lse2, lse)
    c_x, r_x, m_x = oracle.lowbit_encode(K, wl.block)
    assert np.array_equal(resid.cpu().numpy(), r_x)
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), m_x.view(np.uint32))
    i_x, n_x, t_x, b_x = oracle.select_topdelta_lowbit(q, c_x, r_x, m_x, wl.block, wl.sink,
                                                       wl.local, wl.delta, wl.margin)
    tau_h, bmax_h = tau.cpu().numpy(), bmax.cpu().numpy()
    tau_up = 1e-6 * (1 + np.abs(t_x))
    tau_down = 1e-3 * (1 + np.abs(t_x))
    assert np.all(tau_h <= t_x + tau_up) and np.all(tau_h >= t_x - tau_down)
    delta, _ = lowbit_bmax_bound(q, c_x, m_x, wl.block, 1.0 / math.sqrt(wl.D))
    dev = np.abs(bmax_h - b_x)
    assert np.all(dev <= delta), float((dev - delta).max())
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    assert cnt_h.max() <= wl.cap
    # the oracle's kept set outside the bound's band is the GPU's
    win = np.unique(oracle.window_tokens(wl.N, wl.sink, wl.local) // wl.block)
    agree = []
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            got = set(idx_h[b, kh, :cnt_h[b, kh]].tolist())
            hs = list(range(kh * wl.g, (kh + 1) * wl.g))
            must, may = lowbit_kept_band(b_x[b], t_x[b], delta[b], wl.margin, win, hs,
                                         tau_up[b], tau_down[b])
            assert set(np.nonzero(must)[0].tolist()) <= got
            assert all(may[j] for j in got)
            agree.append(got == set(i_x[b, kh, :n_x[b, kh]].tolist()))
    agree = float(np.mean(agree))
    # recall of the exact top-delta rule on the full-precision keys
    lists, _, _ = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
    rec = []
    for b in range(wl.B):
        for h in range(wl.Hq):
            kept = set(idx_h[b, h // wl.g, :cnt_h[b, h // wl.g]].tolist())
            rec.append(np.mean([t // wl.block in kept for t in lists[b][h]]))
    assert np.mean(rec) >= 0.999
    khat_x = oracle.bf16_round(oracle.lowbit_reconstruct(c_x, r_x, m_x, wl.block))
    O_ref, lse_ref = oracle.attend_blocks(q, khat_x, V, idx_h, wl.block, count=cnt_h)
    err = max_abs(O32.cpu().numpy(), O_ref)
    assert err <= 2e-3
    print(f"low-bit top-delta: {cnt_h.mean() / wl.nb:.1%} of blocks kept, recall "
          f"{np.mean(rec):.4f}, lists equal to the oracle's on {agree:.0%} of heads, max-abs O "
          f"error {err:.2e}, {time.time() - t0:.1f}s")


def test_full_prefill():
    t0 = time.time()
    wl = get_workload("sparse_prefill_bf16")
    inp = make_inputs(wl)
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    flags = sa.SA_FORCE_SINK | sa.SA_FORCE_LOCAL | sa.SA_CAUSAL
    idx, cnt, _ = sa.sa_select_topk(Qd, sk, wl.k, flags=flags, q_block=wl.block)
    O32, lse = sa.sa_sparse_prefill(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Q, K, V = (widen(x, "bf16") for x in (inp.Q, inp.K, inp.V))
    Qb, Kb = oracle.prefill_pool_queries(Q, wl.block, wl.g), oracle.sketch(K, wl.block)
    scale = 1.0 / math.sqrt(wl.D)
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    M = wl.nb
    assert int(cnt_h.sum()) == wl.Hkv * 5075
    for kh in range(wl.Hkv):
        r_all = Kb[0, kh] @ Qb[0, kh].T * scale          # r_all[j, i]
        for i in range(M):
            r = np.full(M, -np.inf)
            r[1:i] = r_all[1:i, i]
            forced = [0] if i == 0 else [0, i]
            check_topk_row(idx_h[0, kh, i, :cnt_h[0, kh, i]], r, wl.k, forced,
                           np.arange(1, max(i, 1)), where=f"kh{kh} i{i}")
        for j, i in zip(inp.needles[0, kh], inp.partners[0, kh]):
            assert j in idx_h[0, kh, i, :cnt_h[0, kh, i]]
    rng = np.random.default_rng(0)
    rows = [(0, h, i * wl.block + o) for h in (0, 31) for i in range(M) for o in (0, wl.block - 1)]
    rows += [(0, int(h), int(t)) for h, t in zip(rng.integers(0, wl.Hq, 256), rng.integers(0, wl.N, 256))]
    rows += [(0, 5, t) for t in range(0, 130)]
    O_ref, lse_ref = oracle.prefill_attend_rows(Q, K, V, idx_h, cnt_h, wl.block, rows)
    hs = torch.tensor([h for _, h, _ in rows], device="cuda")
    ts = torch.tensor([t for _, _, t in rows], device="cuda")
    got = O32[0, hs, ts].cpu().numpy()
    gl = lse[0, hs, ts].cpu().numpy()
    err = max_abs(got, O_ref)
    assert err <= 2e-3, err
    assert max_abs(gl, lse_ref) <= 1e-4
    print(f"prefill: {len(rows)} sampled rows, max-abs O error {err:.2e}, {time.time() - t0:.1f}s")
