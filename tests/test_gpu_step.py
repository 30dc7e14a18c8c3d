"""GPU parity of the one-launch decode step (scores, selection, split-K
attention and merge in one kernel; SA_STEP_MODE=1) against the float64 oracle.

The step's kv heads run on XCD teams that exchange candidates and partials
through their L2; these cases cover several team shapes (1 to 8 heads per XCD,
so 32 down to 4 splits per head), g = 1..8, D = 64 and 128, blocks of 64 and
128, ragged caches, splits without rows, every block kept, only the forced
blocks kept, and a score profile whose best blocks all sit in one split (the
whole-row fallback).  Selections must match the oracle outside the 1e-5 tie
band; outputs (float32 mode) within 2e-3 of the oracle on the GPU's lists and
within 1e-5 of the standalone block decode on the same lists; the sketch row
of the newest block is rebuilt; the workspace's error word stays zero; a
repeated call is bitwise identical.
"""
import os

import numpy as np
import pytest

import oracle
from tests.parity_util import check_topk_row, max_abs, to_dev
from workloads import get_workload, make_inputs
from oracle.attention import widen

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import top_sparse_attention_mean_amd as sa  # noqa: E402

STEP_CASES = [
    ("long_decode_bf16", {"N": 65536}),                                    # 8 heads: 32 splits each
    ("long_decode_bf16", {"N": 262144 - 64 * 7 - 19, "Hq": 16, "Hkv": 2}),  # ragged, 2 teams busy
    ("gqa_decode_bf16", {"B": 8, "N": 8192}),                              # 64 heads: 4 splits each
    ("gqa_decode_bf16", {"B": 3, "Hq": 8, "Hkv": 8, "N": 5000}),           # g = 1, 24 heads
    ("gqa_decode_bf16", {"B": 2, "Hq": 8, "Hkv": 4, "N": 3000, "D": 64}),   # g = 2, D = 64
    ("gqa_decode_bf16", {"B": 1, "Hq": 8, "Hkv": 2, "N": 20000, "block": 128, "k": 20}),
    ("gqa_decode_bf16", {"B": 1, "Hq": 4, "Hkv": 1, "N": 1000, "k": 6, "needles": 2}),  # splits with no rows
    ("gqa_decode_bf16", {"B": 2, "Hq": 8, "Hkv": 2, "N": 1500, "k": 30, "needles": 2}),  # k >= nb
    ("gqa_decode_bf16", {"B": 2, "Hq": 8, "Hkv": 2, "N": 4000, "k": 2, "needles": 2}),   # forced only
]


@pytest.fixture(autouse=True)
def _one_launch_step(monkeypatch):
    """Every call of sa_decode_step in this module runs the one-launch step."""
    monkeypatch.setenv("SA_STEP_MODE", "1")


def _case(name, over):
    wl = get_workload(name, **over)
    inp = make_inputs(wl)
    return wl, inp, widen(inp.Q, "bf16"), widen(inp.K, "bf16"), widen(inp.V, "bf16")


def _run_step(wl, Qd, Kd, Vd, sk, upd, ws):
    score = torch.empty(wl.B, wl.Hkv, wl.nb, dtype=torch.float32, device="cuda")
    O, lse, idx, cnt = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block, update_block=upd,
                                         score=score, out_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    return O, lse, idx, cnt, score


def _ws(wl):
    return torch.zeros(sa.workspace_bytes(sa.SA_OP_DECODE_STEP, wl.B, wl.Hq, wl.Hkv, wl.N, wl.D,
                                          wl.block, wl.k), dtype=torch.uint8, device="cuda")


def _check_step(wl, inp, q, K, V, O, lse, idx, cnt, where):
    sc_ref = oracle.block_scores(q, oracle.sketch(K, wl.block))
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    nb = wl.nb
    forced = [0, nb - 1] if nb > 1 else [0]
    for b in range(wl.B):
        for kh in range(wl.Hkv):
            n = int(cnt_h[b, kh])
            assert n == min(wl.k, nb), (where, b, kh, n)
            assert np.all(idx_h[b, kh, n:] == -1)
            if wl.k >= nb:
                assert idx_h[b, kh, :n].tolist() == list(range(nb))
            else:
                check_topk_row(idx_h[b, kh, :n], sc_ref[b, kh], wl.k, forced,
                               np.arange(1, nb - 1), where=f"{where} b{b} kh{kh}")
    O_ref, lse_ref = oracle.attend_blocks(q, K, V, idx_h, wl.block, count=cnt_h)
    err = max_abs(O.cpu().numpy(), O_ref)
    assert err <= 2e-3, (where, err)
    assert max_abs(lse.cpu().numpy(), lse_ref) <= 1e-4
    return err


@pytest.mark.parametrize("name,over", STEP_CASES)
def test_step_parity(name, over):
    wl, inp, q, K, V = _case(name, over)
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk_full = sa.sa_build_sketch(Kd, wl.block)
    sk = sk_full.clone()
    upd = wl.nb - 1
    sk[:, :, upd] = 0                                   # stale newest block, rebuilt by the step
    ws = _ws(wl)
    O, lse, idx, cnt, score = _run_step(wl, Qd, Kd, Vd, sk, upd, ws)
    assert int(ws[:4].view(torch.int32).item()) == 0    # no wait ran out
    assert torch.equal(sk, sk_full)
    err = _check_step(wl, inp, q, K, V, O, lse, idx, cnt, f"{name} {over}")
    # scores: the standalone selection's, bit for bit (the rebuilt block to rounding)
    _, _, score2 = sa.sa_select_topk(Qd, sk_full, wl.k, want_score=True)
    sc, sc2 = score.cpu().numpy(), score2.cpu().numpy()
    assert max_abs(sc[:, :, upd], sc2[:, :, upd]) <= 1e-6 * max(1.0, np.abs(sc2).max())
    sc[:, :, upd] = sc2[:, :, upd] = 0
    np.testing.assert_array_equal(sc, sc2)
    # the block decode on the same lists agrees to P's 16-bit rounding
    O2, lse2 = sa.sa_sparse_decode(Qd, Kd, Vd, idx, cnt, block=wl.block, out_dtype=torch.float32)
    assert max_abs(O.cpu().numpy(), O2.cpu().numpy()) <= 1e-5
    assert max_abs(lse.cpu().numpy(), lse2.cpu().numpy()) <= 1e-5
    # repeatable on the same workspace (the counters reset themselves), bf16 out = RNE of f32
    Ob, lseb, idxb, cntb = sa.sa_decode_step(Qd, Kd, Vd, sk, wl.k, block=wl.block, ws=ws)
    O3, lse3, idx3, cnt3, _ = _run_step(wl, Qd, Kd, Vd, sk, upd, ws)
    assert torch.equal(idx, idx3) and torch.equal(cnt, cnt3)
    assert torch.equal(O, O3) and torch.equal(lse, lse3)
    assert torch.equal(idx, idxb)
    assert torch.equal(Ob, O.to(torch.bfloat16))
    assert int(ws[:4].view(torch.int32).item()) == 0
    print(f"{name} {over}: max-abs O error {err:.2e}")


def test_step_fallback_to_whole_row():
    """Needle blocks all in one split (block ids 64 i fall in split 0 for any
    split count dividing 64): that split holds more of the top set than it
    publishes, its weakest published candidate makes the cut, and every split
    selects from the whole row instead.  The selection must still be exact."""
    wl = get_workload("long_decode_bf16", Hq=16, Hkv=2, needles=4)
    inp = make_inputs(wl)
    Kf = widen(inp.K, "bf16").astype(np.float32)
    q = widen(inp.Q, "bf16")
    g = wl.g
    for kh in range(wl.Hkv):
        qh = q[0, kh * g:(kh + 1) * g].mean(0)
        qh /= np.linalg.norm(qh)
        for i in range(1, 41):                    # 40 > the 16 a split publishes
            Kf[0, kh, 64 * i * wl.block:(64 * i + 1) * wl.block] += (3.0 * qh).astype(np.float32)
    from workloads import f32_to_bf16_bits
    Kb = f32_to_bf16_bits(Kf)
    K = widen(Kb, "bf16")
    V = widen(inp.V, "bf16")
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(Kb, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    ws = _ws(wl)
    O, lse, idx, cnt, _ = _run_step(wl, Qd, Kd, Vd, sk, -1, ws)
    assert int(ws[:4].view(torch.int32).item()) == 0
    _check_step(wl, inp, q, K, V, O, lse, idx, cnt, "fallback")
    idx_h = idx.cpu().numpy()
    for kh in range(wl.Hkv):
        assert {64 * i for i in range(1, 41)} <= set(idx_h[0, kh].tolist())


@pytest.mark.parametrize("mode", ["2", "3", "0"])
def test_step_coherence_modes(mode):
    """Device-coherent publication throughout (2) and the republish path taken
    when a member runs off its team's XCD (3) give bitwise the plain one-launch
    step's result; the two-kernel step (0) the same selection and outputs to
    1e-5."""
    wl, inp, q, K, V = _case("gqa_decode_bf16", {"B": 4, "N": 9000})
    Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
    sk = sa.sa_build_sketch(Kd, wl.block)
    O, lse, idx, cnt, score = _run_step(wl, Qd, Kd, Vd, sk, wl.nb - 1, _ws(wl))
    os.environ["SA_STEP_MODE"] = mode          # the fixture restores it
    ws = _ws(wl)
    O2, lse2, idx2, cnt2, score2 = _run_step(wl, Qd, Kd, Vd, sk, wl.nb - 1, ws)
    O3, lse3, idx3, cnt3, _ = _run_step(wl, Qd, Kd, Vd, sk, wl.nb - 1, ws)
    os.environ["SA_STEP_MODE"] = "1"
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    assert torch.equal(idx2, idx3) and torch.equal(O2, O3)
    if mode == "0":
        assert max_abs(O.cpu().numpy(), O2.cpu().numpy()) <= 1e-5
        assert max_abs(lse.cpu().numpy(), lse2.cpu().numpy()) <= 1e-5
    else:
        assert int(ws[:4].view(torch.int32).item()) == 0
        assert torch.equal(O, O2) and torch.equal(lse, lse2) and torch.equal(score, score2)
    _check_step(wl, inp, q, K, V, O2, lse2, idx2, cnt2, f"mode {mode}")
