"""GPU test of sa_decode_step_noalloc, the decode step that takes no
workspace (its scratch is the library's per-GPU array).

Two calls in a row, the second with a smaller input (other heads, length and
k, so the scratch layout moves), and the first shape again: each must give
bitwise the outputs of sa_decode_step on a freshly zeroed workspace (same
kernels, same split counts), on the two-kernel step and on the one-launch
step, whose counters sit elsewhere in the scratch.
"""
import os

import pytest

from tests.parity_util import to_dev
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import top_sparse_attention_mean_amd as sa  # noqa: E402

CALLS = [
    ("gqa_decode_bf16", {"B": 4, "N": 9000}),
    ("gqa_decode_bf16", {"B": 2, "Hq": 8, "Hkv": 2, "N": 3000, "k": 20, "needles": 2}),
    ("gqa_decode_bf16", {"B": 4, "N": 9000}),
]


def _outputs(wl, dev):
    return (torch.full((wl.B, wl.Hkv, wl.k), -7, dtype=torch.int32, device=dev),
            torch.full((wl.B, wl.Hkv), -7, dtype=torch.int32, device=dev),
            torch.full((wl.B, wl.Hkv, wl.nb), -7.0, dtype=torch.float32, device=dev),
            torch.full((wl.B, wl.Hq, wl.D), -7.0, dtype=torch.float32, device=dev),
            torch.full((wl.B, wl.Hq), -7.0, dtype=torch.float32, device=dev))


@pytest.mark.parametrize("mode", ["0", "1"])
def test_noalloc_matches_decode_step(mode, monkeypatch):
    monkeypatch.setenv("SA_STEP_MODE", mode)
    dev = torch.device("cuda:0")
    for i, (name, over) in enumerate(CALLS):
        wl = get_workload(name, **over)
        inp = make_inputs(wl)
        print(f"mode {mode} call {i}: {name} {over}", flush=True)
        Qd, Kd, Vd = to_dev(inp.Q, "bf16"), to_dev(inp.K, "bf16"), to_dev(inp.V, "bf16")
        sk0 = sa.sa_build_sketch(Kd, wl.block)
        sk0[:, :, wl.nb - 1] = 0                  # stale newest block, rebuilt by the step
        sk1, sk2 = sk0.clone(), sk0.clone()
        idx1, cnt1, sc1, O1, lse1 = _outputs(wl, dev)
        ws = torch.zeros(sa.workspace_bytes(sa.SA_OP_DECODE_STEP, wl.B, wl.Hq, wl.Hkv, wl.N,
                                            wl.D, wl.block, wl.k), dtype=torch.uint8, device=dev)
        sa.sa_decode_step(Qd, Kd, Vd, sk1, wl.k, block=wl.block, update_block=wl.nb - 1,
                          idx=idx1, count=cnt1, score=sc1, O=O1, lse=lse1, ws=ws)
        idx2, cnt2, sc2, O2, lse2 = _outputs(wl, dev)
        sa.sa_decode_step_noalloc(Qd, Kd, Vd, sk2, wl.k, block=wl.block,
                                  update_block=wl.nb - 1, idx=idx2, count=cnt2, score=sc2,
                                  O=O2, lse=lse2)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2), (mode, i)
        assert torch.equal(sc1, sc2) and torch.equal(sk1, sk2), (mode, i)
        assert torch.equal(O1, O2) and torch.equal(lse1, lse2), (mode, i)
        assert int((cnt2 == min(wl.k, wl.nb)).all()), (mode, i)


def test_noalloc_refuses_oversized_shape():
    """A shape whose workspace exceeds the scratch is refused on the host."""
    B, Hq, Hkv, N, D, block, k = 32, 1024, 128, 256, 128, 64, 2
    assert sa.workspace_bytes(sa.SA_OP_DECODE_STEP, B, Hq, Hkv, N, D, block, k) > 16 << 20
    dev = torch.device("cuda:0")
    Q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=dev)
    K = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device=dev)
    sk = torch.zeros(B, Hkv, N // block, D, dtype=torch.float32, device=dev)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    O = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    with pytest.raises(sa.SAError, match="16 MiB"):
        sa.sa_decode_step_noalloc(Q, K, K, sk, k, block=block, idx=idx, count=cnt, O=O)
    assert os.environ.get("SA_STEP_MODE") is None
