"""Helpers for the GPU parity tests (no test functions here).

Selection rule: the GPU's kept set must equal the oracle's, except inside the
near-tie band around the oracle's cut score c (the last free slot's score):
band = {j : |s_j - c| <= 1e-5 * max(|c|, |s_j|)} (s in float64).  Candidates
above the band must be kept, candidates below it must not, and the GPU must
keep as many band members as the oracle does.
"""
import numpy as np

REL_TIE = 1e-5


def to_dev(arr, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def check_topk_row(got, scores, k, forced, cand, where=""):
    """got: kept block ids (GPU); scores: float64 oracle scores [nb];
    forced: always-kept ids; cand: candidate ids (ascending).  Returns the
    number of band-resolved ties."""
    got = [int(x) for x in got]
    assert got == sorted(got), f"{where}: not ascending {got}"
    assert len(set(got)) == len(got), f"{where}: duplicates {got}"
    gs = set(got)
    for f in forced:
        assert f in gs, f"{where}: forced block {f} missing"
    cand = np.asarray(cand, dtype=np.int64)
    nfree = min(k - len(forced), cand.size)
    free_got = gs - set(forced)
    assert free_got <= set(cand.tolist()), f"{where}: kept a non-candidate {sorted(free_got)}"
    assert len(free_got) == nfree, f"{where}: kept {len(free_got)} free blocks, want {nfree}"
    if nfree == 0 or nfree == cand.size:
        return 0
    s = np.where(np.isnan(scores), -np.inf, scores)
    order = cand[np.lexsort((cand, -s[cand]))]
    want = set(order[:nfree].tolist())
    c = s[order[nfree - 1]]
    sc = s[cand]
    band = np.abs(sc - c) <= REL_TIE * np.maximum(np.abs(c), np.abs(sc))
    inband = set(cand[band].tolist())
    for j in cand.tolist():
        if j in inband:
            continue
        assert (j in free_got) == (j in want), (
            f"{where}: block {j} (score {s[j]:.9g}, cut {c:.9g}) kept={j in free_got} want={j in want}")
    assert len(free_got & inband) == len(want & inband), f"{where}: wrong number of tie-band picks"
    return len(inband) - 1 if len(inband) > 1 else 0


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def bf16_rne_of_f32(x):
    """Bits of round-to-nearest-even bf16 of float32 values (test-side copy)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
