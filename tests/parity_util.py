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


def lowbit_bmax_bound(q, codes, meta, block, scale):
    """Per (b, query head, block) bound on how far a provisional block maximum
    computed with int8-quantised weights can sit from the float64 thumbnail
    product q . t of the oracle.

    With w_c = q_c * step_c and the quantisation unit ws = max_c |w_c| / 127,
    rounding each weight to a multiple of ws moves it by at most ws / 2 (plus
    float32 rounding of w, 1/ws and w / ws, far below 1e-4 of a unit), so a
    token's code term moves by at most ws / 2 * sum_c code_c and the block
    maximum by at most that over the block's largest code sum.  The float32
    thumbnail differs from lo + code * step by half a float32 unit, and the
    kernel's own float32 sums (q . lo over D channels, one product, one add,
    the scale) add at most D * 2^-23 of the magnitudes involved.
    Returns (delta [B, Hq, nb], ws [B, Hq, nb])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, N = codes.shape[1], codes.shape[2]
    g = Hq // Hkv
    nb = -(-N // block)
    lo = meta[:, :, :, 0, :].astype(np.float64)
    step = meta[:, :, :, 1, :].astype(np.float64)
    csum = codes.astype(np.int64).sum(-1)                      # [B, Hkv, N]
    cmax = np.zeros((B, Hkv, nb))
    for j in range(nb):
        cmax[:, :, j] = csum[:, :, j * block:min((j + 1) * block, N)].max(-1)
    delta = np.zeros((B, Hq, nb))
    wsa = np.zeros((B, Hq, nb))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            w = np.abs(q[b, h][None, :] * step[b, kh])          # [nb, D]
            ws = w.max(-1) / 127.0
            qlo = np.abs(q[b, h][None, :] * lo[b, kh]).sum(-1)
            lev = (np.abs(q[b, h])[None, :] * (np.abs(lo[b, kh]) + 3 * step[b, kh])).sum(-1)
            quant = ws / 2 * (1 + 1e-4) * cmax[b, kh]
            fp = D * 2.0 ** -23 * qlo + 2.0 ** -22 * lev + 2.0 ** -20 * (qlo + 3 * w.sum(-1))
            delta[b, h] = scale * (quant + fp) + 1e-7
            wsa[b, h] = ws
    return delta, wsa


def lowbit_kept_band(b_x, t_x, delta, margin, forced, hs, tau_up, tau_down):
    """The blocks a low-bit filter must keep (must) and may keep (may) for one
    (b, kv head): the oracle's provisional maxima b_x [Hq, nb] against its
    thresholds t_x [Hq], widened by the per-block bound delta [Hq, nb] and by
    how far the filter's threshold may sit above (tau_up) or below (tau_down)
    the oracle's; `forced` blocks are kept always."""
    nb = b_x.shape[-1]
    must = np.zeros(nb, bool)
    may = np.zeros(nb, bool)
    must[forced] = may[forced] = True
    for h in hs:
        must |= b_x[h] >= t_x[h] - margin + delta[h] + tau_up[h]
        may |= b_x[h] >= t_x[h] - margin - delta[h] - tau_down[h]
    return must, may
