"""Benchmark of the sparse-decode hot path on one MI355X.

A step is one whole decode step of one attention layer at N = 256K keys
(B=1, Hq=64, Hkv=8, d=128, bf16, 64-token blocks, top-82 blocks ~2 %):
refresh the sketch of the newest block, score all 4096 block sketches per KV
group, select the top-k (sink + local forced), split-K sparse attention over
the selected blocks and the log-sum-exp merge.  Inputs are resident in HBM
before timing starts.  R distinct layer copies (K, V, sketch, and a different
query per layer) are cycled so that the 256 MiB Infinity Cache cannot serve
repeated steps.

Prints ONE JSON line (rank 0, N = 1).  Other workloads: --workload NAME.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode µs/step + achieved HBM GB/s (% of peak) at N=256K, top-2% blocks"
HBM_PEAK_GBPS = 8000.0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def decode_bytes(wl) -> dict:
    """Algorithmic bytes of one decode step (what the method must move)."""
    e = 2 if wl.dtype == "bf16" else 4
    sketch = wl.B * wl.Hkv * wl.nb * wl.D * 4
    kv = wl.B * wl.Hkv * min(wl.k, wl.nb) * wl.block * wl.D * e * 2
    q = wl.B * wl.Hq * wl.D * e
    out = wl.B * wl.Hq * wl.D * e + wl.B * wl.Hq * 4
    upd = wl.B * wl.Hkv * wl.block * wl.D * e + wl.B * wl.Hkv * wl.D * 4
    sel = wl.B * wl.Hkv * wl.k * 4 * 2
    return {"sketch": sketch, "kv": kv, "q": q, "out": out, "update": upd, "select_io": sel,
            "total": sketch + kv + q + out + upd + sel}


def time_loop(fn, n, stream):
    """Eager timing: n Python-issued launches back to back (includes host launch cost)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / n   # us per call


def graph_trials(fn, calls, R, trials=10, warmup=1):
    """Capture `calls` calls fn(i % R) as one HIP graph and replay it `trials`
    times after `warmup` untimed replays.  Each replay is timed with HIP events
    recorded on the replay stream, the stream the kernels run on; a short
    device-side spin queued first keeps the stream busy while the host
    enqueues the replay, so the start event cannot run ahead of the graph.
    Returns (median, min, max) microseconds per call over the trials."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for r in range(min(calls, R)):  # one eager pass outside capture
            fn(r)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fn(i % R)
    torch.cuda.synchronize()
    per = []
    with torch.cuda.stream(s):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        for _ in range(trials):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(200000)
            start.record(s)
            g.replay()
            end.record(s)
            end.synchronize()
            per.append(start.elapsed_time(end) * 1e3 / calls)
    torch.cuda.synchronize()
    per.sort()
    return per[len(per) // 2], per[0], per[-1]


def graph_time(fn, R, n_replay, warmup=3):
    """Median microseconds per call of fn(0..R-1) over at least ten timed
    graph replays (see graph_trials)."""
    reps = max(1, n_replay // 10)
    med, _, _ = graph_trials(fn, R * reps, R, trials=10, warmup=max(1, warmup // reps))
    return med


def _blas_threads() -> int:
    """Threads the oracle's BLAS uses: OMP_NUM_THREADS within this process's CPU set."""
    n = len(os.sched_getaffinity(0))
    return min(int(os.environ.get("OMP_NUM_THREADS", "0")) or n, n)


def cpu_baseline(inp, wl, budget_s: float = 12.0) -> dict:
    """The float64 oracle timed on this host on a bounded sample of steps."""
    import numpy as np
    import oracle
    from oracle.attention import widen
    threads = _blas_threads()
    q, K, V = (widen(x, wl.dtype) for x in (inp.Q, inp.K, inp.V))
    t_sk = time.perf_counter()
    sk = oracle.sketch(K, wl.block)                      # amortised at prefill: timed apart
    t_sk = time.perf_counter() - t_sk
    steps, t0 = 0, time.perf_counter()
    while True:
        j = wl.nb - 1                                    # newest block refreshed each step
        sk[:, :, j] = K[:, :, j * wl.block:].mean(axis=2)
        sc = oracle.block_scores(q, sk)
        idx = oracle.select_topk_all(sc, wl.k)
        oracle.attend_blocks(q, K, V, idx, wl.block)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 200:
            break
    return {"value": round(el / steps * 1e6, 1), "unit": "us/step", "cores": threads,
            "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"{steps} full decode steps of {wl.name} (float64 NumPy, "
                      f"BLAS threads={threads}); sketch build excluded (amortised at prefill)",
            "o1_sketch_build_us": round(t_sk * 1e6, 1)}


# The sources the counted kernel (the selecting split-K decode of the step)
# and its launch configuration are built from.
COUNTED_SOURCES = ["k_decode.hip", "sa_decode_core.h", "sa_device.h", "sa_internal.h",
                   "sa_select_core.h"]


def kernel_source_hash(sources=None) -> str:
    """SHA-256 over the sources of the counted kernels (counter data goes stale with them)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_sparse_attention_mean_amd", "csrc")
    for path in [os.path.join(csrc, f) for f in (sources or COUNTED_SOURCES)]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


PREFILL_SOURCES = ["k_prefill.hip", "sa_device.h", "sa_internal.h"]


def load_counter_json(kind: str, workload: str, sources):
    """The committed counter summary profiles/<kind>_<workload>.json, or None
    when there is none or the listed kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d if d.get("source_sha256") == kernel_source_hash(sources) else None


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    d = load_counter_json(f"traffic_{kernel}", workload, COUNTED_SOURCES)
    return d and d.get("hbm_bytes_per_launch")


def _layers(wl, R, dev):
    """R layer copies of (Q, K, V, sketch) resident in HBM, plus each layer's block scores."""
    import numpy as np
    import torch
    import top_sparse_attention_mean_amd as sa
    from tests.parity_util import to_dev
    from workloads import make_inputs
    inp = make_inputs(wl)
    K0, V0 = to_dev(inp.K, wl.dtype, dev), to_dev(inp.V, wl.dtype, dev)
    sk0 = sa.sa_build_sketch(K0, wl.block)
    Ks = [K0] + [K0.clone() for _ in range(R - 1)]
    Vs = [V0] + [V0.clone() for _ in range(R - 1)]
    sks = [sk0] + [sk0.clone() for _ in range(R - 1)]
    rng = np.random.default_rng(1000 + wl.seed)
    Qs = [to_dev(inp.Q, wl.dtype, dev)] + [
        to_dev(rng.standard_normal(inp.Q.shape, dtype=np.float32).astype(np.float32), "f32",
               dev).to(torch.bfloat16 if wl.dtype == "bf16" else torch.float32)
        for _ in range(R - 1)]
    scores = [sa.sa_select_topk(Qs[r], sks[r], wl.k, want_score=True)[2] for r in range(R)]
    return inp, Qs, Ks, Vs, sks, scores


DOMINANT_BF16 = "k_decode_blocks_mfma (sa_select_decode: top-k + split-K attention + merge)"
DOMINANT_F32 = "k_decode_blocks_valu (sa_sparse_decode on the step's lists: split-K + merge)"


def bench_decode(args, name=None, calls=None, layers=None, extras=True) -> dict:
    """One decode step per call (sa_decode_step), timed as HIP-graph replays of
    `calls` steps cycling `layers` layer copies, median of args.trials replays."""
    import math
    import torch
    import top_sparse_attention_mean_amd as sa
    from workloads import get_workload

    wl = get_workload(name or args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = layers or args.layers
    K = calls or args.steps
    inp, Qs, Ks, Vs, sks, scores = _layers(wl, R, dev)
    B, Hq, Hkv, D = wl.B, wl.Hq, wl.Hkv, wl.D
    idx = torch.empty(B, Hkv, wl.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    O = torch.empty(B, Hq, D, dtype=Qs[0].dtype, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    wsb = sa.workspace_bytes(sa.SA_OP_DECODE_STEP, B, Hq, Hkv, wl.N, D, wl.block, wl.k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    upd = wl.nb - 1

    def step(i, w=ws):
        r = i % R
        sa.sa_decode_step(Qs[r], Ks[r], Vs[r], sks[r], wl.k, block=wl.block, update_block=upd,
                          idx=idx, count=cnt, O=O, lse=lse, ws=w)

    warm = max(1, math.ceil(args.warmup / K))
    med, lo, hi = graph_trials(step, K, R, trials=args.trials, warmup=warm)
    by = decode_bytes(wl)
    gbps = by["total"] / (med * 1e-6) / 1e9
    bf = wl.dtype == "bf16"
    # the dominant kernel on its own, same graph timing: the selecting split-K
    # decode on each layer's block scores (bf16), or the block decode on the
    # step's lists (float32); its algorithmic bytes are the selected K and V
    # blocks, Q, O + lse and the index lists
    dws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, wl.N, D,
                                         wl.block, wl.k), dtype=torch.uint8, device=dev)
    step(0)
    if bf:
        dom = lambda i: sa.sa_select_decode(Qs[i % R], Ks[i % R], Vs[i % R], scores[i % R], wl.k,
                                            block=wl.block, idx=idx, count=cnt, O=O, lse=lse,
                                            ws=dws)
    else:
        idx0, cnt0 = idx.clone(), cnt.clone()
        dom = lambda i: sa.sa_sparse_decode(Qs[i % R], Ks[i % R], Vs[i % R], idx0, cnt0,
                                            block=wl.block, O=O, lse=lse, ws=dws)
    t_dom, _, _ = graph_trials(dom, K, R, trials=args.trials, warmup=warm)
    dom_bytes = by["kv"] + by["q"] + by["out"] + by["select_io"]
    ach = dom_bytes / (t_dom * 1e-6) / 1e9
    res = {
        "metric": METRIC,
        "value": round(med, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(med / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, " + (
            "AR(1) drift, " if wl.drift_var else "") + (
            "4 outlier channels x8, " if wl.outlier_channels else "") + "planted needle blocks)",
        "config": {"workload": wl.name, "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "N": wl.N,
                   "block": wl.block, "k": wl.k, "layers_cycled": R,
                   "step": "sketch update (newest block) + score + top-k + split-K + merge"},
        "trials": {"count": args.trials, "steps_per_trial": K, "us_per_step_min": round(lo, 3),
                   "us_per_step_median": round(med, 3), "us_per_step_max": round(hi, 3)},
        "achieved_GBps": round(gbps, 1),
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_step": by["total"],
        "algorithmic_bytes": {k2: v for k2, v in by.items() if k2 != "total"},
        "timing": f"HIP graph of {K} steps (one per layer copy, {R} copies cycled) replayed "
                  f"{args.trials} times after {warm} untimed replay(s), HIP events on the replay "
                  "stream; value = median over the replays",
        "kernels_us": {"dominant kernel alone": round(t_dom, 3),
                       "rest of the step (scoring kernel, newest-block refresh, boundary)":
                           round(max(med - t_dom, 0.0), 3)},
        "roofline": {"bound": "hbm",
                     "kernel": DOMINANT_BF16 if bf else DOMINANT_F32,
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("select_decode", wl.name) if bf else None,
                     "traffic_source": (f"profiles/traffic_select_decode_{wl.name}.md: rocprofv3 "
                                        "--pmc FETCH_SIZE and WRITE_SIZE of this kernel, scaled by "
                                        "the same counters on a plain copy of known size; null "
                                        "when the kernel sources changed since they were taken")
                     if bf else None,
                     "algorithmic_bytes": dom_bytes, "avg_us": round(t_dom, 3)},
    }
    if res["roofline"]["traffic"]:
        # counter bytes over the same live launch time (what the kernel actually moved)
        res["roofline"]["traffic_GBps"] = round(res["roofline"]["traffic"] / (t_dom * 1e-6) / 1e9, 1)
    if not bf:
        res["roofline"]["note"] = ("latency-bound: one launch moves under 0.3 MB, so GB/s says "
                                   "little; the figure is the step time")
    if extras:
        res["eager_us_per_step"] = round(time_loop(step, min(args.steps, 500), st), 3)
        # the same step without the newest block's sketch refresh
        def step_norefresh(i):
            r = i % R
            sa.sa_decode_step(Qs[r], Ks[r], Vs[r], sks[r], wl.k, block=wl.block, update_block=-1,
                              idx=idx, count=cnt, O=O, lse=lse, ws=ws)
        t_nr, _, _ = graph_trials(step_norefresh, min(K, 10 * R), R, trials=args.trials)
        res["us_per_step_without_sketch_update"] = round(t_nr, 3)
        # achievable stream rate: a plain device copy of 1 GiB (2 GiB moved)
        cx = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        cy.copy_(cx)
        t_cp, _, _ = graph_trials(lambda i: cy.copy_(cx), 4, 1, trials=args.trials)
        res["copy_achievable_GBps"] = round(2 * cx.numel() * 4 / (t_cp * 1e-6) / 1e9, 1)
        del cx, cy
        # the one-launch form of the same step (k_step.hip), its own workspace
        os.environ["SA_STEP_MODE"] = "1"
        try:
            ws2 = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            t_one, _, _ = graph_trials(lambda i: step(i, ws2), min(K, 10 * R), R,
                                       trials=args.trials)
        finally:
            del os.environ["SA_STEP_MODE"]
        # unfused path for context: standalone selection kernel, then block decode
        sws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_TOPK, B, Hq, Hkv, 1, D, 1, wl.nb),
                          dtype=torch.uint8, device=dev)
        n_rep = max(10, min(K, 10 * R) // R)
        t_sel = graph_time(lambda r: sa.sa_select_topk(Qs[r], sks[r], wl.k, idx=idx, count=cnt,
                                                       ws=sws), R, n_rep)
        t_dec = graph_time(lambda r: sa.sa_sparse_decode(Qs[r], Ks[r], Vs[r], idx, cnt,
                                                         block=wl.block, O=O, lse=lse, ws=dws),
                           R, n_rep)
        # dense reference: the same block decode with every block selected
        all_idx = torch.arange(wl.nb, dtype=torch.int32, device=dev).repeat(B, Hkv, 1).contiguous()
        all_cnt = torch.full((B, Hkv), wl.nb, dtype=torch.int32, device=dev)
        dn_ws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, wl.N, D,
                                               wl.block, wl.nb), dtype=torch.uint8, device=dev)
        t_dense = graph_time(lambda r: sa.sa_sparse_decode(Qs[r], Ks[r], Vs[r], all_idx, all_cnt,
                                                           block=wl.block, O=O, lse=lse,
                                                           ws=dn_ws), R, 10)
        res["one_launch_step_us"] = round(t_one, 3)
        res["unfused_us"] = {"sa_select_topk": round(t_sel, 3), "sa_sparse_decode": round(t_dec, 3)}
        res["dense_decode_us"] = round(t_dense, 2)
        res["sparse_vs_dense_speedup"] = round(t_dense / med, 2)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget if extras else 6.0)
    return res


def bench_threshold(args, which: str = "threshold") -> dict:
    """Threshold variants at full size, then token-mode a5 + a6.

    which = "threshold": row a4 with the workload's tau (exact scores of every
    key, keep s >= tau - eps, ordered compaction).
    which = "topdelta": the threshold comes from the pseudo-maximum over the
    sink and local tokens (tau = m~ - delta), computed on the GPU in the same
    call, then the same scan and compaction.
    """
    import numpy as np
    import torch
    import oracle
    import top_sparse_attention_mean_amd as sa
    from oracle.attention import widen
    from tests.parity_util import to_dev
    from workloads import get_workload, make_inputs
    wl = get_workload("threshold_decode_bf16" if which == "threshold" else "topdelta_decode_bf16")
    dev = torch.device("cuda:0")
    inp = make_inputs(wl)
    q, K, V = (widen(x, wl.dtype) for x in (inp.Q, inp.K, inp.V))
    R = 2                                                        # 2 x 1 GiB of K/V > Infinity Cache
    Qs = [to_dev(inp.Q, wl.dtype, dev) for _ in range(R)]
    Kd = to_dev(inp.K, wl.dtype, dev)
    Ks = [Kd] + [Kd.clone() for _ in range(R - 1)]
    Vd = to_dev(inp.V, wl.dtype, dev)
    Vs = [Vd] + [Vd.clone() for _ in range(R - 1)]
    B, Hq, Hkv, D, N = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N
    idx = torch.empty(B, Hq, wl.cap, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Hq, wl.cap, dtype=torch.float32, device=dev)
    cnt = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    O = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    dws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, 0, wl.cap),
                      dtype=torch.uint8, device=dev)
    if which == "threshold":
        _, tau32 = oracle.threshold_tau(q, K, wl.percentile)    # the workload's tau (input)
        tau.copy_(torch.from_numpy(tau32))
        tws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_THRESHOLD, B, Hq, Hkv, N, D, 0,
                                             wl.cap), dtype=torch.uint8, device=dev)

        def sel(r):
            sa.sa_select_threshold(Qs[r], Ks[r], tau, wl.cap, idx=idx, score=sc, count=cnt,
                                   ws=tws)
        call = "sa_select_threshold (k_threshold_mfma + k_threshold_compact)"
    else:
        tws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_TOPDELTA, B, Hq, Hkv, N, D, 0,
                                             wl.cap), dtype=torch.uint8, device=dev)

        def sel(r):
            sa.sa_select_topdelta(Qs[r], Ks[r], wl.sink, wl.local, wl.delta, wl.cap, idx=idx,
                                  score=sc, count=cnt, tau=tau, ws=tws)
        call = ("sa_select_topdelta (k_pseudo_max_mfma + k_threshold_mfma + "
                "k_threshold_compact)")

    def dec(r):
        sa.sa_sparse_decode(Qs[r], Ks[r], Vs[r], idx, cnt, mode=sa.SA_IDX_TOKENS, score=sc,
                            O=O, lse=lse, ws=dws)

    n = max(4, args.steps // 20)
    t_pass = graph_time(lambda r: (sel(r), dec(r)), R, n)
    t_sel = graph_time(sel, R, n)
    e = 2
    kept = int(cnt.sum().item())
    assert int(cnt.max().item()) <= wl.cap, "list capacity exceeded"
    win = 0 if which == "threshold" else B * Hkv * len(oracle.window_tokens(N, wl.sink, wl.local)) * D * e
    scan_bytes = B * Hkv * N * D * e + B * Hq * D * e + B * Hq * 4
    list_bytes = B * Hq * wl.cap * 8 + B * Hq * 4
    v_bytes = kept * D * e
    ach = (scan_bytes + win + kept * 8) / (t_sel * 1e-6) / 1e9
    res = {
        "workload": wl.name, "us_per_pass": round(t_pass, 2),
        "pass": (("threshold scan + compaction" if which == "threshold" else
                  "pseudo-max + threshold scan + compaction") + f" ({call.split(' ')[0]}) "
                 "+ token-mode decode"),
        "kernels_us": {call: round(t_sel, 2),
                       "sa_sparse_decode tokens (k_decode_tokens)": round(max(t_pass - t_sel, 0), 2)},
        "kept_tokens": kept, "kept_fraction": round(kept / (B * Hq * N), 5),
        "algorithmic_bytes_per_pass": scan_bytes + win + list_bytes + v_bytes,
        "roofline": {"bound": "hbm", "kernel": "k_threshold_mfma (full K scan; the call also runs "
                     "the small compaction kernel" + (")" if which == "threshold" else
                                                      " and the pseudo-max kernel)"),
                     "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes": scan_bytes + win + kept * 8,
                     "avg_us": round(t_sel, 2)},
    }
    if which == "topdelta":
        res["delta"], res["sink"], res["local"] = wl.delta, wl.sink, wl.local
    if not args.no_cpu:
        # the oracle on the same arrays: selection, then attention
        t0 = time.perf_counter()
        if which == "threshold":
            lists, _ = oracle.select_threshold(q, K, tau32.astype(np.float64))
        else:
            lists, _, _ = oracle.select_topdelta(q, K, wl.sink, wl.local, wl.delta)
        oracle.attend_tokens(q, K, V, lists)
        t_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(t_cpu * 1e6, 1), "unit": "us/pass",
                               "cores": _blas_threads(), "kind": "oracle",
                               "sample": "one full pass (all 256 heads, float64)"}
    return res


def bench_pruned(args) -> dict:
    """Sphere-pruned threshold selection on the clustered workload: the bound
    kernel, then the scan of the live segments only, the compaction and the
    token-mode decode.  The unpruned scan on the same arrays is timed beside it."""
    import numpy as np
    import torch
    import oracle
    import top_sparse_attention_mean_amd as sa
    from oracle.attention import widen
    from tests.parity_util import to_dev
    from workloads import get_workload, make_inputs
    wl = get_workload("clustered_threshold_bf16")
    dev = torch.device("cuda:0")
    inp = make_inputs(wl)
    q, K, V = (widen(x, wl.dtype) for x in (inp.Q, inp.K, inp.V))
    _, tau32 = oracle.threshold_tau(q, K, wl.percentile)        # the workload's tau (input)
    R = 2
    Qs = [to_dev(inp.Q, wl.dtype, dev) for _ in range(R)]
    Kd = to_dev(inp.K, wl.dtype, dev)
    Ks = [Kd] + [Kd.clone() for _ in range(R - 1)]
    Vd = to_dev(inp.V, wl.dtype, dev)
    Vs = [Vd] + [Vd.clone() for _ in range(R - 1)]
    B, Hq, Hkv, D, N, blk, S = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N, wl.block, wl.subspaces
    sks = [sa.sa_build_sketch(k, blk) for k in Ks]                  # built once, at prefill
    rads = [sa.sa_build_radius(k, sk, blk, S) for k, sk in zip(Ks, sks)]
    tau = torch.from_numpy(tau32).to(dev)
    idx = torch.empty(B, Hq, wl.cap, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Hq, wl.cap, dtype=torch.float32, device=dev)
    cnt = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    nseg = -(-N // 128)
    live = torch.empty(B, Hkv, nseg, dtype=torch.uint8, device=dev)
    O = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    pws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_PRUNED, B, Hq, Hkv, N, D, blk, wl.cap),
                      dtype=torch.uint8, device=dev)
    tws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_THRESHOLD, B, Hq, Hkv, N, D, 0, wl.cap),
                      dtype=torch.uint8, device=dev)
    dws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, 0, wl.cap),
                      dtype=torch.uint8, device=dev)

    def sel(r):
        sa.sa_select_threshold_pruned(Qs[r], Ks[r], sks[r], rads[r], tau, wl.cap, blk, idx=idx,
                                      score=sc, count=cnt, live=live, ws=pws)

    def sel0(r):
        sa.sa_select_threshold(Qs[r], Ks[r], tau, wl.cap, idx=idx, score=sc, count=cnt, ws=tws)

    def dec(r):
        sa.sa_sparse_decode(Qs[r], Ks[r], Vs[r], idx, cnt, mode=sa.SA_IDX_TOKENS, score=sc,
                            O=O, lse=lse, ws=dws)

    n = max(4, args.steps // 20)
    t_sel0 = graph_time(sel0, R, n)
    t_pass = graph_time(lambda r: (sel(r), dec(r)), R, n)
    t_sel = graph_time(sel, R, n)
    e = 2
    kept = int(cnt.sum().item())
    nb = -(-N // blk)
    bps = 128 // blk
    lv = live.cpu().numpy()
    frac = float(np.stack([(lv >> i) & 1 for i in range(bps)], -1).reshape(B, Hkv, -1)[:, :, :nb].mean())
    bound_bytes = B * Hkv * nb * (D + S) * 4 + B * Hq * D * e + B * Hq * 4
    scan_bytes = int(round(frac * B * Hkv * N * D * e))
    ach = (bound_bytes + scan_bytes + kept * 8) / (t_sel * 1e-6) / 1e9
    res = {
        "workload": wl.name, "us_per_pass": round(t_pass, 2), "subspaces": S,
        "pass": "sphere bounds + scan of the live blocks + compaction "
                "(sa_select_threshold_pruned) + token-mode decode",
        "kernels_us": {"sa_select_threshold_pruned (k_prune + k_threshold_mfma + "
                       "k_threshold_compact)": round(t_sel, 2),
                       "sa_sparse_decode tokens (k_decode_tokens)": round(max(t_pass - t_sel, 0), 2),
                       "unpruned sa_select_threshold on the same arrays": round(t_sel0, 2)},
        "scanned_block_fraction": round(frac, 4), "kept_tokens": kept,
        "roofline": {"bound": "hbm", "kernel": "k_threshold_mfma over the live blocks (the "
                     "call also runs the bound and compaction kernels)", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes": bound_bytes + scan_bytes + kept * 8,
                     "avg_us": round(t_sel, 2)},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        lists, _, _ = oracle.select_threshold_pruned(q, K, tau32.astype(np.float64), blk, S)
        oracle.attend_tokens(q, K, V, lists)
        t_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(t_cpu * 1e6, 1), "unit": "us/pass",
                               "cores": _blas_threads(), "kind": "oracle",
                               "sample": "one full pass (all 256 heads, float64; sketch and "
                                         "radius included)"}
    return res


def bench_lowbit(args) -> dict:
    """Top-delta over 2-bit key thumbnails (pseudo-max from the window's refined
    keys, thumbnail scan and block filter, refined keys of the kept blocks) and
    block-mode attention over them; the codec runs once, when the cache is
    written.  The exact top-delta pass on the same arrays is timed beside it."""
    import numpy as np
    import torch
    import oracle
    import top_sparse_attention_mean_amd as sa
    from oracle.attention import widen
    from tests.parity_util import to_dev
    from workloads import get_workload, make_inputs
    wl = get_workload("lowbit_topdelta_bf16")
    dev = torch.device("cuda:0")
    inp = make_inputs(wl)
    R = 2
    Qs = [to_dev(inp.Q, wl.dtype, dev) for _ in range(R)]
    Kd = to_dev(inp.K, wl.dtype, dev)
    Ks = [Kd] + [Kd.clone() for _ in range(R - 1)]
    Vd = to_dev(inp.V, wl.dtype, dev)
    Vs = [Vd] + [Vd.clone() for _ in range(R - 1)]
    B, Hq, Hkv, D, N, blk = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N, wl.block
    nb = -(-N // blk)
    enc = [sa.sa_encode_keys(k, blk) for k in Ks]
    torch.cuda.synchronize()
    t_e0 = time.perf_counter()
    sa.sa_encode_keys(Ks[0], blk, codes=enc[0][0], resid=enc[0][1], meta=enc[0][2])
    torch.cuda.synchronize()
    t_enc = (time.perf_counter() - t_e0) * 1e6
    khats = [torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device=dev) for _ in range(R)]
    idx = torch.empty(B, Hkv, wl.cap, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    O = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    lws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_LOWBIT, B, Hq, Hkv, N, D, blk, wl.cap),
                      dtype=torch.uint8, device=dev)
    dws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, blk, wl.cap),
                      dtype=torch.uint8, device=dev)
    # the exact top-delta pass on the same arrays
    tcap = 4096
    tidx = torch.empty(B, Hq, tcap, dtype=torch.int32, device=dev)
    tsc = torch.empty(B, Hq, tcap, dtype=torch.float32, device=dev)
    tcnt = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    tws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_TOPDELTA, B, Hq, Hkv, N, D, 0, tcap),
                      dtype=torch.uint8, device=dev)
    tdws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, 0, tcap),
                       dtype=torch.uint8, device=dev)

    def sel(r):
        c, rs, m = enc[r]
        sa.sa_select_topdelta_lowbit(Qs[r], c, rs, m, blk, wl.sink, wl.local, wl.delta, wl.margin,
                                     wl.cap, khat=khats[r], idx=idx, count=cnt, tau=tau, ws=lws)

    def dec(r):
        sa.sa_sparse_decode(Qs[r], khats[r], Vs[r], idx, cnt, block=blk, O=O, lse=lse, ws=dws)

    def exact(r):
        sa.sa_select_topdelta(Qs[r], Ks[r], wl.sink, wl.local, wl.delta, tcap, idx=tidx, score=tsc,
                              count=tcnt, ws=tws)
        sa.sa_sparse_decode(Qs[r], Ks[r], Vs[r], tidx, tcnt, mode=sa.SA_IDX_TOKENS, score=tsc, O=O,
                            lse=lse, ws=tdws)

    fws = torch.zeros(sa.workspace_bytes(sa.SA_OP_DECODE_LOWBIT, B, Hq, Hkv, N, D, blk, wl.cap),
                      dtype=torch.uint8, device=dev)

    def fused(r):
        c, rs, m = enc[r]
        sa.sa_decode_topdelta_lowbit(Qs[r], c, rs, m, Vs[r], blk, wl.sink, wl.local, wl.delta,
                                     wl.margin, wl.cap, khat=khats[r], idx=idx, count=cnt,
                                     tau=tau, O=O, lse=lse, ws=fws)

    def fused0(r):
        c, rs, m = enc[r]
        sa.sa_decode_topdelta_lowbit(Qs[r], c, rs, m, Vs[r], blk, wl.sink, wl.local, wl.delta,
                                     0.0, wl.cap, khat=khats[r], idx=idx, count=cnt, tau=tau,
                                     O=O, lse=lse, ws=fws)

    n = max(4, args.steps // 20)
    t_fused0 = graph_time(fused0, R, n)
    kept0 = int(cnt.sum().item())
    t_fused = graph_time(fused, R, n)
    t_pass = graph_time(lambda r: (sel(r), dec(r)), R, n)
    t_sel = graph_time(sel, R, n)
    t_exact = graph_time(exact, R, n)
    kept = int(cnt.sum().item())
    e = 2
    scan_bytes = B * Hkv * (N * D // 4 + nb * 2 * D * 4) + B * Hq * D * e + B * Hq * 4
    refine_bytes = kept * blk * D * (1 + 1 / 4) + kept * 3 * D * 4 + kept * blk * D * e
    ach = scan_bytes / (t_sel * 1e-6) / 1e9
    res = {
        "workload": wl.name, "us_per_pass": round(t_fused, 2), "margin": wl.margin,
        "pass": "window refined keys + pseudo-max + thumbnail scan + block list + split-K "
                "attention over the kept blocks with keys rebuilt from codes and residuals in "
                "the kernel (sa_decode_topdelta_lowbit)",
        "kernels_us": {"sa_decode_topdelta_lowbit (fused refinement)": round(t_fused, 2),
                       "two-pass form: sa_select_topdelta_lowbit (refined keys written)":
                           round(t_sel, 2),
                       "two-pass form: sa_sparse_decode blocks over the refined keys":
                           round(max(t_pass - t_sel, 0), 2),
                       "two-pass form, whole": round(t_pass, 2),
                       "exact top-delta pass on the same arrays (sa_select_topdelta + token "
                       "decode)": round(t_exact, 2),
                       "sa_encode_keys, once per cache (host-timed, one call)": round(t_enc, 1)},
        "kept_block_fraction": round(kept / (B * Hkv * nb), 4),
        "margin_0": {"us_per_pass": round(t_fused0, 2),
                     "kept_block_fraction": round(kept0 / (B * Hkv * nb), 4),
                     "note": "the same fused pass with the filter at tau itself (margin 0)"},
        "scan_bytes_per_token": D // 4 + 2 * D * 4 / blk,
        "roofline": {"bound": "hbm", "kernel": "k_thumb_scan (2-bit codes + block ranges; the "
                     "call also runs the window decode, pseudo-max, list and refine kernels)",
                     "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes": int(scan_bytes),
                     "refine_bytes": int(refine_bytes), "avg_us": round(t_sel, 2)},
    }
    if not args.no_cpu:
        q, K, V = (widen(x, wl.dtype) for x in (inp.Q, inp.K, inp.V))
        t0 = time.perf_counter()
        c_x, r_x, m_x = oracle.lowbit_encode(K, blk)
        t_cpu_enc = time.perf_counter() - t0
        t0 = time.perf_counter()
        i_x, n_x, _, _ = oracle.select_topdelta_lowbit(q, c_x, r_x, m_x, blk, wl.sink, wl.local,
                                                       wl.delta, wl.margin)
        kx = oracle.bf16_round(oracle.lowbit_reconstruct(c_x, r_x, m_x, blk))
        oracle.attend_blocks(q, kx, V, i_x, blk, count=n_x)
        t_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(t_cpu * 1e6, 1), "unit": "us/pass",
                               "cores": _blas_threads(), "kind": "oracle",
                               "sample": f"one full pass (all 256 heads, float64); the codec "
                                         f"({t_cpu_enc:.1f} s) not included"}
    return res


def bench_prefill(args) -> dict:
    """Block-sparse causal prefill (rows a1 pooling, a3, a7) at its full size."""
    import numpy as np
    import torch
    import oracle
    import top_sparse_attention_mean_amd as sa
    from oracle.attention import widen
    from tests.parity_util import to_dev
    from workloads import get_workload, make_inputs
    wl = get_workload("sparse_prefill_bf16")
    dev = torch.device("cuda:0")
    inp = make_inputs(wl)
    Qd, Kd, Vd = (to_dev(x, wl.dtype, dev) for x in (inp.Q, inp.K, inp.V))
    B, Hq, Hkv, D, L, blk = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N, wl.block
    M = wl.nb
    flags = sa.SA_FORCE_SINK | sa.SA_FORCE_LOCAL | sa.SA_CAUSAL
    sk = sa.sa_build_sketch(Kd, blk)
    idx = torch.empty(B, Hkv, M, wl.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, M, dtype=torch.int32, device=dev)
    O = torch.empty(B, Hq, L, D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=dev)
    sws = torch.zeros(sa.workspace_bytes(sa.SA_OP_SELECT_TOPK, B, Hq, Hkv, L, D, blk, M),
                      dtype=torch.uint8, device=dev)

    def sketch(r):
        sa.sa_build_sketch(Kd, blk, out=sk)

    def select(r):
        sa.sa_select_topk(Qd, sk, wl.k, flags=flags, q_block=blk, idx=idx, count=cnt, ws=sws)

    def attend(r):
        sa.sa_sparse_prefill(Qd, Kd, Vd, idx, cnt, block=blk, O=O, lse=lse)

    n = max(3, args.steps // 100)
    t_sk = graph_time(sketch, 1, n)
    t_sel = graph_time(select, 1, n)
    t_att = graph_time(attend, 1, n)
    tiles = int(cnt.sum().item()) * (Hq // Hkv)
    flops = tiles * 4.0 * blk * blk * D                   # QK^T + PV per 128x128 tile
    # causal-exact: the diagonal tile of each query block holds blk (blk + 1) / 2
    # (query, key) pairs, not blk^2
    diag = B * Hq * M
    flops_exact = (tiles - diag) * 4.0 * blk * blk * D + diag * 4.0 * D * blk * (blk + 1) / 2
    tflops = flops / (t_att * 1e-6) / 1e12
    busy = load_counter_json("mfma_prefill", wl.name, PREFILL_SOURCES)
    res = {
        "workload": wl.name, "us_per_pass": round(t_sk + t_sel + t_att, 2),
        "pass": "key sketch (blocks of 128) + pooled-query selection + MFMA sparse attention",
        "kernels_us": {"sa_build_sketch (k_sketch)": round(t_sk, 2),
                       "sa_select_topk causal (k_sketch pooling Q + k_prefill_select)": round(t_sel, 2),
                       "sa_sparse_prefill (k_prefill_bf16)": round(t_att, 2)},
        "tiles_per_head_group": int(cnt.sum().item()),
        "roofline": {"bound": "mfma", "kernel": "k_prefill_bf16 (bf16 32x32x16 MFMA, fp32 accumulate)",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "flops_per_launch": flops, "avg_us": round(t_att, 2),
                     "causal_exact_flops": flops_exact,
                     "causal_exact_frac": round(flops_exact / (t_att * 1e-6) / 1e12 / 2500.0, 4),
                     "mfma_busy": busy and busy.get("mfma_busy_frac"),
                     "mfma_busy_source": (f"profiles/mfma_prefill_{wl.name}.md: rocprofv3 --pmc "
                                          "SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE of this "
                                          "kernel; null when its sources changed since")},
    }
    if not args.no_cpu:
        # the oracle: selection for every row of every kv head, attention on a row sample
        Q, K, V = (widen(x, wl.dtype) for x in (inp.Q, inp.K, inp.V))
        t0 = time.perf_counter()
        Qb, Kb = oracle.prefill_pool_queries(Q, blk, wl.g), oracle.sketch(K, blk)
        oi, oc = oracle.prefill_select(Qb, Kb, wl.k)
        t_osel = time.perf_counter() - t0
        rng = np.random.default_rng(0)
        rows = [(0, int(h), int(t)) for h, t in zip(rng.integers(0, Hq, 512), rng.integers(0, L, 512))]
        t0 = time.perf_counter()
        oracle.prefill_attend_rows(Q, K, V, oi, oc, blk, rows)
        t_row = (time.perf_counter() - t0) / len(rows)
        res["cpu_baseline"] = {
            "value": round((t_osel + t_row * B * Hq * L) * 1e6, 1), "unit": "us/pass",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"selection of every row timed whole ({t_osel:.1f} s); attention timed "
                      f"on 512 random rows and scaled to all {B * Hq * L} rows"}
    return res


def bench_mass(args) -> dict:
    """The attention-mass selector at the prefill size (dense causal attention,
    one pass per 128 key blocks) and the recall of the sketch selector against
    it over every query block."""
    import numpy as np
    import torch
    import oracle
    import top_sparse_attention_mean_amd as sa
    from oracle.attention import widen
    from tests.parity_util import to_dev
    from workloads import get_workload, make_inputs
    wl = get_workload("sparse_prefill_bf16")
    dev = torch.device("cuda:0")
    inp = make_inputs(wl)
    Qd, Kd = (to_dev(x, wl.dtype, dev) for x in (inp.Q, inp.K))
    B, Hq, Hkv, D, L, blk = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N, wl.block
    M, kf = wl.nb, wl.k - 2
    flags = sa.SA_FORCE_SINK | sa.SA_FORCE_LOCAL | sa.SA_CAUSAL
    sk = sa.sa_build_sketch(Kd, blk)
    sidx, scnt, _ = sa.sa_select_topk(Qd, sk, wl.k, flags=flags, q_block=blk)
    midx = torch.empty(B, Hkv, M, kf, dtype=torch.int32, device=dev)
    mcnt = torch.empty(B, Hkv, M, dtype=torch.int32, device=dev)
    mws = torch.zeros(sa.workspace_bytes(sa.SA_OP_MASS_SELECT, B, Hq, Hkv, L, D, blk, kf),
                      dtype=torch.uint8, device=dev)

    def run(r):
        sa.sa_mass_select(Qd, Kd, kf, block=blk, idx=midx, count=mcnt, ws=mws)

    n = 3
    t_mass = graph_time(run, 1, n, warmup=1)
    # per-query supports once, eagerly: how much of each row's own top-k the
    # block-shared top-k of its query block holds (b_sel = 1 against 128)
    _, _, _, rows = sa.sa_mass_select(Qd, Kd, kf, block=blk, per_row=True, ws=mws)
    torch.cuda.synchronize()
    ri, rc = rows[0].cpu().numpy(), rows[1].cpu().numpy()
    del rows
    mi_all = midx.cpu().numpy()
    shared = []
    for b in range(B):
        for kh in range(Hkv):
            for t in range(2 * blk, L, 7):
                n_r = int(rc[b, kh, t])
                own = set(ri[b, kh, t, :n_r].tolist())
                blk_sel = set(mi_all[b, kh, t // blk].tolist()) - {-1}
                shared.append(len(own & blk_sel) / n_r)
    si, sc = sidx.cpu().numpy(), scnt.cpu().numpy()
    mi, mc = midx.cpu().numpy(), mcnt.cpu().numpy()
    # recall of the sketch selector's free blocks against the mass top-k, over
    # the query blocks i >= 9 of every kv head (below, nearly every earlier
    # block is kept and the recall is 1 by construction)
    rec = []
    for b in range(B):
        for kh in range(Hkv):
            for i in range(9, M):
                want = set(mi[b, kh, i, :mc[b, kh, i]].tolist())
                got = set(si[b, kh, i, :sc[b, kh, i]].tolist()) - {0, i}
                rec.append(len(want & got) / len(want))
    tiles = B * Hkv * M * (M + 1) // 2 * (Hq // Hkv)
    passes = -(-M // 128)
    # QK^T of every causal tile twice: the statistics pass and the mass passes
    # (each chunk's pass scores only that chunk's blocks)
    flops = 2 * tiles * 2.0 * blk * blk * D
    tflops = flops / (t_mass * 1e-6) / 1e12
    res = {
        "workload": wl.name, "us_per_call": round(t_mass, 1), "k_free": kf,
        "dense_passes": passes,
        "sketch_recall_of_mass_topk": round(float(np.mean(rec)), 4),
        "recall_over": f"query blocks 9..{M - 1} of every kv head ({len(rec)} blocks)",
        "per_row_topk_held_by_block_shared_topk": round(float(np.mean(shared)), 4),
        "query_blocks": len(rec),
        "roofline": {"bound": "mfma", "kernel": "k_prefill_bf16 scores of every causal tile, "
                     "twice (row statistics, then block masses; the call also reduces and "
                     "selects)",
                     "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "flops_per_call": flops, "avg_us": round(t_mass, 1)},
    }
    if not args.no_cpu:
        Q, K = (widen(x, wl.dtype) for x in (inp.Q, inp.K))
        qb = [M - 4, M - 3, M - 2, M - 1]
        t0 = time.perf_counter()
        o8 = oracle.mass_oracle(Q, K, blk, k_free=kf, qblocks=qb)
        t_cpu = time.perf_counter() - t0
        # the same recall against O8 itself on these blocks, and whether the GPU
        # mass selector's lists equal O8's there
        r8, same = [], []
        for (b, kh, i), (_, sel8) in o8.items():
            want = set(sel8.tolist())
            got = set(si[b, kh, i, :sc[b, kh, i]].tolist()) - {0, i}
            r8.append(len(want & got) / len(want))
            same.append(want == set(mi[b, kh, i, :mc[b, kh, i]].tolist()))
        res["o8_check"] = {"query_blocks": qb, "kv_heads": Hkv,
                           "sketch_recall_vs_o8": round(float(np.mean(r8)), 4),
                           "gpu_mass_lists_equal_o8": f"{sum(same)}/{len(same)}"}
        work = sum(i + 1 for i in qb) / (M * (M + 1) / 2)
        res["cpu_baseline"] = {"value": round(t_cpu / work * 1e6, 1), "unit": "us/call",
                               "cores": _blas_threads(), "kind": "oracle",
                               "sample": f"the last 4 query blocks of each kv head timed "
                                         f"({t_cpu:.1f} s) and scaled by their share of the "
                                         f"causal work ({work:.4f})"}
    return res


def pmc_run(args) -> dict:
    """Short run for rocprofv3 counter passes: a plain device copy of known size
    (the counters' calibration) and the dominant kernel on every layer copy."""
    import torch
    import top_sparse_attention_mean_amd as sa
    from workloads import get_workload
    wl = get_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nbytes = 256 << 20
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    R = args.layers
    _, Qs, Ks, Vs, sks, _ = _layers(wl, R, dev)
    ws = torch.zeros(sa.workspace_bytes(sa.SA_OP_DECODE_STEP, wl.B, wl.Hq, wl.Hkv, wl.N, wl.D,
                                        wl.block, wl.k), dtype=torch.uint8, device=dev)
    for _ in range(3):
        for r in range(R):
            sa.sa_decode_step(Qs[r], Ks[r], Vs[r], sks[r], wl.k, block=wl.block,
                              update_block=wl.nb - 1, ws=ws)
    torch.cuda.synchronize()
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
            "decode_step_dispatches": 3 * R, "workload": wl.name,
            "source_sha256": kernel_source_hash()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long_decode_bf16")
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--trials", type=int, default=10, help="timed graph replays (median taken)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the threshold, top-delta, pruned, low-bit and prefill variant "
                    "measurements")
    ap.add_argument("--variant",
                    choices=["threshold", "topdelta", "pruned", "lowbit", "prefill", "mass"],
                    help="run only this variant measurement and print its JSON")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short run for rocprofv3 counter passes (no timing output)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the hot path is "
              "single-GPU and no multi-GPU configuration is measured.", file=sys.stderr)
        return 2
    if int(os.environ.get("RANK", "0")) != 0:
        return 0
    if args.pmc_run:
        res = pmc_run(args)
    elif args.variant:
        res = (bench_prefill(args) if args.variant == "prefill" else
               bench_mass(args) if args.variant == "mass" else
               bench_pruned(args) if args.variant == "pruned" else
               bench_lowbit(args) if args.variant == "lowbit" else
               bench_threshold(args, args.variant))
    else:
        res = bench_decode(args)
        if not args.no_variants:
            import gc
            import torch
            # the other decode configurations at their full sizes (reported beside the metric)
            res["configs"] = {}
            for nm, calls, layers in (("tiny_decode_f32", 200, 4), ("gqa_decode_bf16", 200, 8)):
                gc.collect()
                torch.cuda.empty_cache()
                c = bench_decode(args, name=nm, calls=calls, layers=layers, extras=False)
                res["configs"][nm] = {k2: c[k2] for k2 in (
                    "value", "unit", "dtype", "config", "trials", "achieved_GBps",
                    "pct_of_hbm_peak", "algorithmic_bytes_per_step", "roofline", "cpu_baseline")
                    if k2 in c}
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"] = {"threshold": bench_threshold(args)}
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"]["topdelta"] = bench_threshold(args, "topdelta")
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"]["pruned"] = bench_pruned(args)
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"]["lowbit"] = bench_lowbit(args)
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"]["prefill"] = bench_prefill(args)
            gc.collect()
            torch.cuda.empty_cache()
            res["variants"]["mass"] = bench_mass(args)
            mv = res["variants"]["mass"]
            res["mass_recall"] = {
                "value": mv["sketch_recall_of_mass_topk"],
                "what": "recall of the pooled-sketch prefill selector's 8 free blocks against "
                        "the attention-mass top-8 (O8's rule), mean over " + mv["recall_over"] +
                        " of sparse_prefill_bf16; masses from the GPU mass selector, whose "
                        "lists are checked against the CPU oracle O8 in o8_check",
                "o8_check": mv.get("o8_check")}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
