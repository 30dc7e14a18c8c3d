"""The workloads of the hot path, by name and shape.

Every workload is a single-layer attention problem over a GQA KV cache laid out
as K, V = [B, Hkv, N, D] and Q = [B, Hq, D] (decode) or [B, Hq, L, D]
(prefill), row-major with D innermost.  Query head h reads kv head h // g,
g = Hq // Hkv.

Needle blocks ("planted" blocks whose keys are pushed towards the group's mean
query) give every selector a known set of blocks it must recover.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "decode_topk" | "decode_threshold" | "decode_topdelta" | "prefill"
    B: int
    Hq: int
    Hkv: int
    D: int
    N: int                    # cached keys (decode) or sequence length L (prefill)
    block: int                # tokens per key block (and per query block in prefill)
    k: int                    # blocks kept per (b, kv head) [per query block in prefill]
    dtype: str                # "f32" | "bf16"
    seed: int
    needles: int              # planted blocks per (b, kv head)
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    drift_var: float = 0.0    # marginal variance of the per-block mean offset
    drift_rho: float = 0.0    # AR(1) coefficient of the drift across blocks
    needle_gain: float = 3.0  # planted keys get + needle_gain * unit query
    percentile: float = 99.0  # threshold workload: per-head score percentile
    cap: int = 1024           # threshold workloads: list capacity per head
    sink: int = 0             # top-delta: leading tokens of the pseudo-max window
    local: int = 0            # top-delta: trailing tokens of the pseudo-max window
    delta: float = 0.0        # top-delta: keep s >= pseudo-max - delta
    anchor_gain: float = 0.0  # sink and local keys get + anchor_gain * unit query
    margin: float = 0.0       # low-bit top-delta: filter at tau - margin
    cluster_spread: float = 0.0  # > 0: keys of block j = mu_j + cluster_spread * noise
    subspaces: int = 1        # pruned threshold: contiguous key subspaces per sphere set
    extra: dict = field(default_factory=dict)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    def scaled(self, **kw) -> "Workload":
        """Same recipe at another size (used for fast parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    # B=1, Hq=4, Hkv=1, d=64, N=4096, 64-token blocks, keep 8 incl. sink+local.
    "tiny_decode_f32": Workload(
        name="tiny_decode_f32", kind="decode_topk", B=1, Hq=4, Hkv=1, D=64,
        N=4096, block=64, k=8, dtype="f32", seed=1, needles=3),
    # B=8, Hq=32, Hkv=8, d=128, N=32K, keep 64 of 512 blocks; 4 outlier
    # channels per kv head scaled x8 in K and V; 16 needles per (b, kv head).
    "gqa_decode_bf16": Workload(
        name="gqa_decode_bf16", kind="decode_topk", B=8, Hq=32, Hkv=8, D=128,
        N=32768, block=64, k=64, dtype="bf16", seed=2, needles=16,
        outlier_channels=4, outlier_scale=8.0),
    # B=1, Hq=64, Hkv=8, d=128, N=256K, keep 82 of 4096 blocks (~2 %);
    # slow AR(1) positional drift of the per-block mean; 32 needles per kv head.
    "long_decode_bf16": Workload(
        name="long_decode_bf16", kind="decode_topk", B=1, Hq=64, Hkv=8, D=128,
        N=262144, block=64, k=82, dtype="bf16", seed=3, needles=32,
        drift_var=0.25, drift_rho=0.99),
    # Same arrays as gqa_decode_bf16; keep every token whose exact score is at
    # least the per-head 99th percentile (~1 % of tokens).
    "threshold_decode_bf16": Workload(
        name="threshold_decode_bf16", kind="decode_threshold", B=8, Hq=32,
        Hkv=8, D=128, N=32768, block=64, k=0, dtype="bf16", seed=2,
        needles=16, outlier_channels=4, outlier_scale=8.0, percentile=99.0,
        cap=1024),
    # The GQA decode shapes and draws with attention concentrated on the sink
    # and local tokens, as "Faster Than Flash" (Metodologia §2) reports of real
    # models: the first 64 and last 64 keys of every kv head, and the needle
    # blocks, get + 16 * q_hat.  Keep every token within delta = 5 of the
    # pseudo-max over those 128 tokens (about 2 % of the cache on these draws).
    "topdelta_decode_bf16": Workload(
        name="topdelta_decode_bf16", kind="decode_topdelta", B=8, Hq=32,
        Hkv=8, D=128, N=32768, block=64, k=0, dtype="bf16", seed=2,
        needles=16, outlier_channels=4, outlier_scale=8.0, needle_gain=16.0,
        cap=4096, sink=64, local=64, delta=5.0, anchor_gain=16.0),
    # The threshold selection over keys that form compact clusters, the
    # setting in which "Sparse Attention as a Range Searching Problem"
    # (Metodologia §2) prunes whole clusters by their bounding spheres: the
    # keys of block j are mu_j + 0.05 * noise with mu_j ~ N(0, I).  Same
    # shapes as the GQA decode config; tau = per-head 99th percentile.
    "clustered_threshold_bf16": Workload(
        name="clustered_threshold_bf16", kind="decode_threshold", B=8, Hq=32,
        Hkv=8, D=128, N=32768, block=64, k=0, dtype="bf16", seed=4,
        needles=16, percentile=99.0, cap=1024, cluster_spread=0.05, subspaces=1),
    # The top-delta arrays, scanned through 2-bit key thumbnails with 8-bit
    # residuals ("Faster Than Flash", Metodologia §1, §3): a block stays when
    # a provisional score reaches tau - 1 for some head of the group.
    "lowbit_topdelta_bf16": Workload(
        name="lowbit_topdelta_bf16", kind="decode_topdelta", B=8, Hq=32,
        Hkv=8, D=128, N=32768, block=64, k=0, dtype="bf16", seed=2,
        needles=16, outlier_channels=4, outlier_scale=8.0, needle_gain=16.0,
        cap=512, sink=64, local=64, delta=5.0, anchor_gain=16.0, margin=1.0),
    # B=1, Hq=32, Hkv=4, d=128, L=64K, 128-token query and key blocks; each
    # query block keeps block 0, its diagonal block and the top-8 earlier blocks.
    "sparse_prefill_bf16": Workload(
        name="sparse_prefill_bf16", kind="prefill", B=1, Hq=32, Hkv=4, D=128,
        N=65536, block=128, k=10, dtype="bf16", seed=5, needles=64),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.scaled(**overrides) if overrides else w
