"""Seeded generators for the workloads in :mod:`workloads.configs`.

Recipe (identical for every workload, so a reader can regenerate any array):

1. ``rng = numpy.random.Generator(numpy.random.PCG64(seed))``.
2. Draw Q, then K, then V as standard normal float32, each in layout order.
3. Clusters (if cluster_spread > 0): draw mu ~ N(0, 1) of shape
   [B, Hkv, nb, D]; the keys of block j become mu_j + cluster_spread * K.
3b. Outlier channels (if any): for each kv head in order, draw that many
   distinct channels uniformly; multiply K and V in those channels by the
   outlier scale.  The channels are shared by every batch row.
4. Positional drift (if any): for K, then V, draw eps ~ N(0, drift_var) of shape
   [B, Hkv, nb, D]; mu_0 = eps_0, mu_j = rho * mu_{j-1} + sqrt(1 - rho^2) eps_j
   (an AR(1) with marginal N(0, drift_var)); add mu_j to every token of block j.
5. Needles, drawn last and added last:
   * decode: for each (b, kv head), ``needles`` distinct blocks from
     [1, nb-2]; every key of such a block gets + gain * q_hat, q_hat being the
     unit-length mean of the group's query heads;
   * decode with anchor_gain > 0 (top-delta workloads): then the first
     ``sink`` and the last ``local`` keys of every (b, kv head) also get
     + anchor_gain * q_hat (no draws, so the other arrays are unchanged);
   * prefill: for each (b, kv head), ``needles`` distinct key blocks j from
     [1, nb-2], then for each a partner query block i drawn uniformly from
     [j+1, nb-1]; every key of block j gets + gain * q_hat_i, q_hat_i being the
     unit-length mean of Q over block i's tokens and the group's heads.
6. bf16 workloads round every array once, at the end, to bf16 with
   round-to-nearest-even and keep the raw 16-bit patterns (uint16).

The draws are always made in float32; needles use the float32 queries.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Union

import numpy as np

from .configs import Workload, get_workload


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return the uint16 bits.

    Inputs here are finite; the rounding is done on the IEEE bit pattern:
    add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24  # chunking keeps the uint64 temporaries small
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step].astype(np.uint64)
        v = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        flat_o[s:s + step] = v.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- containers
@dataclass
class DecodeInputs:
    wl: Workload
    Q: np.ndarray            # [B, Hq, D]     float32 or uint16 (bf16 bits)
    K: np.ndarray            # [B, Hkv, N, D]
    V: np.ndarray            # [B, Hkv, N, D]
    needles: np.ndarray      # [B, Hkv, n_needles] int64 block ids
    outlier_channels: Optional[np.ndarray] = None  # [Hkv, n_out]

    @property
    def dtype(self) -> str:
        return self.wl.dtype


@dataclass
class PrefillInputs:
    wl: Workload
    Q: np.ndarray            # [B, Hq, L, D]
    K: np.ndarray            # [B, Hkv, L, D]
    V: np.ndarray            # [B, Hkv, L, D]
    needles: np.ndarray      # [B, Hkv, n_needles] key block ids j
    partners: np.ndarray     # [B, Hkv, n_needles] query block ids i (> j)

    @property
    def dtype(self) -> str:
        return self.wl.dtype


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def _drift(rng: np.random.Generator, X: np.ndarray, wl: Workload) -> None:
    """Add an AR(1) per-block mean offset to X [B, Hkv, N, D] in place."""
    B, H, N, D = X.shape
    nb = -(-N // wl.block)
    sd = np.float32(np.sqrt(wl.drift_var))
    eps = rng.standard_normal((B, H, nb, D), dtype=np.float32) * sd
    mu = np.empty_like(eps)
    mu[:, :, 0] = eps[:, :, 0]
    a = np.float32(wl.drift_rho)
    c = np.float32(np.sqrt(1.0 - wl.drift_rho ** 2))
    for j in range(1, nb):
        mu[:, :, j] = a * mu[:, :, j - 1] + c * eps[:, :, j]
    for j in range(nb):
        X[:, :, j * wl.block:(j + 1) * wl.block, :] += mu[:, :, j][:, :, None, :]


def make_decode_inputs(wl: Workload, seed: Optional[int] = None) -> DecodeInputs:
    if wl.kind not in ("decode_topk", "decode_threshold", "decode_topdelta"):
        raise ValueError(f"{wl.name} is not a decode workload")
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, Hq, Hkv, D, N = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N
    g, nb = wl.g, wl.nb
    Q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    K = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)

    if wl.cluster_spread > 0:
        mu = rng.standard_normal((B, Hkv, nb, D), dtype=np.float32)
        w = np.float32(wl.cluster_spread)
        for j in range(nb):
            K[:, :, j * wl.block:(j + 1) * wl.block] = (
                mu[:, :, j][:, :, None, :] + w * K[:, :, j * wl.block:(j + 1) * wl.block])

    outl = None
    if wl.outlier_channels:
        outl = np.stack([rng.choice(D, size=wl.outlier_channels, replace=False)
                         for _ in range(Hkv)])
        s = np.float32(wl.outlier_scale)
        for kh in range(Hkv):
            K[:, kh, :, outl[kh]] *= s
            V[:, kh, :, outl[kh]] *= s

    if wl.drift_var > 0:
        _drift(rng, K, wl)
        _drift(rng, V, wl)

    n_need = min(wl.needles, max(nb - 2, 0))
    needles = np.zeros((B, Hkv, n_need), dtype=np.int64)
    for b in range(B):
        for kh in range(Hkv):
            if n_need:
                needles[b, kh] = rng.choice(np.arange(1, nb - 1), size=n_need, replace=False)
    gain = np.float32(wl.needle_gain)
    for b in range(B):
        for kh in range(Hkv):
            qm = Q[b, kh * g:(kh + 1) * g].mean(axis=0, dtype=np.float64)
            qhat = (qm / np.linalg.norm(qm)).astype(np.float32)
            for j in needles[b, kh]:
                K[b, kh, j * wl.block:min((j + 1) * wl.block, N)] += gain * qhat
            if wl.anchor_gain > 0:
                a = np.float32(wl.anchor_gain) * qhat
                K[b, kh, :min(wl.sink, N)] += a
                K[b, kh, max(N - wl.local, 0):] += a

    return DecodeInputs(wl, _store(Q, wl.dtype), _store(K, wl.dtype),
                        _store(V, wl.dtype), needles, outl)


def make_prefill_inputs(wl: Workload, seed: Optional[int] = None) -> PrefillInputs:
    if wl.kind != "prefill":
        raise ValueError(f"{wl.name} is not a prefill workload")
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, Hq, Hkv, D, L = wl.B, wl.Hq, wl.Hkv, wl.D, wl.N
    g, nb, blk = wl.g, wl.nb, wl.block
    Q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    K = rng.standard_normal((B, Hkv, L, D), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, L, D), dtype=np.float32)

    n_need = min(wl.needles, max(nb - 2, 0))
    needles = np.zeros((B, Hkv, n_need), dtype=np.int64)
    partners = np.zeros((B, Hkv, n_need), dtype=np.int64)
    for b in range(B):
        for kh in range(Hkv):
            if n_need:
                js = rng.choice(np.arange(1, nb - 1), size=n_need, replace=False)
                needles[b, kh] = js
                partners[b, kh] = [rng.integers(j + 1, nb) for j in js]
    gain = np.float32(wl.needle_gain)
    for b in range(B):
        for kh in range(Hkv):
            for j, i in zip(needles[b, kh], partners[b, kh]):
                qm = Q[b, kh * g:(kh + 1) * g, i * blk:min((i + 1) * blk, L)].mean(
                    axis=(0, 1), dtype=np.float64)
                qhat = (qm / np.linalg.norm(qm)).astype(np.float32)
                K[b, kh, j * blk:min((j + 1) * blk, L)] += gain * qhat

    return PrefillInputs(wl, _store(Q, wl.dtype), _store(K, wl.dtype),
                         _store(V, wl.dtype), needles, partners)


def make_inputs(wl: Union[Workload, str], seed: Optional[int] = None, **overrides):
    if isinstance(wl, str):
        wl = get_workload(wl, **overrides)
    elif overrides:
        wl = wl.scaled(**overrides)
    if wl.kind == "prefill":
        return make_prefill_inputs(wl, seed)
    return make_decode_inputs(wl, seed)
