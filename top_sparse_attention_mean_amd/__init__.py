"""Python binding of the gfx950 top-k block-sparse attention library (libsa.so).

Argument marshalling only: every function takes torch tensors that live on the
GPU, passes their device pointers and the current HIP stream to the C ABI in
``include/sa.h`` and raises if the library reports an error.  All arithmetic
runs in the library's HIP kernels; there is no CPU fallback, and importing this
module fails loudly when ``libsa.so`` has not been built.

bf16 tensors are passed as ``torch.bfloat16`` (raw 16-bit patterns); float32 as
``torch.float32``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python top_sparse_attention_mean_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_F32, SA_BF16 = 0, 1
SA_FORCE_SINK, SA_FORCE_LOCAL, SA_CAUSAL = 1, 2, 4
SA_IDX_BLOCKS, SA_IDX_TOKENS = 0, 1
(SA_OP_SELECT_TOPK, SA_OP_SELECT_THRESHOLD, SA_OP_SPARSE_DECODE, SA_OP_DECODE_STEP,
 SA_OP_SELECT_TOPDELTA, SA_OP_SELECT_PRUNED, SA_OP_SELECT_LOWBIT, SA_OP_MASS_SELECT,
 SA_OP_DECODE_LOWBIT) = range(9)

EXPORTS = ["sa_build_sketch", "sa_build_radius", "sa_encode_keys", "sa_decode_keys",
           "sa_select_topk", "sa_select_threshold", "sa_select_topdelta",
           "sa_select_threshold_pruned", "sa_select_topdelta_lowbit", "sa_decode_topdelta_lowbit",
           "sa_mass_select",
           "sa_sparse_decode",
           "sa_sparse_prefill", "sa_select_decode", "sa_decode_step", "sa_decode_step_noalloc",
           "sa_workspace_bytes",
           "sa_status_str",
           "sa_last_error", "sa_version"]

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_U = ctypes.c_uint


def _sig(name, restype, *args):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(args)
    return f


_build_sketch = _sig("sa_build_sketch", _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P)
_select_topk = _sig("sa_select_topk", _I, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I, _U, _F,
                    _P, _P, _P, _P, _Z, _P)
_select_threshold = _sig("sa_select_threshold", _I, _P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _I,
                         _P, _P, _P, _P, _Z, _P)
_build_radius = _sig("sa_build_radius", _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P)
_select_threshold_pruned = _sig("sa_select_threshold_pruned", _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                _I, _I, _P, _P, _P, _F, _I, _P, _P, _P, _P, _P, _Z, _P)
_encode_keys = _sig("sa_encode_keys", _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P)
_decode_keys = _sig("sa_decode_keys", _I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _I, _P,
                    _P)
_select_topdelta_lowbit = _sig("sa_select_topdelta_lowbit", _I, _P, _P, _P, _P, _I, _I, _I, _I,
                               _I, _I, _I, _I, _F, _F, _F, _I, _P, _P, _P, _P, _P, _P, _Z, _P)
_decode_topdelta_lowbit = _sig("sa_decode_topdelta_lowbit", _I, _P, _P, _P, _P, _P, _I, _I, _I,
                               _I, _I, _I, _I, _I, _F, _F, _F, _I, _P, _P, _P, _P, _P, _P, _I,
                               _P, _P, _Z, _P)
_mass_select = _sig("sa_mass_select", _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                    _P, _P, _P, _P, _Z, _P)
_select_topdelta = _sig("sa_select_topdelta", _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                        _F, _I, _P, _P, _P, _P, _P, _Z, _P)
_sparse_decode = _sig("sa_sparse_decode", _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                      _P, _P, _I, _P, _P, _I, _P, _P, _Z, _P)
_sparse_prefill = _sig("sa_sparse_prefill", _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                       _P, _I, _P, _I, _P, _P)
_decode_step = _sig("sa_decode_step", _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _I, _F,
                    _P, _P, _P, _P, _I, _P, _P, _Z, _P)
_decode_step_noalloc = _sig("sa_decode_step_noalloc", _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                            _P, _I, _I, _F, _P, _P, _P, _P, _I, _P, _P)
_select_decode = _sig("sa_select_decode", _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _U,
                      _F, _P, _P, _P, _I, _P, _P, _Z, _P)
_workspace_bytes = _sig("sa_workspace_bytes", _Z, _I, _I, _I, _I, _I, _I, _I, _I)
_status_str = _sig("sa_status_str", ctypes.c_char_p, _I)
_last_error = _sig("sa_last_error", ctypes.c_char_p)
_version = _sig("sa_version", _I)


class SAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _status_str(status).decode()
        detail = _last_error().decode()
        super().__init__(f"{where}: {msg}: {detail}")


def _check(st: int, where: str) -> None:
    if st != SA_OK:
        raise SAError(st, where)


def version() -> int:
    return _version()


def workspace_bytes(op: int, B: int, Hq: int, Hkv: int, N: int, D: int, block: int, k: int) -> int:
    n = _workspace_bytes(op, B, Hq, Hkv, N, D, block, k)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace query")
    return n


# ------------------------------------------------------------------ helpers
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    dev = None
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"tensors must live on one device ({dev} and {t.device})")


_FP = (torch.bfloat16, torch.float32)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _need(t: Optional[torch.Tensor], name: str, shape=None, dtypes=None) -> None:
    """Raise ValueError unless t (when given) has this shape and one of these
    dtypes.  Runs before anything is launched: a wrong size or element type
    would otherwise make a kernel read or write past the end of a buffer."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)} "
                         f"(got {t.dtype})")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _rank(t: torch.Tensor, name: str, n: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions (got shape {tuple(t.shape)})")


def _qk_shapes(Q: torch.Tensor, K: torch.Tensor):
    """(B, Hq, D, Hkv, N) of a decode query [B, Hq, D] and a cache [B, Hkv, N, D]
    of the same dtype."""
    _rank(Q, "Q", 3)
    _rank(K, "K", 4)
    B, Hq, D = Q.shape
    Hkv, N = K.shape[1], K.shape[2]
    _need(Q, "Q", None, _FP)
    _need(K, "K", (B, Hkv, N, D), (Q.dtype,))
    return B, Hq, D, Hkv, N


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


_ws_cache = {}


def workspace(nbytes: int, device, key=()) -> torch.Tensor:
    """A zero-filled device workspace of at least nbytes, one per (device, key).

    The library keeps arrival counters and histograms in the workspace and
    leaves them at zero after every call, so a workspace may be reused by
    later calls of the same operation and shape (the key); a different layout
    gets its own buffer.
    """
    k = (torch.device(device), tuple(key))
    ws = _ws_cache.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=k[0])
        _ws_cache[k] = ws
    return ws


# ------------------------------------------------------------------ entry points
def sa_build_sketch(X: torch.Tensor, block: int, head_pool: int = 1, blk_begin: int = 0,
                    blk_end: Optional[int] = None, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Per-block mean sketch of X [B, H, N, D] -> float32 [B, H/head_pool, nb, D]."""
    _rank(X, "X", 4)
    _need(X, "X", None, _FP)
    B, H, N, D = X.shape
    nb = -(-N // block)
    if head_pool < 1 or H % head_pool:
        raise ValueError(f"head_pool ({head_pool}) must divide H ({H})")
    _need(out, "out", (B, H // head_pool, nb, D), _F32)
    _dev(X, out)
    if blk_end is None:
        blk_end = nb
    if out is None:
        out = torch.empty(B, H // head_pool, nb, D, dtype=torch.float32, device=X.device)
    _check(_build_sketch(_ptr(X), _dt(X), B, H, N, D, block, head_pool, blk_begin, blk_end,
                         _ptr(out), _stream(stream)), "sa_build_sketch")
    return out


def sa_build_radius(X: torch.Tensor, sketch: torch.Tensor, block: int, S: int = 1,
                    blk_begin: int = 0, blk_end: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Bounding-sphere radii of X [B, H, N, D] around its block sketch
    [B, H, nb, D], per subspace of D/S channels -> float32 [B, H, nb, S]
    (only blocks [blk_begin, blk_end) are written)."""
    _rank(X, "X", 4)
    _need(X, "X", None, _FP)
    B, H, N, D = X.shape
    nb = -(-N // block)
    _need(sketch, "sketch", (B, H, nb, D), _F32)
    _need(out, "out", (B, H, nb, S), _F32)
    _dev(X, sketch, out)
    if blk_end is None:
        blk_end = nb
    if out is None:
        out = torch.empty(B, H, nb, S, dtype=torch.float32, device=X.device)
    _check(_build_radius(_ptr(X), _dt(X), B, H, N, D, block, S, blk_begin, blk_end, _ptr(sketch),
                         _ptr(out), _stream(stream)), "sa_build_radius")
    return out


def sa_encode_keys(K: torch.Tensor, block: int, blk_begin: int = 0,
                   blk_end: Optional[int] = None, codes=None, resid=None, meta=None,
                   stream=None):
    """2-bit thumbnails + 8-bit residuals of K [B, H, N, D] -> codes uint8
    [B, H, N, D/4], resid int8 [B, H, N, D], meta float32 [B, H, nb, 3, D]."""
    _rank(K, "K", 4)
    _need(K, "K", None, _FP)
    B, H, N, D = K.shape
    nb = -(-N // block)
    _need(codes, "codes", (B, H, N, D // 4), (torch.uint8,))
    _need(resid, "resid", (B, H, N, D), (torch.int8,))
    _need(meta, "meta", (B, H, nb, 3, D), _F32)
    _dev(K, codes, resid, meta)
    if blk_end is None:
        blk_end = nb
    dev = K.device
    if codes is None:
        codes = torch.zeros(B, H, N, D // 4, dtype=torch.uint8, device=dev)
    if resid is None:
        resid = torch.zeros(B, H, N, D, dtype=torch.int8, device=dev)
    if meta is None:
        meta = torch.zeros(B, H, nb, 3, D, dtype=torch.float32, device=dev)
    _check(_encode_keys(_ptr(K), _dt(K), B, H, N, D, block, blk_begin, blk_end, _ptr(codes),
                        _ptr(resid), _ptr(meta), _stream(stream)), "sa_encode_keys")
    return codes, resid, meta


def sa_decode_keys(codes: torch.Tensor, resid: torch.Tensor, meta: torch.Tensor, block: int,
                   idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                   blk_begin: int = 0, blk_end: Optional[int] = None,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Refined bf16 keys of the listed blocks (or a block range) into out
    [B, H, N, D] (zeros elsewhere when out is allocated here)."""
    _rank(resid, "resid", 4)
    _need(resid, "resid", None, (torch.int8,))
    B, H, N, D = resid.shape
    nb = -(-N // block)
    _need(codes, "codes", (B, H, N, D // 4), (torch.uint8,))
    _need(meta, "meta", (B, H, nb, 3, D), _F32)
    if idx is not None:
        _rank(idx, "idx", 3)
        _need(idx, "idx", (B, H, idx.shape[-1]), _I32)
        if count is None:
            raise ValueError("a block list needs its count")
    _need(count, "count", (B, H), _I32)
    _need(out, "out", (B, H, N, D), (torch.bfloat16,))
    _dev(codes, resid, meta, idx, count, out)
    if blk_end is None:
        blk_end = nb
    if out is None:
        out = torch.zeros(B, H, N, D, dtype=torch.bfloat16, device=codes.device)
    stride = idx.shape[-1] if idx is not None else 0
    _check(_decode_keys(_ptr(codes), _ptr(resid), _ptr(meta), B, H, N, D, block, _ptr(idx),
                        _ptr(count), stride, blk_begin, blk_end, _ptr(out), _stream(stream)),
           "sa_decode_keys")
    return out


def sa_select_topk(Q: torch.Tensor, ksketch: torch.Tensor, k: int,
                   flags: int = SA_FORCE_SINK | SA_FORCE_LOCAL, scale: float = 0.0,
                   Hkv: Optional[int] = None, q_block: int = 1,
                   idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                   score: Optional[torch.Tensor] = None, want_score: bool = False,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """Top-k block selection.

    Decode: Q [B, Hq, D] -> idx [B, Hkv, k], count [B, Hkv] (score [B, Hkv, nb]).
    Causal prefill (flags & SA_CAUSAL): Q [B, Hq, L, D], q_block = key block ->
    idx [B, Hkv, M, k], count [B, Hkv, M] (score [B, Hkv, M, nb]).
    """
    _rank(ksketch, "ksketch", 4)
    _need(ksketch, "ksketch", None, _F32)
    B, Hkv_, nb, D = ksketch.shape
    Hkv = Hkv or Hkv_
    causal = bool(flags & SA_CAUSAL)
    _rank(Q, "Q", 4 if causal else 3)
    Hq = Q.shape[1]
    Lq = Q.shape[2] if causal else 1
    _need(Q, "Q", (B, Hq, Lq, D) if causal else (B, Hq, D), _FP)
    if causal and Hkv != Hkv_:
        raise ValueError(f"the key sketch has {Hkv_} kv heads, Hkv = {Hkv}")
    M = -(-Lq // q_block)
    rows = (B, Hkv, M) if causal else (B, Hkv)
    _need(idx, "idx", (*rows, k), _I32)
    _need(count, "count", rows, _I32)
    _need(score, "score", (*rows, nb), _F32)
    _dev(Q, ksketch, idx, count, score)
    if idx is None:
        idx = torch.empty(*rows, k, dtype=torch.int32, device=Q.device)
    if count is None:
        count = torch.empty(*rows, dtype=torch.int32, device=Q.device)
    if score is None and want_score:
        score = torch.empty(*rows, nb, dtype=torch.float32, device=Q.device)
    need = workspace_bytes(SA_OP_SELECT_TOPK, B, Hq, Hkv, Lq, D, q_block, nb)
    if ws is None:
        ws = workspace(need, Q.device, ("select", B, Hq, Hkv, Lq, D, q_block, nb))
    _check(_select_topk(_ptr(Q), _dt(Q), B, Hq, Hkv, Lq, D, q_block, _ptr(ksketch), nb, k, flags,
                        scale, _ptr(idx), _ptr(count), _ptr(score), _ptr(ws), ws.numel(),
                        _stream(stream)), "sa_select_topk")
    return idx, count, score


def sa_select_threshold(Q: torch.Tensor, K: torch.Tensor, tau: torch.Tensor, cap: int,
                        scale: float = 0.0, idx=None, score=None, count=None, ws=None,
                        stream=None):
    """Half-space selection: every token with q . k * scale >= tau[b, h].

    Returns idx [B, Hq, cap] (ascending, -1 padded), score [B, Hq, cap] and
    count [B, Hq] (the true count, which may exceed cap).
    """
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    _need(tau, "tau", (B, Hq), _F32)
    _need(idx, "idx", (B, Hq, cap), _I32)
    _need(score, "score", (B, Hq, cap), _F32)
    _need(count, "count", (B, Hq), _I32)
    _dev(Q, K, tau, idx, score, count)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hq, cap, dtype=torch.int32, device=dev)
    if score is None:
        score = torch.empty(B, Hq, cap, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    need = workspace_bytes(SA_OP_SELECT_THRESHOLD, B, Hq, Hkv, N, D, 0, cap)
    if ws is None:
        ws = workspace(need, dev, ("threshold", B, Hq, Hkv, N, D, cap))
    _check(_select_threshold(_ptr(Q), _ptr(K), _dt(Q), B, Hq, Hkv, N, D, _ptr(tau), scale, cap,
                             _ptr(idx), _ptr(score), _ptr(count), _ptr(ws), ws.numel(),
                             _stream(stream)), "sa_select_threshold")
    return idx, score, count


def sa_select_threshold_pruned(Q: torch.Tensor, K: torch.Tensor, sketch: torch.Tensor,
                               radius: torch.Tensor, tau: torch.Tensor, cap: int, block: int,
                               scale: float = 0.0, idx=None, score=None, count=None, live=None,
                               ws=None, stream=None):
    """Half-space selection with blocks pruned by their bounding spheres first.

    sketch [B, Hkv, nb, D] and radius [B, Hkv, nb, S] as built on K.  Returns
    idx, score, count (as sa_select_threshold) and live [B, Hkv, ceil(N/128)]
    uint8: bit i of a 128-token segment's byte is set when its i-th block was
    scanned.
    """
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    nb = -(-N // block)
    _rank(radius, "radius", 4)
    S = radius.shape[-1]
    _need(sketch, "sketch", (B, Hkv, nb, D), _F32)
    _need(radius, "radius", (B, Hkv, nb, S), _F32)
    _need(tau, "tau", (B, Hq), _F32)
    _need(idx, "idx", (B, Hq, cap), _I32)
    _need(score, "score", (B, Hq, cap), _F32)
    _need(count, "count", (B, Hq), _I32)
    _need(live, "live", (B, Hkv, -(-N // 128)), (torch.uint8,))
    _dev(Q, K, sketch, radius, tau, idx, score, count, live)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hq, cap, dtype=torch.int32, device=dev)
    if score is None:
        score = torch.empty(B, Hq, cap, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    if live is None:
        live = torch.empty(B, Hkv, -(-N // 128), dtype=torch.uint8, device=dev)
    need = workspace_bytes(SA_OP_SELECT_PRUNED, B, Hq, Hkv, N, D, block, cap)
    if ws is None:
        ws = workspace(need, dev, ("pruned", B, Hq, Hkv, N, D, cap))
    _check(_select_threshold_pruned(_ptr(Q), _ptr(K), _dt(Q), B, Hq, Hkv, N, D, block, S,
                                    _ptr(sketch), _ptr(radius), _ptr(tau), scale, cap,
                                    _ptr(idx), _ptr(score), _ptr(count), _ptr(live), _ptr(ws),
                                    ws.numel(), _stream(stream)), "sa_select_threshold_pruned")
    return idx, score, count, live


def sa_select_topdelta_lowbit(Q: torch.Tensor, codes: torch.Tensor, resid: torch.Tensor,
                              meta: torch.Tensor, block: int, sink: int, local: int, delta: float,
                              margin: float, kcap: int, scale: float = 0.0, khat=None, idx=None,
                              count=None, tau=None, want_bmax: bool = False, ws=None,
                              stream=None):
    """Top-delta block filter over 2-bit thumbnails; refined keys of the kept
    blocks into khat.  Returns idx [B, Hkv, kcap], count [B, Hkv], tau [B, Hq],
    bmax [B, Hq, nb] (or None) and khat [B, Hkv, N, D] bf16."""
    _rank(Q, "Q", 3)
    _rank(resid, "resid", 4)
    B, Hq, D = Q.shape
    _, Hkv, N, _ = resid.shape
    nb = -(-N // block)
    _need(Q, "Q", None, (torch.bfloat16,))
    _need(resid, "resid", (B, Hkv, N, D), (torch.int8,))
    _need(codes, "codes", (B, Hkv, N, D // 4), (torch.uint8,))
    _need(meta, "meta", (B, Hkv, nb, 3, D), _F32)
    _need(khat, "khat", (B, Hkv, N, D), (torch.bfloat16,))
    _need(idx, "idx", (B, Hkv, kcap), _I32)
    _need(count, "count", (B, Hkv), _I32)
    _need(tau, "tau", (B, Hq), _F32)
    _dev(Q, codes, resid, meta, khat, idx, count, tau)
    dev = Q.device
    if khat is None:
        khat = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device=dev)
    if idx is None:
        idx = torch.empty(B, Hkv, kcap, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if tau is None:
        tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    bmax = torch.empty(B, Hq, nb, dtype=torch.float32, device=dev) if want_bmax else None
    need = workspace_bytes(SA_OP_SELECT_LOWBIT, B, Hq, Hkv, N, D, block, kcap)
    if ws is None:
        ws = workspace(need, dev, ("lowbit", B, Hq, Hkv, N, D, block))
    _check(_select_topdelta_lowbit(_ptr(Q), _ptr(codes), _ptr(resid), _ptr(meta), B, Hq, Hkv, N,
                                   D, block, sink, local, delta, margin, scale, kcap, _ptr(idx),
                                   _ptr(count), _ptr(tau), _ptr(bmax), _ptr(khat), _ptr(ws),
                                   ws.numel(), _stream(stream)), "sa_select_topdelta_lowbit")
    return idx, count, tau, bmax, khat


def sa_decode_topdelta_lowbit(Q: torch.Tensor, codes: torch.Tensor, resid: torch.Tensor,
                              meta: torch.Tensor, V: torch.Tensor, block: int, sink: int,
                              local: int, delta: float, margin: float, kcap: int,
                              scale: float = 0.0, out_dtype=None, khat=None, idx=None,
                              count=None, tau=None, O=None, lse=None, want_bmax: bool = False,
                              want_lse: bool = True, ws=None, stream=None):
    """The whole low-bit top-delta decode: the thumbnail filter, then the
    split-K attention over the kept blocks with their keys rebuilt from codes
    and residuals inside the kernel.  Returns O [B, Hq, D], lse [B, Hq], idx,
    count, tau and bmax (or None); khat holds only the window blocks' rows."""
    _rank(Q, "Q", 3)
    _rank(resid, "resid", 4)
    B, Hq, D = Q.shape
    _, Hkv, N, _ = resid.shape
    nb = -(-N // block)
    _need(Q, "Q", None, (torch.bfloat16,))
    _need(resid, "resid", (B, Hkv, N, D), (torch.int8,))
    _need(codes, "codes", (B, Hkv, N, D // 4), (torch.uint8,))
    _need(meta, "meta", (B, Hkv, nb, 3, D), _F32)
    _need(V, "V", (B, Hkv, N, D), (torch.bfloat16,))
    _need(khat, "khat", (B, Hkv, N, D), (torch.bfloat16,))
    _need(idx, "idx", (B, Hkv, kcap), _I32)
    _need(count, "count", (B, Hkv), _I32)
    _need(tau, "tau", (B, Hq), _F32)
    _need(O, "O", (B, Hq, D), (out_dtype,) if out_dtype else _FP)
    _need(lse, "lse", (B, Hq), _F32)
    _dev(Q, codes, resid, meta, V, khat, idx, count, tau, O, lse)
    dev = Q.device
    if khat is None:
        khat = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device=dev)
    if idx is None:
        idx = torch.empty(B, Hkv, kcap, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if tau is None:
        tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    if O is None:
        O = torch.empty(B, Hq, D, dtype=out_dtype or Q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    bmax = torch.empty(B, Hq, nb, dtype=torch.float32, device=dev) if want_bmax else None
    need = workspace_bytes(SA_OP_DECODE_LOWBIT, B, Hq, Hkv, N, D, block, kcap)
    if ws is None:
        ws = workspace(need, dev, ("decode_lowbit", B, Hq, Hkv, N, D, block, kcap))
    _check(_decode_topdelta_lowbit(_ptr(Q), _ptr(codes), _ptr(resid), _ptr(meta), _ptr(V), B, Hq,
                                   Hkv, N, D, block, sink, local, delta, margin, scale, kcap,
                                   _ptr(idx), _ptr(count), _ptr(tau), _ptr(bmax), _ptr(khat),
                                   _ptr(O), _dt(O), _ptr(lse), _ptr(ws), ws.numel(),
                                   _stream(stream)), "sa_decode_topdelta_lowbit")
    return O, lse, idx, count, tau, bmax


def sa_mass_select(Q: torch.Tensor, K: torch.Tensor, k_free: int, block: int = 128,
                   scale: float = 0.0, want_mass: bool = False, per_row: bool = False,
                   idx=None, count=None, ws=None, stream=None):
    """Attention-mass top-k per (b, kv head, query block) from dense causal
    attention: idx [B, Hkv, M, k_free] ascending, count [B, Hkv, M], mass
    [B, Hkv, M, M] when asked, and with per_row the per-query supports
    (row_idx [B, Hkv, L, k_free], row_count [B, Hkv, L], row_mass [B, Hkv, L, M]);
    returns (idx, count, mass, rows) with rows = (row_idx, row_count, row_mass) or None."""
    _rank(Q, "Q", 4)
    _rank(K, "K", 4)
    B, Hq, L, D = Q.shape
    Hkv = K.shape[1]
    M = -(-L // block)
    _need(Q, "Q", None, _FP)
    _need(K, "K", (B, Hkv, L, D), (Q.dtype,))
    _need(idx, "idx", (B, Hkv, M, k_free), _I32)
    _need(count, "count", (B, Hkv, M), _I32)
    _dev(Q, K, idx, count)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hkv, M, k_free, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, M, dtype=torch.int32, device=dev)
    mass = torch.empty(B, Hkv, M, M, dtype=torch.float32, device=dev) if want_mass else None
    rows = None
    if per_row:
        rows = (torch.empty(B, Hkv, L, k_free, dtype=torch.int32, device=dev),
                torch.empty(B, Hkv, L, dtype=torch.int32, device=dev),
                torch.empty(B, Hkv, L, M, dtype=torch.float32, device=dev))
    ri, rc, rm = rows if rows else (None, None, None)
    need = workspace_bytes(SA_OP_MASS_SELECT, B, Hq, Hkv, L, D, block, k_free)
    if ws is None:
        ws = workspace(need, dev, ("mass", B, Hq, Hkv, L, D, block))
    _check(_mass_select(_ptr(Q), _ptr(K), _dt(Q), B, Hq, Hkv, L, D, block, k_free, scale,
                        _ptr(mass), _ptr(idx), _ptr(count), _ptr(rm), _ptr(ri), _ptr(rc),
                        _ptr(ws), ws.numel(), _stream(stream)), "sa_mass_select")
    return idx, count, mass, rows


def sa_select_topdelta(Q: torch.Tensor, K: torch.Tensor, sink: int, local: int, delta: float,
                       cap: int, scale: float = 0.0, idx=None, score=None, count=None, tau=None,
                       ws=None, stream=None):
    """Top-delta selection: keep tokens with q . k * scale >= m~ - delta, m~ the
    largest score over the first `sink` and the last `local` tokens.

    Returns idx [B, Hq, cap] (ascending, -1 padded), score [B, Hq, cap],
    count [B, Hq] (the true count, which may exceed cap) and tau [B, Hq], the
    threshold the scan used.
    """
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    _need(idx, "idx", (B, Hq, cap), _I32)
    _need(score, "score", (B, Hq, cap), _F32)
    _need(count, "count", (B, Hq), _I32)
    _need(tau, "tau", (B, Hq), _F32)
    _dev(Q, K, idx, score, count, tau)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hq, cap, dtype=torch.int32, device=dev)
    if score is None:
        score = torch.empty(B, Hq, cap, dtype=torch.float32, device=dev)
    if count is None:
        count = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    if tau is None:
        tau = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    need = workspace_bytes(SA_OP_SELECT_TOPDELTA, B, Hq, Hkv, N, D, 0, cap)
    if ws is None:
        ws = workspace(need, dev, ("topdelta", B, Hq, Hkv, N, D, cap))
    _check(_select_topdelta(_ptr(Q), _ptr(K), _dt(Q), B, Hq, Hkv, N, D, sink, local, delta, scale,
                            cap, _ptr(idx), _ptr(score), _ptr(count), _ptr(tau), _ptr(ws),
                            ws.numel(), _stream(stream)), "sa_select_topdelta")
    return idx, score, count, tau


def sa_sparse_decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                     count: Optional[torch.Tensor] = None, mode: int = SA_IDX_BLOCKS,
                     block: int = 64, score: Optional[torch.Tensor] = None, scale: float = 0.0,
                     out_dtype: Optional[torch.dtype] = None, O: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, want_lse: bool = True, ws=None,
                     stream=None):
    """Exact attention over the selected blocks/tokens: O [B, Hq, D], lse [B, Hq]."""
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    _need(V, "V", (B, Hkv, N, D), (Q.dtype,))
    rows = (B, Hkv) if mode == SA_IDX_BLOCKS else (B, Hq)
    _rank(idx, "idx", 3)
    _need(idx, "idx", (*rows, idx.shape[-1]), _I32)
    _need(count, "count", rows, _I32)
    _need(score, "score", (B, Hq, idx.shape[-1]) if mode == SA_IDX_TOKENS else None, _F32)
    od = out_dtype or Q.dtype
    _need(O, "O", (B, Hq, D), (od,) if out_dtype else _FP)
    _need(lse, "lse", (B, Hq), _F32)
    _dev(Q, K, V, idx, count, score, O, lse)
    dev = Q.device
    if O is None:
        O = torch.empty(B, Hq, D, dtype=od, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    stride = idx.shape[-1]
    blk = block if mode == SA_IDX_BLOCKS else 0
    need = workspace_bytes(SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, blk, stride)
    if ws is None:
        ws = workspace(need, dev, ("decode", B, Hq, Hkv, N, D, blk, stride))
    _check(_sparse_decode(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, N, D, scale, mode, block,
                          _ptr(idx), _ptr(count), stride, _ptr(score), _ptr(O), _dt(O), _ptr(lse),
                          _ptr(ws), ws.numel(), _stream(stream)), "sa_sparse_decode")
    return O, lse


def sa_sparse_prefill(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                      count: torch.Tensor, block: int = 128, scale: float = 0.0,
                      out_dtype: Optional[torch.dtype] = None, O=None, lse=None,
                      want_lse: bool = True, stream=None):
    """Block-sparse causal prefill: O [B, Hq, L, D], lse [B, Hq, L]."""
    _rank(Q, "Q", 4)
    _rank(K, "K", 4)
    B, Hq, L, D = Q.shape
    Hkv = K.shape[1]
    M = -(-L // block)
    _need(Q, "Q", None, _FP)
    _need(K, "K", (B, Hkv, L, D), (Q.dtype,))
    _need(V, "V", (B, Hkv, L, D), (Q.dtype,))
    _rank(idx, "idx", 4)
    _need(idx, "idx", (B, Hkv, M, idx.shape[-1]), _I32)
    _need(count, "count", (B, Hkv, M), _I32)
    od = out_dtype or Q.dtype
    _need(O, "O", (B, Hq, L, D), (od,) if out_dtype else _FP)
    _need(lse, "lse", (B, Hq, L), _F32)
    _dev(Q, K, V, idx, count, O, lse)
    dev = Q.device
    if O is None:
        O = torch.empty(B, Hq, L, D, dtype=od, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, L, dtype=torch.float32, device=dev)
    _check(_sparse_prefill(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, L, D, scale, block,
                           _ptr(idx), _ptr(count), idx.shape[-1], _ptr(O), _dt(O), _ptr(lse),
                           _stream(stream)), "sa_sparse_prefill")
    return O, lse


def sa_decode_step(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, ksketch: torch.Tensor,
                   k: int, block: int = 64, update_block: int = -1, scale: float = 0.0,
                   out_dtype=None, idx=None, count=None, score=None, O=None, lse=None,
                   want_lse: bool = True, ws=None, stream=None):
    """One decode step: optional sketch update of one block, top-k select, sparse attention."""
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    nb = -(-N // block)
    _need(V, "V", (B, Hkv, N, D), (Q.dtype,))
    _need(ksketch, "ksketch", (B, Hkv, nb, D), _F32)
    _need(idx, "idx", (B, Hkv, k), _I32)
    _need(count, "count", (B, Hkv), _I32)
    _need(score, "score", (B, Hkv, nb), _F32)
    _need(O, "O", (B, Hq, D), (out_dtype,) if out_dtype else _FP)
    _need(lse, "lse", (B, Hq), _F32)
    _dev(Q, K, V, ksketch, idx, count, score, O, lse)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty(B, Hq, D, dtype=out_dtype or Q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    need = workspace_bytes(SA_OP_DECODE_STEP, B, Hq, Hkv, N, D, block, k)
    if ws is None:
        ws = workspace(need, dev, ("step", B, Hq, Hkv, N, D, block, k))
    _check(_decode_step(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, N, D, block,
                        _ptr(ksketch), update_block, k, scale, _ptr(idx), _ptr(count),
                        _ptr(score), _ptr(O), _dt(O), _ptr(lse), _ptr(ws), ws.numel(),
                        _stream(stream)), "sa_decode_step")
    return O, lse, idx, count


def sa_decode_step_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                           ksketch: torch.Tensor, k: int, block: int = 64, update_block: int = -1,
                           scale: float = 0.0, idx=None, count=None, score=None, O=None, lse=None,
                           stream=None):
    """sa_decode_step with the library's per-GPU scratch as its workspace.  The
    caller passes every output (idx, count, O; lse and score optional), so the
    call allocates nothing."""
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    nb = -(-N // block)
    _need(V, "V", (B, Hkv, N, D), (Q.dtype,))
    _need(ksketch, "ksketch", (B, Hkv, nb, D), _F32)
    _need(idx, "idx", (B, Hkv, k), _I32)
    _need(count, "count", (B, Hkv), _I32)
    _need(score, "score", (B, Hkv, nb), _F32)
    _need(O, "O", (B, Hq, D), _FP)
    _need(lse, "lse", (B, Hq), _F32)
    _dev(Q, K, V, ksketch, idx, count, score, O, lse)
    if idx is None or count is None or O is None:
        raise ValueError("sa_decode_step_noalloc needs idx, count and O from the caller")
    _check(_decode_step_noalloc(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, N, D, block,
                                _ptr(ksketch), update_block, k, scale, _ptr(idx), _ptr(count),
                                _ptr(score), _ptr(O), _dt(O), _ptr(lse), _stream(stream)),
           "sa_decode_step_noalloc")
    return O, lse, idx, count


def sa_select_decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, score: torch.Tensor,
                     k: int, block: int = 64, flags: int = SA_FORCE_SINK | SA_FORCE_LOCAL,
                     scale: float = 0.0, out_dtype=None, idx=None, count=None, O=None, lse=None,
                     want_lse: bool = True, ws=None, stream=None):
    """Top-k selection from block scores fused with the split-K sparse decode."""
    B, Hq, D, Hkv, N = _qk_shapes(Q, K)
    nb = -(-N // block)
    _need(V, "V", (B, Hkv, N, D), (Q.dtype,))
    _need(score, "score", (B, Hkv, nb), _F32)
    _need(idx, "idx", (B, Hkv, k), _I32)
    _need(count, "count", (B, Hkv), _I32)
    _need(O, "O", (B, Hq, D), (out_dtype,) if out_dtype else _FP)
    _need(lse, "lse", (B, Hq), _F32)
    _dev(Q, K, V, score, idx, count, O, lse)
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if O is None:
        O = torch.empty(B, Hq, D, dtype=out_dtype or Q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    need = workspace_bytes(SA_OP_SPARSE_DECODE, B, Hq, Hkv, N, D, block, k)
    if ws is None:
        ws = workspace(need, dev, ("select_decode", B, Hq, Hkv, N, D, block, k))
    _check(_select_decode(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, N, D, block,
                          _ptr(score), k, flags, scale, _ptr(idx), _ptr(count), _ptr(O), _dt(O),
                          _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)), "sa_select_decode")
    return O, lse, idx, count


__all__ = [n for n in dir() if n.startswith("sa_") or n.startswith("SA_")] + [
    "workspace", "workspace_bytes", "version", "SAError", "LIB_PATH", "EXPORTS"]
