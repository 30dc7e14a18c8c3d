"""The Python binding rejects tensors of the wrong shape, element type or
device before anything is launched.

Every call here passes CPU tensors: a call whose shapes and dtypes are right
gets as far as the device check ("must live on the GPU") and a call with a
wrong one must fail earlier, on the shape or dtype, naming the argument.  So
none of them reaches the library, and they run without a GPU.
"""
import os

import pytest

torch = pytest.importorskip("torch")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if not os.path.exists(os.path.join(ROOT, "top_sparse_attention_mean_amd", "libsa.so")):
    pytest.skip("libsa.so not built (run __graft_entry__.build())", allow_module_level=True)
import top_sparse_attention_mean_amd as sa  # noqa: E402

bf, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64
B, Hq, Hkv, N, D, BLK, K = 2, 8, 2, 256, 64, 64, 3
NB = N // BLK


def e(*shape, dtype=bf):
    return torch.empty(*shape, dtype=dtype)


def raises(match, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError), match=match):
        fn(*a, **kw)


def test_reaches_the_device_check_when_arguments_are_right():
    raises("GPU", sa.sa_sparse_decode, e(B, Hq, D), e(B, Hkv, N, D), e(B, Hkv, N, D),
           e(B, Hkv, K, dtype=i32), e(B, Hkv, dtype=i32), block=BLK)
    raises("GPU", sa.sa_decode_step, e(B, Hq, D), e(B, Hkv, N, D), e(B, Hkv, N, D),
           e(B, Hkv, NB, D, dtype=f32), K, block=BLK)


def test_sparse_decode_checks():
    Q, Kc, V = e(B, Hq, D), e(B, Hkv, N, D), e(B, Hkv, N, D)
    idx, cnt = e(B, Hkv, K, dtype=i32), e(B, Hkv, dtype=i32)
    # float32 query with a bf16 cache: the kernel would read K as float32
    raises("K must have dtype", sa.sa_sparse_decode, e(B, Hq, D, dtype=f32), Kc, V, idx, cnt)
    raises("V must have dtype", sa.sa_sparse_decode, Q, Kc, e(B, Hkv, N, D, dtype=f32), idx, cnt)
    raises("V must have shape", sa.sa_sparse_decode, Q, Kc, e(B, Hkv, N - 1, D), idx, cnt)
    # int64 lists (torch.arange's default) would be read as int32 pairs
    raises("idx must have dtype", sa.sa_sparse_decode, Q, Kc, V, e(B, Hkv, K, dtype=i64), cnt)
    raises("count must have dtype", sa.sa_sparse_decode, Q, Kc, V, idx, e(B, Hkv, dtype=i64))
    raises("idx must have shape", sa.sa_sparse_decode, Q, Kc, V, e(B, Hkv - 1, K, dtype=i32), cnt)
    raises("count must have shape", sa.sa_sparse_decode, Q, Kc, V, idx, e(B, Hkv + 1, dtype=i32))
    raises("O must have shape", sa.sa_sparse_decode, Q, Kc, V, idx, cnt, O=e(B, Hq - 1, D))
    raises("O must have dtype", sa.sa_sparse_decode, Q, Kc, V, idx, cnt, out_dtype=f32,
           O=e(B, Hq, D))
    raises("lse must have shape", sa.sa_sparse_decode, Q, Kc, V, idx, cnt, lse=e(B, dtype=f32))
    raises("lse must have dtype", sa.sa_sparse_decode, Q, Kc, V, idx, cnt, lse=e(B, Hq))
    # token mode: per query-head lists and scores
    raises("idx must have shape", sa.sa_sparse_decode, Q, Kc, V, idx, e(B, Hq, dtype=i32),
           mode=sa.SA_IDX_TOKENS)
    raises("score must have shape", sa.sa_sparse_decode, Q, Kc, V, e(B, Hq, 9, dtype=i32),
           e(B, Hq, dtype=i32), mode=sa.SA_IDX_TOKENS, score=e(B, Hq, 8, dtype=f32))
    raises("Q must have 3 dimensions", sa.sa_sparse_decode, e(B, Hq, 1, D), Kc, V, idx, cnt)
    raises("Q must have dtype", sa.sa_sparse_decode, e(B, Hq, D, dtype=torch.float16),
           e(B, Hkv, N, D, dtype=torch.float16), e(B, Hkv, N, D, dtype=torch.float16), idx, cnt)


def test_prefill_checks():
    L, M = 512, 4
    Q, Kc, V = e(1, Hq, L, 128), e(1, Hkv, L, 128), e(1, Hkv, L, 128)
    idx, cnt = e(1, Hkv, M, 10, dtype=i32), e(1, Hkv, M, dtype=i32)
    raises("K must have dtype", sa.sa_sparse_prefill, e(1, Hq, L, 128, dtype=f32), Kc, V, idx, cnt)
    raises("V must have shape", sa.sa_sparse_prefill, Q, Kc, e(1, Hkv, L - 128, 128), idx, cnt)
    raises("idx must have dtype", sa.sa_sparse_prefill, Q, Kc, V, e(1, Hkv, M, 10, dtype=i64), cnt)
    raises("idx must have shape", sa.sa_sparse_prefill, Q, Kc, V, e(1, Hkv, M - 1, 10, dtype=i32),
           cnt)
    raises("count must have shape", sa.sa_sparse_prefill, Q, Kc, V, idx, e(1, Hkv, dtype=i32))
    raises("O must have shape", sa.sa_sparse_prefill, Q, Kc, V, idx, cnt, O=e(1, Hq, L, 64))
    raises("lse must have shape", sa.sa_sparse_prefill, Q, Kc, V, idx, cnt,
           lse=e(1, Hq, L - 1, dtype=f32))


def test_decode_step_and_select_decode_checks():
    Q, Kc, V = e(B, Hq, D), e(B, Hkv, N, D), e(B, Hkv, N, D)
    sk = e(B, Hkv, NB, D, dtype=f32)
    raises("ksketch must have dtype", sa.sa_decode_step, Q, Kc, V, e(B, Hkv, NB, D), K, block=BLK)
    raises("ksketch must have shape", sa.sa_decode_step, Q, Kc, V, e(B, Hkv, NB + 1, D, dtype=f32),
           K, block=BLK)
    raises("idx must have shape", sa.sa_decode_step, Q, Kc, V, sk, K, block=BLK,
           idx=e(B, Hkv, K - 1, dtype=i32))
    raises("score must have shape", sa.sa_decode_step, Q, Kc, V, sk, K, block=BLK,
           score=e(B, Hkv, NB - 1, dtype=f32))
    raises("V must have dtype", sa.sa_decode_step, Q, Kc, e(B, Hkv, N, D, dtype=f32), sk, K,
           block=BLK)
    raises("score must have shape", sa.sa_select_decode, Q, Kc, V, e(B, Hkv, NB + 3, dtype=f32),
           K, block=BLK)
    raises("count must have dtype", sa.sa_select_decode, Q, Kc, V, e(B, Hkv, NB, dtype=f32), K,
           block=BLK, count=e(B, Hkv, dtype=i64))


def test_selection_checks():
    Q, Kc = e(B, Hq, D), e(B, Hkv, N, D)
    sk = e(B, Hkv, NB, D, dtype=f32)
    raises("ksketch must have dtype", sa.sa_select_topk, Q, e(B, Hkv, NB, D), K)
    raises("Q must have shape", sa.sa_select_topk, e(B + 1, Hq, D), sk, K)
    raises("idx must have shape", sa.sa_select_topk, Q, sk, K, idx=e(B, Hkv, K + 1, dtype=i32))
    raises("score must have dtype", sa.sa_select_topk, Q, sk, K, score=e(B, Hkv, NB))
    raises("Q must have 4 dimensions", sa.sa_select_topk, Q, sk, K,
           flags=sa.SA_FORCE_SINK | sa.SA_CAUSAL, q_block=BLK)
    tau = e(B, Hq, dtype=f32)
    raises("tau must have shape", sa.sa_select_threshold, Q, Kc, e(B, Hkv, dtype=f32), 16)
    raises("count must have dtype", sa.sa_select_threshold, Q, Kc, tau, 16,
           count=e(B, Hq, dtype=i64))
    raises("K must have dtype", sa.sa_select_topdelta, Q, e(B, Hkv, N, D, dtype=f32), 64, 64, 5.0,
           16)
    raises("idx must have shape", sa.sa_select_topdelta, Q, Kc, 64, 64, 5.0, 16,
           idx=e(B, Hq, 15, dtype=i32))
    rad = e(B, Hkv, NB, 1, dtype=f32)
    raises("sketch must have shape", sa.sa_select_threshold_pruned, Q, Kc, e(B, Hkv, 3, D, dtype=f32),
           rad, tau, 16, BLK)
    raises("live must have shape", sa.sa_select_threshold_pruned, Q, Kc, sk, rad, tau, 16, BLK,
           live=e(B, Hkv, 1, dtype=torch.uint8))
    raises("K must have shape", sa.sa_mass_select, e(1, Hq, 512, 128), e(1, Hkv, 256, 128), 8)


def test_sketch_codec_and_lowbit_checks():
    Kc = e(B, Hkv, N, D)
    raises("out must have shape", sa.sa_build_sketch, Kc, BLK, out=e(B, Hkv, NB - 1, D, dtype=f32))
    raises("head_pool", sa.sa_build_sketch, Kc, BLK, head_pool=3)
    raises("X must have dtype", sa.sa_build_sketch, e(B, Hkv, N, D, dtype=i32), BLK)
    raises("sketch must have shape", sa.sa_build_radius, Kc, e(B, Hkv, NB, D + 1, dtype=f32), BLK)
    raises("codes must have shape", sa.sa_encode_keys, Kc, BLK,
           codes=e(B, Hkv, N, D, dtype=torch.uint8))
    codes = e(B, Hkv, N, D // 4, dtype=torch.uint8)
    resid = e(B, Hkv, N, D, dtype=torch.int8)
    meta = e(B, Hkv, NB, 3, D, dtype=f32)
    raises("meta must have shape", sa.sa_decode_keys, codes, resid, e(B, Hkv, NB, 2, D, dtype=f32),
           BLK)
    raises("needs its count", sa.sa_decode_keys, codes, resid, meta, BLK,
           idx=e(B, Hkv, 4, dtype=i32))
    raises("Q must have dtype", sa.sa_select_topdelta_lowbit, e(B, Hq, D, dtype=f32), codes, resid,
           meta, BLK, 64, 64, 5.0, 1.0, 8)
    raises("khat must have shape", sa.sa_select_topdelta_lowbit, e(B, Hq, D), codes, resid, meta,
           BLK, 64, 64, 5.0, 1.0, 8, khat=e(B, Hkv, N - 1, D))
