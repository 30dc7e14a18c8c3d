"""C-ABI tests that need no GPU.

The library must load, export every function include/sa.h declares, and reject
bad arguments on the host with the documented status codes before any HIP call
(so these calls are safe without a GPU).  Every call below violates at least
one documented precondition, so none of them reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")
LIB = os.path.join(ROOT, "top_sparse_attention_mean_amd", "libsa.so")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
SINK, LOCAL, CAUSAL = 1, 2, 4
A = 0x10000          # an aligned stand-in address; never dereferenced here
MIS = 0x10004        # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libsa.so not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    P, I, F, Z, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint
    L.sa_build_sketch.argtypes = [P, I, I, I, I, I, I, I, I, I, P, P]
    L.sa_select_topk.argtypes = [P, I, I, I, I, I, I, I, P, I, I, U, F, P, P, P, P, Z, P]
    L.sa_select_threshold.argtypes = [P, P, I, I, I, I, I, I, P, F, I, P, P, P, P, Z, P]
    L.sa_select_topdelta.argtypes = [P, P, I, I, I, I, I, I, I, I, F, F, I, P, P, P, P, P, Z, P]
    L.sa_build_radius.argtypes = [P, I, I, I, I, I, I, I, I, I, P, P, P]
    L.sa_encode_keys.argtypes = [P, I, I, I, I, I, I, I, I, P, P, P, P]
    L.sa_mass_select.argtypes = [P, P, I, I, I, I, I, I, I, I, F, P, P, P, P, P, P, P, Z, P]
    L.sa_decode_keys.argtypes = [P, P, P, I, I, I, I, I, P, P, I, I, I, P, P]
    L.sa_select_topdelta_lowbit.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, F, F, F, I, P, P,
                                            P, P, P, P, Z, P]
    L.sa_select_threshold_pruned.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P, P, F, I, P, P, P,
                                             P, P, Z, P]
    L.sa_sparse_decode.argtypes = [P, P, P, I, I, I, I, I, I, F, I, I, P, P, I, P, P, I, P, P, Z, P]
    L.sa_sparse_prefill.argtypes = [P, P, P, I, I, I, I, I, I, F, I, P, P, I, P, I, P, P]
    L.sa_decode_step.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, I, F, P, P, P, P, I, P, P, Z, P]
    L.sa_select_decode.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, U, F, P, P, P, I, P, P, Z, P]
    L.sa_decode_topdelta_lowbit.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, F, F, F, I, P, P,
                                            P, P, P, P, I, P, P, Z, P]
    L.sa_decode_step_noalloc.argtypes = [P, P, P, I, I, I, I, I, I, I, P, I, I, F, P, P, P, P, I, P,
                                         P]
    L.sa_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    L.sa_workspace_bytes.restype = Z
    L.sa_status_str.restype = ctypes.c_char_p
    L.sa_last_error.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sa_status|size_t|const char\*|int)\s+(sa_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["sa_build_sketch", "sa_build_radius", "sa_encode_keys", "sa_decode_keys",
              "sa_select_topk", "sa_select_threshold", "sa_select_topdelta",
              "sa_select_threshold_pruned", "sa_select_topdelta_lowbit",
              "sa_decode_topdelta_lowbit", "sa_mass_select",
              "sa_sparse_decode", "sa_sparse_prefill", "sa_select_decode", "sa_decode_step",
              "sa_decode_step_noalloc", "sa_workspace_bytes",
              "sa_status_str",
              "sa_last_error", "sa_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in sa.h but not exported"


def test_binding_names_match_header():
    pytest.importorskip("torch")
    if not os.path.exists(LIB):
        pytest.skip("libsa.so not built")
    import top_sparse_attention_mean_amd as sa
    assert sorted(sa.EXPORTS) == declared_functions()
    for n in declared_functions():
        if n not in ("sa_workspace_bytes", "sa_status_str", "sa_last_error", "sa_version"):
            assert callable(getattr(sa, n))


def test_status_strings_and_version(lib):
    assert lib.sa_status_str(0) == b"ok"
    assert lib.sa_status_str(3) == b"workspace too small"
    assert lib.sa_version() >= 100


def test_workspace_sizes(lib):
    # decode select: one float score per block of every (b, kv head)
    assert lib.sa_workspace_bytes(0, 1, 64, 8, 1, 128, 1, 4096) == 8 * 4096 * 4
    # threshold staging grows with B * Hq * N
    a = lib.sa_workspace_bytes(1, 8, 32, 8, 32768, 128, 0, 1024)
    assert a >= 8 * 32 * 32768 * 8
    # decode partials: one float per (b, head, split, column); ~256 selected
    # tokens per split -> ceil(82 * 64 / 256) = 21 splits at the 256K workload
    assert lib.sa_workspace_bytes(2, 1, 64, 8, 262144, 128, 64, 82) >= 64 * 21 * 130 * 4
    assert lib.sa_workspace_bytes(2, 0, 64, 8, 262144, 128, 64, 82) == ctypes.c_size_t(-1).value
    assert lib.sa_workspace_bytes(9, 1, 1, 1, 1, 64, 64, 1) == ctypes.c_size_t(-1).value
    # top-delta: the threshold staging plus one float threshold per (b, head)
    assert lib.sa_workspace_bytes(4, 8, 32, 8, 32768, 128, 0, 1024) >= a + 8 * 32 * 4
    # pruned threshold: the staging plus one flag per (b, kv head, 128-token segment)
    assert lib.sa_workspace_bytes(5, 8, 32, 8, 32768, 128, 64, 1024) >= a + 8 * 8 * 256


def test_sketch_validation(lib):
    # null input
    assert lib.sa_build_sketch(None, 1, 1, 8, 4096, 128, 64, 1, 0, 64, A, None) == INVALID
    # misaligned output
    assert lib.sa_build_sketch(A, 1, 1, 8, 4096, 128, 64, 1, 0, 64, MIS, None) == INVALID
    # unsupported D
    assert lib.sa_build_sketch(A, 1, 1, 8, 4096, 96, 64, 1, 0, 64, A, None) == UNSUPPORTED
    # head_pool must divide H
    assert lib.sa_build_sketch(A, 1, 1, 8, 4096, 128, 64, 3, 0, 64, A, None) == INVALID
    # block range beyond nb
    assert lib.sa_build_sketch(A, 1, 1, 8, 4096, 128, 64, 1, 0, 65, A, None) == INVALID
    assert b"outside" in lib.sa_last_error()
    # unknown dtype
    assert lib.sa_build_sketch(A, 7, 1, 8, 4096, 128, 64, 1, 0, 64, A, None) == INVALID


def test_select_validation(lib):
    args = dict(Q=A, dt=1, B=1, Hq=64, Hkv=8, Lq=1, D=128, qb=1, sk=A, nb=4096, k=82,
                fl=SINK | LOCAL, sc=0.0, idx=A, cnt=A, score=None, ws=A, wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return lib.sa_select_topk(a["Q"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["Lq"], a["D"],
                                  a["qb"], a["sk"], a["nb"], a["k"], a["fl"], a["sc"], a["idx"],
                                  a["cnt"], a["score"], a["ws"], a["wsb"], None)

    assert call(Hq=60) == INVALID                 # Hq % Hkv != 0
    assert call(k=1) == INVALID                   # k below the two forced blocks
    assert call(k=0) == INVALID
    assert call(nb=9000) == UNSUPPORTED           # too many blocks for one LDS row
    assert call(wsb=100) == WORKSPACE             # no room for the scores
    assert call(fl=8) == INVALID                  # unknown flag
    assert call(Lq=128) == INVALID                # multi-row query needs SA_CAUSAL
    assert call(idx=None) == INVALID
    assert call(fl=SINK | LOCAL | CAUSAL, Lq=65536, qb=128, nb=256, ws=A) == INVALID  # nb < M
    assert call(fl=SINK | LOCAL | CAUSAL, Lq=65536, qb=128, nb=512, wsb=16) == WORKSPACE


def test_threshold_validation(lib):
    f = lib.sa_select_threshold
    assert f(A, A, 1, 8, 32, 8, 32768, 128, None, 0.0, 1024, A, A, A, A, 1 << 30, None) == INVALID
    assert f(A, A, 1, 8, 32, 8, 32768, 128, A, 0.0, 0, A, A, A, A, 1 << 30, None) == INVALID
    assert f(A, A, 1, 8, 48, 8, 32768, 128, A, 0.0, 1024, A, A, A, A, 1 << 30, None) == UNSUPPORTED
    assert f(A, A, 1, 8, 32, 8, 32768, 128, A, 0.0, 1024, A, A, A, A, 1024, None) == WORKSPACE


def test_topdelta_validation(lib):
    f = lib.sa_select_topdelta
    base = [A, A, 1, 8, 32, 8, 32768, 128, 64, 64, 5.0, 0.0, 1024, A, A, A, None, A, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(8, -1) == INVALID                 # negative sink
    assert call(9, -5) == INVALID                 # negative local
    a = list(base)
    a[8], a[9] = 0, 0                             # empty window
    assert f(*a) == INVALID
    assert b"empty" in lib.sa_last_error()
    assert call(10, -1.0) == INVALID              # delta < 0
    assert call(10, float("nan")) == INVALID
    assert call(12, 0) == INVALID                 # cap
    assert call(16, MIS) == INVALID               # misaligned tau
    assert call(4, 48) == UNSUPPORTED             # bf16 g = 6
    assert call(18, 1024) == WORKSPACE
    assert call(1, None) == INVALID               # K


def test_radius_validation(lib):
    f = lib.sa_build_radius
    base = [A, 1, 1, 8, 32768, 128, 64, 1, 0, 512, A, A, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(7, 3) == UNSUPPORTED              # S does not divide D
    assert call(7, 32) == UNSUPPORTED             # subspaces of 4 channels
    a = list(base)
    a[5], a[7] = 64, 16                           # D = 64: 4-channel subspaces
    assert f(*a) == UNSUPPORTED
    assert call(6, 0) == INVALID                  # block
    assert call(11, MIS) == INVALID               # misaligned radius
    assert call(10, None) == INVALID              # sketch
    assert call(9, 513) == INVALID                # block range past nb
    assert call(8, 600) == INVALID and call(8, -1) == INVALID   # begin past end / negative


def test_pruned_threshold_validation(lib):
    f = lib.sa_select_threshold_pruned
    base = [A, A, 1, 8, 32, 8, 32768, 128, 64, 1, A, A, A, 0.0, 1024, A, A, A, None, A, 1 << 30,
            None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(8, 48) == UNSUPPORTED             # block must divide the 128-token segment
    assert call(8, 256) == UNSUPPORTED
    assert call(9, 5) == UNSUPPORTED              # S
    assert call(11, None) == INVALID              # radius
    assert call(12, None) == INVALID              # tau
    assert call(18, MIS) == INVALID               # misaligned live
    assert call(20, 4096) == WORKSPACE
    assert call(4, 48) == UNSUPPORTED             # bf16 g = 6


def test_lowbit_validation(lib):
    enc = lib.sa_encode_keys
    eb = [A, 1, 1, 8, 32768, 128, 64, 0, 512, A, A, A, None]

    def ecall(i, v):
        a = list(eb)
        a[i] = v
        return enc(*a)

    assert ecall(5, 96) == UNSUPPORTED            # D
    assert ecall(8, 513) == INVALID               # block range
    assert ecall(9, None) == INVALID              # codes
    assert ecall(11, MIS) == INVALID              # misaligned meta
    dec = lib.sa_decode_keys
    db = [A, A, A, 1, 8, 32768, 128, 64, None, None, 0, 0, 600, A, None]
    assert dec(*db) == INVALID                    # range past nb (no list)
    a = list(db)
    a[8], a[10] = A, 0                            # a list with stride 0
    assert dec(*a) == INVALID
    sel = lib.sa_select_topdelta_lowbit
    sb = [A, A, A, A, 1, 64, 8, 32768, 128, 64, 64, 64, 5.0, 1.0, 0.0, 512, A, A, None, None, A,
          A, 1 << 30, None]

    def scall(i, v):
        a = list(sb)
        a[i] = v
        return sel(*a)

    assert scall(9, 32) == UNSUPPORTED            # block
    assert scall(5, 48) == UNSUPPORTED            # g = 6
    assert scall(13, -1.0) == INVALID             # margin
    assert scall(12, float("nan")) == INVALID     # delta
    assert scall(15, 0) == INVALID                # kcap
    assert scall(20, None) == INVALID             # khat
    assert scall(22, 100) == WORKSPACE
    a = list(sb)
    a[10], a[11] = 0, 0                           # empty window
    assert sel(*a) == INVALID
    fused = lib.sa_decode_topdelta_lowbit
    fb = [A, A, A, A, A, 1, 64, 8, 32768, 128, 64, 64, 64, 5.0, 1.0, 0.0, 512, A, A, None, None,
          A, A, 1, None, A, 1 << 30, None]

    def fcall(i, v):
        a = list(fb)
        a[i] = v
        return fused(*a)

    assert fcall(4, None) == INVALID              # V
    assert fcall(22, None) == INVALID             # O
    assert fcall(23, 7) == INVALID                # output dtype
    assert fcall(16, 1921) == UNSUPPORTED         # more listed blocks than the splits can stage
    assert fcall(10, 32) == UNSUPPORTED           # block
    assert fcall(26, 4096) == WORKSPACE           # the selection's and the decode's workspace


def test_mass_select_validation(lib):
    f = lib.sa_mass_select
    base = [A, A, 1, 1, 32, 4, 65536, 128, 128, 8, 0.0, None, A, A, None, None, None, A, 1 << 40,
            None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(2, 0) == UNSUPPORTED              # fp32
    assert call(7, 64) == UNSUPPORTED             # D
    assert call(8, 64) == UNSUPPORTED             # block
    assert call(9, 0) == INVALID and call(9, 65) == INVALID   # k_free
    assert call(12, None) == INVALID              # idx
    assert call(18, 1024) == WORKSPACE
    assert call(4, 30) == INVALID                 # Hq % Hkv
    assert call(15, A) == INVALID                 # row_idx without row_mass / row_count
    assert call(6, 9 * 1024 * 1024) == UNSUPPORTED   # one kv head past the 32-bit buffer range


def test_decode_validation(lib):
    f = lib.sa_sparse_decode
    base = [A, A, A, 1, 1, 64, 8, 262144, 128, 0.0, 0, 64, A, A, 82, None, A, 1, A, A, 1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(0, None) == INVALID               # Q
    assert call(11, 32) == UNSUPPORTED            # bf16 block mode needs 64/128
    assert call(10, 5) == INVALID                 # unknown mode
    assert call(20, 64) == WORKSPACE
    assert call(5, 48) == UNSUPPORTED             # g = 6
    assert call(7, 9 * 1024 * 1024) == UNSUPPORTED   # one kv head past the 32-bit buffer range
    a = list(base)
    a[10], a[13] = 1, None                        # token mode without counts
    assert f(*a) == INVALID


def test_prefill_validation(lib):
    f = lib.sa_sparse_prefill
    base = [A, A, A, 1, 1, 32, 4, 65536, 128, 0.0, 128, A, A, 10, A, 1, A, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(3, 0) == UNSUPPORTED              # float32 prefill
    assert call(10, 32) == UNSUPPORTED            # 32-token blocks (64 and 128 only)
    assert call(8, 96) == UNSUPPORTED             # D = 96 (64 and 128 only)
    assert call(12, None) == INVALID              # count
    assert call(13, 0) == INVALID                 # kmax
    assert call(7, 9 * 1024 * 1024) == UNSUPPORTED   # one kv head past the 32-bit buffer range


def test_decode_step_validation(lib):
    f = lib.sa_decode_step
    base = [A, A, A, 1, 1, 64, 8, 262144, 128, 64, A, 4095, 82, 0.0, A, A, None, A, 1, A, A,
            1 << 30, None]
    a = list(base)
    a[11] = 4096                                  # update_block past the last block
    assert f(*a) == INVALID
    a = list(base)
    a[21] = 128                                   # workspace
    assert f(*a) == WORKSPACE


def test_decode_step_noalloc_validation(lib):
    """Argument errors return before the scratch lookup (no HIP call), and a
    shape whose workspace exceeds the 16 MiB scratch is refused."""
    f = lib.sa_decode_step_noalloc
    base = [A, A, A, 1, 1, 64, 8, 262144, 128, 64, A, 4095, 82, 0.0, A, A, None, A, 1, A, None]
    a = list(base)
    a[11] = 4096                                  # update_block past the last block
    assert f(*a) == INVALID
    a = list(base)
    a[5] = 63                                     # Hq not a multiple of Hkv
    assert f(*a) == INVALID
    a = list(base)
    a[10] = MIS                                   # misaligned sketch
    assert f(*a) == INVALID
    a = list(base)
    a[4], a[5], a[6] = 64, 64 * 64, 64 * 8        # B = 64: far more than 16 MiB of workspace
    assert f(*a) == WORKSPACE
    assert b"16 MiB" in lib.sa_last_error()


def test_select_decode_validation(lib):
    f = lib.sa_select_decode
    base = [A, A, A, 1, 1, 64, 8, 262144, 128, 64, A, 82, SINK | LOCAL, 0.0, A, A, A, 1, A, A,
            1 << 30, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)

    assert call(10, None) == INVALID              # score
    assert call(15, None) == INVALID              # count
    assert call(12, CAUSAL) == INVALID            # prefill flag
    assert call(11, 1) == INVALID                 # k below the two forced blocks
    assert call(9, 16) == UNSUPPORTED             # 16384 blocks per row
    assert call(9, 32) == UNSUPPORTED             # bf16 block mode needs 64/128
    assert call(20, 64) == WORKSPACE


def test_binding_binds_every_entry_point():
    """Every exported entry point has a ctypes signature and a wrapper in the binding."""
    sa = pytest.importorskip("top_sparse_attention_mean_amd")
    for n in sa.EXPORTS:
        assert hasattr(sa, "_" + n[len("sa_"):]), f"no ctypes signature for {n}"
    for n in ["sa_build_sketch", "sa_build_radius", "sa_encode_keys", "sa_decode_keys",
              "sa_select_topk", "sa_select_threshold", "sa_select_topdelta",
              "sa_select_threshold_pruned", "sa_select_topdelta_lowbit",
              "sa_decode_topdelta_lowbit", "sa_mass_select",
              "sa_sparse_decode", "sa_sparse_prefill", "sa_select_decode", "sa_decode_step"]:
        assert callable(getattr(sa, n)), n
