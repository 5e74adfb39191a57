"""C-ABI checks that need no GPU: the library loads, exports every function
include/aqgemv.h declares, and rejects invalid calls with the documented
status before any HIP call (fake, never-dereferenced pointers are used).
"""
import ctypes
import os
import re

import pytest

import affine_quantized_gemv_amd as aqg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aqgemv.h")
HAS_GPU_NODE = os.path.exists("/dev/kfd")

A16 = 0x10000            # fake, 16-byte aligned device addresses
B16 = 0x20000
C16 = 0x30000
D16 = 0x40000
E16 = 0x50000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aqg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return aqg.load()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    expected = {"aqg_abi_version", "aqg_status_string", "aqg_workspace_bytes", "aqg_gemv_bf16",
                "aqg_swiglu_bf16", "aqg_unpack_codes", "aqg_dispatch_path", "aqg_path_name",
                "aqg_gemv_bf16_argmax", "aqg_gemv_argmax_noalloc"} | \
               {"aqg_gemv_affine_q%d" % b for b in range(2, 9)} | \
               {"aqg_gemv_affine_q%d_argmax" % b for b in range(2, 9)} | \
               {"aqg_swiglu_affine_q%d" % b for b in range(2, 9)} | \
               {"aqg_gemv_bf16_multi"} | {"aqg_gemv_affine_q%d_multi" % b for b in range(2, 9)} | \
               {"aqg_stream_read"} | {"aqg_gemm_affine_q%d" % b for b in range(2, 9)}
    assert set(names) == expected


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert aqg.abi_version() == 1
    for s in range(6):
        assert aqg.status_string(s).startswith(
            ["AQG_OK", "AQG_ERR_INVALID_ARG", "AQG_ERR_UNSUPPORTED", "AQG_ERR_ALIGNMENT",
             "AQG_ERR_LAUNCH", "AQG_ERR_DEVICE"][s])
    assert aqg.status_string(99) == "unknown aqg status"
    assert aqg.workspace_bytes(4, 1, 100, 1024) == 0
    assert aqg.workspace_bytes(aqg.AQG_KIND_SWIGLU, 4, 4096, 1536) == 0


def dense(lib, x=A16, W=B16, y=C16, M=1, N=16, K=64, out=0, ws=None, wsb=0):
    return lib.aqg_gemv_bf16(x, W, y, M, N, K, out, ws, wsb, None)


def affine(lib, bits=4, x=A16, Wq=B16, s=D16, b=E16, y=C16, M=1, N=16, K=64, out=0):
    return getattr(lib, "aqg_gemv_affine_q%d" % bits)(x, Wq, s, b, y, M, N, K, out, None, 0, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(W=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(y=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(N=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(K=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=-1), aqg.AQG_ERR_INVALID_ARG),
    (dict(out=2), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=33), aqg.AQG_ERR_UNSUPPORTED),
    (dict(K=12), aqg.AQG_ERR_UNSUPPORTED),
    (dict(x=A16 + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(W=B16 + 4), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=C16 + 1), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=C16 + 2, out=1), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=A16), aqg.AQG_ERR_INVALID_ARG),          # output overlaps x
    (dict(y=B16 + 16), aqg.AQG_ERR_INVALID_ARG),     # output overlaps W
])
def test_dense_validation(lib, kwargs, status):
    assert dense(lib, **kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(Wq=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(s=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(b=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(K=96), aqg.AQG_ERR_UNSUPPORTED),            # groups other than 64 are refused
    (dict(K=32), aqg.AQG_ERR_UNSUPPORTED),
    (dict(M=40), aqg.AQG_ERR_UNSUPPORTED),
    (dict(Wq=B16 + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(s=D16 + 1), aqg.AQG_ERR_ALIGNMENT),
    (dict(s=D16 + 2), aqg.AQG_ERR_ALIGNMENT),         # scales and biases: 4-byte aligned
    (dict(b=E16 + 2), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=D16), aqg.AQG_ERR_INVALID_ARG),           # output overlaps scales
])
def test_affine_validation(lib, kwargs, status):
    for bits in range(2, 9):
        assert affine(lib, bits=bits, **kwargs) == status


def test_swiglu_affine_validation(lib):
    for b in range(2, 9):
        f = getattr(lib, "aqg_swiglu_affine_q%d" % b)
        ok = (A16, B16, D16, E16, 0x60000, 0x70000, 0x80000, C16, 1, 16, 64, 0, None, 0, None)
        args = list(ok)
        assert f(*[None if i == 4 else a for i, a in enumerate(args)]) == aqg.AQG_ERR_INVALID_ARG   # no Wu
        assert f(*[None if i == 5 else a for i, a in enumerate(args)]) == aqg.AQG_ERR_INVALID_ARG   # no up scales
        assert f(*[0x70002 if i == 5 else a for i, a in enumerate(args)]) == aqg.AQG_ERR_ALIGNMENT
        assert f(*[96 if i == 10 else a for i, a in enumerate(args)]) == aqg.AQG_ERR_UNSUPPORTED  # K % 64
        assert f(*[0x80000 if i == 7 else a for i, a in enumerate(args)]) == aqg.AQG_ERR_INVALID_ARG  # out on up biases
        if not HAS_GPU_NODE:
            assert f(*args) == aqg.AQG_ERR_DEVICE
    assert aqg.workspace_bytes(aqg.AQG_KIND_SWIGLU_AFFINE + 4, 8, 4096, 1536) == 0


def test_swiglu_validation(lib):
    f = lib.aqg_swiglu_bf16
    assert f(A16, B16, None, C16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(A16, B16, D16 + 8, C16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_ALIGNMENT
    assert f(A16, B16, D16, C16, 33, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(A16, B16, D16, D16, 1, 16, 64, 0, None, 0, None) == aqg.AQG_ERR_INVALID_ARG


def test_unpack_validation(lib):
    f = lib.aqg_unpack_codes
    assert f(4, None, A16, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(4, B16, None, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG
    assert f(1, B16, A16, 4, 64, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(9, B16, A16, 4, 64, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(4, B16, A16, 4, 100, None) == aqg.AQG_ERR_UNSUPPORTED
    assert f(4, B16 + 4, A16, 4, 64, None) == aqg.AQG_ERR_ALIGNMENT
    assert f(4, B16, B16, 4, 64, None) == aqg.AQG_ERR_INVALID_ARG


@pytest.mark.skipif(HAS_GPU_NODE, reason="only meaningful where no GPU can be reached")
def test_valid_call_without_gpu_reports_device_error(lib):
    """Arguments pass validation, then the device check fails: nothing is launched."""
    assert dense(lib) == aqg.AQG_ERR_DEVICE
    assert affine(lib) == aqg.AQG_ERR_DEVICE
    assert lib.aqg_unpack_codes(4, B16, A16, 4, 64, None) == aqg.AQG_ERR_DEVICE


def test_python_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        aqg.gemv_bf16(x, torch.zeros(4, 64, dtype=torch.bfloat16))


def test_dispatch_query_names_the_families_the_gpu_tests_cover(lib):
    """The exactness tests state the kernel family of each case; the library's
    dispatch query (no launch; 256 CUs without a device) must agree, so a
    change of thresholds cannot move a case off the kernel it pins unnoticed."""
    import test_gpu_exact
    for family, bits, M, N, K in test_gpu_exact.CASES:
        assert aqg.dispatch_path(bits, M, N, K)[0] == family, (family, bits, M, N, K)


def test_dispatch_query_refuses_what_the_calls_refuse(lib):
    cols = ctypes.c_int(0)
    assert lib.aqg_dispatch_path(4, 33, 100, 1024, ctypes.byref(cols)) == -aqg.AQG_ERR_UNSUPPORTED
    assert lib.aqg_dispatch_path(4, 1, 100, 1000, ctypes.byref(cols)) == -aqg.AQG_ERR_UNSUPPORTED
    assert lib.aqg_dispatch_path(0, 0, 100, 1024, ctypes.byref(cols)) == -aqg.AQG_ERR_INVALID_ARG
    assert lib.aqg_dispatch_path(1, 1, 100, 1024, None) == -aqg.AQG_ERR_INVALID_ARG
    assert lib.aqg_path_name(99) == b"unknown"
    p = lib.aqg_dispatch_path(0, 1, 1536, 1536, ctypes.byref(cols))
    assert p >= 0 and cols.value == 1 and lib.aqg_path_name(p) == b"piece"


F16 = 0x60000
G16 = 0x70000
WS = 0x1000000


def argmax_dense(lib, x=A16, W=B16, val=F16, idx=G16, M=1, N=16, K=64, ws=WS, wsb=None):
    if wsb is None:
        wsb = aqg.workspace_bytes(aqg.AQG_KIND_ARGMAX_DENSE, M, N, K) if 0 < M <= 32 and N > 0 and K > 0 else 0
    return lib.aqg_gemv_bf16_argmax(x, W, val, idx, M, N, K, ws, wsb, None)


def test_argmax_workspace_sizes_follow_the_kernel(lib):
    """Fused epilogue (large N): partials only; otherwise fp32 y plus the
    chunk partials.  Every size is nonzero (a workspace is always needed)."""
    K = aqg.AQG_KIND_ARGMAX_DENSE
    big = aqg.workspace_bytes(K, 16, 100000, 1536)
    small = aqg.workspace_bytes(K, 16, 1536, 1536)
    assert big == 32 * 32 * 256 * 8                      # 32 rows x 32 producers per CU x 256 CUs
    assert small >= 16 * 1536 * 4
    assert aqg.workspace_bytes(K + 4, 4, 151936, 1024) == big
    assert aqg.workspace_bytes(K + 3, 4, 50000, 1024) >= 4 * 50000 * 4
    assert aqg.workspace_bytes(K, 33, 100, 1024) == 0


@pytest.mark.parametrize("kwargs,status", [
    (dict(val=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(idx=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(ws=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(wsb=16), aqg.AQG_ERR_INVALID_ARG),             # shorter than the workspace the shape needs
    (dict(M=33), aqg.AQG_ERR_UNSUPPORTED),
    (dict(K=12), aqg.AQG_ERR_UNSUPPORTED),
    (dict(val=F16 + 2), aqg.AQG_ERR_ALIGNMENT),
    (dict(ws=WS + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(idx=F16), aqg.AQG_ERR_INVALID_ARG),            # outputs overlap
    (dict(val=A16), aqg.AQG_ERR_INVALID_ARG),            # output overlaps x
    (dict(ws=B16), aqg.AQG_ERR_INVALID_ARG),             # workspace overlaps W
])
def test_argmax_validation(lib, kwargs, status):
    assert argmax_dense(lib, **kwargs) == status
    f = lib.aqg_gemv_affine_q4_argmax
    if "W" not in kwargs:
        kw = dict(kwargs)
        M = kw.get("M", 1)
        wsb = kw.get("wsb", aqg.workspace_bytes(aqg.AQG_KIND_ARGMAX_DENSE + 4, M, 16, kw.get("K", 64))
                     if M <= 32 else 0)
        assert f(kw.get("x", A16), B16, D16, E16, kw.get("val", F16), kw.get("idx", G16), M, 16, kw.get("K", 64),
                 kw.get("ws", WS), wsb, None) == status


@pytest.mark.skipif(HAS_GPU_NODE, reason="only meaningful where no GPU can be reached")
def test_valid_argmax_without_gpu_reports_device_error(lib):
    assert argmax_dense(lib) == aqg.AQG_ERR_DEVICE


def test_multi_validation(lib):
    P = ctypes.c_void_p
    f = lib.aqg_gemv_bf16_multi

    def call(Ws, ys, Ns, M=1, K=64):
        return f(A16, len(Ns), (P * len(Ws))(*Ws), (P * len(ys))(*ys), (ctypes.c_int * len(Ns))(*Ns), M, K, 0,
                 None, 0, None)
    W = [0x100000, 0x200000, 0x300000]
    Y = [0x400000, 0x500000, 0x600000]
    assert f(A16, 0, None, None, None, 1, 64, 0, None, 0, None) == aqg.AQG_ERR_INVALID_ARG
    assert call([], [], []) == aqg.AQG_ERR_UNSUPPORTED                       # P = 0
    assert call(W + W[:2], Y + Y[:2], [16] * 5) == aqg.AQG_ERR_UNSUPPORTED   # P = 5
    assert call(W, Y, [16, 0, 16]) == aqg.AQG_ERR_INVALID_ARG                # an empty projection
    assert call(W, Y, [16, 16, 16], M=33) == aqg.AQG_ERR_UNSUPPORTED
    assert call(W, Y, [16, 16, 16], K=12) == aqg.AQG_ERR_UNSUPPORTED
    assert call([W[0], W[1] + 8, W[2]], Y, [16, 16, 16]) == aqg.AQG_ERR_ALIGNMENT
    assert call(W, [Y[0], Y[0] + 4, Y[2]], [16, 16, 16]) == aqg.AQG_ERR_INVALID_ARG   # outputs overlap
    assert call(W, [Y[0], W[2], Y[2]], [16, 16, 16]) == aqg.AQG_ERR_INVALID_ARG      # output on a weight
    if not HAS_GPU_NODE:
        assert call(W, Y, [16, 16, 16]) == aqg.AQG_ERR_DEVICE
    g = lib.aqg_gemv_affine_q4_multi
    S = [0x700000, 0x710000, 0x720000]
    B = [0x800000, 0x810000, 0x820000]
    args = lambda s: (A16, 3, (P * 3)(*W), (P * 3)(*s), (P * 3)(*B), (P * 3)(*Y), (ctypes.c_int * 3)(16, 16, 16),
                      1, 64, 0, None, 0, None)
    assert g(*args([S[0], 0, S[2]])) == aqg.AQG_ERR_INVALID_ARG           # a null scale array entry
    assert g(*args([S[0], S[1] + 2, S[2]])) == aqg.AQG_ERR_ALIGNMENT


# ------------------------------------------------ affine prompt GEMM

def gemm_ws_closed_form(bits, M, K):
    """x operands (M rounded up to 64) x K bf16, then the pieces (3 per row
    and group for 8 bits, else 6) over groups rounded up to 32, each part
    rounded up to 256 bytes."""
    Mp = -(-M // 64) * 64
    Gp = -(-(K // 64) // 32) * 32
    up = lambda v: -(-v // 256) * 256
    return up(Mp * K * 2) + up((3 if bits == 8 else 6) * Mp * Gp * 2)


def gemm_split_closed_form(M, N, K, cus=256):
    """Workgroups per tile splitting its groups, as the header states it: the
    wavefront split (WN, WK) in (8, 1), (4, 2), (2, 4), the widest giving
    three quarters of the CUs a tile, else the one with the most tiles; then,
    if the tiles leave more than a quarter of the CUs idle, the smallest ks in
    2..8 that fills three quarters with at least 2 groups per wavefront chunk
    (ks WK dividing the groups), else the largest such ks."""
    G = K // 64
    tm = -(-M // 64)
    best, best_t = (8, 1), -1
    for wn, wk in ((8, 1), (4, 2), (2, 4)):
        if G % wk:
            continue
        t = -(-N // (64 * wn)) * tm
        if 4 * t >= 3 * cus:
            best, best_t = (wn, wk), t
            break
        if t > best_t:
            best, best_t = (wn, wk), t
    wn, wk = best
    T = -(-N // (64 * wn)) * tm
    if 4 * T >= 3 * cus:
        return 1
    ks = 1
    for k in range(2, 9):
        if G % (wk * k) or G // (wk * k) < 2:
            continue
        ks = k
        if 4 * T * k >= 3 * cus:
            break
    return ks


def gemm_ws_full(bits, M, N, K):
    ks = gemm_split_closed_form(M, N, K)
    part = -(-ks * M * N * 4 // 256) * 256 if ks > 1 else 0
    return gemm_ws_closed_form(bits, M, K) + part


@pytest.mark.parametrize("bits", range(2, 9))
def test_gemm_workspace_bytes(bits):
    """The size query: the operands (always required) plus, where the tiles
    are split, the partial products; 14336-row matrices are never split, the
    1024- and 3584-row ones of the prompt shapes are."""
    kind = aqg.AQG_KIND_GEMM_AFFINE + bits
    for M, K in [(1, 64), (33, 1024), (64, 1536), (65, 4096), (512, 4096), (1000, 3584)]:
        for N in (100, 1024, 3584, 14336):
            assert aqg.workspace_bytes(kind, M, N, K) == gemm_ws_full(bits, M, N, K), (M, N, K)
    assert gemm_split_closed_form(128, 14336, 4096) == 1
    assert gemm_split_closed_form(128, 1024, 3584) == 7
    assert gemm_split_closed_form(128, 3584, 1024) == 2
    assert aqg.workspace_bytes(kind, 0, 100, 1024) == 0
    assert aqg.workspace_bytes(kind, 33, 100, 96) == 0               # K not a multiple of 64
    assert aqg.workspace_bytes(kind, aqg.GEMM_MAX_M + 1, 100, 64) == 0


def gemm(lib, bits=4, x=A16, Wq=B16, s=D16, b=E16, y=C16, M=40, N=16, K=64, out=0, ws=0x100000, wsb=None):
    if wsb is None:
        wsb = gemm_ws_closed_form(bits, M, K) if M > 0 and K > 0 else 0
    return getattr(lib, "aqg_gemm_affine_q%d" % bits)(x, Wq, s, b, y, M, N, K, out, ws, wsb, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(Wq=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(s=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(b=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(y=None), aqg.AQG_ERR_INVALID_ARG),
    (dict(M=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(N=0), aqg.AQG_ERR_INVALID_ARG),
    (dict(out=3), aqg.AQG_ERR_INVALID_ARG),
    (dict(ws=None), aqg.AQG_ERR_INVALID_ARG),            # the workspace is required
    (dict(wsb=1024), aqg.AQG_ERR_INVALID_ARG),           # and must hold the x operands and pieces
    (dict(K=96), aqg.AQG_ERR_UNSUPPORTED),
    (dict(M=aqg.GEMM_MAX_M + 1), aqg.AQG_ERR_UNSUPPORTED),
    (dict(x=A16 + 8), aqg.AQG_ERR_ALIGNMENT),
    (dict(Wq=B16 + 4), aqg.AQG_ERR_ALIGNMENT),
    (dict(ws=0x100008), aqg.AQG_ERR_ALIGNMENT),
    (dict(s=D16 + 2), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=C16 + 2, out=1), aqg.AQG_ERR_ALIGNMENT),
    (dict(y=A16), aqg.AQG_ERR_INVALID_ARG),              # output overlaps x
    (dict(ws=B16), aqg.AQG_ERR_INVALID_ARG),             # workspace overlaps Wq
    (dict(ws=C16), aqg.AQG_ERR_INVALID_ARG),             # workspace overlaps y
])
def test_gemm_validation(lib, kwargs, status):
    for bits in range(2, 9):
        assert gemm(lib, bits=bits, **kwargs) == status


def test_gemm_accepts_decode_and_prompt_sizes_up_to_the_device_check(lib):
    """Valid arguments get past validation (to the device check: no GPU here,
    or the call is made on one)."""
    if HAS_GPU_NODE:
        pytest.skip("a GPU node is present: the call would launch")
    far = [(i + 1) << 30 for i in range(6)]   # arrays 1 GiB apart: no overlap
    for M in (1, 32, 33, 4096):
        assert gemm(lib, M=M, K=1024, x=far[0], Wq=far[1], s=far[2], b=far[3], y=far[4],
                    ws=far[5]) == aqg.AQG_ERR_DEVICE


def test_gemm_dispatch_query():
    for bits in range(2, 9):
        path, cols = aqg.dispatch_path(aqg.AQG_KIND_GEMM_AFFINE + bits, 512, 14336, 4096)
        assert path == "affine_gemm" and cols == 64
    with pytest.raises(aqg.AqgError):
        aqg.dispatch_path(aqg.AQG_KIND_GEMM_AFFINE + 4, 40, 100, 96)
