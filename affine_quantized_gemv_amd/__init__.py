"""Small-M decode projections on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libaqgemv.so`` (include/aqgemv.h).
PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the device is not gfx950, calls raise.

    y = gemv_bf16(x, W)                       # y[M,N] = x[M,K] . W[N,K]^T
    y = gemv_affine(x, Wq, scales, biases, 4) # affine 4-bit, groups of 64
    o = swiglu_bf16(x, Wg, Wu)                # silu(x.Wg^T) * (x.Wu^T)
    q = unpack_codes(Wq, bits, K)             # uint8 codes, test hook

Shapes, layouts and status codes are documented in include/aqgemv.h.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "lib_path", "load", "AqgError", "abi_version", "status_string", "workspace_bytes", "dispatch_path",
    "gemv_bf16", "gemv_affine", "swiglu_bf16", "swiglu_affine", "unpack_codes", "gemv_bf16_argmax",
    "gemv_affine_argmax", "gemv_bf16_multi", "gemv_affine_multi", "gemm_affine",
    "gemv_affine_q2", "gemv_affine_q3", "gemv_affine_q4", "gemv_affine_q5",
    "gemv_affine_q6", "gemv_affine_q7", "gemv_affine_q8",
    "AQG_OK", "AQG_ERR_INVALID_ARG", "AQG_ERR_UNSUPPORTED", "AQG_ERR_ALIGNMENT",
    "AQG_ERR_LAUNCH", "AQG_ERR_DEVICE", "AQG_OUT_BF16", "AQG_OUT_F32",
]

AQG_OK, AQG_ERR_INVALID_ARG, AQG_ERR_UNSUPPORTED, AQG_ERR_ALIGNMENT, AQG_ERR_LAUNCH, AQG_ERR_DEVICE = range(6)
AQG_OUT_BF16, AQG_OUT_F32 = 0, 1
AQG_KIND_DENSE, AQG_KIND_SWIGLU, AQG_KIND_SWIGLU_AFFINE, AQG_KIND_ARGMAX_DENSE = 0, 9, 16, 32
AQG_KIND_GEMM_AFFINE = 48      # + bits: affine prompt GEMM (any M)
GEMM_MAX_M = 65536             # AQG_GEMM_MAX_M

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_lock = threading.Lock()


def lib_path() -> str:
    return os.path.join(_HERE, "libaqgemv.so")


class AqgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, status_string(status) if _lib else status))


def load():
    """Load libaqgemv.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError("libaqgemv.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.aqg_abi_version.restype = I
        lib.aqg_abi_version.argtypes = []
        lib.aqg_status_string.restype = ctypes.c_char_p
        lib.aqg_status_string.argtypes = [I]
        lib.aqg_workspace_bytes.restype = Z
        lib.aqg_workspace_bytes.argtypes = [I, I, I, I]
        lib.aqg_gemv_bf16.restype = I
        lib.aqg_gemv_bf16.argtypes = [P, P, P, I, I, I, I, P, Z, P]
        for b in range(2, 9):
            f = getattr(lib, "aqg_gemv_affine_q%d" % b)
            f.restype = I
            f.argtypes = [P, P, P, P, P, I, I, I, I, P, Z, P]
        lib.aqg_swiglu_bf16.restype = I
        lib.aqg_swiglu_bf16.argtypes = [P, P, P, P, I, I, I, I, P, Z, P]
        lib.aqg_unpack_codes.restype = I
        lib.aqg_unpack_codes.argtypes = [I, P, P, I, I, P]
        for b in range(2, 9):
            f = getattr(lib, "aqg_swiglu_affine_q%d" % b)
            f.restype = I
            f.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, Z, P]
        PP = ctypes.POINTER(ctypes.c_void_p)
        IP = ctypes.POINTER(ctypes.c_int)
        lib.aqg_gemv_bf16_multi.restype = I
        lib.aqg_gemv_bf16_multi.argtypes = [P, I, PP, PP, IP, I, I, I, P, Z, P]
        for b in range(2, 9):
            f = getattr(lib, "aqg_gemv_affine_q%d_multi" % b)
            f.restype = I
            f.argtypes = [P, I, PP, PP, PP, PP, IP, I, I, I, P, Z, P]
        lib.aqg_gemv_bf16_argmax.restype = I
        lib.aqg_gemv_bf16_argmax.argtypes = [P, P, P, P, I, I, I, P, Z, P]
        for b in range(2, 9):
            f = getattr(lib, "aqg_gemv_affine_q%d_argmax" % b)
            f.restype = I
            f.argtypes = [P, P, P, P, P, P, I, I, I, P, Z, P]
        for b in range(2, 9):
            f = getattr(lib, "aqg_gemm_affine_q%d" % b)
            f.restype = I
            f.argtypes = [P, P, P, P, P, I, I, I, I, P, Z, P]
        lib.aqg_gemv_argmax_noalloc.restype = I
        lib.aqg_gemv_argmax_noalloc.argtypes = [I, P, P, P, P, P, P, I, I, I, P]
        lib.aqg_stream_read.restype = I
        lib.aqg_stream_read.argtypes = [P, Z, P, P]
        lib.aqg_dispatch_path.restype = I
        lib.aqg_dispatch_path.argtypes = [I, I, I, I, ctypes.POINTER(I)]
        lib.aqg_path_name.restype = ctypes.c_char_p
        lib.aqg_path_name.argtypes = [I]
        _lib = lib
        return lib


def abi_version() -> int:
    return load().aqg_abi_version()


def status_string(status: int) -> str:
    return load().aqg_status_string(int(status)).decode()


def workspace_bytes(kind: int, M: int, N: int, K: int) -> int:
    return int(load().aqg_workspace_bytes(kind, M, N, K))


def dispatch_path(kind: int, M: int, N: int, K: int):
    """(path name, kernel columns) a call would run on (test hook; launches nothing)."""
    cols = ctypes.c_int(0)
    p = load().aqg_dispatch_path(kind, M, N, K, ctypes.byref(cols))
    if p < 0:
        raise AqgError(-p, "aqg_dispatch_path")
    return load().aqg_path_name(p).decode(), cols.value


# ------------------------------------------------------------ marshalling

def _check(status: int, what: str) -> None:
    if status != AQG_OK:
        raise AqgError(status, what)


def _dev(t: torch.Tensor, name: str, dtypes, ndim: int = 2) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype not in dtypes:
        raise ValueError("%s must have dtype in %s, got %s" % (name, dtypes, t.dtype))
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-D tensor" % (name, ndim))
    return t


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _out(out, M: int, N: int, out_dtype, like: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty((M, N), dtype=out_dtype, device=like.device)
    _dev(out, "out", (torch.bfloat16, torch.float32))
    if tuple(out.shape) != (M, N):
        raise ValueError("out must have shape %s" % ((M, N),))
    return out


def _odt(t: torch.Tensor) -> int:
    return AQG_OUT_F32 if t.dtype == torch.float32 else AQG_OUT_BF16


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _ws(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def gemv_bf16(x: torch.Tensor, W: torch.Tensor, out_dtype=torch.bfloat16, out=None, workspace=None):
    """y[M,N] = x[M,K] . W[N,K]^T (bf16 in, fp32 accumulate, bf16 or fp32 out)."""
    _dev(x, "x", (torch.bfloat16,))
    _dev(W, "W", (torch.bfloat16,))
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, %d]" % K)
    y = _out(out, M, N, out_dtype, x)
    ws, wsb = _ws(workspace)
    _check(load().aqg_gemv_bf16(_p(x), _p(W), _p(y), M, N, K, _odt(y), ws, wsb, _stream(x)),
           "aqg_gemv_bf16")
    return y


def gemv_affine(x: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                bits: int, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Affine b-bit GEMV: y = x . (scale*q + bias)^T with groups of 64 along K.

    Wq: int32/uint32 [N, K*bits/32] (LSB-first bit stream per row);
    scales, biases: bf16 [N, K/64].
    """
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(x, "x", (torch.bfloat16,))
    _dev(Wq, "Wq", (torch.int32, torch.uint32))
    _dev(scales, "scales", (torch.bfloat16,))
    _dev(biases, "biases", (torch.bfloat16,))
    M, K = x.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 32 != K * bits:
        raise ValueError("Wq must be [N, K*bits/32]")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales and biases must be [N, K/64]")
    y = _out(out, M, N, out_dtype, x)
    ws, wsb = _ws(workspace)
    fn = getattr(load(), "aqg_gemv_affine_q%d" % bits)
    _check(fn(_p(x), _p(Wq), _p(scales), _p(biases), _p(y), M, N, K, _odt(y), ws, wsb, _stream(x)),
           "aqg_gemv_affine_q%d" % bits)
    return y


def _affine_b(bits):
    def f(x, Wq, scales, biases, out_dtype=torch.bfloat16, out=None, workspace=None):
        return gemv_affine(x, Wq, scales, biases, bits, out_dtype, out, workspace)
    f.__name__ = "gemv_affine_q%d" % bits
    f.__doc__ = "Affine %d-bit GEMV (see gemv_affine)." % bits
    return f


gemv_affine_q2 = _affine_b(2)
gemv_affine_q3 = _affine_b(3)
gemv_affine_q4 = _affine_b(4)
gemv_affine_q5 = _affine_b(5)
gemv_affine_q6 = _affine_b(6)
gemv_affine_q7 = _affine_b(7)
gemv_affine_q8 = _affine_b(8)


def swiglu_bf16(x: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, out_dtype=torch.bfloat16,
                out=None, workspace=None):
    """out[M,N] = silu(x.Wg^T) * (x.Wu^T), fp32 inside."""
    _dev(x, "x", (torch.bfloat16,))
    _dev(Wg, "Wg", (torch.bfloat16,))
    _dev(Wu, "Wu", (torch.bfloat16,))
    M, K = x.shape
    N = Wg.shape[0]
    if tuple(Wg.shape) != (N, K) or tuple(Wu.shape) != (N, K):
        raise ValueError("Wg and Wu must both be [N, %d]" % K)
    y = _out(out, M, N, out_dtype, x)
    ws, wsb = _ws(workspace)
    _check(load().aqg_swiglu_bf16(_p(x), _p(Wg), _p(Wu), _p(y), M, N, K, _odt(y), ws, wsb, _stream(x)),
           "aqg_swiglu_bf16")
    return y


def _affine_check(Wq, scales, biases, bits: int, N: int, K: int, name: str):
    _dev(Wq, name + " Wq", (torch.int32, torch.uint32))
    _dev(scales, name + " scales", (torch.bfloat16,))
    _dev(biases, name + " biases", (torch.bfloat16,))
    if tuple(Wq.shape) != (N, K * bits // 32):
        raise ValueError("%s Wq must be [%d, %d]" % (name, N, K * bits // 32))
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("%s scales and biases must be [%d, %d]" % (name, N, K // 64))


def swiglu_affine(x: torch.Tensor, gate, up, bits: int, out_dtype=torch.bfloat16, out=None, workspace=None):
    """out[M,N] = silu(x.Wg^T) * (x.Wu^T) with affine b-bit Wg and Wu, fp32 inside.

    gate, up: (Wq int32/uint32 [N, K*bits/32], scales bf16 [N, K/64],
    biases bf16 [N, K/64]) each.
    """
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(x, "x", (torch.bfloat16,))
    M, K = x.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    N = gate[0].shape[0]
    _affine_check(*gate, bits, N, K, "gate")
    _affine_check(*up, bits, N, K, "up")
    y = _out(out, M, N, out_dtype, x)
    ws, wsb = _ws(workspace)
    fn = getattr(load(), "aqg_swiglu_affine_q%d" % bits)
    _check(fn(_p(x), _p(gate[0]), _p(gate[1]), _p(gate[2]), _p(up[0]), _p(up[1]), _p(up[2]), _p(y),
              M, N, K, _odt(y), ws, wsb, _stream(x)), "aqg_swiglu_affine_q%d" % bits)
    return y


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _multi_out(out, M: int, Ns, out_dtype, like):
    if out is None:
        return [torch.empty((M, n), dtype=out_dtype, device=like.device) for n in Ns]
    if len(out) != len(Ns):
        raise ValueError("one output per projection")
    return [_out(o, M, n, out_dtype, like) for o, n in zip(out, Ns)]


def gemv_bf16_multi(x: torch.Tensor, Ws, out_dtype=torch.bfloat16, out=None, workspace=None):
    """[x . W_p^T for each W_p] (1..4 dense projections of the same x) in one call."""
    _dev(x, "x", (torch.bfloat16,))
    M, K = x.shape
    for i, W in enumerate(Ws):
        _dev(W, "W[%d]" % i, (torch.bfloat16,))
        if W.shape[1] != K:
            raise ValueError("W[%d] must be [N, %d]" % (i, K))
    Ns = [W.shape[0] for W in Ws]
    ys = _multi_out(out, M, Ns, out_dtype, x)
    ws, wsb = _ws(workspace)
    _check(load().aqg_gemv_bf16_multi(_p(x), len(Ws), _ptrs(Ws), _ptrs(ys), (ctypes.c_int * len(Ns))(*Ns),
                                      M, K, _odt(ys[0]), ws, wsb, _stream(x)), "aqg_gemv_bf16_multi")
    return ys


def gemv_affine_multi(x: torch.Tensor, mats, bits: int, out_dtype=torch.bfloat16, out=None, workspace=None):
    """[x . (scale*q + bias)_p^T for each (Wq, scales, biases)_p] of one width, in one call."""
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(x, "x", (torch.bfloat16,))
    M, K = x.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    Ns = []
    for i, (Wq, sc, bi) in enumerate(mats):
        N = Wq.shape[0]
        _affine_check(Wq, sc, bi, bits, N, K, "projection %d" % i)
        Ns.append(N)
    ys = _multi_out(out, M, Ns, out_dtype, x)
    ws, wsb = _ws(workspace)
    fn = getattr(load(), "aqg_gemv_affine_q%d_multi" % bits)
    _check(fn(_p(x), len(mats), _ptrs([m[0] for m in mats]), _ptrs([m[1] for m in mats]),
              _ptrs([m[2] for m in mats]), _ptrs(ys), (ctypes.c_int * len(Ns))(*Ns), M, K, _odt(ys[0]),
              ws, wsb, _stream(x)), "aqg_gemv_affine_q%d_multi" % bits)
    return ys


def _argmax_out(M: int, like: torch.Tensor, out):
    if out is None:
        return (torch.empty(M, dtype=torch.float32, device=like.device),
                torch.empty(M, dtype=torch.int32, device=like.device))
    val, idx = out
    _dev(val, "out[0]", (torch.float32,), ndim=1)
    _dev(idx, "out[1]", (torch.int32,), ndim=1)
    if val.shape[0] != M or idx.shape[0] != M:
        raise ValueError("argmax outputs must have %d rows" % M)
    return val, idx


def _argmax_ws(kind: int, M: int, N: int, K: int, like: torch.Tensor, workspace):
    need = workspace_bytes(kind, M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace needs %d bytes" % need)
    return workspace


def gemm_affine(x: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                bits: int, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Affine b-bit prompt GEMM: the product of gemv_affine for any M (up to
    GEMM_MAX_M rows of x).  workspace: a device tensor of at least
    workspace_bytes(AQG_KIND_GEMM_AFFINE + bits, M, N, K) bytes (allocated
    here when None)."""
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(x, "x", (torch.bfloat16,))
    M, K = x.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    N = Wq.shape[0]
    _affine_check(Wq, scales, biases, bits, N, K, "W")
    y = _out(out, M, N, out_dtype, x)
    ws = _argmax_ws(AQG_KIND_GEMM_AFFINE + bits, M, N, K, x, workspace)
    fn = getattr(load(), "aqg_gemm_affine_q%d" % bits)
    _check(fn(_p(x), _p(Wq), _p(scales), _p(biases), _p(y), M, N, K, _odt(y), _p(ws),
              ws.numel() * ws.element_size(), _stream(x)), "aqg_gemm_affine_q%d" % bits)
    return y


def gemv_bf16_argmax(x: torch.Tensor, W: torch.Tensor, out=None, workspace=None):
    """(max value fp32 [M], index int32 [M]) of each row of x . W^T; the lowest
    index wins ties; the logits are not written."""
    _dev(x, "x", (torch.bfloat16,))
    _dev(W, "W", (torch.bfloat16,))
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, %d]" % K)
    val, idx = _argmax_out(M, x, out)
    ws = _argmax_ws(AQG_KIND_ARGMAX_DENSE, M, N, K, x, workspace)
    _check(load().aqg_gemv_bf16_argmax(_p(x), _p(W), _p(val), _p(idx), M, N, K, *_ws(ws), _stream(x)),
           "aqg_gemv_bf16_argmax")
    return val, idx


def gemv_affine_argmax(x: torch.Tensor, Wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                       bits: int, out=None, workspace=None):
    """Row argmax of the affine b-bit GEMV (see gemv_affine and gemv_bf16_argmax)."""
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(x, "x", (torch.bfloat16,))
    _dev(Wq, "Wq", (torch.int32, torch.uint32))
    _dev(scales, "scales", (torch.bfloat16,))
    _dev(biases, "biases", (torch.bfloat16,))
    M, K = x.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 32 != K * bits:
        raise ValueError("Wq must be [N, K*bits/32]")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales and biases must be [N, K/64]")
    val, idx = _argmax_out(M, x, out)
    ws = _argmax_ws(AQG_KIND_ARGMAX_DENSE + bits, M, N, K, x, workspace)
    fn = getattr(load(), "aqg_gemv_affine_q%d_argmax" % bits)
    _check(fn(_p(x), _p(Wq), _p(scales), _p(biases), _p(val), _p(idx), M, N, K, *_ws(ws), _stream(x)),
           "aqg_gemv_affine_q%d_argmax" % bits)
    return val, idx


def unpack_codes(Wq: torch.Tensor, bits: int, K: int, out=None) -> torch.Tensor:
    """codes[N, K] uint8 through the kernels' own unpack path."""
    if bits not in range(2, 9):
        raise ValueError("bits must be in 2..8")
    _dev(Wq, "Wq", (torch.int32, torch.uint32))
    N = Wq.shape[0]
    if Wq.shape[1] * 32 != K * bits:
        raise ValueError("Wq must be [N, K*bits/32]")
    if out is None:
        codes = torch.empty((N, K), dtype=torch.uint8, device=Wq.device)
    else:
        codes = _dev(out, "out", (torch.uint8,))
        if tuple(codes.shape) != (N, K) or codes.device != Wq.device:
            raise ValueError("out must be a uint8 [%d, %d] tensor on %s" % (N, K, Wq.device))
    _check(load().aqg_unpack_codes(bits, _p(Wq), _p(codes), N, K, _stream(Wq)), "aqg_unpack_codes")
    return codes
