"""MI355X-native Q8_0 block-quantized contraction (``qdot_t``) -- Python binding.

Thin ctypes binding over the C-ABI library ``libq8qdot.so`` built from
``csrc/`` for gfx950 (declarations: ``include/q8qdot.h``).  The functions keep
the C names.  They only marshal arguments -- check dtypes, shapes, devices and
contiguity of torch tensors, pass their device pointers and the current HIP
stream -- and raise :class:`Q8Error` on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no CPU fallback: when
the library is missing, every call raises.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import _build

LIB_PATH = _build.LIB_PATH

Q8_OK = 0
Q8_EINVAL = -1
Q8_ENULL = -2
Q8_EALIGN = -3
Q8_ELAUNCH = -4
Q8_ERANGE = -5

# Every symbol include/q8qdot.h declares.
EXPORTS = ("q8_qdot", "q8_qdot_stream", "q8_qmma", "q8_qdot_partials", "q8_qdot_path",
           "q8_qdot_ws_size", "q8_qdot_ws", "q8_qmma_ws", "q8_qdot_ws_partials", "q8_qdot_noalloc",
           "q8_q50_qdot", "q8_q50_qmma", "q8_q50_partials", "q8_q50_path",
           "q8_quantize", "q8_strerror", "q8_version")

_lock = threading.Lock()
_lib = None


class Q8Error(RuntimeError):
    """A non-zero q8_status from the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, _strerror(status), status))


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (no build, no fallback)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                "libq8qdot.so is not built (%s). Build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` or "
                "`python gemm_q8_qdot_amd/_build.py`." % p)
        lib = ctypes.CDLL(p)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.q8_qdot.restype = ci
        lib.q8_qdot.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci]
        lib.q8_qdot_stream.restype = ci
        lib.q8_qdot_stream.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
        lib.q8_qmma.restype = ci
        lib.q8_qmma.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
        for name in ("q8_q50_qdot", "q8_q50_qmma"):
            getattr(lib, name).restype = ci
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
        lib.q8_q50_partials.restype = ci
        lib.q8_q50_partials.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        lib.q8_qdot_partials.restype = ci
        lib.q8_qdot_partials.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        for name in ("q8_qdot_ws", "q8_qmma_ws"):
            getattr(lib, name).restype = ci
            getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp, ctypes.c_size_t, vp]
        lib.q8_qdot_noalloc.restype = ci
        lib.q8_qdot_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
        lib.q8_qdot_ws_size.restype = ci
        lib.q8_qdot_ws_size.argtypes = [ci, ci, ci, ctypes.POINTER(ctypes.c_size_t)]
        lib.q8_qdot_ws_partials.restype = ci
        lib.q8_qdot_ws_partials.argtypes = [vp, vp, vp, ci, ci, ci, vp]
        lib.q8_qdot_path.restype = ci
        lib.q8_qdot_path.argtypes = [ci, ci, ci]
        lib.q8_q50_path.restype = ci
        lib.q8_q50_path.argtypes = [ci, ci, ci]
        lib.q8_quantize.restype = ci
        lib.q8_quantize.argtypes = [vp, vp, vp, ci, ci, vp]
        lib.q8_strerror.restype = ctypes.c_char_p
        lib.q8_strerror.argtypes = [ci]
        lib.q8_version.restype = ci
        lib.q8_version.argtypes = []
        if path is None:
            _lib = lib
        return lib


def ensure_built() -> str:
    """Build the library when it is absent (tests, smoke, bench)."""
    if not os.path.exists(LIB_PATH):
        _build.build()
    return LIB_PATH


def _strerror(status: int) -> str:
    try:
        return load().q8_strerror(status).decode()
    except Exception:  # library missing while formatting an error
        return "status %d" % status


def _check(status: int, what: str) -> None:
    if status != Q8_OK:
        raise Q8Error(status, what)


# ----------------------------------------------------------------- raw pointers
# Integer device addresses; ``stream`` is a hipStream_t as an int (0 = null).

def q8_qdot_raw(A: int, AS: int, W: int, WS: int, C: int, M: int, N: int, K: int,
                stream: int = 0) -> int:
    """``q8_qdot_stream`` on raw device addresses; returns the status."""
    return load().q8_qdot_stream(A, AS, W, WS, C, M, N, K, stream or None)


def q8_qmma_raw(A: int, AS: int, W: int, WST: int, C: int, M: int, N: int, K: int,
                stream: int = 0) -> int:
    """``q8_qmma`` (weight scales ``[K/32, N]``) on raw device addresses; returns the status."""
    return load().q8_qmma(A, AS, W, WST, C, M, N, K, stream or None)


def q8_q50_qdot_raw(A: int, AS: int, W5: int, WS: int, C: int, M: int, N: int, K: int,
                    stream: int = 0, ws_t: bool = False) -> int:
    """``q8_q50_qdot`` (or, with ``ws_t``, ``q8_q50_qmma``) on raw device addresses."""
    f = load().q8_q50_qmma if ws_t else load().q8_q50_qdot
    return f(A, AS, W5, WS, C, M, N, K, stream or None)


def q8_qdot_ws_raw(A: int, AS: int, W: int, WS: int, C: int, M: int, N: int, K: int,
                   workspace: int, ws_bytes: int, stream: int = 0, ws_t: bool = False) -> int:
    """``q8_qdot_ws`` (or, with ``ws_t``, ``q8_qmma_ws``) on raw device addresses."""
    f = load().q8_qmma_ws if ws_t else load().q8_qdot_ws
    return f(A, AS, W, WS, C, M, N, K, workspace or None, ws_bytes, stream or None)


def q8_qdot_noalloc_raw(A: int, AS: int, W: int, WS: int, C: int, M: int, N: int, K: int,
                        stream: int = 0) -> int:
    """``q8_qdot_noalloc`` (the split form in the library's static scratch) on raw addresses."""
    return load().q8_qdot_noalloc(A, AS, W, WS, C, M, N, K, stream or None)


def q8_qdot_ws_partials_raw(A: int, W: int, P: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().q8_qdot_ws_partials(A, W, P, M, N, K, stream or None)


def q8_q50_partials_raw(A: int, W5: int, P: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().q8_q50_partials(A, W5, P, M, N, K, stream or None)


def q8_qdot_partials_raw(A: int, W: int, P: int, M: int, N: int, K: int, stream: int = 0) -> int:
    return load().q8_qdot_partials(A, W, P, M, N, K, stream or None)


def q8_quantize_raw(X: int, Q: int, D: int, rows: int, K: int, stream: int = 0) -> int:
    return load().q8_quantize(X, Q, D, rows, K, stream or None)


# -------------------------------------------------------------- torch tensors

def _torch():
    import torch
    return torch


def _current_stream(dev) -> int:
    torch = _torch()
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.numel() and not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major, densely packed)" % name)


def _ptr(t) -> int:
    return t.data_ptr() if t.numel() else 0


def q8_qdot(A, AS, W, WS, C=None, stream=None):
    """``C[M, N] = qdot_t(A, AS, W, WS)`` on the GPU (f32 output).

    ``A`` int8 ``[M, K]``, ``AS`` f32 ``[M, K/32]``, ``W`` int8 ``[N, K]``,
    ``WS`` f32 ``[N, K/32]``; ``C`` f32 ``[M, N]`` (allocated when omitted).
    Runs on ``stream`` (a torch stream, default: the current stream).
    """
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    KB = K // 32
    _need(A, torch.int8, (M, K), "A")
    _need(AS, torch.float32, (M, KB), "AS")
    _need(W, torch.int8, (N, K), "W")
    _need(WS, torch.float32, (N, KB), "WS")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _need(C, torch.float32, (M, N), "C")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    st = load().q8_qdot_stream(_ptr(A), _ptr(AS), _ptr(W), _ptr(WS), _ptr(C), M, N, K, s or None)
    _check(st, "q8_qdot")
    return C


q8_qdot_stream = q8_qdot


def q8_qmma(A, AS, W, WST, C=None, stream=None):
    """``C[M, N] = qmma_t(A, AS, W, WST)``: as :func:`q8_qdot` with the weight
    scales stored transposed, ``WST`` f32 ``[K/32, N]``."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    KB = K // 32
    _need(A, torch.int8, (M, K), "A")
    _need(AS, torch.float32, (M, KB), "AS")
    _need(W, torch.int8, (N, K), "W")
    _need(WST, torch.float32, (KB, N), "WST")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _need(C, torch.float32, (M, N), "C")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    st = load().q8_qmma(_ptr(A), _ptr(AS), _ptr(W), _ptr(WST), _ptr(C), M, N, K, s or None)
    _check(st, "q8_qmma")
    return C


def q8_qdot_partials(A, W, P=None, stream=None):
    """Per-block int32 partials ``P[M, N, K/32]`` from the same kernel ``q8_qdot`` uses."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    _need(A, torch.int8, (M, K), "A")
    _need(W, torch.int8, (N, K), "W")
    if P is None:
        P = torch.empty((M, N, K // 32), dtype=torch.int32, device=A.device)
    _need(P, torch.int32, (M, N, K // 32), "P")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    st = load().q8_qdot_partials(_ptr(A), _ptr(W), _ptr(P), M, N, K, s or None)
    _check(st, "q8_qdot_partials")
    return P


def q8_qdot_ws_size(M: int, N: int, K: int) -> int:
    """Workspace bytes ``q8_qdot_ws`` / ``q8_qmma_ws`` use for this shape on the
    current device (0: the shape does not take the split form)."""
    n = ctypes.c_size_t(0)
    _check(load().q8_qdot_ws_size(M, N, K, ctypes.byref(n)), "q8_qdot_ws_size")
    return int(n.value)


def workspace(M: int, N: int, K: int, device=None):
    """A zero-filled uint8 device tensor of ``q8_qdot_ws_size(M, N, K)`` bytes
    (at least one byte), for the ``*_ws`` entries."""
    torch = _torch()
    return torch.zeros(max(1, q8_qdot_ws_size(M, N, K)), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def _ws_call(A, AS, W, WS, workspace, C, stream, ws_t):
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    KB = K // 32
    _need(A, torch.int8, (M, K), "A")
    _need(AS, torch.float32, (M, KB), "AS")
    _need(W, torch.int8, (N, K), "W")
    _need(WS, torch.float32, (KB, N) if ws_t else (N, KB), "WST" if ws_t else "WS")
    _need(workspace, torch.uint8, (workspace.numel(),), "workspace")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _need(C, torch.float32, (M, N), "C")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    f = load().q8_qmma_ws if ws_t else load().q8_qdot_ws
    st = f(_ptr(A), _ptr(AS), _ptr(W), _ptr(WS), _ptr(C), M, N, K, _ptr(workspace),
           workspace.numel(), s or None)
    _check(st, "q8_qmma_ws" if ws_t else "q8_qdot_ws")
    return C


def q8_qdot_ws(A, AS, W, WS, workspace, C=None, stream=None):
    """:func:`q8_qdot` with a caller workspace (a zero-filled uint8 tensor, see
    :func:`workspace`); shapes with few output tiles split the contraction
    across workgroups."""
    return _ws_call(A, AS, W, WS, workspace, C, stream, False)


def q8_qmma_ws(A, AS, W, WST, workspace, C=None, stream=None):
    """:func:`q8_qmma` with a caller workspace (see :func:`q8_qdot_ws`)."""
    return _ws_call(A, AS, W, WST, workspace, C, stream, True)


def q8_qdot_ws_partials(A, W, P=None, stream=None):
    """Per-block int32 partials from the kernel ``q8_qdot_ws`` uses for the shape."""
    torch = _torch()
    M, K = A.shape
    N = W.shape[0]
    _need(A, torch.int8, (M, K), "A")
    _need(W, torch.int8, (N, K), "W")
    if P is None:
        P = torch.empty((M, N, K // 32), dtype=torch.int32, device=A.device)
    _need(P, torch.int32, (M, N, K // 32), "P")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    st = load().q8_qdot_ws_partials(_ptr(A), _ptr(W), _ptr(P), M, N, K, s or None)
    _check(st, "q8_qdot_ws_partials")
    return P


def _q50_call(A, AS, W5, WS, C, stream, ws_t):
    torch = _torch()
    M, K = A.shape
    N = W5.shape[0]
    KB = K // 32
    _need(A, torch.int8, (M, K), "A")
    _need(AS, torch.float32, (M, KB), "AS")
    _need(W5, torch.uint8, (N, KB * 20), "W5")
    _need(WS, torch.float32, (KB, N) if ws_t else (N, KB), "WST" if ws_t else "WS")
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    _need(C, torch.float32, (M, N), "C")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    f = load().q8_q50_qmma if ws_t else load().q8_q50_qdot
    _check(f(_ptr(A), _ptr(AS), _ptr(W5), _ptr(WS), _ptr(C), M, N, K, s or None),
           "q8_q50_qmma" if ws_t else "q8_q50_qdot")
    return C


def q8_q50_qdot(A, AS, W5, WS, C=None, stream=None):
    """``C = q50_qdot_t(A, AS, W5, WS)``: Q5_0 weights ``W5`` uint8 ``[N, K/32*20]``, ``WS [N, K/32]``."""
    return _q50_call(A, AS, W5, WS, C, stream, False)


def q8_q50_qmma(A, AS, W5, WST, C=None, stream=None):
    """``C = q50_qmma_t(A, AS, W5, WST)``: as :func:`q8_q50_qdot` with ``WST [K/32, N]``."""
    return _q50_call(A, AS, W5, WST, C, stream, True)


def q8_q50_partials(A, W5, P=None, stream=None):
    """Per-block int32 partials against Q5_0 weights, ``P[M, N, K/32]``."""
    torch = _torch()
    M, K = A.shape
    N = W5.shape[0]
    _need(A, torch.int8, (M, K), "A")
    _need(W5, torch.uint8, (N, K // 32 * 20), "W5")
    if P is None:
        P = torch.empty((M, N, K // 32), dtype=torch.int32, device=A.device)
    _need(P, torch.int32, (M, N, K // 32), "P")
    s = stream.cuda_stream if stream is not None else _current_stream(A.device)
    _check(load().q8_q50_partials(_ptr(A), _ptr(W5), _ptr(P), M, N, K, s or None), "q8_q50_partials")
    return P


def q8_quantize(X, Q=None, D=None, stream=None):
    """Q8_0-quantize f32 rows ``X [rows, K]`` -> ``(Q int8 [rows, K], D f32 [rows, K/32])``."""
    torch = _torch()
    rows, K = X.shape
    _need(X, torch.float32, (rows, K), "X")
    if Q is None:
        Q = torch.empty((rows, K), dtype=torch.int8, device=X.device)
    if D is None:
        D = torch.empty((rows, K // 32), dtype=torch.float32, device=X.device)
    _need(Q, torch.int8, (rows, K), "Q")
    _need(D, torch.float32, (rows, K // 32), "D")
    s = stream.cuda_stream if stream is not None else _current_stream(X.device)
    st = load().q8_quantize(_ptr(X), _ptr(Q), _ptr(D), rows, K, s or None)
    _check(st, "q8_quantize")
    return Q, D


def q8_qdot_path(M: int, N: int, K: int) -> int:
    """0 = wave64 matvec, 1 = MFMA GEMM (K split across a workgroup), 2 = MFMA GEMM (LDS-staged
    128 x 224 tiles), 3 = MFMA GEMM (64 x 64 tiles over all of K through an LDS ring)."""
    st = load().q8_qdot_path(M, N, K)
    if st < 0:
        raise Q8Error(st, "q8_qdot_path")
    return st


def q8_q50_path(M: int, N: int, K: int) -> int:
    """Q5_0 weights (16-byte aligned): 0 = Q5_0 matvec, 1 = K-split MFMA GEMM, 3 = 64 x 64-tile
    ring GEMM decoding each stage in LDS."""
    st = load().q8_q50_path(M, N, K)
    if st < 0:
        raise Q8Error(st, "q8_q50_path")
    return st


def q8_strerror(status: int) -> str:
    return load().q8_strerror(status).decode()


def q8_version() -> int:
    return int(load().q8_version())
