"""Q8_0 qdot oracle -- TEST INFRASTRUCTURE ONLY.

Plain CPU statement of the Q8_0 block contraction (``qdot_t``), used to check
the GPU library.  Only ``tests/``, the smoke check and the benchmark's CPU
baseline leg may import this package; the GPU product never does, and this
package never imports the product.

What it computes (Phobos documentation pages):

* "Phobos Language Spec", section "Quantized built-ins", Q8_0 table, row
  ``qdot_t``: ``out[i, j] = sum_b a_scales[i, b] * w_scales[j, b] *
  sum_{k in b} a[i, k] * w[j, k]`` with 32-wide blocks, scales ``[M, K/32]``
  and ``[N, K/32]``.
* "Quantized built-ins and formats", section "Q8_0": signed bytes, one scale
  per 32 values, activations quantized the same way, integer inner sums.

The arithmetic lives in ``q8_oracle.c`` (plain C, OpenMP over independent
outputs only); this module builds it with gcc when no library is present and
marshals NumPy arrays.  ``brute.py`` holds the exact-rational brute force used
to pin it on tiny shapes.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
(exact rationals, closed forms, integer invariants, quantizer properties and a
hand-derived worked example under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point this at a deliberately broken build of q8_oracle.c to show
# that the pins catch a planted mistake.
_LIB_OVERRIDE = os.environ.get("Q8_ORACLE_LIB")
BLOCK = 32

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile ``q8_oracle.c`` into ``liboracle.so`` (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = BUILD_FLAGS.split() + ["-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                if not os.path.exists(_LIB_PATH):
                    build()
                lib = ctypes.CDLL(_LIB_PATH)
            p = ctypes.c_void_p
            i64 = ctypes.c_int64
            lib.q8o_num_threads.restype = ctypes.c_int
            lib.q8o_num_threads.argtypes = []
            lib.q8o_set_num_threads.restype = None
            lib.q8o_set_num_threads.argtypes = [ctypes.c_int]
            lib.q8o_quantize_rows.restype = ctypes.c_int
            lib.q8o_quantize_rows.argtypes = [p, i64, i64, p, p]
            lib.q8o_block_partials.restype = ctypes.c_int
            lib.q8o_block_partials.argtypes = [p, p, p, i64, i64, i64]
            lib.q8o_qdot_f64.restype = ctypes.c_int
            lib.q8o_qdot_f64.argtypes = [p, p, p, p, i64, i64, i64, p, p]
            lib.q8o_qdot_f64_at.restype = ctypes.c_int
            lib.q8o_qdot_f64_at.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p, p]
            lib.q8o_qmma_f64.restype = ctypes.c_int
            lib.q8o_qmma_f64.argtypes = [p, p, p, p, i64, i64, i64, p, p]
            lib.q8o_qmma_f64_at.restype = ctypes.c_int
            lib.q8o_qmma_f64_at.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p, p]
            lib.q8o_q50_decode.restype = ctypes.c_int
            lib.q8o_q50_decode.argtypes = [p, p, i64, i64]
            lib.q8o_q50_block_partials.restype = ctypes.c_int
            lib.q8o_q50_block_partials.argtypes = [p, p, p, i64, i64, i64]
            lib.q8o_q50_f64.restype = ctypes.c_int
            lib.q8o_q50_f64.argtypes = [p, p, p, p, ctypes.c_int, i64, i64, i64, p, p]
            lib.q8o_q50_f64_at.restype = ctypes.c_int
            lib.q8o_q50_f64_at.argtypes = [p, p, p, p, ctypes.c_int, i64, i64, i64, p, p, i64, p, p]
            lib.q8o_block_partials_at.restype = ctypes.c_int
            lib.q8o_block_partials_at.argtypes = [p, p, i64, i64, i64, p, p, i64, p]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().q8o_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later calls (its OpenMP loops)."""
    _load().q8o_set_num_threads(int(n))


BUILD_FLAGS = "gcc -O2 -std=c11 -fopenmp -ffp-contract=off"


def quantize_rows(x: np.ndarray):
    """Q8_0-quantize f32 rows ``x [rows, K]`` -> ``(q int8 [rows, K], d f32 [rows, K/32])``.

    Per 32-block: ``d = f32(max|x| / 127)``, ``q = clamp(rint(x / d), -127, 127)``
    in f32 with ties-to-even, and ``d == 0`` gives ``q == 0`` (a reading: the
    pages do not say how Q8_0 values are produced).
    """
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((rows, K), np.int8)
    d = np.empty((rows, K // BLOCK), np.float32)
    rc = _load().q8o_quantize_rows(_ptr(x), rows, K, _ptr(q), _ptr(d))
    if rc:
        raise ValueError("q8o_quantize_rows failed: %d" % rc)
    return q, d


def _check_ops(A, W):
    A = _c(A, np.int8)
    W = _c(W, np.int8)
    if A.ndim != 2 or W.ndim != 2 or A.shape[1] != W.shape[1]:
        raise ValueError("A [M,K] and W [N,K] must share K")
    if A.shape[1] % BLOCK:
        raise ValueError("K must be a multiple of 32")
    return A, W


def block_partials(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Integer block partials ``P[i, j, b] = sum_{k in b} A[i,k] * W[j,k]`` (int32 ``[M, N, K/32]``)."""
    A, W = _check_ops(A, W)
    M, K = A.shape
    N = W.shape[0]
    P = np.empty((M, N, K // BLOCK), np.int32)
    rc = _load().q8o_block_partials(_ptr(A), _ptr(W), _ptr(P), M, N, K)
    if rc:
        raise ValueError("q8o_block_partials failed: %d" % rc)
    return P


def _check_scales(A, AS, W, WS):
    M, K = A.shape
    N = W.shape[0]
    AS = _c(AS, np.float32)
    WS = _c(WS, np.float32)
    if AS.shape != (M, K // BLOCK) or WS.shape != (N, K // BLOCK):
        raise ValueError("scales must be AS [M, K/32] and WS [N, K/32]")
    return AS, WS


def qdot_f64(A, AS, W, WS):
    """The ``qdot_t`` definition in f64: returns ``(out [M,N], abs_terms [M,N])`` (float64)."""
    A, W = _check_ops(A, W)
    AS, WS = _check_scales(A, AS, W, WS)
    M, K = A.shape
    N = W.shape[0]
    out = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    rc = _load().q8o_qdot_f64(_ptr(A), _ptr(AS), _ptr(W), _ptr(WS), M, N, K,
                             _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_qdot_f64 failed: %d" % rc)
    return out, mag


def qdot_f64_at(A, AS, W, WS, ii, jj):
    """The definition at sampled positions ``(ii[s], jj[s])``: ``(out [S], abs_terms [S])``."""
    A, W = _check_ops(A, W)
    AS, WS = _check_scales(A, AS, W, WS)
    M, K = A.shape
    N = W.shape[0]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D and equal length")
    out = np.empty(ii.shape[0], np.float64)
    mag = np.empty(ii.shape[0], np.float64)
    rc = _load().q8o_qdot_f64_at(_ptr(A), _ptr(AS), _ptr(W), _ptr(WS), M, N, K,
                                _ptr(ii), _ptr(jj), ii.shape[0], _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_qdot_f64_at failed: %d" % rc)
    return out, mag


def _check_scales_t(A, AS, W, WST):
    M, K = A.shape
    N = W.shape[0]
    AS = _c(AS, np.float32)
    WST = _c(WST, np.float32)
    if AS.shape != (M, K // BLOCK) or WST.shape != (K // BLOCK, N):
        raise ValueError("scales must be AS [M, K/32] and WST [K/32, N]")
    return AS, WST


def qmma_f64(A, AS, W, WST):
    """The ``qmma_t`` definition in f64 (weight scales ``WST [K/32, N]``): ``(out, abs_terms)``."""
    A, W = _check_ops(A, W)
    AS, WST = _check_scales_t(A, AS, W, WST)
    M, K = A.shape
    N = W.shape[0]
    out = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    rc = _load().q8o_qmma_f64(_ptr(A), _ptr(AS), _ptr(W), _ptr(WST), M, N, K,
                             _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_qmma_f64 failed: %d" % rc)
    return out, mag


def qmma_f64_at(A, AS, W, WST, ii, jj):
    """``qmma_t`` at sampled positions ``(ii[s], jj[s])``: ``(out [S], abs_terms [S])``."""
    A, W = _check_ops(A, W)
    AS, WST = _check_scales_t(A, AS, W, WST)
    M, K = A.shape
    N = W.shape[0]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D and equal length")
    out = np.empty(ii.shape[0], np.float64)
    mag = np.empty(ii.shape[0], np.float64)
    rc = _load().q8o_qmma_f64_at(_ptr(A), _ptr(AS), _ptr(W), _ptr(WST), M, N, K,
                                _ptr(ii), _ptr(jj), ii.shape[0], _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_qmma_f64_at failed: %d" % rc)
    return out, mag


def block_partials_at(A, W, ii, jj):
    """Integer partials at sampled positions: int32 ``[S, K/32]``."""
    A, W = _check_ops(A, W)
    M, K = A.shape
    N = W.shape[0]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    P = np.empty((ii.shape[0], K // BLOCK), np.int32)
    rc = _load().q8o_block_partials_at(_ptr(A), _ptr(W), M, N, K, _ptr(ii), _ptr(jj),
                                      ii.shape[0], _ptr(P))
    if rc:
        raise ValueError("q8o_block_partials_at failed: %d" % rc)
    return P


# ------------------------------------------------------------------ Q5_0

Q50_BLOCK_BYTES = 20


def _check_q50(A, W5):
    A = _c(A, np.int8)
    W5 = _c(W5, np.uint8)
    if A.ndim != 2 or W5.ndim != 2 or A.shape[1] % BLOCK:
        raise ValueError("A [M,K] with K % 32 == 0 and W5 [N, K/32*20]")
    if W5.shape[1] != A.shape[1] // BLOCK * Q50_BLOCK_BYTES:
        raise ValueError("W5 must be [N, K/32 * 20] bytes")
    return A, W5


def q50_decode(W5: np.ndarray, K: int) -> np.ndarray:
    """Q5_0 blocks ``W5 [N, K/32*20]`` (uint8) -> values ``int8 [N, K]`` in ``[-16, 15]``."""
    W5 = _c(W5, np.uint8)
    N = W5.shape[0]
    if K % BLOCK or W5.shape[1] != K // BLOCK * Q50_BLOCK_BYTES:
        raise ValueError("W5 must be [N, K/32 * 20] bytes")
    Wd = np.empty((N, K), np.int8)
    rc = _load().q8o_q50_decode(_ptr(W5), _ptr(Wd), N, K)
    if rc:
        raise ValueError("q8o_q50_decode failed: %d" % rc)
    return Wd


def q50_block_partials(A, W5) -> np.ndarray:
    """Integer block partials against Q5_0 weights: int32 ``[M, N, K/32]``."""
    A, W5 = _check_q50(A, W5)
    M, K = A.shape
    N = W5.shape[0]
    P = np.empty((M, N, K // BLOCK), np.int32)
    rc = _load().q8o_q50_block_partials(_ptr(A), _ptr(W5), _ptr(P), M, N, K)
    if rc:
        raise ValueError("q8o_q50_block_partials failed: %d" % rc)
    return P


def _q50_f64(A, AS, W5, WS, ws_t):
    A, W5 = _check_q50(A, W5)
    M, K = A.shape
    N = W5.shape[0]
    AS = _c(AS, np.float32)
    WS = _c(WS, np.float32)
    want = (K // BLOCK, N) if ws_t else (N, K // BLOCK)
    if AS.shape != (M, K // BLOCK) or WS.shape != want:
        raise ValueError("scales must be AS [M, K/32] and WS %s" % (want,))
    out = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    rc = _load().q8o_q50_f64(_ptr(A), _ptr(AS), _ptr(W5), _ptr(WS), int(ws_t), M, N, K,
                            _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_q50_f64 failed: %d" % rc)
    return out, mag


def q50_qdot_f64(A, AS, W5, WS):
    """``q50_qdot_t`` in f64 (weight scales ``[N, K/32]``): ``(out, abs_terms)``."""
    return _q50_f64(A, AS, W5, WS, False)


def q50_qmma_f64(A, AS, W5, WST):
    """``q50_qmma_t`` in f64 (weight scales ``[K/32, N]``): ``(out, abs_terms)``."""
    return _q50_f64(A, AS, W5, WST, True)


def q50_f64_at(A, AS, W5, WS, ws_t, ii, jj):
    """Q5_0 contraction at sampled positions: ``(out [S], abs_terms [S])``."""
    A, W5 = _check_q50(A, W5)
    M, K = A.shape
    N = W5.shape[0]
    AS = _c(AS, np.float32)
    WS = _c(WS, np.float32)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    out = np.empty(ii.shape[0], np.float64)
    mag = np.empty(ii.shape[0], np.float64)
    rc = _load().q8o_q50_f64_at(_ptr(A), _ptr(AS), _ptr(W5), _ptr(WS), int(ws_t), M, N, K,
                               _ptr(ii), _ptr(jj), ii.shape[0], _ptr(out), _ptr(mag))
    if rc:
        raise ValueError("q8o_q50_f64_at failed: %d" % rc)
    return out, mag


def within_tolerance(C, out64, abs64, rel=1e-5, absol=1e-6):
    """The acceptance bound ``|C - out64| <= rel * abs64 + absol`` elementwise."""
    C = np.asarray(C, np.float64)
    return np.abs(C - out64) <= rel * abs64 + absol
