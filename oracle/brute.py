"""Exact-rational brute force for tiny shapes -- TEST INFRASTRUCTURE ONLY.

Two formulations of the Q8_0 contraction in exact rational arithmetic
(``fractions.Fraction`` of the f32 scales, which are dyadic rationals):

* ``exact_definition``: the ``qdot_t`` row of the Q8_0 table ("Phobos Language
  Spec", section "Quantized built-ins"): scale-product times integer block sum.
* ``exact_dequantized``: the dot product of the dequantized rows,
  ``sum_k (AS[i, b(k)] * A[i, k]) * (WS[j, b(k)] * W[j, k])`` -- the plain-tile
  formulation the "Quantized built-ins and formats" page mentions under Q8_0
  (bytes converted to float, scale applied per block).

* ``exact_definition_qmma``: the ``qmma_t`` row of the same table, whose
  weight scales are stored transposed, ``w_scales[b][j]`` (``[K/32, N]``).

By distributivity the first two are equal as rationals; the tests assert that, and
that the f64 oracle lies within its rounding bound of them.  Pure Python
loops: only for tiny M, N, K.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

BLOCK = 32


def exact_definition(A, AS, W, WS):
    """``[[Fraction]]``: sum_b AS[i,b]*WS[j,b]*sum_{k in b} A[i,k]*W[j,k]."""
    A = np.asarray(A)
    W = np.asarray(W)
    M, K = A.shape
    N = W.shape[0]
    KB = K // BLOCK
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            total = Fraction(0)
            for b in range(KB):
                p = 0
                for t in range(BLOCK):
                    k = b * BLOCK + t
                    p += int(A[i, k]) * int(W[j, k])
                total += Fraction(float(AS[i, b])) * Fraction(float(WS[j, b])) * p
            row.append(total)
        out.append(row)
    return out


def exact_dequantized(A, AS, W, WS):
    """``[[Fraction]]``: sum_k (AS[i,k//32]*A[i,k]) * (WS[j,k//32]*W[j,k])."""
    A = np.asarray(A)
    W = np.asarray(W)
    M, K = A.shape
    N = W.shape[0]
    out = []
    for i in range(M):
        a_deq = [Fraction(float(AS[i, k // BLOCK])) * int(A[i, k]) for k in range(K)]
        row = []
        for j in range(N):
            total = Fraction(0)
            for k in range(K):
                total += a_deq[k] * (Fraction(float(WS[j, k // BLOCK])) * int(W[j, k]))
            row.append(total)
        out.append(row)
    return out


def exact_abs_terms(A, AS, W, WS):
    """``[[Fraction]]``: sum_b |AS[i,b]*WS[j,b]*P[i,j,b]| in exact arithmetic."""
    A = np.asarray(A)
    W = np.asarray(W)
    M, K = A.shape
    N = W.shape[0]
    KB = K // BLOCK
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            total = Fraction(0)
            for b in range(KB):
                p = sum(int(A[i, b * BLOCK + t]) * int(W[j, b * BLOCK + t]) for t in range(BLOCK))
                total += abs(Fraction(float(AS[i, b])) * Fraction(float(WS[j, b])) * p)
            row.append(total)
        out.append(row)
    return out


def exact_definition_qmma(A, AS, W, WST):
    """``[[Fraction]]``: sum_b AS[i,b]*WST[b,j]*sum_{k in b} A[i,k]*W[j,k] (``WST [K/32, N]``)."""
    A = np.asarray(A)
    W = np.asarray(W)
    M, K = A.shape
    N = W.shape[0]
    KB = K // BLOCK
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            total = Fraction(0)
            for b in range(KB):
                p = sum(int(A[i, b * BLOCK + t]) * int(W[j, b * BLOCK + t]) for t in range(BLOCK))
                total += Fraction(float(AS[i, b])) * Fraction(float(WST[b, j])) * p
            row.append(total)
        out.append(row)
    return out


def q50_values_py(W5_row, K):
    """Pure-Python Q5_0 decode of one weight row (``K/32 * 20`` bytes) into ``K`` ints.

    Written from the q50 rows of the Q8_0 table ("Phobos Language Spec",
    "Quantized built-ins"): per 32 values the qh word (little-endian, bit e =
    bit 4 of element e), then 16 bytes, byte e = element e (low nibble) and
    element e + 16 (high nibble); value = q - 16.
    """
    vals = []
    for b in range(K // BLOCK):
        blk = [int(x) for x in W5_row[b * 20:(b + 1) * 20]]
        qh = blk[0] | (blk[1] << 8) | (blk[2] << 16) | (blk[3] << 24)
        for e in range(BLOCK):
            byte = blk[4 + (e % 16)]
            nib = (byte & 15) if e < 16 else (byte >> 4)
            vals.append((nib | (((qh >> e) & 1) << 4)) - 16)
    return vals


def exact_definition_q50(A, AS, W5, WS, ws_t=False):
    """``[[Fraction]]``: the q50 contraction; ``WS`` is ``[N, K/32]`` or, with ``ws_t``, ``[K/32, N]``."""
    A = np.asarray(A)
    W5 = np.asarray(W5)
    M, K = A.shape
    N = W5.shape[0]
    KB = K // BLOCK
    wv = [q50_values_py(W5[j], K) for j in range(N)]
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            total = Fraction(0)
            for b in range(KB):
                p = sum(int(A[i, b * BLOCK + t]) * wv[j][b * BLOCK + t] for t in range(BLOCK))
                ws = WS[b, j] if ws_t else WS[j, b]
                total += Fraction(float(AS[i, b])) * Fraction(float(ws)) * p
            row.append(total)
        out.append(row)
    return out
