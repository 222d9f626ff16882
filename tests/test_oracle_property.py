"""Property-based pins of the oracle (CPU): random tiny cases drawn by
hypothesis, checked against exact rational arithmetic and brute force.

- qdot_f64 / qmma_f64 against the qdot_t / qmma_t definition evaluated in
  exact rationals (oracle.brute), within the f64 rounding bound of a
  KB-term sum whose terms each round once ("Phobos Language Spec",
  "Quantized built-ins", Q8_0 table);
- block_partials against a NumPy int64 brute force over the full byte range
  (-128 included), and the |P| <= 32 * 128^2 bound;
- quantize_rows: |x - d q| <= d / 2 (plus f32 slack), the block maximum maps
  to +-127, signs kept, a zero block gives d = 0.
"""
import numpy as np
import pytest

import oracle
from oracle import brute

hyp = pytest.importorskip("hypothesis")
st = pytest.importorskip("hypothesis.strategies")
from hypothesis import given, settings, HealthCheck  # noqa: E402

SETTINGS = settings(max_examples=60, deadline=None, database=None,
                    suppress_health_check=[HealthCheck.too_slow])

f32_scale = st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, allow_infinity=False, width=32)


@st.composite
def contraction(draw, transposed=False):
    M = draw(st.integers(1, 3))
    N = draw(st.integers(1, 3))
    KB = draw(st.integers(1, 4))
    K = 32 * KB
    A = np.array(draw(st.lists(st.integers(-128, 127), min_size=M * K, max_size=M * K)), np.int8).reshape(M, K)
    W = np.array(draw(st.lists(st.integers(-128, 127), min_size=N * K, max_size=N * K)), np.int8).reshape(N, K)
    AS = np.array(draw(st.lists(f32_scale, min_size=M * KB, max_size=M * KB)), np.float32).reshape(M, KB)
    shape = (KB, N) if transposed else (N, KB)
    WS = np.array(draw(st.lists(f32_scale, min_size=N * KB, max_size=N * KB)), np.float32).reshape(shape)
    return A, AS, W, WS


@SETTINGS
@given(contraction())
def test_qdot_f64_matches_exact_rationals(case):
    A, AS, W, WS = case
    ex = brute.exact_definition(A, AS, W, WS)
    ex_abs = brute.exact_abs_terms(A, AS, W, WS)
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    KB = A.shape[1] // 32
    for i in range(A.shape[0]):
        for j in range(W.shape[0]):
            bound = 2.0 * KB * 2.0 ** -53 * float(ex_abs[i][j])
            assert abs(out[i, j] - float(ex[i][j])) <= bound
            assert abs(mag[i, j] - float(ex_abs[i][j])) <= bound


@SETTINGS
@given(contraction(transposed=True))
def test_qmma_f64_matches_exact_rationals(case):
    A, AS, W, WST = case
    ex = brute.exact_definition_qmma(A, AS, W, WST)
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    KB = A.shape[1] // 32
    for i in range(A.shape[0]):
        for j in range(W.shape[0]):
            bound = 2.0 * KB * 2.0 ** -53 * float(mag[i, j]) + 1e-300
            assert abs(out[i, j] - float(ex[i][j])) <= bound


@SETTINGS
@given(contraction())
def test_block_partials_brute_force(case):
    A, _, W, _ = case
    M, K = A.shape
    N = W.shape[0]
    P = oracle.block_partials(A, W)
    ref = np.einsum("ibk,jbk->ijb", A.astype(np.int64).reshape(M, K // 32, 32),
                    W.astype(np.int64).reshape(N, K // 32, 32))
    assert np.array_equal(P.astype(np.int64), ref)
    assert np.abs(ref).max() <= 32 * 128 * 128


@SETTINGS
@given(st.lists(st.floats(min_value=-1e4, max_value=1e4, allow_nan=False, width=32), min_size=32, max_size=32),
       st.booleans())
def test_quantizer_block_properties(vals, zero):
    x = np.zeros((1, 32), np.float32) if zero else np.array(vals, np.float32).reshape(1, 32)
    Q, D = oracle.quantize_rows(x)
    q = Q[0].astype(np.int64)
    d = float(D[0, 0])
    amax = float(np.abs(x).max())
    if amax == 0.0:
        assert d == 0.0 and (q == 0).all()
        return
    assert d == float(np.float32(np.float32(amax) / np.float32(127.0)))
    assert np.abs(q).max() == 127
    assert (np.abs(q) <= 127).all()
    nz = x[0] != 0
    assert (np.sign(q[nz & (q != 0)]) == np.sign(x[0][nz & (q != 0)])).all()
    err = np.abs(x[0].astype(np.float64) - d * q)
    assert (err <= d / 2 + 1e-6 * amax).all()
