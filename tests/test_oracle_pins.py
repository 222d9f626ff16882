"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties the oracle to something fixed independently: a hand-derived
worked example (tests/golden), exact rational arithmetic, closed forms of the
Q8_0 definition, integer invariants, or NumPy's own integer matmul.  The
definition pinned is the ``qdot_t`` row of the Q8_0 table ("Phobos Language
Spec", section "Quantized built-ins"), restated under "Quantized built-ins and
formats", section "Q8_0".
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_golden():
    g = _load_golden("qdot_worked_2x2x64.json")
    A = np.array(g["A"], np.int8)
    W = np.array(g["W"], np.int8)
    AS = np.array(g["AS"], np.float32)
    WS = np.array(g["WS"], np.float32)
    P = oracle.block_partials(A, W)
    assert P.tolist() == g["P"]
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    assert out.tolist() == g["out"]
    assert mag.tolist() == g["abs_terms"]
    # sampled entry point agrees on the same positions
    ii = np.array([0, 0, 1, 1])
    jj = np.array([0, 1, 0, 1])
    o2, m2 = oracle.qdot_f64_at(A, AS, W, WS, ii, jj)
    assert o2.tolist() == [v for row in g["out"] for v in row]
    assert m2.tolist() == [v for row in g["abs_terms"] for v in row]
    assert oracle.block_partials_at(A, W, ii, jj).tolist() == [p for row in g["P"] for p in row]


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 32, 1), (2, 3, 64, 2), (3, 2, 96, 3),
                                        (4, 4, 256, 4), (1, 4, 256, 5)])
def test_exact_rational_bruteforce(M, N, K, seed):
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 100)
    AS = synth.random_scales((M, K // 32), seed + 200, 1e-4, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 300, 1e-4, 10.0)
    ex_def = brute.exact_definition(A, AS, W, WS)
    ex_deq = brute.exact_dequantized(A, AS, W, WS)
    ex_abs = brute.exact_abs_terms(A, AS, W, WS)
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    KB = K // 32
    for i in range(M):
        for j in range(N):
            # the definition and the dequantized dot are the same rational
            assert ex_def[i][j] == ex_deq[i][j]
            # f64 oracle: each term s*p rounds once (s exact), KB-term sum
            bound = 2.0 * KB * 2.0 ** -53 * float(ex_abs[i][j])
            assert abs(out[i, j] - float(ex_def[i][j])) <= bound
            assert abs(mag[i, j] - float(ex_abs[i][j])) <= bound


@pytest.mark.parametrize("M,N,K,seed", [(2, 3, 64, 11), (3, 5, 128, 12), (1, 2, 96, 13)])
def test_qmma_exact_rational_bruteforce(M, N, K, seed):
    """qmma_t (weight scales [K/32, N]) against exact rationals; N != K/32 so a
    transposed index reads a different scale."""
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 100)
    AS = synth.random_scales((M, K // 32), seed + 200, 1e-4, 10.0)
    WST = synth.random_scales((K // 32, N), seed + 300, 1e-4, 10.0)
    ex = brute.exact_definition_qmma(A, AS, W, WST)
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    KB = K // 32
    for i in range(M):
        for j in range(N):
            bound = 2.0 * KB * 2.0 ** -53 * float(mag[i, j]) + 1e-300
            assert abs(out[i, j] - float(ex[i][j])) <= bound
    o2, m2 = oracle.qmma_f64_at(A, AS, W, WST, np.repeat(np.arange(M), N), np.tile(np.arange(N), M))
    assert np.array_equal(o2, out.ravel()) and np.array_equal(m2, mag.ravel())


def test_qmma_is_qdot_with_transposed_scales():
    """Storing the weight scales transposed changes nothing else: same terms in
    the same block order, so the f64 results agree bit for bit."""
    A = synth.random_i8((5, 320), 21)
    W = synth.random_i8((7, 320), 22)
    AS = synth.random_scales((5, 10), 23, 1e-3, 1.0)
    WS = synth.random_scales((7, 10), 24, 1e-3, 1.0)
    o1, m1 = oracle.qdot_f64(A, AS, W, WS)
    o2, m2 = oracle.qmma_f64(A, AS, W, np.ascontiguousarray(WS.T))
    assert np.array_equal(o1, o2) and np.array_equal(m1, m2)


def test_partials_match_numpy_int64_and_bound():
    M, N, K = 5, 7, 320
    A = synth.random_i8((M, K), 11)
    W = synth.random_i8((N, K), 12)
    P = oracle.block_partials(A, W)
    KB = K // 32
    ref = np.einsum("ibt,jbt->ijb", A.reshape(M, KB, 32).astype(np.int64),
                    W.reshape(N, KB, 32).astype(np.int64))
    assert P.dtype == np.int32
    assert np.array_equal(P.astype(np.int64), ref)
    assert np.abs(ref).max() <= 32 * 128 * 128


def test_partials_extreme_bytes():
    # -128 is a legal byte although the quantizer never emits it; the
    # largest block sum is 32 * (-128)^2 = 2^19 and must not wrap.
    K = 64
    A = np.full((1, K), -128, np.int8)
    W = np.full((2, K), -128, np.int8)
    W[1] = 127
    P = oracle.block_partials(A, W)
    assert P[0, 0].tolist() == [524288, 524288]
    assert P[0, 1].tolist() == [-128 * 127 * 32] * 2


def test_unit_scales_is_integer_matmul():
    M, N, K = 6, 5, 192
    A = synth.random_i8((M, K), 21)
    W = synth.random_i8((N, K), 22)
    ones_a = np.ones((M, K // 32), np.float32)
    ones_w = np.ones((N, K // 32), np.float32)
    out, mag = oracle.qdot_f64(A, ones_a, W, ones_w)
    ref = A.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(out, ref.astype(np.float64))


def test_all_ones_gives_K():
    for K in (32, 96, 4096):
        A = np.ones((2, K), np.int8)
        W = np.ones((3, K), np.int8)
        out, _ = oracle.qdot_f64(A, np.ones((2, K // 32), np.float32), W,
                                 np.ones((3, K // 32), np.float32))
        assert np.all(out == K)


def test_constant_scales_factor_out():
    M, N, K = 3, 4, 128
    A = synth.random_i8((M, K), 31)
    W = synth.random_i8((N, K), 32)
    ca, cw = np.float32(0.375), np.float32(-1.25)
    out, _ = oracle.qdot_f64(A, np.full((M, K // 32), ca, np.float32), W,
                             np.full((N, K // 32), cw, np.float32))
    ref = float(ca) * float(cw) * (A.astype(np.int64) @ W.astype(np.int64).T)
    assert np.array_equal(out, ref)


def test_one_hot_activation_selects_weight():
    # A[i] = e_k: out[i, j] = AS[i, k//32] * WS[j, k//32] * W[j, k]
    K, N = 256, 6
    ks = [0, 31, 32, 100, 255]
    A = np.zeros((len(ks), K), np.int8)
    for i, k in enumerate(ks):
        A[i, k] = 1
    W = synth.random_i8((N, K), 41)
    AS = synth.random_scales((len(ks), K // 32), 42)
    WS = synth.random_scales((N, K // 32), 43)
    out, _ = oracle.qdot_f64(A, AS, W, WS)
    for i, k in enumerate(ks):
        b = k // 32
        for j in range(N):
            assert out[i, j] == float(AS[i, b]) * float(WS[j, b]) * int(W[j, k])


def test_scales_index_by_block_not_transposed():
    # Distinct scale per block: a wrong block index or a transposed scale
    # array changes the result.  Only block 2 of row 0 is non-zero.
    K = 128
    A = np.zeros((2, K), np.int8)
    W = np.zeros((3, K), np.int8)
    A[0, 64:96] = 2
    W[1, 64:96] = 3
    AS = np.array([[1, 2, 4, 8], [16, 32, 64, 128]], np.float32)
    WS = np.array([[1, 3, 5, 7], [9, 11, 13, 15], [17, 19, 21, 23]], np.float32)
    out, _ = oracle.qdot_f64(A, AS, W, WS)
    expect = np.zeros((2, 3))
    expect[0, 1] = 4 * 13 * (32 * 6)
    assert np.array_equal(out, expect)


def test_single_block_K32():
    A = synth.random_i8((3, 32), 51)
    W = synth.random_i8((2, 32), 52)
    AS = synth.random_scales((3, 1), 53)
    WS = synth.random_scales((2, 1), 54)
    out, _ = oracle.qdot_f64(A, AS, W, WS)
    p = A.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(out, AS.astype(np.float64) * WS.astype(np.float64).T * p)


def test_zero_scale_block_contributes_nothing():
    K = 96
    A = synth.random_i8((2, K), 61)
    W = synth.random_i8((2, K), 62)
    AS = np.ones((2, 3), np.float32)
    WS = np.ones((2, 3), np.float32)
    WS[:, 1] = 0.0
    out, _ = oracle.qdot_f64(A, AS, W, WS)
    keep = np.r_[0:32, 64:96]
    ref = A[:, keep].astype(np.int64) @ W[:, keep].astype(np.int64).T
    assert np.array_equal(out, ref.astype(np.float64))


# ---------------------------------------------------------------- quantizer


def test_quantizer_golden_block():
    g = _load_golden("quantize_worked_block.json")
    x = np.array([g["x"]], np.float32)
    q, d = oracle.quantize_rows(x)
    assert d.tolist() == [[g["d"]]]
    assert q[0].tolist() == g["q"]
    z = np.array([g["zero_block"]["x"]], np.float32)
    qz, dz = oracle.quantize_rows(z)
    assert dz.tolist() == [[0.0]] and qz[0].tolist() == g["zero_block"]["q"]
    nb = g["nonpower_scale_block"]
    qn, dn = oracle.quantize_rows(np.array([nb["x"]], np.float32))
    assert dn.tolist() == [[nb["d"]]]
    assert qn[0].tolist() == nb["q"]


def test_quantizer_properties():
    x = synth.random_f32((16, 512), 71)
    x[3, 32:64] = 0.0                     # a zero block
    x[5, :32] *= np.float32(1e-3)         # a small block
    q, d = oracle.quantize_rows(x)
    KB = x.shape[1] // 32
    xb = x.reshape(16, KB, 32).astype(np.float64)
    qb = q.reshape(16, KB, 32).astype(np.int64)
    db = d.astype(np.float64)[..., None]
    amax = np.abs(xb).max(axis=2)
    # the scale is max|x|/127 rounded once to f32
    assert np.array_equal(d, (amax / 127.0).astype(np.float32))
    # reconstruction error at most half a step (plus f32 slack in x/d)
    err = np.abs(xb - db * qb)
    assert np.all(err <= db * (0.5 + 2.0 ** -16))
    # signs kept, never -128, never beyond 127
    assert np.all((qb == 0) | (np.sign(qb) == np.sign(xb)))
    assert q.min() >= -127 and q.max() <= 127
    # the block maximum maps to +-127
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, arg[..., None], axis=2)[..., 0]
    nz = amax > 0
    assert np.all(np.abs(top[nz]) == 127)
    # zero block
    assert d[3, 1] == 0.0 and np.all(q[3, 32:64] == 0)


def test_quantizer_power_of_two_invariance():
    x = synth.random_f32((4, 256), 81)
    q1, d1 = oracle.quantize_rows(x)
    for e in (-20, -3, 5, 30):
        s = np.float32(2.0 ** e)
        q2, d2 = oracle.quantize_rows(x * s)
        assert np.array_equal(q1, q2)
        assert np.array_equal(d2, d1 * s)


def test_quantize_then_contract_approximates_float_dot():
    # End-to-end sanity of the format: the Q8_0 contraction of quantized
    # rows approximates the f64 dot product of the original rows within the
    # quantization error bound sum_k (|a| ea + |w| ew + ea ew).
    K = 1024
    a = synth.random_f32((2, K), 91)
    w = synth.random_f32((3, K), 92, 0.02)
    qa, da = oracle.quantize_rows(a)
    qw, dw = oracle.quantize_rows(w)
    out, _ = oracle.qdot_f64(qa, da, qw, dw)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    ea = np.repeat(da.astype(np.float64), 32, axis=1) * 0.5 * (1 + 2 ** -16)
    ew = np.repeat(dw.astype(np.float64), 32, axis=1) * 0.5 * (1 + 2 ** -16)
    bound = (np.abs(a) @ ew.T + ea @ np.abs(w).T + ea @ ew.T)
    assert np.all(np.abs(out - ref) <= bound)


def test_tolerance_helper():
    out = np.array([1.0, -2.0])
    mag = np.array([1.0, 3.0])
    assert oracle.within_tolerance(np.array([1.0 + 5e-6, -2.0]), out, mag).all()
    assert not oracle.within_tolerance(np.array([1.0 + 3e-5, -2.0]), out, mag).all()


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.zeros((1, 33), np.float32))
    with pytest.raises(ValueError):
        oracle.block_partials(np.zeros((1, 32), np.int8), np.zeros((1, 64), np.int8))
    with pytest.raises(ValueError):
        oracle.qdot_f64(np.zeros((1, 32), np.int8), np.zeros((1, 2), np.float32),
                        np.zeros((1, 32), np.int8), np.zeros((1, 1), np.float32))


# ------------------------------------------------------------------ Q5_0

def _q50_golden():
    g = json.load(open(os.path.join(GOLDEN, "q50_worked_blocks.json")))
    W5 = np.frombuffer(bytes.fromhex("".join(g["blocks_hex"])), np.uint8)[None, :].copy()
    A = np.array(g["A"], np.int8)
    return g, A, W5


def test_q50_golden_worked_blocks():
    g, A, W5 = _q50_golden()
    K = g["K"]
    assert oracle.q50_decode(W5, K)[0].tolist() == g["values"]
    P = oracle.q50_block_partials(A, W5)
    assert P[:, 0, :].tolist() == g["P"]
    ones_a = np.ones((A.shape[0], K // 32), np.float32)
    ones_w = np.ones((1, K // 32), np.float32)
    out, mag = oracle.q50_qdot_f64(A, ones_a, W5, ones_w)
    assert out[:, 0].tolist() == g["out_unit_scales"]
    out_t, _ = oracle.q50_qmma_f64(A, ones_a, W5, ones_w.T.copy())
    assert out_t[:, 0].tolist() == g["out_unit_scales"]


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 32, 31), (2, 3, 64, 32), (3, 2, 96, 33)])
def test_q50_exact_rational_bruteforce(M, N, K, seed):
    A = synth.random_i8((M, K), seed)
    W5 = synth.random_q50(N, K, seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-3, 10.0)
    KB = K // 32
    for ws_t in (False, True):
        W_scales = np.ascontiguousarray(WS.T) if ws_t else WS
        ex = brute.exact_definition_q50(A, AS, W5, W_scales, ws_t)
        out, mag = (oracle.q50_qmma_f64 if ws_t else oracle.q50_qdot_f64)(A, AS, W5, W_scales)
        # the sampled form, at every position listed twice in a scrambled order
        ii = np.tile(np.repeat(np.arange(M), N), 2)[::-1].copy()
        jj = np.tile(np.tile(np.arange(N), M), 2)[::-1].copy()
        o_at, m_at = oracle.q50_f64_at(A, AS, W5, W_scales, ws_t, ii, jj)
        for i in range(M):
            for j in range(N):
                bound = 2.0 * KB * 2.0 ** -53 * float(mag[i, j]) + 1e-300
                assert abs(out[i, j] - float(ex[i][j])) <= bound
        for s in range(ii.shape[0]):
            i, j = int(ii[s]), int(jj[s])
            bound = 2.0 * KB * 2.0 ** -53 * float(mag[i, j]) + 1e-300
            assert abs(o_at[s] - float(ex[i][j])) <= bound
            assert m_at[s] == mag[i, j]
    # the pure-Python decoder and the oracle's agree value for value
    Wd = oracle.q50_decode(W5, K)
    for j in range(N):
        assert Wd[j].tolist() == brute.q50_values_py(W5[j], K)


def test_q50_decode_properties():
    K = 256
    W5 = synth.random_q50(40, K, 77)
    Wd = oracle.q50_decode(W5, K).astype(np.int32)
    assert Wd.min() >= -16 and Wd.max() <= 15
    # uniform bytes give every code
    assert set(np.unique(Wd).tolist()) == set(range(-16, 16))
    # flipping bit e of a block's qh word moves exactly element e by 16
    for e in (0, 5, 15, 16, 30, 31):
        W5b = W5.copy()
        qh_byte = 20 * 3 + e // 8          # block 3 of every row
        W5b[:, qh_byte] ^= np.uint8(1 << (e % 8))
        Wb = oracle.q50_decode(W5b, K).astype(np.int32)
        diff = Wb - Wd
        assert (np.abs(diff[:, 96 + e]) == 16).all()
        diff[:, 96 + e] = 0
        assert not diff.any()
    # the nibbles of byte e feed elements e and e + 16 only
    W5c = W5.copy()
    W5c[:, 20 * 2 + 4 + 7] ^= np.uint8(0x21)   # block 2, byte 7: low bit 0, high bit 1
    Wc = oracle.q50_decode(W5c, K).astype(np.int32)
    d = Wc - Wd
    assert (np.abs(d[:, 64 + 7]) == 1).all() and (np.abs(d[:, 64 + 23]) == 2).all()
    d[:, 64 + 7] = 0
    d[:, 64 + 23] = 0
    assert not d.any()


def test_q50_partials_equal_q8_partials_of_decoded_values():
    A = synth.random_i8((3, 320), 81)
    W5 = synth.random_q50(5, 320, 82)
    P5 = oracle.q50_block_partials(A, W5)
    P8 = oracle.block_partials(A, oracle.q50_decode(W5, 320))
    assert np.array_equal(P5, P8)
    assert np.abs(P5).max() <= 32 * 128 * 16


def test_cancelling_blocks_discriminate_half_block_scaling():
    # The GPU parity test built on synth.cancelling_blocks is only worth
    # something if the tolerance rejects arithmetic that scales half-block
    # sums before the exact block sum is formed.  Check that here, on the
    # host: the construction holds, an f32 accumulation of the exact block
    # sums passes the bar everywhere, and the same accumulation fed the two
    # half-block sums separately fails it on most outputs.
    M, N, K = 3, 200, 2048
    A, AS, W, WS = synth.cancelling_blocks(M, N, K, 17)
    KB = K // 32
    Ab = A.reshape(M, KB, 32).astype(np.int64)
    Wb = W.reshape(N, KB, 32).astype(np.int64)
    lo = np.einsum("mbt,nbt->mnb", Ab[:, :, :16], Wb[:, :, :16])
    hi = np.einsum("mbt,nbt->mnb", Ab[:, :, 16:], Wb[:, :, 16:])
    P = oracle.block_partials(A, W)
    assert np.array_equal(P, lo + hi)
    assert np.abs(P).max() <= 127 and np.abs(lo).min() >= 60000
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    s = AS[:, None, :] * WS[None, :, :]                 # f32 products
    exact = np.zeros((M, N), np.float32)
    halves = np.zeros((M, N), np.float32)
    for b in range(KB):
        exact = exact + s[:, :, b] * P[:, :, b].astype(np.float32)
        halves = halves + s[:, :, b] * lo[:, :, b].astype(np.float32)
        halves = halves + s[:, :, b] * hi[:, :, b].astype(np.float32)
    assert exact.dtype == np.float32 and halves.dtype == np.float32
    assert oracle.within_tolerance(exact, out, mag).all()
    assert oracle.within_tolerance(halves, out, mag).mean() < 0.7
