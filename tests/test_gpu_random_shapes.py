"""GPU: seeded random shapes through every entry point, against the oracle.

The shapes are drawn once from a fixed seed so that each dispatch regime is
reached several times with sizes nobody picked by hand: one activation row,
small batches (2..7 rows), the K-split GEMM (few output tiles), the
LDS-staged GEMM (M >= 128 and many tiles, short K) and the 64 x 64-tile GEMM
over all of K (medium M x N, short K; and, two workgroups per compute unit,
shapes the staged GEMM would take but is slower on, and shapes past one
round of its tiles, Q5_0 weights included); N and K/32 are
ragged (any value; one activation row up to 600 blocks, past the 16 KiB
rows of the one-row kernels).  Each case runs q8_qdot, q8_qmma (the same
scales transposed), q8_q50_qdot and q8_q50_qmma (Q5_0 weights) and both
partials entries.  Bar: int32 partials bit-exact; f32 outputs within
``1e-5 * sum_b |AS*WS*P| + 1e-6`` of the oracle.  Sizes keep the oracle to
about a second per case.
"""
import sys

import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6
MAX_MNK = 60_000_000      # multiply-adds per case (staged-GEMM cases excepted)


def _draw_cases(per_regime=6, seed=20261202):
    """(M, N, K) triples, `per_regime` for each dispatch regime."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(per_regime):       # one activation row, rows up to 600 blocks
        K = 32 * int(rng.integers(1, 601))
        cases.append((1, int(rng.integers(1, max(2, min(5000, MAX_MNK // K)) + 1)), K))
    for _ in range(per_regime):       # small batches
        M, K = int(rng.integers(2, 8)), 32 * int(rng.integers(1, 513))
        cases.append((M, int(rng.integers(1, max(2, min(5000, MAX_MNK // (M * K))) + 1)), K))
    for _ in range(per_regime):       # few output tiles: the K-split GEMM
        M, K = int(rng.integers(8, 601)), 32 * int(rng.integers(1, 513))
        cases.append((M, int(rng.integers(1, max(2, min(600, MAX_MNK // (M * K))) + 1)), K))
    for _ in range(per_regime):       # many tiles: the LDS-staged GEMM, short K
        # (one round of 128 x 224 tiles, and more than 4.1 tiles of 64 x 64
        # per compute unit, so the staged GEMM is the faster)
        M = int(rng.integers(128, 601))
        n_lo = max(224 * (-(-128 // -(-M // 128))), 64 * (-(-1050 // -(-M // 64))))
        n_hi = 224 * (256 // -(-M // 128))
        cases.append((M, int(rng.integers(n_lo, n_hi + 1)), 32 * int(rng.integers(1, 9))))
    for _ in range(per_regime):       # 520..1000 tiles of 32 x 32 (three or four
        # rounds on 256 compute units), one round of 64 x 64 tiles, too few
        # 128 x 224 tiles: the 64 x 64-tile GEMM over all of K, short K
        M = int(rng.integers(64, 601))
        mt = -(-M // 32)
        nt = int(rng.integers(-(-520 // mt), 1000 // mt + 1))
        N = 32 * nt - int(rng.integers(0, 32))
        cases.append((M, N, 32 * int(rng.integers(1, 9))))
    for _ in range(per_regime):       # shapes the staged GEMM would take with at
        # most 4.1 tiles of 64 x 64 per compute unit: the 64 x 64-tile GEMM,
        # two workgroups per unit, short K
        M = int(rng.integers(128, 601))
        n_lo = 224 * (-(-128 // -(-M // 128)))
        n_hi = min(224 * (256 // -(-M // 128)), 64 * (1049 // -(-M // 64)))
        cases.append((M, int(rng.integers(n_lo, n_hi + 1)), 32 * int(rng.integers(1, 9))))
    for _ in range(per_regime):       # 257..600 tiles of 64 x 64, too few staged
        # tiles: the 64 x 64-tile GEMM, two workgroups per unit (Q5_0 weights
        # too: K/32 a multiple of 4)
        M = int(rng.integers(64, 601))
        mt = -(-M // 64)
        nt = int(rng.integers(-(-257 // mt), 600 // mt + 1))
        N = 64 * nt - int(rng.integers(0, 64))
        cases.append((M, N, 128))
    return cases


CASES = _draw_cases()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _close(C, out, mag, what):
    ok = oracle.within_tolerance(C, out, mag, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        raise AssertionError("%s: %d/%d outside tolerance; first bad %s C=%r oracle=%r"
                             % (what, len(bad), ok.size, bad[:5].tolist(),
                                C[tuple(bad[0])], out[tuple(bad[0])]))


def _equal(Pg, Pref, what):
    if not np.array_equal(Pg, Pref):
        bad = np.argwhere(Pg != Pref)
        raise AssertionError("%s: %d partials differ; first %s gpu=%r oracle=%r"
                             % (what, len(bad), bad[:3].tolist(), Pg[tuple(bad[0])], Pref[tuple(bad[0])]))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shape_all_entries(dev, case):
    M, N, K = CASES[case]
    path = q8.q8_qdot_path(M, N, K)
    print("[random] case %d M=%d N=%d K=%d path=%d" % (case, M, N, K, path), flush=True)
    sys.stdout.flush()
    seed = 7000 + 11 * case
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    W5 = synth.random_q50(N, K, seed + 2)
    AS = synth.random_scales((M, K // 32), seed + 3, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), seed + 4, 1e-3, 1.0)
    WST = np.ascontiguousarray(WS.T)
    tA, tAS, tW, tW5 = _dev(A, dev), _dev(AS, dev), _dev(W, dev), _dev(W5, dev)
    tWS, tWST = _dev(WS, dev), _dev(WST, dev)

    C1 = q8.q8_qdot(tA, tAS, tW, tWS)
    C2 = q8.q8_qmma(tA, tAS, tW, tWST)
    C3 = q8.q8_q50_qdot(tA, tAS, tW5, tWS)
    C4 = q8.q8_q50_qmma(tA, tAS, tW5, tWST)
    P1 = q8.q8_qdot_partials(tA, tW)
    P2 = q8.q8_q50_partials(tA, tW5)
    torch.cuda.synchronize()

    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _close(C1.cpu().numpy(), out, mag, "q8_qdot")
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _close(C2.cpu().numpy(), out, mag, "q8_qmma")
    out, mag = oracle.q50_qdot_f64(A, AS, W5, WS)
    _close(C3.cpu().numpy(), out, mag, "q8_q50_qdot")
    out, mag = oracle.q50_qmma_f64(A, AS, W5, WST)
    _close(C4.cpu().numpy(), out, mag, "q8_q50_qmma")
    _equal(P1.cpu().numpy(), oracle.block_partials(A, W), "q8_qdot_partials")
    _equal(P2.cpu().numpy(), oracle.q50_block_partials(A, W5), "q8_q50_partials")


def test_cases_reach_every_path():
    # each regime of the draw lands on its dispatch path (0 matvec,
    # 1 K-split GEMM, 2 LDS-staged GEMM, 3 64 x 64-tile GEMM over all of K)
    paths = [q8.q8_qdot_path(M, N, K) for M, N, K in CASES]
    per = len(CASES) // 7
    assert paths[:2 * per] == [0] * (2 * per)
    assert paths[2 * per:3 * per] == [1] * per
    assert paths[3 * per:4 * per] == [2] * per, CASES[3 * per:4 * per]
    assert paths[4 * per:] == [3] * (3 * per), CASES[4 * per:]
    assert [q8.q8_q50_path(M, N, K) for M, N, K in CASES[6 * per:]] == [3] * per, CASES[6 * per:]
