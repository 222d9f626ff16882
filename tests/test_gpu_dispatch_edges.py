"""GPU: shapes on both sides of every GEMM dispatch boundary, against the oracle.

The M >= 8 dispatch turns on counts of tiles: more 64 x 64 tiles than
compute units switches the ring GEMM to its two-workgroups-per-unit form;
128 staged tiles of 128 x 224 admit the staged GEMM, which gives way to the
ring GEMM at up to 4.1 of its tiles per unit per staged round; Q5_0 weights
take the ring GEMM only past one round of its tiles.  Each shape here sits
one tile either side of such a line (on a 256-compute-unit MI355X), with a
short K (one partial stage where K/32 = 3) so the oracle stays quick; every
Q8_0 entry and the Q5_0 entry are checked (f32 within tolerance, int32
partials bit-exact), and the kernel each reaches is asserted.
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

# (M, N, K, Q8_0 path, Q5_0 path)
EDGES = [
    (64, 16384, 128, 3, 1),     # 256 ring tiles: one workgroup per unit
    (64, 16448, 128, 3, 3),     # 257: two per unit
    (64, 16448, 96, 3, 1),      # the same, K/32 = 3 (a partial stage; Q5_0 on the K-split GEMM)
    (256, 14336, 128, 3, 3),    # 128 staged tiles, 896 ring tiles: the ring GEMM
    (127, 28672, 128, 3, 3),    # M below the staged GEMM's 128 rows
    (384, 11136, 128, 3, 3),    # 150 staged tiles, 1044 ring tiles (<= 4.1 per unit)
    (384, 11200, 128, 2, 3),    # 150 staged tiles, 1050 ring tiles: the staged GEMM
    (640, 14336, 128, 2, 3),    # two staged rounds, 2240 ring tiles: the staged GEMM
    (512, 16000, 128, 3, 3),    # two staged rounds (288), 2000 ring tiles: the ring GEMM
]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU dispatch tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _close(C, out, mag, what):
    ok = oracle.within_tolerance(C, out, mag, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        raise AssertionError("%s: %d/%d outside tolerance, first %s" % (what, len(bad), ok.size, bad[:4].tolist()))


@pytest.mark.parametrize("M,N,K,p8,p5", EDGES)
def test_dispatch_edges(dev, M, N, K, p8, p5):
    print("[edges] M=%d N=%d K=%d paths %d/%d" % (M, N, K, p8, p5), flush=True)
    sys.stdout.flush()
    assert q8.q8_qdot_path(M, N, K) == p8
    assert q8.q8_q50_path(M, N, K) == p5
    seed = M * 3 + N + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-3, 1.0)
    W5 = synth.random_q50(N, K, seed + 4)
    WST = np.ascontiguousarray(WS.T)
    tA, tAS, tW, tWS, tW5, tWST = (_dev(x, dev) for x in (A, AS, W, WS, W5, WST))
    C1 = q8.q8_qdot(tA, tAS, tW, tWS)
    C2 = q8.q8_qmma(tA, tAS, tW, tWST)
    P = q8.q8_qdot_partials(tA, tW)
    C5 = q8.q8_q50_qdot(tA, tAS, tW5, tWS)
    P5 = q8.q8_q50_partials(tA, tW5)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _close(C1.cpu().numpy(), out, mag, "q8_qdot")
    _close(C2.cpu().numpy(), out, mag, "q8_qmma")
    assert np.array_equal(P.cpu().numpy(), oracle.block_partials(A, W)), "q8_qdot_partials"
    out5, mag5 = oracle.q50_qdot_f64(A, AS, W5, WS)
    _close(C5.cpu().numpy(), out5, mag5, "q8_q50_qdot")
    assert np.array_equal(P5.cpu().numpy(), oracle.q50_block_partials(A, W5)), "q8_q50_partials"
