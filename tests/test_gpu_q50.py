"""GPU parity of the Q5_0-weight entries (q8_q50_qdot, q8_q50_qmma,
q8_q50_partials) against the oracle's q50 definitions, element by element.

Bar: int32 partials bit-exact; f32 within ``1e-5 * sum_b |AS*WS*P| + 1e-6``.
Weights are seeded uniform bytes (every byte pattern is a valid Q5_0
block), so all 32 codes and all qh bit patterns occur.  Shapes reach the
matvec (M < 8, K <= 16384: one activation row, a batch staged in LDS, or a
batch too large for LDS taken a row at a time), the 64 x 64-tile ring GEMM
(shapes whose Q8_0 GEMM is the staged or the ring one and whose 64 x 64
tiles outnumber the compute units, with K/32 a multiple of 4 and an aligned
weight array) and the K-split GEMM (everything else),
blocks per row not a multiple of 4 (rows that start 4- but not 16-byte
aligned), ragged M and N, and a weight array that starts 4 bytes past a
16-byte boundary.
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


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _case(M, N, K, seed):
    A = synth.random_i8((M, K), seed)
    W5 = synth.random_q50(N, K, seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-3, 1.0)
    return A, AS, W5, WS


def _check(A, AS, W5, WS, dev, what, misalign=False):
    M, K = A.shape
    N = W5.shape[0]
    print("[q50] %s M=%d N=%d K=%d misalign=%d" % (what, M, N, K, misalign), flush=True)
    sys.stdout.flush()
    tA, tAS = _dev(A, dev), _dev(AS, dev)
    if misalign:
        big = torch.empty(W5.size + 4, dtype=torch.uint8, device=dev)
        big[4:] = torch.from_numpy(W5.ravel()).to(dev)
        tW5 = big[4:].view(W5.shape)
        assert tW5.data_ptr() % 16 == 4
    else:
        tW5 = _dev(W5, dev)
    WST = np.ascontiguousarray(WS.T)
    C1 = q8.q8_q50_qdot(tA, tAS, tW5, _dev(WS, dev))
    C2 = q8.q8_q50_qmma(tA, tAS, tW5, _dev(WST, dev))
    P = q8.q8_q50_partials(tA, tW5)
    torch.cuda.synchronize()
    Pref = oracle.q50_block_partials(A, W5)
    Pg = P.cpu().numpy()
    if not np.array_equal(Pg, Pref):
        bad = np.argwhere(Pg != Pref)
        raise AssertionError("%s: %d partials differ; first %s gpu=%r oracle=%r"
                             % (what, len(bad), bad[:3].tolist(), Pg[tuple(bad[0])], Pref[tuple(bad[0])]))
    for name, C, ws_t in (("q50_qdot", C1, False), ("q50_qmma", C2, True)):
        out, mag = oracle.q50_qmma_f64(A, AS, W5, WST) if ws_t else oracle.q50_qdot_f64(A, AS, W5, WS)
        ok = oracle.within_tolerance(C.cpu().numpy(), out, mag, REL, ABS)
        if not ok.all():
            bad = np.argwhere(~ok)
            raise AssertionError("%s %s: %d/%d outside tolerance, first %s"
                                 % (what, name, len(bad), ok.size, bad[:5].tolist()))


SHAPES = [
    (1, 14336, 4096), (1, 4096, 14336), (1, 37, 96), (3, 129, 2080), (7, 300, 1024),  # matvec
    (1, 9, 16416), (2, 100, 16416),                                                     # K-split, long K
    (8, 37, 96), (64, 4096, 4096), (127, 300, 4160), (512, 1024, 4096), (33, 65, 160),  # K-split
    # small batches read the weights once for all rows when the rows fit in
    # LDS: four rows to a weight group (K <= 2048), one row of 65..96 blocks
    # (blocks past K/32 in some lanes), 96..448 blocks, the largest rows at
    # M = 2 and 3; larger batches of long rows fall back to one grid row per
    # activation row
    (7, 4096, 2048), (2, 1, 32), (4, 14336, 4096), (5, 333, 2080), (2, 3000, 6144),
    (5, 1000, 8192), (3, 500, 14336), (2, 65, 16384), (6, 777, 14336), (7, 129, 16384),
    # one row: rows of 4 to 288 blocks, one to several rows per wave group,
    # a single weight row
    (1, 1000, 128), (1, 333, 1536), (1, 777, 1664), (1, 5000, 3200), (1, 4096, 6272),
    (1, 3000, 9216), (1, 1, 4096),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_q50_shapes(dev, M, N, K):
    A, AS, W5, WS = _case(M, N, K, 5000 + M + N + K)
    _check(A, AS, W5, WS, dev, "shape")


# The ring GEMM (two workgroups per compute unit): shapes whose Q8_0
# dispatch is the ring GEMM (520 x 2100, 512 x 4096, 600 x 2000, 129 x 14336)
# and the staged one (385 x 14336); ragged M and N, one to 36 stages.
RING = [(520, 2100, 1024), (512, 4096, 512), (600, 2000, 1152), (129, 14336, 128),
        (385, 14336, 128), (520, 2100, 128)]


@pytest.mark.parametrize("M,N,K", RING)
def test_q50_ring_gemm_shapes(dev, M, N, K):
    assert q8.q8_q50_path(M, N, K) == 3
    A, AS, W5, WS = _case(M, N, K, 5500 + M + N + K)
    _check(A, AS, W5, WS, dev, "ring")


def test_q50_ring_fallbacks(dev):
    # shapes the ring GEMM would take, run on the K-split GEMM: K/32 not a
    # multiple of 4, and a weight array only 4-byte aligned
    assert q8.q8_q50_path(520, 2100, 1056) == 1
    A, AS, W5, WS = _case(520, 2100, 1056, 5600)
    _check(A, AS, W5, WS, dev, "ring shape, K/32 = 33")
    assert q8.q8_q50_path(520, 2100, 1024) == 3
    A, AS, W5, WS = _case(520, 2100, 1024, 5601)
    _check(A, AS, W5, WS, dev, "ring shape, misaligned", misalign=True)


@pytest.mark.parametrize("M,N,K", [(1, 200, 4096), (16, 200, 1056)])
def test_q50_misaligned_weights(dev, M, N, K):
    A, AS, W5, WS = _case(M, N, K, 6100 + M)
    _check(A, AS, W5, WS, dev, "misaligned", misalign=True)


def test_q50_extreme_codes(dev):
    # all-zero blocks (every value -16) and all-ones blocks (every value 15)
    # against -128 / 127 activations: the largest block sums
    M, N, K = 9, 64, 256
    A = np.where(np.arange(K)[None, :] % 2 == 0, -128, 127).astype(np.int8).repeat(M, 0)
    W5 = np.zeros((N, K // 32 * 20), np.uint8)
    W5[N // 2:] = 0xFF
    AS = np.full((M, K // 32), 0.5, np.float32)
    WS = np.full((N, K // 32), 0.25, np.float32)
    _check(A, AS, W5, WS, dev, "extreme")
    _check(A[:1], AS[:1], W5, WS, dev, "extreme-matvec")
    # weight scales of 2^110 / 2^126 against activation scales of their
    # inverse: the GEMM's fast epilogue overflows and the tile is recomputed
    # in the plain order
    for b, e in ((1, 110), (5, 126)):
        WS[5:30, b] = np.float32(2.0 ** e)
        AS[:, b] = np.float32(2.0 ** -e)
    _check(A, AS, W5, WS, dev, "huge weight scales")
    _check(A[:1], AS[:1], W5, WS, dev, "huge weight scales (matvec)")


def test_q50_ring_extreme_codes(dev):
    # the same extremes on the ring GEMM (M = 520, N = 2100, K = 256), whose
    # non-finite fallback decodes the weight blocks straight from memory
    M, N, K = 520, 2100, 256
    assert q8.q8_q50_path(M, N, K) == 3
    A = np.where(np.arange(K)[None, :] % 2 == 0, -128, 127).astype(np.int8).repeat(M, 0)
    W5 = synth.random_q50(N, K, 5700)
    W5[:64] = 0
    W5[64:128] = 0xFF
    AS = np.full((M, K // 32), 0.5, np.float32)
    WS = np.full((N, K // 32), 0.25, np.float32)
    _check(A, AS, W5, WS, dev, "ring extreme")
    for b, e in ((1, 110), (5, 126)):
        WS[5:30, b] = np.float32(2.0 ** e)
        AS[:, b] = np.float32(2.0 ** -e)
    _check(A, AS, W5, WS, dev, "ring huge weight scales")
