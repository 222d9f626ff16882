"""How the contraction splits across GPUs, shown on one GPU.

Splitting along N (each GPU holds a slab of W's rows and WS's rows, A and AS
replicated) needs no exchange: every output column is computed from its own
weight row only.  Splitting along K on 32-block boundaries gives each GPU an
f32 partial of every output, which one all-reduce would sum; the int32 block
partials are those of the unsplit contraction, block for block.  Here every
shard is one call of the library on its slice, run one after the other on
cuda:0, and the pieces are put together on the host.

Bar: for one activation row or a small batch (M < 8, the decode kernels)
an output column's arithmetic does not depend on N, so the N-shards equal
the unsplit output bit for bit; for M >= 8 the dispatch may pick another
GEMM kernel for the slab, so each shard is held to the oracle's tolerance.
Block partials are bit-exact in every split.  The K-shards' f32 partial
outputs, summed in f64, are within the sum of the shards' bounds,
``1e-5 * sum_b |AS*WS*P| + S * 1e-6`` for S shards.
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
SHARDS = 8


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU shard tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _operands(M, N, K, seed, outliers=False):
    a32 = synth.activations_f32(M, K, seed, (seed + 1) if outliers else None)
    w32 = synth.weights_f32(N, K, seed + 2)
    A, AS = oracle.quantize_rows(a32)
    W, WS = oracle.quantize_rows(w32)
    return A, AS, W, WS


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (4, 2048, 4096), (64, 1024, 4096)])
def test_split_along_n(dev, M, N, K):
    _say("[shard] N split M=%d N=%d K=%d into %d" % (M, N, K, SHARDS))
    A, AS, W, WS = _operands(M, N, K, 700 + M)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C_full = q8.q8_qdot(tA, tAS, tW, tWS)
    P_full = q8.q8_qdot_partials(tA, tW)
    n = N // SHARDS
    C_parts, P_parts = [], []
    for s in range(SHARDS):
        # a slab of whole weight rows is contiguous: no copy
        Ws, WSs = tW[s * n:(s + 1) * n], tWS[s * n:(s + 1) * n]
        C_parts.append(q8.q8_qdot(tA, tAS, Ws, WSs))
        P_parts.append(q8.q8_qdot_partials(tA, Ws))
    torch.cuda.synchronize()
    C_full = C_full.cpu().numpy()
    C_cat = np.concatenate([c.cpu().numpy() for c in C_parts], axis=1)
    P_cat = np.concatenate([p.cpu().numpy() for p in P_parts], axis=1)
    assert np.array_equal(P_cat, P_full.cpu().numpy()), "N-shard partials differ from the unsplit ones"
    assert np.array_equal(P_cat, oracle.block_partials(A, W)), "N-shard partials differ from the oracle"
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    assert oracle.within_tolerance(C_cat, out, mag, REL, ABS).all(), "N-shard output out of tolerance"
    if M < 8:
        assert np.array_equal(C_cat.view(np.int32), C_full.view(np.int32)), \
            "decode-kernel N-shards differ from the unsplit output"


@pytest.mark.parametrize("M,N,K,outliers", [(1, 4096, 14336, True), (64, 512, 8192, False)])
def test_split_along_k(dev, M, N, K, outliers):
    _say("[shard] K split M=%d N=%d K=%d into %d" % (M, N, K, SHARDS))
    A, AS, W, WS = _operands(M, N, K, 800 + M, outliers)
    KB = K // 32
    kb = KB // SHARDS
    assert kb * SHARDS == KB
    C_sum = np.zeros((M, N), dtype=np.float64)
    P_parts = []
    for s in range(SHARDS):
        b0, b1 = s * kb, (s + 1) * kb
        # a K slice of row-major operands is strided: each GPU would hold
        # its own contiguous copy
        tA = _dev(A[:, 32 * b0:32 * b1], dev)
        tW = _dev(W[:, 32 * b0:32 * b1], dev)
        tAS = _dev(AS[:, b0:b1], dev)
        tWS = _dev(WS[:, b0:b1], dev)
        C = q8.q8_qdot(tA, tAS, tW, tWS)
        P = q8.q8_qdot_partials(tA, tW)
        torch.cuda.synchronize()
        C_sum += C.cpu().numpy().astype(np.float64)
        P_parts.append(P.cpu().numpy())
    P_cat = np.concatenate(P_parts, axis=2)
    assert np.array_equal(P_cat, oracle.block_partials(A, W)), "K-shard partials differ from the oracle"
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    err = np.abs(C_sum - out)
    bound = REL * mag + SHARDS * ABS
    assert (err <= bound).all(), "K-shard sum off by %.3g x its bound" % float((err / bound).max())
