"""GPU: the entry points captured in a HIP graph and replayed.

The library launches only kernels (no memset or copy nodes; K = 0 fills C
with a kernel), so a caller may capture its calls.  Each case captures one
call per dispatch path on a side stream, then replays the graph several
times with eager work and synchronizations between the replays: the output
is poisoned with NaN before every replay, and every replay must reproduce
the eager result bit for bit (same kernel, same inputs, fixed summation
order), which the oracle also checks once.
"""
import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU graph tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _case(M, N, K, seed):
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-3, 1.0)
    return A, AS, W, WS


def _replay_and_compare(g, out, eager, what):
    for r in range(REPLAYS):
        out.fill_(float("nan"))              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), \
            "%s: replay %d differs from the eager result" % (what, r)


# matvec (M = 1, a small batch, rows over 16 KiB), K-split GEMM, staged GEMM,
# 64 x 64-tile GEMM over all of K (one workgroup per unit, and two), the
# empty sum (K = 0)
SHAPES = [(1, 4096, 4096), (4, 2000, 4096), (1, 300, 16416), (64, 1024, 1024),
          (385, 14336, 512), (300, 2000, 1056), (256, 14336, 512), (3, 77, 0)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_qdot_graph_replay(dev, M, N, K):
    A, AS, W, WS = _case(M, N, K, 31 + M + N + K)
    tA, tAS, tW, tWS = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (A, AS, W, WS))
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    q8.q8_qdot(tA, tAS, tW, tWS, C)
    torch.cuda.synchronize()
    eager = C.cpu().numpy().copy()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    assert oracle.within_tolerance(eager, out, mag).all()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q8.q8_qdot(tA, tAS, tW, tWS, C, stream=s)
    torch.cuda.synchronize()
    _replay_and_compare(g, C, eager, "q8_qdot %dx%dx%d path %d" % (M, N, K, q8.q8_qdot_path(M, N, K)))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (40, 7000, 1056), (520, 2100, 1024)])
def test_q50_graph_replay(dev, M, N, K):
    # Q5_0 weights: the matvec, the K-split GEMM and the ring GEMM
    A, AS, _, WS = _case(M, N, K, 41 + M + N + K)
    W5 = synth.random_q50(N, K, 42 + M)
    tA, tAS, tW5, tWS = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (A, AS, W5, WS))
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    q8.q8_q50_qdot(tA, tAS, tW5, tWS, C)
    torch.cuda.synchronize()
    eager = C.cpu().numpy().copy()
    out, mag = oracle.q50_qdot_f64(A, AS, W5, WS)
    assert oracle.within_tolerance(eager, out, mag).all()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q8.q8_q50_qdot(tA, tAS, tW5, tWS, C, stream=s)
    torch.cuda.synchronize()
    _replay_and_compare(g, C, eager, "q8_q50_qdot %dx%dx%d path %d" % (M, N, K, q8.q8_q50_path(M, N, K)))


def test_partials_and_quantize_graph_replay(dev):
    M, N, K = 64, 300, 2048
    A, AS, W, WS = _case(M, N, K, 77)
    tA, tW = (torch.from_numpy(x).to(dev) for x in (A, W))
    P = torch.empty((M, N, K // 32), dtype=torch.int32, device=dev)
    X = torch.from_numpy(synth.random_f32((M, K), 78)).to(dev)
    Q = torch.empty((M, K), dtype=torch.int8, device=dev)
    D = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q8.q8_qdot_partials(tA, tW, P, stream=s)
            q8.q8_quantize(X, Q, D, stream=s)
    torch.cuda.synchronize()
    Pref = oracle.block_partials(A, W)
    Qref, Dref = oracle.quantize_rows(X.cpu().numpy())
    for r in range(REPLAYS):
        P.fill_(-1)
        Q.fill_(0)
        D.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(P.cpu().numpy(), Pref), "partials, replay %d" % r
        assert np.array_equal(Q.cpu().numpy(), Qref), "quantized bytes, replay %d" % r
        assert np.array_equal(D.cpu().numpy(), Dref), "scales, replay %d" % r
