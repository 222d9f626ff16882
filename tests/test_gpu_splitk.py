"""GPU parity of the workspace entries (q8_qdot_ws, q8_qmma_ws,
q8_qdot_ws_partials): the split-K GEMM against the oracle.

Bar: int32 partials bit-exact; f32 within ``1e-5 * sum_b |AS*WS*P| + 1e-6``;
the result bit-identical from call to call (the partial tiles are added in
slice order whichever workgroup finishes last), and the workspace's tile
counters back at zero after every call, so the next call (any shape) finds
it ready.  Inputs are seeded (``synth``) and quantized by the oracle.
"""
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
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    return A, AS, W, WS


def _tiles(M, N):
    return ((M + 63) // 64) * ((N + 63) // 64)


def _assert_close(C, out, mag, what):
    ok = oracle.within_tolerance(C, out, mag, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        raise AssertionError("%s: %d/%d outside tolerance, first %s" % (what, len(bad), ok.size,
                                                                        bad[:5].tolist()))


def _counters_zero(ws, M, N):
    # the workspace starts with 4096 bytes of tile counters
    return int(torch.count_nonzero(ws[:4096]).item()) == 0


# long contractions (K >= 8192) with few output tiles: the long-K
# workload's shape at M = 32, ragged blocks per slice, ragged M and N,
# several M tiles, the smallest M
SPLIT = [(32, 4096, 14336), (64, 4096, 8224), (40, 1000, 8320), (100, 300, 8320),
         (129, 700, 8192), (8, 64, 8192), (64, 1024, 16384)]


@pytest.mark.parametrize("M,N,K", SPLIT)
def test_split_parity(dev, M, N, K):
    need = q8.q8_qdot_ws_size(M, N, K)
    assert need > 0, "shape expected to take the split form"
    print("[splitk] M=%d N=%d K=%d workspace %d bytes" % (M, N, K, need), flush=True)
    A, AS, W, WS = _case(M, N, K, 900 + M + N + K)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    ws = q8.workspace(M, N, K, dev)
    C1 = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)
    C2 = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)
    P = q8.q8_qdot_ws_partials(tA, tW)
    WST = np.ascontiguousarray(WS.T)
    C3 = q8.q8_qmma_ws(tA, tAS, tW, _dev(WST, dev), ws)
    torch.cuda.synchronize()
    assert _counters_zero(ws, M, N), "tile counters not reset"
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32)), "not deterministic"
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C1.cpu().numpy(), out, mag, "q8_qdot_ws")
    out_t, mag_t = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C3.cpu().numpy(), out_t, mag_t, "q8_qmma_ws")
    Pref = oracle.block_partials(A, W)
    Pg = P.cpu().numpy()
    if not np.array_equal(Pg, Pref):
        bad = np.argwhere(Pg != Pref)
        raise AssertionError("%d partials differ; first %s gpu=%r oracle=%r"
                             % (len(bad), bad[:3].tolist(), Pg[tuple(bad[0])], Pref[tuple(bad[0])]))


def test_long_k_workload_at_m32(dev):
    # the long-contraction workload (N = 4096, K = 14336, activations with
    # outliers) drawn with 32 activation rows instead of one
    w = synth.WORKLOADS[2]
    a32, w32 = synth.workload_f32(w, M=32)
    A, AS = oracle.quantize_rows(a32)
    W, WS = oracle.quantize_rows(w32)
    M, N, K = A.shape[0], W.shape[0], A.shape[1]
    assert q8.q8_qdot_ws_size(M, N, K) > 0
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    ws = q8.workspace(M, N, K, dev)
    C = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)
    P = q8.q8_qdot_ws_partials(tA, tW)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "long K, M=32")
    assert np.array_equal(P.cpu().numpy(), oracle.block_partials(A, W))


def test_shared_workspace_across_shapes(dev):
    # one workspace (sized for the largest) serving different shapes in turn
    shapes = [(32, 4096, 8192), (40, 1000, 8320), (32, 4096, 8192), (100, 300, 8320)]
    size = max(q8.q8_qdot_ws_size(*s) for s in shapes)
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)
    for k, (M, N, K) in enumerate(shapes):
        A, AS, W, WS = _case(M, N, K, 1200 + k)
        C = q8.q8_qdot_ws(*(_dev(x, dev) for x in (A, AS, W, WS)), ws)
        torch.cuda.synchronize()
        out, mag = oracle.qdot_f64(A, AS, W, WS)
        _assert_close(C.cpu().numpy(), out, mag, "shared workspace %s" % ((M, N, K),))


def test_small_workspace_falls_back(dev):
    # too small a workspace: exactly the plain entry (same kernel, same bits)
    M, N, K = 64, 2048, 8192
    assert q8.q8_qdot_ws_size(M, N, K) > 1024
    A, AS, W, WS = _case(M, N, K, 1300)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    small = torch.zeros(1024, dtype=torch.uint8, device=dev)
    C1 = q8.q8_qdot_ws(tA, tAS, tW, tWS, small)
    C2 = q8.q8_qdot(tA, tAS, tW, tWS)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_shapes_without_split_match_plain_entry(dev):
    # shapes that do not take the split form run the plain entry's kernel
    for (M, N, K) in [(1, 4096, 4096), (4, 300, 1024), (512, 14336, 256), (9, 37, 96),
                      (64, 4096, 4096)]:
        assert q8.q8_qdot_ws_size(M, N, K) == 0
        A, AS, W, WS = _case(M, N, K, 1400 + M)
        tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
        ws = torch.zeros(64, dtype=torch.uint8, device=dev)
        C1 = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)
        C2 = q8.q8_qdot(tA, tAS, tW, tWS)
        torch.cuda.synchronize()
        assert torch.equal(C1.view(torch.int32), C2.view(torch.int32)), (M, N, K)


def test_split_huge_weight_scales(dev):
    # fast-epilogue overflow: the affected waves recompute in the plain order
    M, N, K = 64, 512, 8192
    A = np.full((M, K), -128, np.int8)
    W = synth.random_i8((N, K), 1500)
    AS = synth.random_scales((M, K // 32), 1501)
    WS = synth.random_scales((N, K // 32), 1502)
    for b, e in ((1, 101), (20, 110), (140, 126)):
        WS[3:100, b] = np.float32(2.0 ** e)
        AS[:, b] = np.float32(2.0 ** -e)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    ws = q8.workspace(M, N, K, dev)
    C = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma_ws(tA, tAS, tW, _dev(WST, dev), ws)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "huge scales")
    out_t, mag_t = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out_t, mag_t, "huge scales (qmma)")


def test_split_graph_replay(dev):
    # captured and replayed: the counters reset inside the kernel, so every
    # replay (with eager calls on the same workspace in between) is exact
    M, N, K = 64, 2048, 8192
    A, AS, W, WS = _case(M, N, K, 1600)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    ws = q8.workspace(M, N, K, dev)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    q8.q8_qdot_ws(tA, tAS, tW, tWS, ws, C)
    torch.cuda.synchronize()
    eager = C.cpu().numpy().copy()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(eager, out, mag, "eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q8.q8_qdot_ws(tA, tAS, tW, tWS, ws, C, stream=s)
    torch.cuda.synchronize()
    for r in range(4):
        C.fill_(float("nan"))
        other = q8.q8_qdot_ws(tA, tAS, tW, tWS, ws)   # eager use of the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), eager.view(np.uint32)), "replay %d" % r
        assert np.array_equal(other.cpu().numpy().view(np.uint32), eager.view(np.uint32))
    assert _counters_zero(ws, M, N)


def test_two_streams_two_workspaces(dev):
    # calls on two streams, each with its own workspace, interleaved: every
    # result is the eager single-stream one, bit for bit
    shapes = [(32, 4096, 8192), (40, 1000, 8320)]
    cases = []
    for k, (M, N, K) in enumerate(shapes):
        host = _case(M, N, K, 1700 + k)
        t = tuple(_dev(x, dev) for x in host)
        ref = q8.q8_qdot_ws(*t, q8.workspace(M, N, K, dev))
        cases.append((t, ref, q8.workspace(M, N, K, dev), (M, N, K)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[], []]
    for rep in range(3):
        for k, (t, ref, ws, (M, N, K)) in enumerate(cases):
            with torch.cuda.stream(streams[k]):
                C = torch.empty((M, N), dtype=torch.float32, device=dev)
                q8.q8_qdot_ws(*t, ws, C, stream=streams[k])
                outs[k].append(C)
    torch.cuda.synchronize()
    for k, (t, ref, ws, shape) in enumerate(cases):
        for C in outs[k]:
            assert torch.equal(C.view(torch.int32), ref.view(torch.int32)), "stream %d %s" % (k, shape)
        assert _counters_zero(ws, *shape[:2])
