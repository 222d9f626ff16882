"""GPU: every kernel writes exactly its output, nothing around it.

Each case places the output (C f32, or P int32) inside a larger buffer whose
surrounding words hold a sentinel bit pattern (at a 4-byte but not 16-byte
aligned address, the documented minimum), calls the C-ABI entry with
the interior address, and checks that (a) the words before and after are
untouched, (b) every output word was written, and (c) the output matches
the oracle (partials bit for bit, f32 within the contraction's tolerance).
The shapes reach every kernel the library dispatches to (``q8_qdot_path``
and the Q5_0 / transposed-scale entries), each with ragged extents.
"""
import sys

import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 4096            # sentinel words on each side of the output
SENTINEL = 0x7FC0DEAD   # a NaN payload no kernel produces as f32, and an unlikely int32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# The outputs (C, P, the quantizer's D) need only 4-byte alignment: they
# start one word past the guard, so no kernel may assume more.
LEAD = GUARD + 1


def _guarded(n, dtype, dev):
    buf = torch.full((LEAD + n + GUARD,), SENTINEL, dtype=torch.int32, device=dev)
    return buf, buf[LEAD:LEAD + n].view(dtype)


def _check_guard(buf, n, what):
    host = buf.cpu().numpy()
    before, inner, after = host[:LEAD], host[LEAD:LEAD + n], host[LEAD + n:]
    assert (before == SENTINEL).all(), "%s: wrote %d words before the output" % (what, (before != SENTINEL).sum())
    assert (after == SENTINEL).all(), "%s: wrote %d words after the output" % (what, (after != SENTINEL).sum())
    unwritten = int((inner == SENTINEL).sum())
    assert unwritten == 0, "%s: %d output words never written" % (what, unwritten)


def _t(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


# (entry, M, N, K): the kernel each shape reaches is in the comment.
CASES = [
    ("qdot", 1, 5000, 4096),      # one-row decode kernel, rows per wave ragged
    ("qdot", 1, 3001, 4096),      # one-row decode kernel, neighbouring-row pairs, odd N
    ("qdot", 1, 3000, 9248),      # one-row decode kernel, prefetching form
    ("qdot", 1, 130, 16416),      # chunked matvec (rows longer than 16 KiB)
    ("qdot", 3, 1000, 4128),      # small-batch matvec
    ("qdot", 70, 300, 1056),      # K-split MFMA GEMM
    ("qdot", 100, 3000, 1056),    # K-split MFMA GEMM, two workgroups per compute unit
    ("qdot", 385, 14336, 96),     # LDS-staged MFMA GEMM, ragged M
    ("qdot", 129, 14336, 96),     # 64 x 64-tile GEMM where the staged one would be slower
    ("qdot", 300, 2000, 1056),    # 64 x 64-tile GEMM over all of K, ragged M, N, K
    ("qdot", 520, 2100, 1056),    # 64 x 64-tile GEMM, two workgroups per compute unit
    ("qmma", 1, 1000, 4096),      # matvec with transposed scales
    ("qmma", 5, 1000, 2080),      # small batch with transposed scales
    ("qmma", 390, 14300, 128),    # staged GEMM with transposed scales
    ("qmma", 270, 1900, 544),     # 64 x 64-tile GEMM with transposed scales
    ("qmma", 520, 2100, 544),     # the same, two workgroups per compute unit
    ("q50", 1, 1001, 4096),       # Q5_0 matvec
    ("q50", 9, 100, 1056),        # Q5_0 K-split GEMM
    ("q50", 40, 7000, 1056),      # Q5_0 K-split GEMM, two workgroups per compute unit
    ("q50", 600, 2000, 1152),     # Q5_0 ring GEMM
    ("q50t", 520, 2100, 1024),    # Q5_0 ring GEMM, two workgroups per compute unit, transposed scales
    ("q50t", 2, 333, 2048),       # Q5_0 matvec, transposed scales
]


def test_cases_reach_every_q8_path():
    paths = {q8.q8_qdot_path(M, N, K) for entry, M, N, K in CASES if entry in ("qdot", "qmma")}
    assert paths == {0, 1, 2, 3}


@pytest.mark.parametrize("entry,M,N,K", CASES)
def test_output_bounds(dev, entry, M, N, K):
    _say("[guard] %s M=%d N=%d K=%d" % (entry, M, N, K))
    KB = K // 32
    seed = M * 131 + N * 7 + K
    A = synth.random_i8((M, K), seed)
    AS = synth.random_scales((M, KB), seed + 1, 1e-3, 1.0)
    WS = synth.random_scales((N, KB), seed + 2, 1e-3, 1.0)
    q50 = entry.startswith("q50")
    ws_t = entry in ("qmma", "q50t")
    W = synth.random_q50(N, K, seed + 3) if q50 else synth.random_i8((N, K), seed + 3)
    WSx = np.ascontiguousarray(WS.T) if ws_t else WS
    tA, tAS, tW, tWS = _t(A, dev), _t(AS, dev), _t(W, dev), _t(WSx, dev)

    cbuf, C = _guarded(M * N, torch.float32, dev)
    C = C.view(M, N)
    if entry == "qdot":
        q8.q8_qdot(tA, tAS, tW, tWS, C)
    elif entry == "qmma":
        q8.q8_qmma(tA, tAS, tW, tWS, C)
    elif entry == "q50":
        q8.q8_q50_qdot(tA, tAS, tW, tWS, C)
    else:
        q8.q8_q50_qmma(tA, tAS, tW, tWS, C)
    pbuf, P = _guarded(M * N * KB, torch.int32, dev)
    P = P.view(M, N, KB)
    if q50:
        q8.q8_q50_partials(tA, tW, P)
    else:
        q8.q8_qdot_partials(tA, tW, P)
    torch.cuda.synchronize()
    _check_guard(cbuf, M * N, entry + " C")
    _check_guard(pbuf, M * N * KB, entry + " P")

    if q50:
        Pref = oracle.q50_block_partials(A, W)
        out, mag = (oracle.q50_qmma_f64 if ws_t else oracle.q50_qdot_f64)(A, AS, W, WSx)
    else:
        Pref = oracle.block_partials(A, W)
        out, mag = (oracle.qmma_f64 if ws_t else oracle.qdot_f64)(A, AS, W, WSx)
    assert np.array_equal(P.cpu().numpy(), Pref)
    assert oracle.within_tolerance(C.cpu().numpy(), out, mag).all()


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 4128), (257, 1056)])
def test_quantize_bounds(dev, rows, K):
    # The quantizer clamps codes to [-127, 127], so -128 marks unwritten bytes.
    _say("[guard] quantize rows=%d K=%d" % (rows, K))
    X = synth.random_f32((rows, K), rows * 7 + K)
    qbuf = torch.full((GUARD + rows * K + GUARD,), -128, dtype=torch.int8, device=dev)
    Q = qbuf[GUARD:GUARD + rows * K].view(rows, K)
    dbuf, D = _guarded(rows * (K // 32), torch.float32, dev)
    D = D.view(rows, K // 32)
    q8.q8_quantize(_t(X, dev), Q, D)
    torch.cuda.synchronize()
    host = qbuf.cpu().numpy()
    assert (host[:GUARD] == -128).all() and (host[GUARD + rows * K:] == -128).all()
    assert not (host[GUARD:GUARD + rows * K] == -128).any()
    _check_guard(dbuf, rows * (K // 32), "quantize D")
    Qref, Dref = oracle.quantize_rows(X)
    assert np.array_equal(Q.cpu().numpy(), Qref)
    assert np.array_equal(D.cpu().numpy().view(np.uint32), Dref.view(np.uint32))


# The workspace entries' split form (K >= 8192, few 64 x 64 tiles), with
# ragged M and N and a partial last slice; the workspace itself sits in a
# guarded buffer too: nothing past the size q8_qdot_ws_size reports may be
# written, and its tile counters must be back at zero.
WS_CASES = [
    ("qdot_ws", 40, 1000, 8320),
    ("qmma_ws", 70, 300, 8224),
    ("noalloc", 33, 700, 9216),
]


@pytest.mark.parametrize("entry,M,N,K", WS_CASES)
def test_split_output_and_workspace_bounds(dev, entry, M, N, K):
    _say("[guard] %s M=%d N=%d K=%d" % (entry, M, N, K))
    KB = K // 32
    need = q8.q8_qdot_ws_size(M, N, K)
    assert need > 0, "shape expected to take the split form"
    seed = M * 131 + N * 7 + K
    A = synth.random_i8((M, K), seed)
    AS = synth.random_scales((M, KB), seed + 1, 1e-3, 1.0)
    WS = synth.random_scales((N, KB), seed + 2, 1e-3, 1.0)
    W = synth.random_i8((N, K), seed + 3)
    ws_t = entry == "qmma_ws"
    WSx = np.ascontiguousarray(WS.T) if ws_t else WS
    tA, tAS, tW, tWS = _t(A, dev), _t(AS, dev), _t(W, dev), _t(WSx, dev)

    cbuf, C = _guarded(M * N, torch.float32, dev)
    C = C.view(M, N)
    # workspace: zero-filled need bytes, then sentinel words
    wbuf = torch.full(((need + 3) // 4 + GUARD,), SENTINEL, dtype=torch.int32, device=dev)
    wbuf[:(need + 3) // 4] = 0
    ws = wbuf.view(torch.uint8)[:need]
    if entry == "qdot_ws":
        q8.q8_qdot_ws(tA, tAS, tW, tWS, ws, C)
    elif entry == "qmma_ws":
        q8.q8_qmma_ws(tA, tAS, tW, tWS, ws, C)
    else:
        st = q8.q8_qdot_noalloc_raw(tA.data_ptr(), tAS.data_ptr(), tW.data_ptr(), tWS.data_ptr(),
                                    C.data_ptr(), M, N, K, torch.cuda.current_stream().cuda_stream)
        assert st == q8.Q8_OK, q8.q8_strerror(st)
    pbuf, P = _guarded(M * N * KB, torch.int32, dev)
    P = P.view(M, N, KB)
    q8.q8_qdot_ws_partials(tA, tW, P)
    torch.cuda.synchronize()
    _check_guard(cbuf, M * N, entry + " C")
    _check_guard(pbuf, M * N * KB, entry + " P")
    host = wbuf.cpu().numpy()
    assert (host[(need + 3) // 4:] == SENTINEL).all(), "%s: wrote past the workspace" % entry
    assert (host[:1024] == 0).all(), "%s: tile counters not reset" % entry
    assert np.array_equal(P.cpu().numpy(), oracle.block_partials(A, W))
    out, mag = (oracle.qmma_f64 if ws_t else oracle.qdot_f64)(A, AS, W, WSx)
    assert oracle.within_tolerance(C.cpu().numpy(), out, mag).all()
