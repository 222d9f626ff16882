"""GPU parity of q8_qmma (the qmma_t form: weight scales stored [K/32, N])
against the oracle's qmma_t definition, element by element.

Same bar as q8_qdot: f32 output within ``1e-5 * sum_b |AS*WST*P| + 1e-6``.
The shapes reach every kernel and every weight-scale load mode: the matvec
(M < 8), the K-split GEMM (few tiles), and the staged GEMM with 16-byte
transposed-scale loads (N % 4 == 0, whole 4-block stages, 16-byte aligned
scales) or dword loads (any other case, including a misaligned array).
"""
import functools
import sys

import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL, ABS = 1e-5, 1e-6


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def _workload(idx):
    w = synth.WORKLOADS[idx]
    a32, w32 = synth.workload_f32(w)
    A, AS = oracle.quantize_rows(a32)
    W, WS = oracle.quantize_rows(w32)
    return A, AS, W, np.ascontiguousarray(WS.T)


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _assert_close(C, out, mag, what):
    ok = oracle.within_tolerance(C, out, mag, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        raise AssertionError("%s: %d/%d outside tolerance; first bad %s C=%r oracle=%r"
                             % (what, len(bad), ok.size, bad[:5].tolist(),
                                C[tuple(bad[0])], out[tuple(bad[0])]))


def _random_case(M, N, K, seed):
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 1.0)
    WST = synth.random_scales((K // 32, N), seed + 3, 1e-3, 1.0)
    return A, AS, W, WST


def _check(A, AS, W, WST, dev, what, misalign=False):
    M, K = A.shape
    N = W.shape[0]
    _say("[qmma] %s M=%d N=%d K=%d path=%d misalign=%d"
         % (what, M, N, K, q8.q8_qdot_path(M, N, K), misalign))
    tA, tAS, tW = (_dev(x, dev) for x in (A, AS, W))
    if misalign:
        # the scales start 4 bytes past a 16-byte boundary
        big = torch.empty(WST.size + 1, dtype=torch.float32, device=dev)
        big[1:] = torch.from_numpy(WST.ravel()).to(dev)
        tWST = big[1:].view(WST.shape)
        assert tWST.data_ptr() % 16 == 4
    else:
        tWST = _dev(WST, dev)
    C = q8.q8_qmma(tA, tAS, tW, tWST)
    torch.cuda.synchronize()
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C.cpu().numpy(), out, mag, what)


@pytest.mark.parametrize("idx", [0, 2, 3])
def test_workload_full_output(dev, idx):
    A, AS, W, WST = _workload(idx)
    _check(A, AS, W, WST, dev, synth.WORKLOADS[idx].name)


def test_workload_prompt_size(dev):
    # the full 512 x 14336 output against the oracle (about 30 G
    # multiply-adds on the host)
    A, AS, W, WST = _workload(4)
    M, N = A.shape[0], W.shape[0]
    _say("[qmma] prompt-size full output path=%d" % q8.q8_qdot_path(M, N, A.shape[1]))
    tA, tAS, tW, tWST = (_dev(x, dev) for x in (A, AS, W, WST))
    C = q8.q8_qmma(tA, tAS, tW, tWST)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    del C
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(Ch, out, mag, "prompt-size qmma")


SHAPES = [
    (1, 37, 1056), (3, 129, 2080), (7, 300, 1024), (5, 64, 4096),      # matvec
    # one row: shares of rows per workgroup that are ragged, several
    # LDS tiles per share, a single row, the two-rows-in-flight form and
    # the one-row form (rows over 12 KiB), rows longer than 16 KiB
    (1, 14300, 4096), (1, 40000, 2048), (1, 1, 64), (1, 3000, 12288), (1, 1000, 13312),
    (1, 2049, 16384), (1, 100, 16416),
    # small batches: the largest LDS footprint (7 rows of 16 KiB and their
    # scales beside the scale tile), several tiles per share, ragged shares
    (7, 500, 16384), (4, 3000, 8192), (2, 14336, 4096), (6, 40000, 1024),
    (9, 37, 96), (33, 100, 4096), (127, 300, 4160), (64, 4099, 128),    # K-split
    (512, 14336, 1024),                                                 # staged, 16-byte scales
    (390, 14302, 1024), (384, 14400, 2080), (392, 14300, 160),          # staged, dword scales
    (512, 7168, 1024), (136, 14300, 160),                               # 64 x 64 tiles, shared units
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes(dev, M, N, K):
    A, AS, W, WST = _random_case(M, N, K, 900 + M + N + K)
    _check(A, AS, W, WST, dev, "shape")


@pytest.mark.parametrize("M,N,K", [(512, 7168, 1024), (64, 4096, 512), (2, 100, 256), (1, 1000, 4096)])
def test_misaligned_scales(dev, M, N, K):
    A, AS, W, WST = _random_case(M, N, K, 55 + M)
    _check(A, AS, W, WST, dev, "misaligned", misalign=True)


def test_qmma_matches_qdot_on_transposed_scales(dev):
    # same data, both layouts: the two entries must agree to the bar (their
    # f32 sums may round differently only if the kernels' orders differ)
    A, AS, W, WST = _random_case(200, 3000, 2048, 4242)
    WS = np.ascontiguousarray(WST.T)
    tA, tAS, tW = (_dev(x, dev) for x in (A, AS, W))
    C1 = q8.q8_qdot(tA, tAS, tW, _dev(WS, dev))
    C2 = q8.q8_qmma(tA, tAS, tW, _dev(WST, dev))
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C1.cpu().numpy(), out, mag, "qdot")
    _assert_close(C2.cpu().numpy(), out, mag, "qmma")
