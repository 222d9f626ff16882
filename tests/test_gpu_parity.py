"""GPU parity: the HIP library against the CPU oracle, element by element.

Bar (stated with the contraction): int32 block partials bit-exact; f32 output
within ``|C - out64| <= 1e-5 * sum_b |AS*WS*P| + 1e-6`` of the f64 oracle;
the GPU quantizer bit-exact with the oracle quantizer (both decide each code
in f32).  Inputs come from the seeded generators in ``synth`` and are
quantized by the oracle on the host, so no oracle input or expected value
comes from the GPU.  Every call goes through the C-ABI (``gemm_q8_qdot_amd``
is a ctypes binding over ``libq8qdot.so``).
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


@functools.lru_cache(maxsize=4)
def _workload(idx):
    w = synth.WORKLOADS[idx]
    a32, w32 = synth.workload_f32(w)
    A, AS = oracle.quantize_rows(a32)
    W, WS = oracle.quantize_rows(w32)
    return A, AS, W, WS


def _dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _run(A, AS, W, WS, dev):
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C = q8.q8_qdot(tA, tAS, tW, tWS)
    P = q8.q8_qdot_partials(tA, tW)
    torch.cuda.synchronize()
    return C.cpu().numpy(), P.cpu().numpy()


def _assert_close(C, out, mag, what):
    ok = oracle.within_tolerance(C, out, mag, REL, ABS)
    if not ok.all():
        bad = np.argwhere(~ok)
        err = np.abs(C.astype(np.float64) - out)
        ratio = err / (REL * mag + ABS)
        k = tuple(np.unravel_index(np.argmax(ratio), ratio.shape))
        raise AssertionError("%s: %d/%d outside tolerance; worst at %s: C=%r oracle=%r "
                             "abs_terms=%r (%.3g x bound); first bad %s"
                             % (what, len(bad), ok.size, k, C[k], out[k], mag[k], ratio[k],
                                bad[:5].tolist()))


def _check_full(A, AS, W, WS, dev, what):
    _say("[parity] %s M=%d N=%d K=%d" % (what, A.shape[0], W.shape[0], A.shape[1]))
    C, P = _run(A, AS, W, WS, dev)
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    Pref = oracle.block_partials(A, W)
    assert P.shape == Pref.shape
    if not np.array_equal(P, Pref):
        bad = np.argwhere(P != Pref)
        raise AssertionError("%s: %d partials differ; first %s gpu=%r oracle=%r"
                             % (what, len(bad), bad[:3].tolist(), P[tuple(bad[0])],
                                Pref[tuple(bad[0])]))
    _assert_close(C, out, mag, what)
    return C, P


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_workload_full_output(dev, idx):
    A, AS, W, WS = _workload(idx)
    _check_full(A, AS, W, WS, dev, synth.WORKLOADS[idx].name)


def _check_partials_sliced(P, A, W, what, rows=32):
    """Every int32 partial of a device P [M, N, K/32] against the oracle.

    P can be gigabytes: it is copied back and compared ``rows`` activation
    rows at a time, each slice against ``oracle.block_partials`` of the same
    rows.
    """
    M = A.shape[0]
    for i0 in range(0, M, rows):
        i1 = min(M, i0 + rows)
        got = P[i0:i1].cpu().numpy()
        ref = oracle.block_partials(A[i0:i1], W)
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            k = tuple(bad[0])
            raise AssertionError("%s: %d partials differ in rows %d..%d; first (%d, %d, %d) "
                                 "gpu=%r oracle=%r" % (what, len(bad), i0, i1 - 1, k[0] + i0, k[1],
                                                       k[2], got[k], ref[k]))


def test_workload_prompt_size(dev):
    # 512 x 14336 x 4096 in the launch configuration the benchmark times:
    # the f32 output in full against the oracle (about 30 G multiply-adds,
    # a second or two on the host's cores), and every one of the 939.5 M
    # int32 block partials (3.8 GB) of the full-size debug launch, which runs
    # the timed kernel's own loop, compared 32 rows at a time.
    idx = 4
    A, AS, W, WS = _workload(idx)
    _say("[parity] %s full output" % synth.WORKLOADS[idx].name)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C = q8.q8_qdot(tA, tAS, tW, tWS)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    del C
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(Ch, out, mag, "c4 C")
    del Ch, out, mag
    _say("[parity] %s all partials" % synth.WORKLOADS[idx].name)
    P = q8.q8_qdot_partials(tA, tW)
    torch.cuda.synchronize()
    _check_partials_sliced(P, A, W, "c4 P")
    del P
    torch.cuda.empty_cache()


# --------------------------------------------------------------- edge shapes

EDGE = [
    (1, 1, 32), (1, 37, 1056), (2, 100, 32), (3, 129, 2080), (5, 64, 4096), (7, 300, 1024),
    (8, 1, 64), (9, 37, 96), (16, 33, 128), (31, 65, 1056), (33, 100, 4096), (63, 129, 320),
    (64, 4096, 32), (65, 224, 2048), (128, 449, 512), (1, 513, 16416), (3, 8, 32800),
    (12, 70, 16416), (4, 4099, 14336), (9, 1, 14336), (127, 300, 4160), (40, 2050, 8224),
]

# One activation row with K <= 16 KiB (the decode kernel, launched as one
# workgroup per compute unit with a grid stride over weight rows): rows per
# wave that do not divide evenly, the prefetching form for rows of 9..14 KiB
# with an odd and an even number of rows per wave, rows of 15 and 16 KiB,
# and K that is not a multiple of 1 KiB.
ROWS = [(1, 5000, 4096), (1, 3000, 9248), (1, 1025, 14336), (1, 2049, 16384), (1, 7, 15360),
        (1, 2048 * 3 + 5, 1056), (1, 100, 8192)]


@pytest.mark.parametrize("M,N,K", ROWS)
def test_decode_rows(dev, M, N, K):
    seed = N * 17 + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _check_full(A, AS, W, WS, dev, "rows")


# Small decode batches (2..7 activation rows): one weight pass for all rows,
# at the decode workloads' sizes and at ragged ones.
BATCH = [(2, 14336, 4096), (4, 4096, 14336), (7, 4096, 4096), (3, 1000, 16384), (5, 333, 1056),
         (6, 2, 32), (7, 300, 16384), (2, 5000, 9216), (4, 2049, 8192)]


@pytest.mark.parametrize("M,N,K", BATCH)
def test_small_batch(dev, M, N, K):
    A = synth.random_i8((M, K), 60 + M)
    W = synth.random_i8((N, K), 61 + M)
    AS = synth.random_scales((M, K // 32), 62 + M, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), 63 + M, 1e-3, 1.0)
    _check_full(A, AS, W, WS, dev, "batch")


# one row, a small batch, the K-split GEMM, the LDS-staged GEMM, the
# 64 x 64-tile GEMM over all of K
@pytest.mark.parametrize("M,N,K", [(1, 3000, 4096), (4, 3000, 4096), (64, 512, 2048), (385, 14336, 256),
                                   (300, 2000, 1024)])
def test_cancelling_half_blocks(dev, M, N, K):
    A, AS, W, WS = synth.cancelling_blocks(M, N, K, 880 + M)
    P = oracle.block_partials(A, W)
    assert np.abs(P).max() <= 128                      # the construction holds
    C, _ = _check_full(A, AS, W, WS, dev, "cancelling halves")
    # the transposed-scale entry takes the same care
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma(_dev(A, dev), _dev(AS, dev), _dev(W, dev), _dev(WST, dev))
    torch.cuda.synchronize()
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out, mag, "cancelling halves (qmma)")


@pytest.mark.parametrize("M,N,K", EDGE)
def test_edge_shapes(dev, M, N, K):
    seed = M * 1000003 + N * 101 + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _check_full(A, AS, W, WS, dev, "edge")


# Subnormal weight scales (below 2^-126) on every third block, against
# activation scales of 1e26 (the largest the M >= 8 epilogue's bound covers
# for such scales, per the header): every path must stay finite and inside
# the bound.  One row, a batch, the K-split GEMM (one round and shared), the
# staged GEMM, the 64 x 64-tile GEMM (one workgroup per unit and shared).
@pytest.mark.parametrize("M,N,K", [(1, 300, 2048), (4, 300, 2048), (9, 300, 2048), (16, 9000, 512),
                                   (385, 14336, 128), (300, 2000, 256), (129, 14336, 128)])
def test_subnormal_weight_scales(dev, M, N, K):
    seed = M * 5 + N + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 1.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    KB = K // 32
    for b in range(0, KB, 3):
        WS[:, b] = np.float32(1e-40) * np.float32(1 + (b % 7))   # subnormal f32
        AS[:, b] = np.float32(1e26)
    assert (WS[:, 0] < np.finfo(np.float32).tiny).all() and (WS[:, 0] > 0).all()
    _check_full(A, AS, W, WS, dev, "subnormal scales")
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma(_dev(A, dev), _dev(AS, dev), _dev(W, dev), _dev(WST, dev))
    torch.cuda.synchronize()
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out, mag, "subnormal scales (qmma)")


def _dev_offset(x, dev, words=1):
    # a device copy of x starting `words` 4-byte words past a fresh
    # allocation's (256-byte aligned) start: 4-byte but not 16-byte aligned
    flat = torch.zeros(x.size + words, dtype=torch.from_numpy(x[:0]).dtype, device=dev)
    flat[words:] = torch.from_numpy(np.ascontiguousarray(x).ravel()).to(dev)
    return flat[words:].view(*x.shape)


# Scales and the output at 4-byte (not 16-byte) aligned addresses on every
# path: the kernels that load scales 16 bytes at a time must fall back to
# dword loads, and no store may assume more than 4-byte alignment.
@pytest.mark.parametrize("M,N,K", [(1, 3000, 4096), (4, 300, 2048), (9, 300, 2048), (16, 9000, 512),
                                   (385, 14336, 128), (300, 2000, 256), (129, 14336, 128)])
def test_misaligned_scales_and_output(dev, M, N, K):
    seed = M * 3 + N + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _say("[parity] misaligned scales and C M=%d N=%d K=%d path=%d" % (M, N, K, q8.q8_qdot_path(M, N, K)))
    tA, tW = _dev(A, dev), _dev(W, dev)
    tAS, tWS = _dev_offset(AS, dev), _dev_offset(WS, dev)
    tWST = _dev_offset(np.ascontiguousarray(WS.T), dev)
    assert tAS.data_ptr() % 16 != 0 and tWS.data_ptr() % 16 != 0 and tWST.data_ptr() % 16 != 0
    C = _dev_offset(np.zeros((M, N), np.float32), dev)
    C2 = _dev_offset(np.zeros((M, N), np.float32), dev, 3)
    q8.q8_qdot(tA, tAS, tW, tWS, C)
    q8.q8_qmma(tA, tAS, tW, tWST, C2)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "misaligned (qdot)")
    _assert_close(C2.cpu().numpy(), out, mag, "misaligned (qmma)")


# The decode kernels form AS * WS in f32 before the block sum, so subnormal
# weight scales against activation scales near 1e36 give ordinary products
# that carry the whole result: a kernel (or a build) that flushed subnormal
# operands to zero would miss every output (checked on the host: the result
# with WS flushed fails the bound everywhere).
@pytest.mark.parametrize("M,N,K", [(1, 300, 2048), (4, 300, 2048), (1, 300, 20480)])
def test_subnormal_scales_decode_kernels(dev, M, N, K):
    A = synth.random_i8((M, K), 61 + M)
    W = synth.random_i8((N, K), 62 + M)
    AS = (np.float32(1e36) * synth.random_scales((M, K // 32), 63 + M, 0.5, 2.0)).astype(np.float32)
    WS = (np.float32(1e-40) * synth.random_scales((N, K // 32), 64 + M, 1.0, 10.0)).astype(np.float32)
    assert (WS < np.finfo(np.float32).tiny).all()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    flushed, _ = oracle.qdot_f64(A, AS, W, np.zeros_like(WS))
    assert not oracle.within_tolerance(flushed.astype(np.float32), out, mag).any()
    assert q8.q8_qdot_path(M, N, K) == 0
    _check_full(A, AS, W, WS, dev, "subnormal scales, decode")
    tA, tAS, tW = _dev(A, dev), _dev(AS, dev), _dev(W, dev)
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma(tA, tAS, tW, _dev(WST, dev))
    W5 = synth.random_q50(N, K, 65 + M)
    C5 = q8.q8_q50_qdot(tA, tAS, _dev(W5, dev), _dev(WS, dev))
    torch.cuda.synchronize()
    out2, mag2 = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out2, mag2, "subnormal scales, decode (qmma)")
    out5, mag5 = oracle.q50_qdot_f64(A, AS, W5, WS)
    _assert_close(C5.cpu().numpy(), out5, mag5, "subnormal scales, decode (Q5_0)")


# Large extents: one activation row of 128 KiB (eight 16 KiB chunks), 200003
# short weight rows (many rows per wave), a batch of 50000 rows, and the
# K-split GEMM over 2048 and 1024 blocks; Q5_0 weights past the 16 Ki values
# of the decode kernel.
LARGE = [(1, 64, 131072), (1, 200003, 256), (3, 50000, 512), (9, 40, 65536), (200, 70, 32768)]


@pytest.mark.parametrize("M,N,K", LARGE)
def test_large_extents(dev, M, N, K):
    seed = M * 7 + N + K // 32
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _check_full(A, AS, W, WS, dev, "large")
    if K > 16384 and N <= 100:
        W5 = synth.random_q50(N, K, seed + 4)
        tA, tAS, tW5, tWS = (_dev(x, dev) for x in (A, AS, W5, WS))
        C5 = q8.q8_q50_qdot(tA, tAS, tW5, tWS)
        P5 = q8.q8_q50_partials(tA, tW5)
        torch.cuda.synchronize()
        out, mag = oracle.q50_qdot_f64(A, AS, W5, WS)
        _assert_close(C5.cpu().numpy(), out, mag, "large (Q5_0)")
        assert np.array_equal(P5.cpu().numpy(), oracle.q50_block_partials(A, W5)), "large (Q5_0) partials"


STAGED = [(385, 14336, 96), (390, 14300, 160), (384, 14400, 2080), (512, 14336, 32)]


@pytest.mark.parametrize("M,N,K", STAGED)
def test_staged_gemm_shapes(dev, M, N, K):
    # Shapes that reach the LDS-staged GEMM, with ragged M, N and a partial
    # last stage of blocks; f32 output and partials in full.
    assert q8.q8_qdot_path(M, N, K) == 2
    seed = M * 7 + N * 3 + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _say("[parity] staged M=%d N=%d K=%d" % (M, N, K))
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C = q8.q8_qdot(tA, tAS, tW, tWS)
    P = q8.q8_qdot_partials(tA, tW)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "staged C")
    _check_partials_sliced(P, A, W, "staged P")


# The K-split GEMM with more 32 x 32 tiles than compute units (eight-wave
# workgroups, two per compute unit): a 16-row decode batch against the
# 14336-row weight, and ragged M, N, K; Q8_0 and Q5_0 weights, both scale
# layouts, partials in full.
KSPLIT_SHARED = [(16, 14336, 1024), (100, 3000, 1056)]


@pytest.mark.parametrize("M,N,K", KSPLIT_SHARED)
def test_ksplit_shared_workgroups(dev, M, N, K):
    assert q8.q8_qdot_path(M, N, K) == 1
    assert -(-M // 32) * -(-N // 32) > 256
    seed = M * 13 + N * 3 + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    W5 = synth.random_q50(N, K, seed + 4)
    _say("[parity] K-split, shared workgroups M=%d N=%d K=%d" % (M, N, K))
    tA, tAS, tW, tWS, tW5 = (_dev(x, dev) for x in (A, AS, W, WS, W5))
    WST = np.ascontiguousarray(WS.T)
    C = q8.q8_qdot(tA, tAS, tW, tWS)
    C2 = q8.q8_qmma(tA, tAS, tW, _dev(WST, dev))
    C5 = q8.q8_q50_qdot(tA, tAS, tW5, tWS)
    P = q8.q8_qdot_partials(tA, tW)
    P5 = q8.q8_q50_partials(tA, tW5)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "K-split shared C")
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out, mag, "K-split shared C (qmma)")
    out, mag = oracle.q50_qdot_f64(A, AS, W5, WS)
    _assert_close(C5.cpu().numpy(), out, mag, "K-split shared C (Q5_0)")
    _check_partials_sliced(P, A, W, "K-split shared P")
    assert np.array_equal(P5.cpu().numpy(), oracle.q50_block_partials(A, W5)), "K-split shared P (Q5_0)"


# The 64 x 64-tile GEMM over all of K: the M=512 workload's 8-way N share at
# its full K, and ragged M, N and K (a partial last stage of blocks).
# the last four have more 64 x 64 tiles than compute units (two workgroups
# share a unit: the 8-wave form of the kernel); the last two are shapes the
# staged GEMM would take but is slower on
WHOLE_K = [(512, 1792, 4096), (300, 2000, 1056), (270, 1900, 544), (512, 4096, 1024), (520, 2100, 1056),
           (129, 14336, 96), (136, 14300, 160)]


@pytest.mark.parametrize("M,N,K", WHOLE_K)
def test_whole_k_gemm_shapes(dev, M, N, K):
    assert q8.q8_qdot_path(M, N, K) == 3
    seed = M * 11 + N * 5 + K
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    _say("[parity] whole-K GEMM M=%d N=%d K=%d" % (M, N, K))
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C = q8.q8_qdot(tA, tAS, tW, tWS)
    P = q8.q8_qdot_partials(tA, tW)
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma(tA, tAS, tW, _dev(WST, dev))
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "whole-K C")
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out, mag, "whole-K C (qmma)")
    _check_partials_sliced(P, A, W, "whole-K P")


# one row, the K-split GEMM (M = 9, and M = 129 with few tiles), the
# LDS-staged GEMM (M = 385 with N = 14336), the 64 x 64-tile GEMM over all
# of K (M = 300, N = 2000; M = 129, N = 14336 with two workgroups per unit)
@pytest.mark.parametrize("M,N,K", [(1, 70, 1024), (9, 70, 1024), (129, 70, 1024), (385, 14336, 256),
                                   (300, 2000, 1024), (129, 14336, 256)])
def test_extreme_bytes_and_scales(dev, M, N, K):
    A = np.full((M, K), -128, np.int8)
    W = synth.random_i8((N, K), 77)
    W[0] = -128
    W[1] = 127
    AS = synth.random_scales((M, K // 32), 78)
    WS = synth.random_scales((N, K // 32), 79)
    AS[:, 3] = 1e30
    WS[:, 3] = 1e-30           # product 1 at block 3
    AS[:, 5] = 1e-30           # tiny contributions at block 5
    WS[:, 7] = 0.0             # zero-scale block
    WS[2] = 0.0                # a whole zero row of scales
    # Weight scales far above 1 against tiny activation scales (products of
    # order 1): 2^101 (the GEMMs' fast epilogue still finite), 2^110 (its
    # bias product overflows) and 2^126 (ws * p overflows before the
    # activation scale) -- the GEMMs recompute such tiles in the plain order.
    # Columns 40..69 keep ordinary scales throughout.
    for b, e in ((1, 101), (6, 110), (2, 126)):
        WS[3:40, b] = np.float32(2.0 ** e)
        AS[:, b] = np.float32(2.0 ** -e)
    if M > 1:
        assert q8.q8_qdot_path(M, N, K) == (2 if M == 385 else 3 if N in (2000, 14336) else 1)
    _check_full(A, AS, W, WS, dev, "extreme")
    WST = np.ascontiguousarray(WS.T)
    C2 = q8.q8_qmma(_dev(A, dev), _dev(AS, dev), _dev(W, dev), _dev(WST, dev))
    torch.cuda.synchronize()
    out, mag = oracle.qmma_f64(A, AS, W, WST)
    _assert_close(C2.cpu().numpy(), out, mag, "extreme (qmma)")


def test_zero_blocks_and_negative_scales(dev):
    M, N, K = 10, 50, 512
    A = synth.random_i8((M, K), 88)
    W = synth.random_i8((N, K), 89)
    A[:, 64:96] = 0
    W[:, 128:160] = 0
    AS = synth.random_scales((M, K // 32), 90) * np.where(np.arange(K // 32) % 3 == 0, -1, 1).astype(np.float32)
    WS = synth.random_scales((N, K // 32), 91)
    _check_full(A, AS, W, WS, dev, "zeros/negative scales")


# ------------------------------------------------------------ determinism etc.

@pytest.mark.parametrize("idx", [1, 3])
def test_deterministic(dev, idx):
    A, AS, W, WS = _workload(idx)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    C1 = q8.q8_qdot(tA, tAS, tW, tWS)
    C2 = q8.q8_qdot(tA, tAS, tW, tWS)
    P1 = q8.q8_qdot_partials(tA, tW)
    P2 = q8.q8_qdot_partials(tA, tW)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    assert torch.equal(P1, P2)


def test_row_chunk_offsets_match_full(dev):
    # Offset pointers into A/AS (a chunk of rows) give the same rows.
    A, AS, W, WS = _workload(3)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    full = q8.q8_qdot(tA, tAS, tW, tWS)
    part = q8.q8_qdot(tA[40:52], tAS[40:52], tW, tWS)
    one = q8.q8_qdot(tA[17:18], tAS[17:18], tW, tWS)
    torch.cuda.synchronize()
    out, mag = oracle.qdot_f64(A[40:52], AS[40:52], W, WS)
    _assert_close(part.cpu().numpy(), out, mag, "row chunk")
    out1, mag1 = oracle.qdot_f64(A[17:18], AS[17:18], W, WS)
    _assert_close(one.cpu().numpy(), out1, mag1, "single row")
    _assert_close(full[40:52].cpu().numpy(), out, mag, "full rows")


def test_output_overwritten_not_accumulated(dev):
    A = synth.random_i8((9, 64), 5)
    W = synth.random_i8((20, 64), 6)
    AS = synth.random_scales((9, 2), 7)
    WS = synth.random_scales((20, 2), 8)
    for M in (1, 9):
        tA, tAS, tW, tWS = (_dev(x, dev) for x in (A[:M], AS[:M], W, WS))
        C = torch.full((M, 20), 12345.0, device=dev)
        q8.q8_qdot(tA, tAS, tW, tWS, C)
        torch.cuda.synchronize()
        out, mag = oracle.qdot_f64(A[:M], AS[:M], W, WS)
        _assert_close(C.cpu().numpy(), out, mag, "overwrite M=%d" % M)


def test_empty_and_zero_K(dev):
    e8 = torch.empty((0, 64), dtype=torch.int8, device=dev)
    C = q8.q8_qdot(e8, torch.empty((0, 2), device=dev), torch.zeros((5, 64), dtype=torch.int8, device=dev),
                   torch.zeros((5, 2), device=dev))
    assert C.shape == (0, 5)
    for M in (1, 9):
        C = torch.full((M, 6), 7.0, device=dev)
        q8.q8_qdot(torch.empty((M, 0), dtype=torch.int8, device=dev), torch.empty((M, 0), device=dev),
                   torch.empty((6, 0), dtype=torch.int8, device=dev), torch.empty((6, 0), device=dev), C)
        torch.cuda.synchronize()
        assert torch.count_nonzero(C).item() == 0


def test_side_stream(dev):
    A, AS, W, WS = _workload(0)
    tA, tAS, tW, tWS = (_dev(x, dev) for x in (A, AS, W, WS))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        C = q8.q8_qdot(tA, tAS, tW, tWS)
    s.synchronize()
    out, mag = oracle.qdot_f64(A, AS, W, WS)
    _assert_close(C.cpu().numpy(), out, mag, "side stream")


# ------------------------------------------------------------------ quantizer

def _quant_check(x, dev, what):
    q_ref, d_ref = oracle.quantize_rows(x)
    Q, D = q8.q8_quantize(_dev(x, dev))
    torch.cuda.synchronize()
    Qn, Dn = Q.cpu().numpy(), D.cpu().numpy()
    assert np.array_equal(Dn.view(np.int32), d_ref.view(np.int32)), what + ": scales differ"
    if not np.array_equal(Qn, q_ref):
        bad = np.argwhere(Qn != q_ref)
        raise AssertionError("%s: %d codes differ, first %s" % (what, len(bad), bad[:3].tolist()))


@pytest.mark.parametrize("idx", [0, 2])
def test_quantizer_workload_rows(dev, idx):
    w = synth.WORKLOADS[idx]
    a32, w32 = synth.workload_f32(w, N=512)
    _quant_check(a32, dev, "activations")
    _quant_check(w32, dev, "weights")


def test_quantizer_golden_and_edges(dev):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantize_worked_block.json")))
    rows = [g["x"], g["zero_block"]["x"], g["nonpower_scale_block"]["x"]]
    x = np.array(rows, np.float32).reshape(1, -1)
    _quant_check(x, dev, "golden")
    Q, D = q8.q8_quantize(_dev(x, dev))
    torch.cuda.synchronize()
    assert Q.cpu().numpy()[0, :32].tolist() == g["q"]
    assert Q.cpu().numpy()[0, 64:96].tolist() == g["nonpower_scale_block"]["q"]
    y = synth.random_f32((37, 4128), 3)
    y[0, :32] = 0.0
    y[1] *= np.float32(1e-30)
    y[2] *= np.float32(1e30)
    y[3, 5] = -y[3, :32].__abs__().max() * 2
    _quant_check(y, dev, "edge rows")
