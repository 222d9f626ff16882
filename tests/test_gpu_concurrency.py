"""Concurrent use of the plain entries: several streams, several host threads.

The plain entries keep no state between calls (no device buffers of their
own; only per-device launch settings, set once), so calls that overlap on
different streams, issued from one host thread or from several, must give
exactly what the same calls give one after another.  Every kernel family is
covered (the one-row and small-batch decode kernels, the three GEMMs, transposed
weight scales, Q5_0 weights, the debug partials and the quantizer).  The
reference is the library's own serial result on the same inputs, so the
comparison is bitwise; the oracle parity of each kernel is covered by the
parity tests.  (The no-allocation entry shares one scratch array per device
and is documented as not safe to overlap; it is not called here.)
"""
import concurrent.futures as cf
import sys

import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STREAMS = 4
ROUNDS = 3

# (entry, M, N, K, expected q8_qdot_path or None)
CASES = [
    ("qdot", 1, 4096, 4096, 0),
    ("qdot", 4, 2048, 4096, 0),
    ("qdot", 64, 1024, 4096, 1),
    ("qdot", 16, 14336, 1024, 1),
    ("qdot", 385, 14336, 1024, 2),
    ("qdot", 256, 14336, 1024, 3),
    ("qdot", 300, 2000, 1056, 3),
    ("qmma", 64, 1024, 4096, 1),
    ("q50", 1, 4096, 4096, None),
    ("q50", 520, 2100, 1024, None),
    ("partials", 16, 512, 4096, 1),
    ("quantize", 512, 0, 4096, None),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU concurrency tests need a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def inputs(dev):
    ins = []
    for n, (kind, M, N, K, path) in enumerate(CASES):
        if path is not None:
            assert q8.q8_qdot_path(M, N, K) == path, (kind, M, N, K)
        seed = 9100 + 10 * n
        KB = K // 32
        if kind == "quantize":
            ins.append((torch.from_numpy(synth.random_f32((M, K), seed)).to(dev),))
            continue
        A = torch.from_numpy(synth.random_i8((M, K), seed)).to(dev)
        AS = torch.from_numpy(synth.random_scales((M, KB), seed + 1)).to(dev)
        if kind == "q50":
            W = torch.from_numpy(synth.random_q50(N, K, seed + 2)).to(dev)
        else:
            W = torch.from_numpy(synth.random_i8((N, K), seed + 2)).to(dev)
        WS = torch.from_numpy(synth.random_scales((N, KB), seed + 3)).to(dev)
        if kind == "qmma":
            WS = WS.t().contiguous()
        ins.append((A, AS, W, WS))
    torch.cuda.synchronize()
    return ins


def _outputs(dev):
    outs = []
    for kind, M, N, K, _ in CASES:
        if kind == "quantize":
            outs.append((torch.empty((M, K), dtype=torch.int8, device=dev),
                         torch.empty((M, K // 32), dtype=torch.float32, device=dev)))
        elif kind == "partials":
            outs.append((torch.empty((M, N, K // 32), dtype=torch.int32, device=dev),))
        else:
            outs.append((torch.empty((M, N), dtype=torch.float32, device=dev),))
    return outs


def _call(n, args, out, stream):
    kind = CASES[n][0]
    if kind == "qdot":
        q8.q8_qdot(*args, C=out[0], stream=stream)
    elif kind == "qmma":
        q8.q8_qmma(*args, C=out[0], stream=stream)
    elif kind == "q50":
        q8.q8_q50_qdot(*args, C=out[0], stream=stream)
    elif kind == "partials":
        q8.q8_qdot_partials(args[0], args[2], P=out[0], stream=stream)
    else:
        q8.q8_quantize(args[0], Q=out[0], D=out[1], stream=stream)


def _host(out):
    return [t.cpu().numpy().view(np.uint8) for t in out]


def _reference(dev, inputs):
    outs = _outputs(dev)
    for n in range(len(CASES)):
        _call(n, inputs[n], outs[n], None)
    torch.cuda.synchronize()
    return [_host(o) for o in outs]


def _compare(ref, got, what):
    for n, (r, g) in enumerate(zip(ref, got)):
        for a, b in zip(r, g):
            assert np.array_equal(a, b), "%s: case %s differs from the serial result" % (what, CASES[n][:4])


def test_overlapping_streams_one_thread(dev, inputs):
    _say("[concurrency] %d streams x %d rounds, one host thread" % (STREAMS, ROUNDS))
    ref = _reference(dev, inputs)
    streams = [torch.cuda.Stream() for _ in range(STREAMS)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[_outputs(dev) for _ in range(ROUNDS)] for _ in range(STREAMS)]
    for r in range(ROUNDS):
        for n in range(len(CASES)):
            for k, s in enumerate(streams):
                _call(n, inputs[n], outs[k][r][n], s)
    torch.cuda.synchronize()
    for k in range(STREAMS):
        for r in range(ROUNDS):
            _compare(ref, [_host(o) for o in outs[k][r]], "stream %d round %d" % (k, r))


def test_host_threads_own_streams(dev, inputs):
    _say("[concurrency] %d host threads, one stream each, %d rounds" % (STREAMS, ROUNDS))
    ref = _reference(dev, inputs)
    streams = [torch.cuda.Stream() for _ in range(STREAMS)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [[_outputs(dev) for _ in range(ROUNDS)] for _ in range(STREAMS)]
    torch.cuda.synchronize()

    def work(k):
        # each thread walks the cases in its own order
        order = list(range(len(CASES)))
        order = order[k % len(order):] + order[:k % len(order)]
        for r in range(ROUNDS):
            for n in order:
                _call(n, inputs[n], outs[k][r][n], streams[k])
        return k

    with cf.ThreadPoolExecutor(max_workers=STREAMS) as ex:
        assert sorted(ex.map(work, range(STREAMS))) == list(range(STREAMS))
    torch.cuda.synchronize()
    for k in range(STREAMS):
        for r in range(ROUNDS):
            _compare(ref, [_host(o) for o in outs[k][r]], "thread %d round %d" % (k, r))
