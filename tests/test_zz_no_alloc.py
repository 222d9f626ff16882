"""GPU: the no-allocation entry (q8_qdot_noalloc) against the workspace entry.

q8_qdot_noalloc is q8_qdot_ws with the library's static scratch array as the
workspace: for the same shape it runs the same kernel with the same split,
so its output must equal q8_qdot_ws's bit for bit, and both must meet the
oracle's bar (``|C - out64| <= 1e-5 * sum_b |AS*WS*P| + 1e-6``).  Two calls
in a row, the second on a smaller input, check that the shared array's
counters come back to zero between calls; a shape that does not split runs
the plain entry.  Calls go through the C-ABI on raw device addresses.
"""
import numpy as np
import pytest

import gemm_q8_qdot_amd as q8
import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "needs a visible gfx950 GPU"
    q8.ensure_built()
    q8.load()
    return torch.device("cuda:0")


def _case(M, N, K, seed, dev):
    A = synth.random_i8((M, K), seed)
    W = synth.random_i8((N, K), seed + 1)
    AS = synth.random_scales((M, K // 32), seed + 2, 1e-3, 10.0)
    WS = synth.random_scales((N, K // 32), seed + 3, 1e-4, 1.0)
    host = (A, AS, W, WS)
    return host, tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in host)


def _run(entry, t, M, N, K, dev, ws=None):
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream().cuda_stream
    ptrs = [x.data_ptr() for x in t] + [C.data_ptr()]
    if ws is None:
        st = entry(*ptrs, M, N, K, sp)
    else:
        st = entry(*ptrs, M, N, K, ws.data_ptr(), ws.numel(), sp)
    assert st == q8.Q8_OK, q8.q8_strerror(st)
    return C


@pytest.mark.parametrize("shapes", [
    [(32, 4096, 14336), (40, 1000, 8320)],    # both split, the second smaller
    [(64, 2048, 8192), (8, 64, 8192)],
    [(64, 4096, 4096), (16, 300, 8192)],      # a plain shape, then a split one
])
def test_noalloc_matches_workspace_entry(dev, shapes):
    for k, (M, N, K) in enumerate(shapes):
        print("[noalloc] call %d: M=%d N=%d K=%d split bytes %d"
              % (k, M, N, K, q8.q8_qdot_ws_size(M, N, K)), flush=True)
        host, t = _case(M, N, K, 4100 + 7 * k + M, dev)
        ws = q8.workspace(M, N, K, dev)
        C0 = _run(q8.q8_qdot_noalloc_raw, t, M, N, K, dev)
        C1 = _run(q8.q8_qdot_ws_raw, t, M, N, K, dev, ws)
        torch.cuda.synchronize()
        assert torch.equal(C0.view(torch.int32), C1.view(torch.int32)), "call %d differs" % k
        out, mag = oracle.qdot_f64(*host)
        assert oracle.within_tolerance(C0.cpu().numpy(), out, mag).all(), "call %d vs oracle" % k
