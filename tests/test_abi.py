"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function ``include/q8qdot.h`` declares,
and reject bad arguments with the documented status before anything is
enqueued.  Only validation paths are called here: each returns before any HIP
runtime call, so no device is touched.
"""
import os
import re

import pytest

import gemm_q8_qdot_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8qdot.h")


@pytest.fixture(scope="module")
def lib():
    q8.ensure_built()
    return q8.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(q8.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def _declared_status_values():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef enum\s*\{(.*?)\}\s*q8_status;", text, flags=re.S).group(1)
    return {k: int(v) for k, v in re.findall(r"\b(Q8_[A-Z]+)\s*=\s*(-?\d+)", body)}


def test_status_values():
    # The five codes of the boundary contract keep their fixed values (a
    # caller written against it reads -4 as a launch failure); the range
    # error is this library's addition and takes the next free value.
    vals = _declared_status_values()
    assert vals == {"Q8_OK": 0, "Q8_EINVAL": -1, "Q8_ENULL": -2, "Q8_EALIGN": -3,
                    "Q8_ELAUNCH": -4, "Q8_ERANGE": -5}
    for name, v in vals.items():
        assert getattr(q8, name) == v, name


def test_version_and_strerror(lib):
    assert q8.q8_version() >= 100
    for st in (0, -1, -2, -3, -4, -5):
        assert q8.q8_strerror(st) and q8.q8_strerror(st) != "unknown status"
    assert q8.q8_strerror(7) == "unknown status"


def test_path_dispatch(lib):
    assert q8.q8_qdot_path(1, 4096, 4096) == 0
    assert q8.q8_qdot_path(7, 4096, 4096) == 0
    assert q8.q8_qdot_path(8, 4096, 4096) == 1
    assert q8.q8_qdot_path(64, 4096, 4096) == 1
    assert q8.q8_qdot_path(512, 14336, 4096) == 2
    assert q8.q8_qdot_path(385, 14336, 96) == 2
    assert q8.q8_qdot_path(129, 14336, 96) == 3   # below the staged GEMM's rule
    assert q8.q8_qdot_path(128, 449, 512) == 1
    # many 32 x 32 tiles but too few 128 x 224 ones: 64 x 64 tiles over all of K
    # (on a 256-compute-unit part: 896 against 224 tiles, 4 rounds against 1)
    assert q8.q8_qdot_path(512, 1792, 4096) == 3
    assert q8.q8_qdot_path(256, 4096, 1024) == 3
    assert q8.q8_qdot_path(128, 4096, 4096) == 1     # 512 against 128 tiles: 2 rounds against 1
    assert q8.q8_qdot_path(16, 40000, 4096) == 1     # 64-row tiles would be three quarters empty
    assert lib.q8_qdot_path(1, 1, 33) == q8.Q8_EINVAL
    assert lib.q8_qdot_path(-1, 1, 32) == q8.Q8_EINVAL


def test_q50_path_dispatch(lib):
    # Q5_0 weights: matvec below 8 rows (K <= 16384), the ring GEMM where the
    # Q8_0 dispatch is the staged or the ring GEMM, its 64 x 64 tiles outnumber
    # the compute units and K/32 is a multiple of 4, else the K-split GEMM
    assert q8.q8_q50_path(1, 14336, 4096) == 0
    assert q8.q8_q50_path(7, 4096, 16384) == 0
    assert q8.q8_q50_path(3, 4096, 16416) == 1        # rows over 16 KiB: one row per grid row
    assert q8.q8_q50_path(64, 4096, 4096) == 1
    assert q8.q8_q50_path(512, 14336, 4096) == 3      # staged for Q8_0
    assert q8.q8_q50_path(512, 4096, 4096) == 3
    assert q8.q8_q50_path(512, 1792, 4096) == 1       # one round of 64 x 64 tiles
    assert q8.q8_q50_path(520, 2100, 1056) == 1       # K/32 = 33
    assert lib.q8_q50_path(1, 1, 33) == q8.Q8_EINVAL
    rng = __import__("numpy").random.default_rng(4243)
    for _ in range(2000):
        M = int(rng.integers(1, 3000))
        N = int(rng.integers(1, 60000))
        K = 32 * int(rng.integers(1, 600))
        want = _expected_path(M, N, K)
        if M <= 7:
            want = 0 if K <= 16384 and N * (K // 32) * 20 < 2 ** 31 - 1 - 2 ** 20 else 1
        else:
            t64 = -(-M // 64) * -(-N // 64)
            want = 3 if want >= 2 and (K // 32) % 4 == 0 and t64 > 256 else 1
        assert q8.q8_q50_path(M, N, K) == want, (M, N, K)


BAD_SHAPES = [(1, 1, 31), (1, 1, -32), (-1, 4, 32), (4, -1, 32), (2, 2, 48)]


@pytest.mark.parametrize("M,N,K", BAD_SHAPES)
def test_bad_shapes_rejected(lib, M, N, K):
    assert q8.q8_qdot_raw(16, 16, 16, 16, 16, M, N, K) == q8.Q8_EINVAL
    assert lib.q8_qdot(16, 16, 16, 16, 16, M, N, K) == q8.Q8_EINVAL
    assert q8.q8_qdot_partials_raw(16, 16, 16, M, N, K) == q8.Q8_EINVAL
    assert q8.q8_qmma_raw(16, 16, 16, 16, 16, M, N, K) == q8.Q8_EINVAL


def test_null_pointers_rejected(lib):
    ok = 4096
    for args in [(0, ok, ok, ok, ok), (ok, 0, ok, ok, ok), (ok, ok, 0, ok, ok),
                 (ok, ok, ok, 0, ok), (ok, ok, ok, ok, 0)]:
        assert q8.q8_qdot_raw(*args, 1, 64, 64) == q8.Q8_ENULL
        assert q8.q8_qdot_raw(*args, 64, 64, 64) == q8.Q8_ENULL
        assert q8.q8_qmma_raw(*args, 1, 64, 64) == q8.Q8_ENULL
        assert q8.q8_qmma_raw(*args, 64, 64, 64) == q8.Q8_ENULL
    assert q8.q8_qdot_partials_raw(0, ok, ok, 8, 8, 64) == q8.Q8_ENULL
    assert q8.q8_qdot_partials_raw(ok, 0, ok, 8, 8, 64) == q8.Q8_ENULL
    assert q8.q8_qdot_partials_raw(ok, ok, 0, 8, 8, 64) == q8.Q8_ENULL
    # K == 0 needs only C
    assert q8.q8_qdot_raw(0, 0, 0, 0, 0, 2, 2, 0) == q8.Q8_ENULL
    assert q8.q8_quantize_raw(0, ok, ok, 1, 32) == q8.Q8_ENULL
    assert q8.q8_quantize_raw(ok, 0, ok, 1, 32) == q8.Q8_ENULL
    assert q8.q8_quantize_raw(ok, ok, 0, 1, 32) == q8.Q8_ENULL


def test_misaligned_pointers_rejected(lib):
    base = 1 << 20
    # A or W off a 16-byte boundary
    assert q8.q8_qdot_raw(base + 8, base, base, base, base, 1, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qdot_raw(base, base, base + 4, base, base, 64, 4, 32) == q8.Q8_EALIGN
    # f32 arrays off a 4-byte boundary
    assert q8.q8_qdot_raw(base, base + 2, base, base, base, 1, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qdot_raw(base, base, base, base + 1, base, 1, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qmma_raw(base, base, base, base + 2, base, 9, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qmma_raw(base + 4, base, base, base, base, 9, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qdot_raw(base, base, base, base, base + 3, 9, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qdot_partials_raw(base, base, base + 2, 9, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_qdot_partials_raw(base + 1, base, base, 9, 4, 32) == q8.Q8_EALIGN
    assert q8.q8_quantize_raw(base + 4, base, base, 1, 32) == q8.Q8_EALIGN
    assert q8.q8_quantize_raw(base, base + 8, base, 1, 32) == q8.Q8_EALIGN
    assert q8.q8_quantize_raw(base, base, base + 2, 1, 32) == q8.Q8_EALIGN


def test_empty_outputs_are_noops(lib):
    # M == 0 or N == 0: nothing launched, pointers not inspected
    assert q8.q8_qdot_raw(0, 0, 0, 0, 0, 0, 5, 64) == q8.Q8_OK
    assert q8.q8_qdot_raw(0, 0, 0, 0, 0, 5, 0, 64) == q8.Q8_OK
    assert q8.q8_qmma_raw(0, 0, 0, 0, 0, 0, 5, 64) == q8.Q8_OK
    assert q8.q8_qdot_partials_raw(0, 0, 0, 0, 3, 64) == q8.Q8_OK
    assert q8.q8_qdot_partials_raw(0, 0, 0, 3, 3, 0) == q8.Q8_OK
    assert q8.q8_quantize_raw(0, 0, 0, 0, 64) == q8.Q8_OK
    assert q8.q8_quantize_raw(0, 0, 0, 4, 0) == q8.Q8_OK
    assert q8.q8_quantize_raw(0, 0, 0, 1, 33) == q8.Q8_EINVAL


def test_q50_validation(lib):
    ok = 4096
    base = 1 << 20
    for ws_t in (False, True):
        # bad shapes, nulls, alignment (W5 needs 4 bytes, A 16)
        assert q8.q8_q50_qdot_raw(16, 16, 16, 16, 16, 2, 2, 48, ws_t=ws_t) == q8.Q8_EINVAL
        assert q8.q8_q50_qdot_raw(0, ok, ok, ok, ok, 1, 64, 64, ws_t=ws_t) == q8.Q8_ENULL
        assert q8.q8_q50_qdot_raw(ok, ok, 0, ok, ok, 9, 64, 64, ws_t=ws_t) == q8.Q8_ENULL
        assert q8.q8_q50_qdot_raw(base, base, base + 2, base, base, 1, 4, 32, ws_t=ws_t) == q8.Q8_EALIGN
        assert q8.q8_q50_qdot_raw(base + 4, base, base, base, base, 9, 4, 32, ws_t=ws_t) == q8.Q8_EALIGN
        assert q8.q8_q50_qdot_raw(0, 0, 0, 0, 0, 0, 4, 32, ws_t=ws_t) == q8.Q8_OK
    assert q8.q8_q50_partials_raw(16, 16, 0, 8, 8, 64) == q8.Q8_ENULL
    assert q8.q8_q50_partials_raw(base, base + 1, base, 8, 8, 64) == q8.Q8_EALIGN
    assert q8.q8_q50_partials_raw(0, 0, 0, 3, 3, 0) == q8.Q8_OK
    # the GEMM path addresses tiles with 32-bit offsets
    assert q8.q8_q50_qdot_raw(16, 16, 16, 16, 16, 8, 4, 2**26) == q8.Q8_ERANGE


def test_range_overflow_rejected(lib):
    big = 2**31 - 32
    assert q8.q8_qdot_partials_raw(16, 16, 16, big, big, big) == q8.Q8_ERANGE
    # the block GEMMs (M >= 8) need 32 * K < 2^31; the matvec does not
    huge_k = 2**26
    assert q8.q8_qdot_raw(16, 16, 16, 16, 16, 8, 4, huge_k) == q8.Q8_ERANGE
    assert q8.q8_qdot_partials_raw(16, 16, 16, 8, 4, huge_k) == q8.Q8_ERANGE
    # qmma_t with M >= 8 addresses the transposed scales with 32-bit offsets
    assert q8.q8_qmma_raw(16, 16, 16, 16, 16, 8, 2**20, 2**15) == q8.Q8_ERANGE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        q8.load(str(tmp_path / "missing.so"))


C_PROGRAM = r"""
#include <stdio.h>
#include "q8qdot.h"

int main(void) {
    int8_t dummy[32];
    printf("version %d\n", q8_version());
    printf("path %d %d %d %d\n", q8_qdot_path(1, 4096, 4096), q8_qdot_path(64, 4096, 4096),
           q8_qdot_path(512, 14336, 4096), q8_qdot_path(1, 1, 33));
    printf("einval %d\n", q8_qdot(dummy, 0, dummy, 0, 0, 1, 1, 33));
    printf("enull %d\n", q8_qdot_stream(0, 0, 0, 0, 0, 1, 1, 32, 0));
    printf("ealign %d\n", q8_qdot_partials(dummy + 1, dummy, (int32_t *)0 + 1, 1, 1, 32, 0));
    printf("empty %d\n", q8_quantize(0, 0, 0, 0, 32, 0));
    printf("strerror %s\n", q8_strerror(Q8_ELAUNCH));
    return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path, lib):
    # The header is plain C (C99, no C++): a C program includes it, links
    # the library and reaches the host-side validation of several entries.
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(q8.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L" + libdir, "-l:" + os.path.basename(q8.LIB_PATH),
           "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().split("\n"))
    assert int(out["version"]) == q8.q8_version()
    assert out["path"].split() == ["0", "1", "2", str(q8.Q8_EINVAL)]
    assert int(out["einval"]) == q8.Q8_EINVAL
    assert int(out["enull"]) == q8.Q8_ENULL
    assert int(out["ealign"]) == q8.Q8_EALIGN
    assert int(out["empty"]) == q8.Q8_OK
    assert out["strerror"] == q8.q8_strerror(q8.Q8_ELAUNCH)


def _expected_path(M, N, K, cus=256):
    """The documented dispatch for Q8_0 weights (header, q8_qdot_path), restated."""
    if M <= 7:
        return 0
    staged_tiles = -(-M // 128) * -(-N // 224)
    t32 = -(-M // 32) * -(-N // 32)
    t64 = -(-M // 64) * -(-N // 64)
    ring_ok = K * 64 <= 2 ** 31 - 1 and t64 <= 0x7FFFFFFF
    if M >= 128 and staged_tiles >= 128 and K * 224 < 2 ** 31:
        # the ring kernel where it has at most 4.1 tiles per unit per staged round
        return 3 if ring_ok and 10 * t64 <= 41 * cus * -(-staged_tiles // cus) else 2
    if ring_ok and 100 * -(-t32 // cus) > 245 * -(-t64 // cus):
        return 3
    return 1


def test_path_dispatch_rule_over_many_shapes(lib):
    # The dispatch query follows one rule for every shape (on this host the
    # library assumes 256 compute units: no device is visible).
    rng = __import__("numpy").random.default_rng(4242)
    for _ in range(4000):
        M = int(rng.integers(1, 3000))
        N = int(rng.integers(1, 60000))
        K = 32 * int(rng.integers(1, 2000))
        assert q8.q8_qdot_path(M, N, K) == _expected_path(M, N, K), (M, N, K)
