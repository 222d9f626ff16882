"""Ahead-of-time build of ``libq8qdot.so`` for gfx950 with hipcc.

Every HIP source is compiled separately (in parallel) and linked into one
shared library next to this file.  No JIT and no torch extension machinery:
the library is a plain C-ABI .so that the binding loads with ctypes.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libq8qdot.so")

SOURCES = ("q8qdot_api.hip", "matvec.hip", "matvec_q50.hip", "qgemm.hip",
           "qgemm_ksplit.hip", "qgemm_splitk.hip", "quantize.hip")
ARCH = "gfx950"

# Packed-FP32 VALU forms are disabled for every device pass; hipcc's host
# pass warns that it does not know the feature, which is harmless.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs (the f32 epilogue reads them with plain VALU ops,
    # no v_accvgpr_read per element).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(REPO, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (need ROCm with gfx950 support)")


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + ["-D" + d for d in defines] + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, out: str = LIB_PATH, defines=()) -> str:
    """Compile every source and link the library; returns its path.

    ``defines`` (``NAME=VALUE`` strings) override the kernels' compile-time
    launch-shape knobs; ``out`` places such a variant elsewhere.
    """
    build_dir = BUILD_DIR if out == LIB_PATH else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
