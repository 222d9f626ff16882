"""Host-side checks of bench.py (no GPU needed).

The benchmark measures one GPU: asked for more it must exit with a message
before touching a device.  The counter record it reports as ``traffic`` is
tied to the kernel sources it was taken on.
"""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_record_is_tied_to_kernel_sources(tmp_path, monkeypatch):
    # a record whose source hash does not match the current kernel source is
    # stale: reported as None, never as a number
    rec = {"q8_fake_workload": {"kernel_source_sha": "0" * 16, "fetch_bytes_per_launch": 10,
                                "write_bytes_per_launch": 5}}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    csrc = tmp_path / "gemm_q8_qdot_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("matvec.hip", "q8_device.h"):
        with open(os.path.join(ROOT, "gemm_q8_qdot_amd", "csrc", name), "rb") as f:
            (csrc / name).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("q8_fake_workload", "matvec.hip") is None
    rec["q8_fake_workload"]["kernel_source_sha"] = bench.kernel_source_sha("matvec.hip")
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("q8_fake_workload", "matvec.hip") == 15
    assert bench.measured_traffic("q8_other", "matvec.hip") is None
