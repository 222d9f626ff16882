"""GPU: bench.py's JSON line carries every field of its reporting contract.

A short run in this process (few steps, the headline workload only, a
one-second oracle sample): the line must name the metric and its unit, the
one-GPU throughput, the timing window, the workload, the roofline of the
dominant kernel (HBM-bound, with the algorithmic bytes it is computed from)
and the CPU oracle baseline with its core count, and the figures must agree
with one another.
"""
import json
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def test_bench_json_contract(capsys, monkeypatch):
    assert torch.cuda.is_available(), "the bench needs a visible gfx950 GPU"
    import bench
    print("[bench-contract] short bench run", file=sys.stderr, flush=True)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "5", "--warmup", "2", "--second", "-1",
                                      "--others", "", "--no-variants", "--cpu-seconds", "1"])
    bench.main()
    out = capsys.readouterr().out.strip().split("\n")
    rec = json.loads(out[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 5 and rec["warmup"] == 2
    assert rec["unit"] == "GB/s" and rec["higher_is_better"] is True
    assert rec["vs_baseline"] is None
    cfg = rec["config"]
    assert cfg["workload"] == "q8_matvec_m1_n14336_k4096"
    assert (cfg["M"], cfg["N"], cfg["K"]) == (1, 14336, 4096)
    assert cfg["kernel"] == "matvec"
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # achieved = the algorithmic bytes of one launch over its mean duration
    bytes_ = roof["algorithmic_bytes_per_launch"]
    assert bytes_ == 14336 * 4096 + 14336 * 128 * 4 + 4096 + 128 * 4 + 14336 * 4
    assert abs(roof["achieved"] - bytes_ / (rec["ms_per_step"] * 1e-3) / 1e9) < 0.01 * roof["achieved"]
    # value = weight bytes per second of the same window
    weights = 14336 * 4096 + 14336 * 128 * 4
    assert abs(rec["value"] - weights / (rec["ms_per_step"] * 1e-3) / 1e9) < 0.01 * rec["value"]
    cpu = rec["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
