"""bench.py's output contract: one JSON line with the fields the benchmark
driver reads.  The multi-GPU refusal runs on the host; the short run needs a GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_default_run_is_the_largest_workload(monkeypatch):
    # With no flags the headline is the 70B FFN-down layer at M = 2048 (the
    # largest single-GPU configuration), fused quantization + GEMM.
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.workload == "ffn_down_m2048" and args.gpus == 1
    from w4a8_quantized_gemm_quantize_amd import inputs
    spec = inputs.WORKLOADS[args.workload]
    assert (spec["m"], spec["k"], spec["n"]) == (2048, 28672, 8192)
    assert all(name in inputs.WORKLOADS for name in bench.SUB_WORKLOADS)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.gpu
def test_short_run_prints_the_contract_line():
    print("CASE bench contract (tiny workload, 7 steps)", flush=True)
    r = subprocess.run([sys.executable, "-u", BENCH, "--workload", "tiny", "--steps", "7",
                        "--warmup", "3", "--cpu-seconds", "1", "--no-quantizer",
                        "--no-extensions", "--no-subworkloads"], capture_output=True,
                       text=True, timeout=600,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 7 and d["warmup"] == 3
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"]
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < roof["achieved"] and 0 < roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"])
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
