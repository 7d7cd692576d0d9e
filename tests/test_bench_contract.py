"""bench.py keeps its output contract: one JSON line with the headline metric, a roofline object for the
dominant kernel and the oracle's CPU baseline; more than one GPU is refused with a message."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_roofline_and_cpu_baseline():
    # a child process (run before any cooperative launch of the test process; see conftest.py)
    cmd = [sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--settle-ms", "0", "--cpu-seconds", "0.3",
           "--no-kernels"]
    print("bench child: " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["unit"] == "GB/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "ln_16x64x256x256"
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0


def test_traffic_is_reported_only_for_unchanged_kernel_code(monkeypatch):
    """roofline.traffic comes from the committed counter summary only while the profiled kernels' code is
    the code that was measured: the hash covers the sources with comments and blank lines removed and the
    extra compiler flags of each, so a change to code or flags changes it and a change to comments alone
    does not."""
    from normalization_ln_forward_amd import build, profiling

    def sha(text):
        return profiling.source_sha(["k.hip"], read=lambda name: text)

    base = "__global__ void k(float* y) {\n    y[0] = 1.0f;  // one\n}\n"
    assert sha(base) == sha("// a kernel\n__global__ void k(float* y) {\n    y[0] = 1.0f;\n}\n\n")
    assert sha(base) == sha("/* a\n   kernel */\n__global__ void k(float* y) {   \n    y[0] = 1.0f; /* x */\n}\n")
    assert sha(base) != sha("__global__ void k(float* y) {\n    y[0] = 2.0f;\n}\n")
    assert sha(base) != sha("__global__ void k(float* y) {\n    y[1] = 1.0f;\n}\n")
    plain = sha(base)
    monkeypatch.setitem(build.EXTRA_FLAGS, "k.hip", ["-mllvm", "-some-option"])
    assert sha(base) != plain
