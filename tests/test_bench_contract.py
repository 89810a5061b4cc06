"""bench.py's output contract: one JSON line with the metric, throughput,
roofline and CPU-baseline fields, and a clear refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_json_line_fields():
    r = _bench("--steps", "3", "--warmup", "1", "--cpu-seconds", "0.2")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["higher_is_better"] is True
    assert rec["dtype"] == "bf16" and rec["config"]["workload"]
    roof = rec["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < roof["frac"] <= 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = rec["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["sample"]
    assert cpu["cores"] == len(os.sched_getaffinity(0)) and cpu["blas_threads"] >= 1
    cfg = rec["config"]
    assert cfg["algorithmic_bytes"] == cfg["algorithmic_kv_bytes"] + cfg["algorithmic_other_bytes"]
    assert cfg["algorithmic_kv_bytes"] > 0.9 * cfg["algorithmic_bytes"]
    # the oracle's rows agree with the GPU's within the bf16 bound the parity tests use
    assert cpu["max_abs_err_vs_gpu"] < 0.05


@pytest.mark.gpu
def test_windowed_mixed_step_runs():
    """The mixed step under a 1024-token sliding window: the imported
    histories skip the pages the builder does not hold below the window."""
    r = _bench("--window", "1024", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-clock")
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    assert rec["config"]["sliding_window"] == 1024 and rec["value"] > 0


@pytest.mark.gpu
def test_chunk_sweep_covers_every_chunk_of_the_long_prompt():
    """--sweep over the chunk workload times the 20,000-token prompt's 40
    chunks in order (512 tokens each at offsets 0, 512, ..., the last 32)."""
    r = _bench("--workload", "chunk", "--sweep", "--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads([l for l in r.stdout.splitlines() if l.startswith("{")][-1])
    rows = rec["sweep"]["per_step"]
    assert [x["chunk_offset"] for x in rows] == [512 * k for k in range(40)]
    assert [x["chunk_tokens"] for x in rows] == [512] * 39 + [32]
    assert all(x["decodes"] == 0 and x["kernel_us"] > 0 for x in rows)
    assert rec["roofline"]["bound"] == "mfma" and 0 < rec["roofline"]["frac"] <= 1
    assert rec["config"]["steps_swept"] == 40 and rec["value"] > 0


def test_sweep_applies_to_the_long_prompt_workloads_only():
    r = _bench("--workload", "mixed", "--sweep", timeout=300)
    assert r.returncode != 0
    assert "--sweep applies to the long and chunk workloads" in (r.stderr + r.stdout)
