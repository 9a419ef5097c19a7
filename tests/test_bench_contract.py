"""The benchmark's output contract: one JSON line with the fields the
measurement reports (metric, value, unit, steps, warm-ups, roofline of the
dominant kernel, the CPU oracle baseline), and a refusal of more than one GPU.
The GPU case runs bench.py in a child process with few steps."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = _run(["--gpus", "2"], timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert not any(ln.startswith("{") for ln in r.stdout.splitlines())


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_one_json_line_with_the_contract_fields():
    r = _run(["--steps", "3", "--warmup", "1", "--cpu-rows", "64", "--sparse-density", "0"], timeout=540)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    line = json.loads(lines[0])
    for key, kind in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)]:
        assert isinstance(line[key], kind), (key, line.get(key))
    assert "vs_baseline" in line
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["warmup"] == 1
    assert line["unit"] == "TFLOP/s" and line["dtype"] == "bf16" and line["higher_is_better"] is True
    assert line["config"]["workload"] == "t2i_2048"
    assert abs(line["value"] - 3.508e12 / (line["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * line["value"]
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2516.6
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert line["check"]["bf16"]["within_spec"] and line["check"]["fp8"]["within_spec"]
    assert line["sustained"]["value"] > 0 and line["mfma_ceiling"]["bf16"]["tflops"] > 0
