"""bench.py's JSON line on a GPU, for a small workload: every field of the
contract, the roofline object and the CPU-oracle baseline."""
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_json_line_fields():
    say("bench.py --workload c1_gelu --steps 5 --warmup 2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "c1_gelu",
                        "--steps", "5", "--warmup", "2"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    out = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in out, k
    assert out["n_gpus"] == 1 and out["steps"] == 5 and out["warmup"] == 2
    assert out["value"] > 0 and out["unit"] == "TFLOP/s" and out["higher_is_better"] is True
    assert out["config"]["workload"].startswith("c1_gelu")
    rl = out["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2516.6
    assert 0 < rl["frac"] < 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > 0
    cb = out["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
