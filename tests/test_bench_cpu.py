"""bench.py's host-side contract, without a GPU: it measures one GPU and says
so for any other count, and its workload table carries the five benchmark
configurations at their sizes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single MI355X" in r.stderr and r.stdout == ""


def test_workload_sizes():
    sys.path.insert(0, ROOT)
    import synth
    w = synth.WORKLOADS
    assert (w["c1_plain"].M, w["c1_plain"].N, w["c1_plain"].K) == (256, 256, 256)
    assert (w["c2_plain"].M, w["c2_plain"].N, w["c2_plain"].K) == (1024, 1024, 1024)
    assert (w["c3_gelu"].M, w["c3_gelu"].N, w["c3_gelu"].K, w["c3_gelu"].act) == (4096, 4096, 4096, "gelu")
    assert (w["c4_relu"].M, w["c4_relu"].N, w["c4_relu"].K) == (3000, 5120, 1000)
    assert w["c4_sigmoid"].act == "sigmoid"
    c5 = w["c5_gelu"]
    assert (c5.M, c5.N, c5.K, c5.dtype, c5.act) == (16384, 14336, 4096, "bf16", "gelu")
