"""bench.py's command line on the CPU: more than one GPU is refused with a
message and a non-zero status, and the counter summariser reduces a
rocprofv3 counter CSV to per-kernel means."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr
    assert res.stdout == ""


def test_counter_summary_means(tmp_path):
    d = tmp_path / "pmc" / "node"
    d.mkdir(parents=True)
    rows = ["Kernel_Name,Counter_Name,Counter_Value",
            "kA,FETCH_SIZE,100", "kA,FETCH_SIZE,300", "kB,FETCH_SIZE,7", "kA,WRITE_SIZE,5"]
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-pmc",
                          str(tmp_path / "pmc")], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = json.loads(res.stdout)
    assert out["kA"]["FETCH_SIZE"] == {"mean": 200.0, "samples": 2}
    assert out["kB"]["FETCH_SIZE"]["mean"] == 7.0
    assert out["kA"]["WRITE_SIZE"]["samples"] == 1
