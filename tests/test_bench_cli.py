"""bench.py on the CPU: more than one GPU is refused with a message and a
non-zero status, the counter summariser reduces a rocprofv3 counter CSV to
per-kernel means, and the roofline takes the bound (HBM bytes or MFMA FLOPs)
that a launch's work needs longest for."""
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


def test_roofline_bound_choice():
    """The roofline of a launch is the bound that takes longer at the MI355X
    peaks: the matrix cores for the long causal workload, HBM for ten queries
    against 4096 keys over 800 heads (841 MB of Q, K, V, O and lse)."""
    sys.path.insert(0, ROOT)
    import bench
    from tiled_attention_04_amd import synth
    c5 = synth.WORKLOADS["c5"]
    r = bench.roofline(c5, "c5", 1, [3.8, 3.9, 4.0], bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["achieved"] - c5.flops() / 3.9e-3 / 1e12) < 1e-3
    assert abs(r["frac"] - r["achieved"] / bench.PEAK_BF16_TFLOPS) < 1e-4
    h800 = synth.EXTRA_WORKLOADS["short10_h800"]
    nbytes = 800 * ((2 * 10 + 2 * 4096) * 64 * 2 + 4 * 10)
    assert bench.algorithmic_bytes(h800) == nbytes
    r = bench.roofline(h800, "short10_h800", 1, [0.2, 0.2], bench.PEAK_BF16_TFLOPS)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert abs(r["achieved"] - nbytes / 0.2e-3 / 1e9) < 1e-2
    assert r["algorithmic_bytes"] == nbytes
