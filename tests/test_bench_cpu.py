"""Host-side checks of bench.py's contract (no GPU needed): the one-GPU rule and
the roofline arithmetic its JSON line reports."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == 2


def test_roofline_entry_divides_work_by_time():
    e = bench.roofline_entry("hbm", 4.0e9, 1.0, "x", "k")          # 4 GB in 1 ms
    assert e["unit"] == "GB/s" and e["achieved"] == 4000.0 and e["peak"] == bench.PEAK_HBM_GBS
    assert e["frac"] == 0.5 and e["avg_us"] == 1000.0 and e["bound"] == "hbm"
    e = bench.roofline_entry("mfma", 2.0e12, 1.0, "x", "k")        # 2 TFLOP in 1 ms
    assert e["unit"] == "TFLOP/s" and e["achieved"] == 2000.0 and e["peak"] == bench.PEAK_FP4_TFLOPS
    e = bench.roofline_entry("mfma_bf16", 1.25e12, 1.0, "x", "k", {"best_us": 990.0})
    assert e["bound"] == "mfma" and e["peak"] == bench.PEAK_BF16_TFLOPS and e["frac"] == 0.5
    assert e["best_us"] == 990.0
    e = bench.roofline_entry("mfma_fp8", 2.5e12, 1.0, "x", "k")
    assert e["peak"] == bench.PEAK_FP8_TFLOPS and e["frac"] == 0.5
