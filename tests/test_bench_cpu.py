"""Host-side checks of bench.py that need no GPU: the one-GPU contract, and
the C++ oracle baseline's bookkeeping on small inputs."""
import json
import os
import subprocess
import sys

import numpy as np

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_reports_rate_threads_and_sample():
    sys.path.insert(0, ROOT)
    import bench

    x = synthetic.normal_bf16((64, 256), 1.0, 9, 0)
    w = synthetic.normal_bf16((96, 256), 0.02, 9, 1)
    res = bench.cpu_baseline([("a", x, w), ("b", x, w)], 0.2)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert res["one_thread"]["cores"] == 1 and res["one_thread"]["value"] > 0
    assert res["numpy_oracle"]["value"] > 0
    json.dumps(res)   # one JSON line


def test_traffic_record_matches_its_kernel_source_or_is_ignored():
    """The committed traffic record carries the SHA-256 of the kernel source it
    was measured with; bench.py reports it only while the source matches."""
    sys.path.insert(0, ROOT)
    import bench

    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_gate_up.json")))
    t = bench.traffic_for_current_kernel()
    assert t is None or t == rec["traffic_bytes_per_launch"]
    assert rec["traffic_bytes_per_launch"] >= rec["algorithmic_bytes_per_launch"] > 0
    assert np.isclose(rec["copy_calibration"]["fetch_factor"], 2.0, rtol=1e-3)
