"""bench.py's command-line contract, on the CPU: more than one GPU is
refused with a message and exit status 2, before any GPU work; the
workload table names the three decode workloads with consistent shapes."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_workload_table():
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.WORKLOADS) == {"batch", "long", "layers"}
    for name, w in bench.WORKLOADS.items():
        assert w["Hq"] % w["Hkv"] == 0 and w["Hq"] // w["Hkv"] in (1, 2, 4, 8), name
        assert w["replicas"] == 1 or w["layers"] == 1, name
    assert bench.WORKLOADS["batch"]["T"] == 32768 and bench.WORKLOADS["batch"]["B"] == 16
