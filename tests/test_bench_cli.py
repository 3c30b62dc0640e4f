"""bench.py's contract parts that run without a GPU: the one-GPU guard and the CPU oracle
baseline's fields (timed on a tiny batch)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    cfg = W.get_config("llama13b", batch=4, num_blocks=512, steps=2)
    w = W.make_workload(cfg, device="cpu")
    r = bench.cpu_baseline(w, 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["runs"] >= 1
    assert "sequences" in r["sample"]
    # The next step's host side (oracle append, block copies, cache write) on the same sample.
    assert r["append_step"]["seconds"] > 0 and r["append_step"]["tokens_per_s"] > 0
