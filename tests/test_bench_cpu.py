"""bench.py's host-side contract, without a GPU: more than one GPU is refused with a
message, and the host description beside the oracle timing is readable."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_host_cpu_description():
    sys.path.insert(0, ROOT)
    import bench
    model, ncpu = bench.host_cpu()
    assert isinstance(model, str) and model
    assert ncpu is None or ncpu >= 1
