"""bench.py's command line, on the host: a request for more than one GPU
is refused with a message and exit status 2 before any device work, since
the library has no multi-GPU path; the workload list names every
workload."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_every_workload_is_listed_in_the_module_docstring():
    sys.path.insert(0, ROOT)
    import bench
    for name in bench.WORKLOADS:
        assert re.search(rf"\n  {name}( \(default\))?\n", bench.__doc__), name
