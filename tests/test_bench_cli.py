"""bench.py command line, host side: it refuses more than one GPU with a
message and exit status 2 before touching a device, and --help lists the
workloads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workloads():
    r = _bench("--help")
    assert r.returncode == 0, r.stderr
    for cfg in ("1024sq", "mixed", "2048sq", "train65k", "edit1024", "edit_mixed"):
        assert cfg in r.stdout
