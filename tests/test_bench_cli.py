"""CPU checks of bench.py's command line (no GPU needed): a request for more
than one GPU is refused with a message and a non-zero status, before any
device work; --help lists the workloads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)


def test_help_lists_workloads():
    r = _run("--help")
    assert r.returncode == 0
    assert "--workload" in r.stdout and "--gpus" in r.stdout
