"""bench.py's command-line contract on the CPU: it measures one GPU only, so
a request for more exits at once with a message, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_names_the_workloads():
    r = run("--help")
    assert r.returncode == 0
    for cfg in ("14b", "1.3b", "int4", "sweep"):
        assert cfg in r.stdout
