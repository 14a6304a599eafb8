"""bench.py's command line on the CPU: a request for several GPUs exits with a
message before anything touches a device, and --help describes the run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_several_gpus_exit_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_help_names_the_workload():
    r = _run("--help")
    assert r.returncode == 0
    assert "T = 65,536" in r.stdout and "--steps" in r.stdout
