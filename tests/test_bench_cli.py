"""bench.py's command line on the CPU: the one-GPU guard and the help text."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_modes():
    r = _bench("--help")
    assert r.returncode == 0
    for flag in ("--workload", "--context", "--op", "--eager", "--partition", "--copy-calibration"):
        assert flag in r.stdout
