"""bench.py's command line on the host: a run on more than one GPU is refused
with a message (the convolution runs on one MI355X) before anything touches a
GPU, and --help lists the workloads and operators."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_workloads_and_operators():
    r = _bench("--help")
    assert r.returncode == 0
    for word in ("--config", "--op", "mole", "grid", "s2act", "--envelope", "--heads", "--cpu-edges"):
        assert word in r.stdout
