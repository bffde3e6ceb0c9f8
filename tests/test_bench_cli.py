"""bench.py's command line on the host: the one-GPU rule and the help text
(no GPU needed; both exit before anything touches a device)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        r = run_bench("--gpus", n)
        assert r.returncode == 2, r
        assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""


def test_help_lists_the_workloads():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--config", "--segments"):
        assert flag in r.stdout
