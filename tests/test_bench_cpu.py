"""Host-side checks of bench.py's command line (no GPU is touched): a run on
more than one GPU is refused with a message, and a non-positive step count is
an argument error."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*argv):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                          cwd=ROOT, capture_output=True, text=True, timeout=120)


def test_bench_refuses_several_gpus():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""   # no JSON line for a refused run


def test_bench_rejects_zero_steps():
    r = _bench("--steps", "0", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "--steps must be at least 1" in r.stderr
