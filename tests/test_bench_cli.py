"""bench.py's command line on the CPU: more than one GPU is refused with a
message (this build measures a single GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_stage_argument_checked():
    from io_aware_exact_03_amd import _lib
    lib = _lib.load()
    A = 4096
    args = [A] * 10 + [1, 1, 8, 64, 1.0, 0, 2, None]
    assert lib.fa_bwd_stage(0, *args) == 1
    assert lib.fa_bwd_stage(4, *args) == 1
