"""Every kernel launches one block per tile up to a grid cap (2^30 blocks,
reached only by multi-terabyte inputs), and beyond it the blocks stride over
the tiles. A child process with the cap lowered to 13 blocks (ZR_MAX_GRID,
read once when the library loads, so it needs a process of its own) runs the
whole bit-exact parity module, which checks the strided loops of the
reduce-scatter, discrete reduce-scatter, all-reduce, all-gather and flatten
kernels against the oracle on every parity case.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu


def test_parity_with_blocks_striding_over_tiles():
    env = dict(os.environ, ZR_MAX_GRID="13")
    cmd = [sys.executable, "-u", "-m", "pytest", os.path.join(ROOT, "tests", "test_gpu_parity.py"),
           "-x", "-q", "-m", "gpu", "-p", "no:cacheprovider", "--timeout", "300",
           "--timeout-method", "thread"]
    print("strided grid: running the parity module with ZR_MAX_GRID=13", flush=True)
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = r.stdout[-2500:] + r.stderr[-1500:]
    print(tail, flush=True)
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout
