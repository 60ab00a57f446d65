"""The kernels' other paths, forced on every parity case.

The reduce-scatter, discrete reduce-scatter, all-reduce and all-gather choose
between 16-byte (quad) access and element-by-element folds or copies from
their inputs' alignment, and the ring-order reduce-scatters choose one-slice
tiles for launches too small to fill the GPU and for the shapes that stream
faster so (bf16 input at K = 8, bf16 -> fp32 above K = 8, when the partitions
are overwritten), and four-slice tiles otherwise.
ZR_FORCE_PATH overrides those choices (read once per process, so each
setting runs the whole bit-exact parity module, and the module of ranks in
different phases, in a child process):

  element  every aligned case also goes element by element (with ZR_DEBUG=1,
           so every call waits for its stream and reports a kernel error
           itself);
  large    small launches, and the one-slice shapes above, take four-slice tiles;
  small    large launches take one-slice tiles.

Ring-order results do not depend on the path, so every case must still be
bit-exact against the oracle.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("env", [{"ZR_FORCE_PATH": "element", "ZR_DEBUG": "1"},
                                 {"ZR_FORCE_PATH": "large"},
                                 {"ZR_FORCE_PATH": "small"}],
                         ids=["element_debug", "large", "small"])
def test_parity_on_forced_paths(env):
    cmd = [sys.executable, "-u", "-m", "pytest", os.path.join(ROOT, "tests", "test_gpu_parity.py"),
           os.path.join(ROOT, "tests", "test_gpu_mixed_phases.py"),
           "-x", "-q", "-m", "gpu", "-p", "no:cacheprovider", "--timeout", "300",
           "--timeout-method", "thread"]
    print(f"forced path: running the parity module with {env}", flush=True)
    r = subprocess.run(cmd, env=dict(os.environ, **env), cwd=ROOT, capture_output=True, text=True,
                       timeout=900)
    tail = r.stdout[-2500:] + r.stderr[-1500:]
    print(tail, flush=True)
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout
    assert "libzr:" not in r.stderr  # the setting was understood
