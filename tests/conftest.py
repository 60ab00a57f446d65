import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the host-side libraries if they are missing (CPU-only runs)."""
    need = [os.path.join(ROOT, "oracle", "liboracle.so"),
            os.path.join(ROOT, "synth", "libsynth_host.so")]
    if all(os.path.exists(p) for p in need):
        return
    from oracle import _build as ob
    from synth import _build as sb
    ob.build()
    sb.build()


_ensure_built()
