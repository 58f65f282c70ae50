import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# The mutation test re-runs the oracle pins against a deliberately broken copy
# of the oracle placed on this path (CPU only).
_MUT = os.environ.get("PD_ORACLE_MUTANT_DIR")
if _MUT:
    sys.path.insert(0, _MUT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
