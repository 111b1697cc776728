import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes on the host)")


def pytest_terminal_summary(terminalreporter):
    """Distribution of the output errors the GPU parity tests measured."""
    mod = sys.modules.get("gpu_helpers")
    if mod is None:
        return
    for dtype, vals in mod.REL_ERRORS.items():
        if vals:
            v = sorted(vals)
            terminalreporter.write_line(
                f"[parity] {dtype}: {len(v)} outputs, max|err|/max|y_ref| median {v[len(v) // 2]:.2e}, "
                f"max {v[-1]:.2e} (tolerance {mod.TOL[dtype]:.0e})")
