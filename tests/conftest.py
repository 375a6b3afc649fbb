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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C ABI")
    config.addinivalue_line("markers", "slow: multi-GB full-size workload")


def pytest_terminal_summary(terminalreporter):
    """Print the parity statistics the GPU tests recorded (code mismatch
    counts and window ratios, worst scale / dequant / attention errors), so
    they appear even in a quiet run."""
    mod = sys.modules.get("parity")
    if mod is None or not getattr(mod, "REPORT", None):
        return
    terminalreporter.write_sep("-", "parity statistics")
    for label, stats in mod.REPORT:
        terminalreporter.write_line("%s: %s" % (label, stats))
